"""Python binding of libbitlinear.so, the fused BitLinear layer for MI355X.

Thin marshalling layer: each function checks tensor dtypes, devices and
shapes, allocates outputs and workspace with PyTorch when the caller does
not pass them, and calls the C entry point of the same name on the current
HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no CPU or PyTorch fallback, and importing a function
raises if the library has not been built (run __graft_entry__.build() or
`python bitlinear_layer_amd/build.py`).

Tensor conventions (see include/bitlinear.h for the full contract):
  x, h        bf16 [M, K] (torch.bfloat16, or int16/uint16 bit patterns)
  rms_weight  fp32 [K]
  W           fp32 [N, K]            packed   uint8 [N, K/4]
  gamma       fp32 [1] (device)      y        fp32 [M, N]
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

BITLINEAR_OK = 0
BITLINEAR_ERR_INVALID_ARG = 1
BITLINEAR_ERR_WORKSPACE = 2
BITLINEAR_ERR_UNSUPPORTED = 3
BITLINEAR_ERR_HIP = 4

BITLINEAR_KERNEL_AUTO = 0
BITLINEAR_KERNEL_GEMV = 1
BITLINEAR_KERNEL_MFMA = 2
BITLINEAR_KERNEL_DECODE = 3

_P = ctypes.c_void_p
_I = ctypes.c_int64
_F = ctypes.c_float
_S = ctypes.c_size_t
_INT = ctypes.c_int

_SIGNATURES = {
    "bitlinear_abi_version": (_INT, []),
    "bitlinear_decode_supported": (_INT, [_I, _I]),
    "bitlinear_last_error": (ctypes.c_char_p, []),
    "bitlinear_packed_bytes": (_S, [_I, _I]),
    "bitlinear_pack_workspace_bytes": (_S, [_I, _I]),
    "bitlinear_pack_weights": (_INT, [_P, _I, _I, _P, _P, _P, _S, _P]),
    "bitlinear_pack_batched_workspace_bytes": (_S, [_I, _I, _I]),
    "bitlinear_pack_weights_batched": (_INT, [_P, _I, _I, _I, _P, _P, _P, _S, _P]),
    "bitlinear_unpack_weights": (_INT, [_P, _I, _I, _P, _P]),
    "bitlinear_forward_workspace_bytes": (_S, [_I, _I, _I]),
    "bitlinear_forward": (_INT, [_P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _S, _P]),
    "bitlinear_forward_ex": (_INT, [_P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _S, _P, _INT]),
    "bitlinear_forward_noalloc": (_INT, [_P, _P, _P, _P, _I, _I, _I, _F, _P, _P]),
    "bitlinear_prepare_activations": (_INT, [_P, _P, _I, _I, _F, _P, _S, _P]),
    "bitlinear_forward_prepared": (_INT, [_P, _P, _I, _I, _I, _P, _P, _S, _P, _INT]),
    "bitlinear_forward_batched_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "bitlinear_forward_batched": (_INT, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _S, _P]),
    "bitlinear_glu_workspace_bytes": (_S, [_I, _I, _I]),
    "bitlinear_glu_forward": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _S, _P]),
    "bitlinear_glu_batched_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "bitlinear_glu_forward_batched": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _S,
                                             _P]),
    "bitlinear_glu_hidden": (_INT, [_P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _S, _P, _INT]),
    "bitlinear_quantize": (_INT, [_P, _P, _I, _I, _F, _P, _P, _P]),
    "bitlinear_ternary_matmul_i32": (_INT, [_P, _P, _I, _I, _I, _P, _P, _S, _P, _INT]),
    "bitlinear_mlgru_scan_workspace_bytes": (_S, [_I, _I, _I]),
    "bitlinear_mlgru_scan": (_INT, [_P, _I, _I, _I, _P, _P, _P, _S, _P]),
    "bitlinear_mlgru_workspace_bytes": (_S, [_I, _I, _I]),
    "bitlinear_mlgru_forward": (_INT, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _S, _P]),
    "bitlinear_layer_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "bitlinear_layer_forward": (_INT, [_P] * 13 + [_I, _I, _I, _I, _F, _P, _P, _P, _S, _P]),
    "bitlinear_backward_workspace_bytes": (_S, [_I, _I, _I]),
    "bitlinear_backward": (_INT, [_P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _P, _S, _P]),
}

_lib = None


class BitlinearError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"bitlinear status {status}: {message}")
        self.status = status


def lib():
    """The loaded libbitlinear.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def exported_symbols():
    return list(_SIGNATURES)


def bitlinear_abi_version():
    return lib().bitlinear_abi_version()


def bitlinear_decode_supported(M, K):
    return bool(lib().bitlinear_decode_supported(M, K))


def bitlinear_last_error():
    return lib().bitlinear_last_error().decode()


def _check(status):
    if status != BITLINEAR_OK:
        raise BitlinearError(status, bitlinear_last_error())


# The raw handle of the current device's current stream.  torch's internal
# hook returns it without building a Stream object (which costs a few
# microseconds per call); the public call is the fallback.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_current_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    """The stream handle for the C ABI (an int; ctypes passes it as void*):
    the given stream, or the current stream of the current device."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and _current_device is not None:
        return _raw_stream(_current_device())
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    """A tensor's device address as an int (ctypes passes it as void*)."""
    return None if t is None else t.data_ptr()


def _dev(t, name, dtypes, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has {t.dim()}")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _out(t, name, dtypes, shape, like):
    """Check a caller-supplied output (or allocate nothing: returns t).

    Outputs reach the kernels as raw pointers, so each is checked before any
    call: dtype, exact shape, contiguity, then that it lives on the same GPU
    as the input `like`.  The checks run in that order, so the shape and
    dtype rejections are testable with CPU tensors."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda or t.get_device() != like.get_device():
        raise ValueError(f"{name} must be on {like.device}, is on {t.device}")
    return t


def _new_or_out(t, name, dtype, shape, like, dtypes=None):
    """A fresh output tensor on like's device, or the caller's, checked."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    return _out(t, name, dtypes or (dtype,), shape, like)


def _workspace(nbytes, ws, like):
    """Workspace of at least nbytes (the library checks the size): a fresh
    byte tensor, or the caller's, which must be a contiguous tensor on like's
    GPU."""
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    else:
        _out(ws, "ws", (ws.dtype,), tuple(ws.shape), like)
    return ws, ws.numel() * ws.element_size()


def _scalar(t, name, n=1):
    """A device fp32 vector of exactly n values (gamma)."""
    _dev(t, name, (torch.float32,))
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} value(s), holds {t.numel()}")
    return t


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

def bitlinear_packed_bytes(N, K):
    return lib().bitlinear_packed_bytes(N, K)


def bitlinear_pack_workspace_bytes(N, K):
    return lib().bitlinear_pack_workspace_bytes(N, K)


def bitlinear_pack_weights(W, packed=None, gamma=None, ws=None, stream=None):
    """fp32 W [N, K] -> (packed uint8 [N, K/4], gamma fp32 [1])."""
    _dev(W, "W", (torch.float32,), 2)
    N, K = W.shape
    packed = _new_or_out(packed, "packed", torch.uint8, (N, K // 4), W)
    gamma = _new_or_out(gamma, "gamma", torch.float32, (1,), W)
    ws, nbytes = _workspace(bitlinear_pack_workspace_bytes(N, K), ws, W)
    _check(lib().bitlinear_pack_weights(_ptr(W), N, K, _ptr(packed), _ptr(gamma), _ptr(ws), nbytes,
                                        _stream(stream)))
    return packed, gamma


def bitlinear_pack_batched_workspace_bytes(B, N, K):
    return lib().bitlinear_pack_batched_workspace_bytes(B, N, K)


def bitlinear_pack_weights_batched(W, packed=None, gamma=None, ws=None, stream=None):
    """fp32 W [B, N, K] -> (packed uint8 [B, N, K/4], gamma fp32 [B]), one
    gamma per matrix."""
    _dev(W, "W", (torch.float32,), 3)
    B, N, K = W.shape
    packed = _new_or_out(packed, "packed", torch.uint8, (B, N, K // 4), W)
    gamma = _new_or_out(gamma, "gamma", torch.float32, (B,), W)
    ws, nbytes = _workspace(bitlinear_pack_batched_workspace_bytes(B, N, K), ws, W)
    _check(lib().bitlinear_pack_weights_batched(_ptr(W), B, N, K, _ptr(packed), _ptr(gamma), _ptr(ws), nbytes,
                                                _stream(stream)))
    return packed, gamma


def bitlinear_unpack_weights(packed, K, w=None, stream=None):
    """packed uint8 [N, K/4] -> int8 [N, K] (code - 1 per weight)."""
    _dev(packed, "packed", (torch.uint8,), 2)
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError("packed does not hold K/4 bytes per row")
    w = _new_or_out(w, "w", torch.int8, (N, K), packed)
    _check(lib().bitlinear_unpack_weights(_ptr(packed), N, K, _ptr(w), _stream(stream)))
    return w


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------

def bitlinear_forward_workspace_bytes(M, N, K):
    return lib().bitlinear_forward_workspace_bytes(M, N, K)


def bitlinear_forward(x, rms_weight, packed, gamma, eps=1e-6, y=None, ws=None, stream=None,
                      kernel=BITLINEAR_KERNEL_AUTO):
    """bf16 x [M, K] -> fp32 y [M, N] through the packed ternary matrix."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_weight, "rms_weight", (torch.float32,), 1)
    _dev(packed, "packed", (torch.uint8,), 2)
    _scalar(gamma, "gamma")
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K or rms_weight.shape[0] != K:
        raise ValueError("x, rms_weight and packed disagree on K")
    y = _new_or_out(y, "y", torch.float32, (M, N), x)
    ws, nbytes = _workspace(bitlinear_forward_workspace_bytes(M, N, K), ws, x)
    _check(lib().bitlinear_forward_ex(_ptr(x), _ptr(rms_weight), _ptr(packed), _ptr(gamma), M, N, K,
                                      float(eps), _ptr(y), _ptr(ws), nbytes, _stream(stream),
                                      int(kernel)))
    return y


def bitlinear_forward_noalloc(x, rms_weight, packed, gamma, y, eps=1e-6, stream=None):
    """bitlinear_forward without a workspace or any allocation: the caller
    passes y fp32 [M, N]; the library's per-GPU scratch holds the activation
    stage (at most BITLINEAR_NOALLOC_SCRATCH_BYTES)."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_weight, "rms_weight", (torch.float32,), 1)
    _dev(packed, "packed", (torch.uint8,), 2)
    _scalar(gamma, "gamma")
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K or rms_weight.shape[0] != K:
        raise ValueError("x, rms_weight and packed disagree on K")
    _out(y, "y", (torch.float32,), (M, N), x)
    _check(lib().bitlinear_forward_noalloc(_ptr(x), _ptr(rms_weight), _ptr(packed), _ptr(gamma), M, N, K,
                                           float(eps), _ptr(y), _stream(stream)))
    return y


def bitlinear_prepare_activations(x, rms_weight, eps=1e-6, N=0, ws=None, stream=None):
    """Quantise x [M, K] into a workspace (returned) for bitlinear_forward_prepared."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_weight, "rms_weight", (torch.float32,), 1)
    M, K = x.shape
    if rms_weight.shape[0] != K:
        raise ValueError("x and rms_weight disagree on K")
    ws, nbytes = _workspace(bitlinear_forward_workspace_bytes(M, N, K), ws, x)
    _check(lib().bitlinear_prepare_activations(_ptr(x), _ptr(rms_weight), M, K, float(eps), _ptr(ws),
                                               nbytes, _stream(stream)))
    return ws


def bitlinear_forward_prepared(ws, packed, gamma, M, y=None, stream=None,
                               kernel=BITLINEAR_KERNEL_AUTO):
    """Ternary product + rescale from a prepared workspace -> y fp32 [M, N]."""
    _dev(packed, "packed", (torch.uint8,), 2)
    _scalar(gamma, "gamma")
    N, K = packed.shape[0], packed.shape[1] * 4
    y = _new_or_out(y, "y", torch.float32, (M, N), packed)
    if ws is not None:
        _out(ws, "ws", (ws.dtype,), tuple(ws.shape), packed)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().bitlinear_forward_prepared(_ptr(packed), _ptr(gamma), M, N, K, _ptr(y), _ptr(ws),
                                            nbytes, _stream(stream), int(kernel)))
    return y


def bitlinear_forward_batched_workspace_bytes(B, M, N, K):
    return lib().bitlinear_forward_batched_workspace_bytes(B, M, N, K)


def bitlinear_forward_batched(x, rms_weight, packed, gamma, eps=1e-6, y=None, ws=None, stream=None):
    """B independent layers: x [B, M, K], rms_weight [B, K], packed [B, N, K/4],
    gamma [B] -> y [B, M, N]."""
    _dev(x, "x", _BF16, 3)
    _dev(rms_weight, "rms_weight", (torch.float32,), 2)
    _dev(packed, "packed", (torch.uint8,), 3)
    B, M, K = x.shape
    _scalar(gamma, "gamma", B)
    N = packed.shape[1]
    if packed.shape[0] != B or tuple(rms_weight.shape) != (B, K):
        raise ValueError("batch dimensions disagree")
    if packed.shape[2] * 4 != K:
        raise ValueError("x and packed disagree on K")
    y = _new_or_out(y, "y", torch.float32, (B, M, N), x)
    ws, nbytes = _workspace(bitlinear_forward_batched_workspace_bytes(B, M, N, K), ws, x)
    _check(lib().bitlinear_forward_batched(_ptr(x), _ptr(rms_weight), _ptr(packed), _ptr(gamma), B, M,
                                           N, K, float(eps), _ptr(y), _ptr(ws), nbytes,
                                           _stream(stream)))
    return y


# --------------------------------------------------------------------------
# GLU channel mixer
# --------------------------------------------------------------------------

def bitlinear_glu_workspace_bytes(M, D, F):
    return lib().bitlinear_glu_workspace_bytes(M, D, F)


def bitlinear_glu_forward(x, rms_w_gu, packed_gu, gamma_gu, rms_w_down, packed_down, gamma_down,
                          eps=1e-6, y=None, ws=None, stream=None):
    """x [M, D] -> y [M, D]: fused gate|up BitLinear (packed_gu [2F, D/4]),
    SiLU(gate) * up as bf16, down BitLinear (packed_down [D, F/4])."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_w_gu, "rms_w_gu", (torch.float32,), 1)
    _dev(packed_gu, "packed_gu", (torch.uint8,), 2)
    _scalar(gamma_gu, "gamma_gu")
    _dev(rms_w_down, "rms_w_down", (torch.float32,), 1)
    _dev(packed_down, "packed_down", (torch.uint8,), 2)
    _scalar(gamma_down, "gamma_down")
    M, D = x.shape
    F = packed_down.shape[1] * 4
    if (tuple(packed_gu.shape) != (2 * F, D // 4) or packed_down.shape[0] != D
            or rms_w_gu.shape[0] != D or rms_w_down.shape[0] != F):
        raise ValueError("GLU matrix shapes disagree with x")
    y = _new_or_out(y, "y", torch.float32, (M, D), x)
    ws, nbytes = _workspace(bitlinear_glu_workspace_bytes(M, D, F), ws, x)
    _check(lib().bitlinear_glu_forward(_ptr(x), _ptr(rms_w_gu), _ptr(packed_gu), _ptr(gamma_gu),
                                       _ptr(rms_w_down), _ptr(packed_down), _ptr(gamma_down), M, D, F,
                                       float(eps), _ptr(y), _ptr(ws), nbytes, _stream(stream)))
    return y


def bitlinear_glu_batched_workspace_bytes(B, M, D, F):
    return lib().bitlinear_glu_batched_workspace_bytes(B, M, D, F)


def bitlinear_glu_forward_batched(x, rms_w_gu, packed_gu, gamma_gu, rms_w_down, packed_down, gamma_down,
                                  eps=1e-6, y=None, ws=None, stream=None):
    """B independent mixers: x [B, M, D], rms_w_gu [B, D], packed_gu [B, 2F, D/4],
    gamma_gu [B], rms_w_down [B, F], packed_down [B, D, F/4], gamma_down [B]
    -> y [B, M, D]."""
    _dev(x, "x", _BF16, 3)
    _dev(rms_w_gu, "rms_w_gu", (torch.float32,), 2)
    _dev(packed_gu, "packed_gu", (torch.uint8,), 3)
    _dev(rms_w_down, "rms_w_down", (torch.float32,), 2)
    _dev(packed_down, "packed_down", (torch.uint8,), 3)
    B, M, D = x.shape
    _scalar(gamma_gu, "gamma_gu", B)
    _scalar(gamma_down, "gamma_down", B)
    F = packed_down.shape[2] * 4
    if (tuple(packed_gu.shape) != (B, 2 * F, D // 4) or tuple(packed_down.shape[:2]) != (B, D)
            or tuple(rms_w_gu.shape) != (B, D) or tuple(rms_w_down.shape) != (B, F)):
        raise ValueError("batched GLU shapes disagree with x")
    y = _new_or_out(y, "y", torch.float32, (B, M, D), x)
    ws, nbytes = _workspace(bitlinear_glu_batched_workspace_bytes(B, M, D, F), ws, x)
    _check(lib().bitlinear_glu_forward_batched(_ptr(x), _ptr(rms_w_gu), _ptr(packed_gu), _ptr(gamma_gu),
                                               _ptr(rms_w_down), _ptr(packed_down), _ptr(gamma_down), B,
                                               M, D, F, float(eps), _ptr(y), _ptr(ws), nbytes,
                                               _stream(stream)))
    return y


def bitlinear_glu_hidden(x, rms_w_gu, packed_gu, gamma_gu, eps=1e-6, h=None, ws=None, stream=None,
                         kernel=BITLINEAR_KERNEL_AUTO):
    """First half of the mixer: h = bf16(SiLU(gate) * up) as int16 bits [M, F]."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_w_gu, "rms_w_gu", (torch.float32,), 1)
    _dev(packed_gu, "packed_gu", (torch.uint8,), 2)
    _scalar(gamma_gu, "gamma_gu")
    M, D = x.shape
    F = packed_gu.shape[0] // 2
    if packed_gu.shape[0] != 2 * F or packed_gu.shape[1] * 4 != D or rms_w_gu.shape[0] != D:
        raise ValueError("GLU gate|up shapes disagree with x")
    h = _new_or_out(h, "h", torch.int16, (M, F), x, _BF16)
    ws, nbytes = _workspace(bitlinear_forward_workspace_bytes(M, 2 * F, D), ws, x)
    _check(lib().bitlinear_glu_hidden(_ptr(x), _ptr(rms_w_gu), _ptr(packed_gu), _ptr(gamma_gu), M, D,
                                      F, float(eps), _ptr(h), _ptr(ws), nbytes, _stream(stream),
                                      int(kernel)))
    return h


# --------------------------------------------------------------------------
# MLGRU token mixer and one layer
# --------------------------------------------------------------------------

def bitlinear_mlgru_scan_workspace_bytes(B, T, d):
    return lib().bitlinear_mlgru_scan_workspace_bytes(B, T, d)


def bitlinear_mlgru_scan(z, state, p=None, ws=None, stream=None):
    """The recurrence from pre-activations z fp32 [B, T, 3d]: returns p bf16
    (int16 bits) [B, T, d]; state fp32 [B, d] is updated in place (h_0 in,
    h_T out)."""
    _dev(z, "z", (torch.float32,), 3)
    B, T, d3 = z.shape
    d = d3 // 3
    if d3 != 3 * d:
        raise ValueError("z must hold 3d pre-activations per token")
    _out(state, "state", (torch.float32,), (B, d), z)
    p = _new_or_out(p, "p", torch.int16, (B, T, d), z, _BF16)
    ws, nbytes = _workspace(bitlinear_mlgru_scan_workspace_bytes(B, T, d), ws, z)
    _check(lib().bitlinear_mlgru_scan(_ptr(z), B, T, d, _ptr(state), _ptr(p), _ptr(ws), nbytes,
                                      _stream(stream)))
    return p


def bitlinear_mlgru_workspace_bytes(B, T, d):
    return lib().bitlinear_mlgru_workspace_bytes(B, T, d)


def _mlgru_weights(d, rms_w_in, packed_in, gamma_in, rms_w_out, packed_out, gamma_out):
    _dev(rms_w_in, "rms_w_in", (torch.float32,), 1)
    _dev(packed_in, "packed_in", (torch.uint8,), 2)
    _scalar(gamma_in, "gamma_in")
    _dev(rms_w_out, "rms_w_out", (torch.float32,), 1)
    _dev(packed_out, "packed_out", (torch.uint8,), 2)
    _scalar(gamma_out, "gamma_out")
    if (tuple(packed_in.shape) != (3 * d, d // 4) or tuple(packed_out.shape) != (d, d // 4)
            or rms_w_in.shape[0] != d or rms_w_out.shape[0] != d):
        raise ValueError("MLGRU matrix shapes disagree with x")


def bitlinear_mlgru_forward(x, rms_w_in, packed_in, gamma_in, rms_w_out, packed_out, gamma_out, state,
                            eps=1e-6, y=None, ws=None, stream=None):
    """Token mixer: x bf16 [B, T, d] -> y fp32 [B, T, d]; packed_in [3d, d/4]
    (rows f | c | g), packed_out [d, d/4]; state fp32 [B, d] updated in
    place (h_0 in, h_T out)."""
    _dev(x, "x", _BF16, 3)
    B, T, d = x.shape
    _mlgru_weights(d, rms_w_in, packed_in, gamma_in, rms_w_out, packed_out, gamma_out)
    _out(state, "state", (torch.float32,), (B, d), x)
    y = _new_or_out(y, "y", torch.float32, (B, T, d), x)
    ws, nbytes = _workspace(bitlinear_mlgru_workspace_bytes(B, T, d), ws, x)
    _check(lib().bitlinear_mlgru_forward(_ptr(x), _ptr(rms_w_in), _ptr(packed_in), _ptr(gamma_in),
                                         _ptr(rms_w_out), _ptr(packed_out), _ptr(gamma_out), B, T, d,
                                         float(eps), _ptr(state), _ptr(y), _ptr(ws), nbytes, _stream(stream)))
    return y


def bitlinear_layer_workspace_bytes(B, T, d, F):
    return lib().bitlinear_layer_workspace_bytes(B, T, d, F)


def bitlinear_layer_forward(x, mlgru_w, glu_w, state, eps=1e-6, out=None, ws=None, stream=None):
    """One layer, u = bf16(x + MLGRU(x)), out = bf16(u + GLU(u)): x bf16
    [B, T, d] -> out bf16 (int16 bits) [B, T, d].  mlgru_w = (rms_w_in,
    packed_in, gamma_in, rms_w_out, packed_out, gamma_out); glu_w = (rms_w_gu,
    packed_gu, gamma_gu, rms_w_down, packed_down, gamma_down); state fp32
    [B, d] updated in place."""
    _dev(x, "x", _BF16, 3)
    B, T, d = x.shape
    _mlgru_weights(d, *mlgru_w)
    rms_w_gu, packed_gu, gamma_gu, rms_w_down, packed_down, gamma_down = glu_w
    _dev(rms_w_gu, "rms_w_gu", (torch.float32,), 1)
    _dev(packed_gu, "packed_gu", (torch.uint8,), 2)
    _scalar(gamma_gu, "gamma_gu")
    _dev(rms_w_down, "rms_w_down", (torch.float32,), 1)
    _dev(packed_down, "packed_down", (torch.uint8,), 2)
    _scalar(gamma_down, "gamma_down")
    F = packed_down.shape[1] * 4
    if (tuple(packed_gu.shape) != (2 * F, d // 4) or packed_down.shape[0] != d
            or rms_w_gu.shape[0] != d or rms_w_down.shape[0] != F):
        raise ValueError("GLU matrix shapes disagree with x")
    _out(state, "state", (torch.float32,), (B, d), x)
    out = _new_or_out(out, "out", torch.int16, (B, T, d), x, _BF16)
    ws, nbytes = _workspace(bitlinear_layer_workspace_bytes(B, T, d, F), ws, x)
    _check(lib().bitlinear_layer_forward(_ptr(x), *[_ptr(t) for t in mlgru_w], *[_ptr(t) for t in glu_w],
                                         B, T, d, F, float(eps), _ptr(state), _ptr(out), _ptr(ws), nbytes,
                                         _stream(stream)))
    return out


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------

def bitlinear_backward_workspace_bytes(M, N, K):
    return lib().bitlinear_backward_workspace_bytes(M, N, K)


def bitlinear_backward(x, rms_weight, packed, gamma, dy, eps=1e-6, dx=None, dg=None, dW=None, ws=None,
                       stream=None):
    """Straight-through backward: x bf16 [M, K], rms_weight [K], packed
    [N, K/4], gamma [1], dy fp32 [M, N] -> (dx [M, K], dg [K], dW [N, K]),
    all fp32."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_weight, "rms_weight", (torch.float32,), 1)
    _dev(packed, "packed", (torch.uint8,), 2)
    _scalar(gamma, "gamma")
    _dev(dy, "dy", (torch.float32,), 2)
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K or tuple(dy.shape) != (M, N) or tuple(rms_weight.shape) != (K,):
        raise ValueError("backward shapes disagree with x")
    dx = _new_or_out(dx, "dx", torch.float32, (M, K), x)
    dg = _new_or_out(dg, "dg", torch.float32, (K,), x)
    dW = _new_or_out(dW, "dW", torch.float32, (N, K), x)
    ws, nbytes = _workspace(bitlinear_backward_workspace_bytes(M, N, K), ws, x)
    _check(lib().bitlinear_backward(_ptr(x), _ptr(rms_weight), _ptr(packed), _ptr(gamma), _ptr(dy), M, N, K,
                                    float(eps), _ptr(dx), _ptr(dg), _ptr(dW), _ptr(ws), nbytes,
                                    _stream(stream)))
    return dx, dg, dW


# --------------------------------------------------------------------------
# stages
# --------------------------------------------------------------------------

def bitlinear_quantize(x, rms_weight, eps=1e-6, q=None, s=None, stream=None):
    """RMSNorm + absmax int8: x [M, K] -> (q int8 [M, K], s fp32 [M])."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_weight, "rms_weight", (torch.float32,), 1)
    M, K = x.shape
    if rms_weight.shape[0] != K:
        raise ValueError("x and rms_weight disagree on K")
    q = _new_or_out(q, "q", torch.int8, (M, K), x)
    s = _new_or_out(s, "s", torch.float32, (M,), x)
    _check(lib().bitlinear_quantize(_ptr(x), _ptr(rms_weight), M, K, float(eps), _ptr(q), _ptr(s),
                                    _stream(stream)))
    return q, s


def bitlinear_ternary_matmul_i32(q, packed, acc=None, ws=None, stream=None,
                                 kernel=BITLINEAR_KERNEL_AUTO):
    """int8 q [M, K] x packed [N, K/4] -> int32 acc [M, N]."""
    _dev(q, "q", (torch.int8,), 2)
    _dev(packed, "packed", (torch.uint8,), 2)
    M, K = q.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError("q and packed disagree on K")
    acc = _new_or_out(acc, "acc", torch.int32, (M, N), q)
    ws, nbytes = _workspace(bitlinear_forward_workspace_bytes(M, N, K), ws, q)
    _check(lib().bitlinear_ternary_matmul_i32(_ptr(q), _ptr(packed), M, N, K, _ptr(acc), _ptr(ws),
                                              nbytes, _stream(stream), int(kernel)))
    return acc
