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


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has {t.dim()}")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _workspace(nbytes, ws, device):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


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
    if packed is None:
        packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    ws, nbytes = _workspace(bitlinear_pack_workspace_bytes(N, K), ws, W.device)
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
    if packed is None:
        packed = torch.empty((B, N, K // 4), dtype=torch.uint8, device=W.device)
    if gamma is None:
        gamma = torch.empty(B, dtype=torch.float32, device=W.device)
    ws, nbytes = _workspace(bitlinear_pack_batched_workspace_bytes(B, N, K), ws, W.device)
    _check(lib().bitlinear_pack_weights_batched(_ptr(W), B, N, K, _ptr(packed), _ptr(gamma), _ptr(ws), nbytes,
                                                _stream(stream)))
    return packed, gamma


def bitlinear_unpack_weights(packed, K, w=None, stream=None):
    """packed uint8 [N, K/4] -> int8 [N, K] (code - 1 per weight)."""
    _dev(packed, "packed", (torch.uint8,), 2)
    N = packed.shape[0]
    if w is None:
        w = torch.empty((N, K), dtype=torch.int8, device=packed.device)
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
    _dev(gamma, "gamma", (torch.float32,))
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K or rms_weight.shape[0] != K:
        raise ValueError("x, rms_weight and packed disagree on K")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    ws, nbytes = _workspace(bitlinear_forward_workspace_bytes(M, N, K), ws, x.device)
    _check(lib().bitlinear_forward_ex(_ptr(x), _ptr(rms_weight), _ptr(packed), _ptr(gamma), M, N, K,
                                      float(eps), _ptr(y), _ptr(ws), nbytes, _stream(stream),
                                      int(kernel)))
    return y


def bitlinear_prepare_activations(x, rms_weight, eps=1e-6, N=0, ws=None, stream=None):
    """Quantise x [M, K] into a workspace (returned) for bitlinear_forward_prepared."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_weight, "rms_weight", (torch.float32,), 1)
    M, K = x.shape
    ws, nbytes = _workspace(bitlinear_forward_workspace_bytes(M, N, K), ws, x.device)
    _check(lib().bitlinear_prepare_activations(_ptr(x), _ptr(rms_weight), M, K, float(eps), _ptr(ws),
                                               nbytes, _stream(stream)))
    return ws


def bitlinear_forward_prepared(ws, packed, gamma, M, y=None, stream=None,
                               kernel=BITLINEAR_KERNEL_AUTO):
    """Ternary product + rescale from a prepared workspace -> y fp32 [M, N]."""
    _dev(packed, "packed", (torch.uint8,), 2)
    _dev(gamma, "gamma", (torch.float32,))
    N, K = packed.shape[0], packed.shape[1] * 4
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=packed.device)
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
    _dev(gamma, "gamma", (torch.float32,), 1)
    B, M, K = x.shape
    N = packed.shape[1]
    if packed.shape[0] != B or rms_weight.shape != (B, K) or gamma.shape[0] != B:
        raise ValueError("batch dimensions disagree")
    if packed.shape[2] * 4 != K:
        raise ValueError("x and packed disagree on K")
    if y is None:
        y = torch.empty((B, M, N), dtype=torch.float32, device=x.device)
    ws, nbytes = _workspace(bitlinear_forward_batched_workspace_bytes(B, M, N, K), ws, x.device)
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
    _dev(gamma_gu, "gamma_gu", (torch.float32,))
    _dev(rms_w_down, "rms_w_down", (torch.float32,), 1)
    _dev(packed_down, "packed_down", (torch.uint8,), 2)
    _dev(gamma_down, "gamma_down", (torch.float32,))
    M, D = x.shape
    F = packed_down.shape[1] * 4
    if packed_gu.shape != (2 * F, D // 4) or packed_down.shape[0] != D:
        raise ValueError("GLU matrix shapes disagree with x")
    if y is None:
        y = torch.empty((M, D), dtype=torch.float32, device=x.device)
    ws, nbytes = _workspace(bitlinear_glu_workspace_bytes(M, D, F), ws, x.device)
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
    _dev(gamma_gu, "gamma_gu", (torch.float32,), 1)
    _dev(rms_w_down, "rms_w_down", (torch.float32,), 2)
    _dev(packed_down, "packed_down", (torch.uint8,), 3)
    _dev(gamma_down, "gamma_down", (torch.float32,), 1)
    B, M, D = x.shape
    F = packed_down.shape[2] * 4
    if (packed_gu.shape != (B, 2 * F, D // 4) or packed_down.shape[:2] != (B, D)
            or rms_w_gu.shape != (B, D) or rms_w_down.shape != (B, F)
            or gamma_gu.shape != (B,) or gamma_down.shape != (B,)):
        raise ValueError("batched GLU shapes disagree with x")
    if y is None:
        y = torch.empty((B, M, D), dtype=torch.float32, device=x.device)
    ws, nbytes = _workspace(bitlinear_glu_batched_workspace_bytes(B, M, D, F), ws, x.device)
    _check(lib().bitlinear_glu_forward_batched(_ptr(x), _ptr(rms_w_gu), _ptr(packed_gu), _ptr(gamma_gu),
                                               _ptr(rms_w_down), _ptr(packed_down), _ptr(gamma_down), B,
                                               M, D, F, float(eps), _ptr(y), _ptr(ws), nbytes,
                                               _stream(stream)))
    return y


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
    _dev(gamma, "gamma", (torch.float32,), 1)
    _dev(dy, "dy", (torch.float32,), 2)
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K or dy.shape != (M, N) or rms_weight.shape != (K,):
        raise ValueError("backward shapes disagree with x")
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.float32, device=x.device)
    if dg is None:
        dg = torch.empty(K, dtype=torch.float32, device=x.device)
    if dW is None:
        dW = torch.empty((N, K), dtype=torch.float32, device=x.device)
    ws, nbytes = _workspace(bitlinear_backward_workspace_bytes(M, N, K), ws, x.device)
    _check(lib().bitlinear_backward(_ptr(x), _ptr(rms_weight), _ptr(packed), _ptr(gamma), _ptr(dy), M, N, K,
                                    float(eps), _ptr(dx), _ptr(dg), _ptr(dW), _ptr(ws), nbytes,
                                    _stream(stream)))
    return dx, dg, dW


def bitlinear_glu_hidden(x, rms_w_gu, packed_gu, gamma_gu, eps=1e-6, h=None, ws=None, stream=None,
                         kernel=BITLINEAR_KERNEL_AUTO):
    """First half of the mixer: h = bf16(SiLU(gate) * up) as int16 bits [M, F]."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_w_gu, "rms_w_gu", (torch.float32,), 1)
    _dev(packed_gu, "packed_gu", (torch.uint8,), 2)
    _dev(gamma_gu, "gamma_gu", (torch.float32,))
    M, D = x.shape
    F = packed_gu.shape[0] // 2
    if h is None:
        h = torch.empty((M, F), dtype=torch.int16, device=x.device)
    ws, nbytes = _workspace(bitlinear_forward_workspace_bytes(M, 2 * F, D), ws, x.device)
    _check(lib().bitlinear_glu_hidden(_ptr(x), _ptr(rms_w_gu), _ptr(packed_gu), _ptr(gamma_gu), M, D,
                                      F, float(eps), _ptr(h), _ptr(ws), nbytes, _stream(stream),
                                      int(kernel)))
    return h


# --------------------------------------------------------------------------
# stages
# --------------------------------------------------------------------------

def bitlinear_quantize(x, rms_weight, eps=1e-6, q=None, s=None, stream=None):
    """RMSNorm + absmax int8: x [M, K] -> (q int8 [M, K], s fp32 [M])."""
    _dev(x, "x", _BF16, 2)
    _dev(rms_weight, "rms_weight", (torch.float32,), 1)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s is None:
        s = torch.empty(M, dtype=torch.float32, device=x.device)
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
    if acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=q.device)
    ws, nbytes = _workspace(bitlinear_forward_workspace_bytes(M, N, K), ws, q.device)
    _check(lib().bitlinear_ternary_matmul_i32(_ptr(q), _ptr(packed), M, N, K, _ptr(acc), _ptr(ws),
                                              nbytes, _stream(stream), int(kernel)))
    return acc
