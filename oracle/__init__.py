"""NumPy front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY.  The oracle is the plain CPU definition of the
BitLinear forward pass that the HIP library is checked against.  Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the library never does.  The functions here only marshal NumPy
arrays into the C routines; all arithmetic is in oracle.c.

Every function of the oracle is pinned by CPU tests against closed forms,
invariants, brute force and the quantisation error bound; none is left
"parity unpinned".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int64
_F = ctypes.c_float

_SIGS = {
    "orc_absmean_gamma": (_F, [_P, _I, _I]),
    "orc_ternarize": (None, [_P, _I, _I, _F, _P]),
    "orc_pack": (ctypes.c_int, [_P, _I, _I, _P]),
    "orc_unpack": (ctypes.c_int, [_P, _I, _I, _P]),
    "orc_bf16_to_float": (_F, [ctypes.c_uint16]),
    "orc_double_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
    "orc_rmsnorm_quant": (None, [_P, _P, _I, _I, _F, _P, _P]),
    "orc_ternary_accumulate": (None, [_P, _P, _I, _I, _I, _P]),
    "orc_rescale": (None, [_P, _F, _P, _I, _I, _P]),
    "orc_bitlinear": (None, [_P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P]),
    "orc_bitlinear_ternary": (None, [_P, _P, _P, _F, _I, _I, _I, _F, _P, _P, _P, _P]),
    "orc_glu": (None, [_P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P]),
    "orc_glu_ternary": (None, [_P, _P, _P, _F, _P, _P, _F, _I, _I, _I, _F, _P, _P]),
    "orc_bitlinear_backward": (None, [_P, _P, _P, _F, _P, _I, _I, _I, _F, _P, _P, _P]),
    "orc_mlgru_scan": (None, [_P, _I, _I, _I, _P, _P]),
    "orc_mlgru_ternary": (None, [_P, _P, _P, _F, _P, _P, _F, _I, _I, _I, _F, _P, _P, _P]),
    "orc_mlgru": (None, [_P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P]),
    "orc_lm_layer_ternary": (None, [_P, _P, _P, _F, _P, _P, _F, _P, _P, _F, _P, _P, _F, _I, _I, _I, _I,
                                    _F, _P, _P, _P]),
}


def lib(path: str = None):
    """Load (once) and return the oracle's shared library."""
    global _lib
    if path is not None:
        return _load(path)
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = _load(_LIB_PATH)
    return _lib


def _load(path):
    h = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    return h


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """Wrapper bound to one loaded copy of the library (tests may load a
    deliberately altered build to check that the pins catch it)."""

    def __init__(self, handle=None):
        self.h = handle if handle is not None else lib()

    # weights ---------------------------------------------------------------
    def gamma(self, W):
        W = _c(W, np.float32)
        return np.float32(self.h.orc_absmean_gamma(_ptr(W), W.shape[0], W.shape[1]))

    def ternarize(self, W, gamma):
        W = _c(W, np.float32)
        w = np.empty(W.shape, np.int8)
        self.h.orc_ternarize(_ptr(W), W.shape[0], W.shape[1], float(gamma), _ptr(w))
        return w

    def pack(self, w):
        w = _c(w, np.int8)
        N, K = w.shape
        out = np.empty((N, K // 4), np.uint8)
        if self.h.orc_pack(_ptr(w), N, K, _ptr(out)) != 0:
            raise ValueError("orc_pack: K must be a multiple of 16 and w in {-1,0,1}")
        return out

    def unpack(self, packed, K):
        packed = _c(packed, np.uint8)
        N = packed.shape[0]
        w = np.empty((N, K), np.int8)
        if self.h.orc_unpack(_ptr(packed), N, K, _ptr(w)) != 0:
            raise ValueError("orc_unpack: bad K or unused code 3")
        return w

    # bf16 ------------------------------------------------------------------
    def bf16_to_float(self, bits):
        return np.float32(self.h.orc_bf16_to_float(int(bits)))

    def double_to_bf16(self, v):
        return int(self.h.orc_double_to_bf16(float(v)))

    # activations -----------------------------------------------------------
    def rmsnorm_quant(self, x_bits, g, eps=1e-6):
        x_bits = _c(x_bits, np.uint16)
        g = _c(g, np.float32)
        M, K = x_bits.shape
        q = np.empty((M, K), np.int8)
        s = np.empty(M, np.float32)
        self.h.orc_rmsnorm_quant(_ptr(x_bits), _ptr(g), M, K, float(eps), _ptr(q), _ptr(s))
        return q, s

    def accumulate(self, q, w):
        q = _c(q, np.int8)
        w = _c(w, np.int8)
        M, K = q.shape
        N = w.shape[0]
        acc = np.empty((M, N), np.int32)
        self.h.orc_ternary_accumulate(_ptr(q), _ptr(w), M, N, K, _ptr(acc))
        return acc

    def rescale(self, acc, gamma, s):
        acc = _c(acc, np.int32)
        s = _c(s, np.float32)
        M, N = acc.shape
        y = np.empty((M, N), np.float64)
        self.h.orc_rescale(_ptr(acc), float(gamma), _ptr(s), M, N, _ptr(y))
        return y

    # compositions ----------------------------------------------------------
    def bitlinear(self, x_bits, g, W, eps=1e-6):
        """Full forward from fp32 master weights.  Returns a dict with y (fp64)
        and every intermediate (gamma, w, q, s, acc)."""
        x_bits = _c(x_bits, np.uint16)
        g = _c(g, np.float32)
        W = _c(W, np.float32)
        M, K = x_bits.shape
        N = W.shape[0]
        y = np.empty((M, N), np.float64)
        gamma = np.empty(1, np.float32)
        w = np.empty((N, K), np.int8)
        q = np.empty((M, K), np.int8)
        s = np.empty(M, np.float32)
        acc = np.empty((M, N), np.int32)
        self.h.orc_bitlinear(_ptr(x_bits), _ptr(g), _ptr(W), M, N, K, float(eps), _ptr(y),
                             _ptr(gamma), _ptr(w), _ptr(q), _ptr(s), _ptr(acc))
        return dict(y=y, gamma=gamma[0], w=w, q=q, s=s, acc=acc)

    def bitlinear_ternary(self, x_bits, g, w, gamma, eps=1e-6):
        x_bits = _c(x_bits, np.uint16)
        g = _c(g, np.float32)
        w = _c(w, np.int8)
        M, K = x_bits.shape
        N = w.shape[0]
        y = np.empty((M, N), np.float64)
        q = np.empty((M, K), np.int8)
        s = np.empty(M, np.float32)
        acc = np.empty((M, N), np.int32)
        self.h.orc_bitlinear_ternary(_ptr(x_bits), _ptr(g), _ptr(w), float(gamma), M, N, K,
                                     float(eps), _ptr(y), _ptr(q), _ptr(s), _ptr(acc))
        return dict(y=y, q=q, s=s, acc=acc)

    def glu(self, x_bits, g_gu, W_gu, g_down, W_down, eps=1e-6):
        x_bits = _c(x_bits, np.uint16)
        M, D = x_bits.shape
        F = W_down.shape[1]
        assert W_gu.shape == (2 * F, D) and W_down.shape == (D, F)
        y = np.empty((M, D), np.float64)
        h = np.empty((M, F), np.uint16)
        self.h.orc_glu(_ptr(x_bits), _ptr(_c(g_gu, np.float32)), _ptr(_c(W_gu, np.float32)),
                       _ptr(_c(g_down, np.float32)), _ptr(_c(W_down, np.float32)),
                       M, D, F, float(eps), _ptr(y), _ptr(h))
        return dict(y=y, h=h)

    def glu_ternary(self, x_bits, g_gu, w_gu, gamma_gu, g_down, w_down, gamma_down, eps=1e-6):
        x_bits = _c(x_bits, np.uint16)
        M, D = x_bits.shape
        F = w_down.shape[1]
        y = np.empty((M, D), np.float64)
        h = np.empty((M, F), np.uint16)
        self.h.orc_glu_ternary(_ptr(x_bits), _ptr(_c(g_gu, np.float32)), _ptr(_c(w_gu, np.int8)),
                               float(gamma_gu), _ptr(_c(g_down, np.float32)),
                               _ptr(_c(w_down, np.int8)), float(gamma_down), M, D, F,
                               float(eps), _ptr(y), _ptr(h))
        return dict(y=y, h=h)

    # MLGRU token mixer and the layer --------------------------------------
    def mlgru_scan(self, z, state=None):
        """z [B, T, 3d] pre-activations (z_f | z_c | z_g per token) ->
        dict(p bf16 [B, T, d], state fp64 [B, d] = h_T); state holds h_0
        (zeros when None)."""
        z = _c(z, np.float64)
        B, T, d3 = z.shape
        d = d3 // 3
        st = np.zeros((B, d), np.float64) if state is None else _c(state, np.float64).copy()
        p = np.empty((B, T, d), np.uint16)
        self.h.orc_mlgru_scan(_ptr(z), B, T, d, _ptr(st), _ptr(p))
        return dict(p=p, state=st)

    def mlgru_ternary(self, x_bits, g_in, w_in, gamma_in, g_out, w_out, gamma_out, state=None,
                      eps=1e-6):
        """x bf16 [B, T, d] -> dict(y fp64 [B, T, d], p bf16 [B, T, d],
        state [B, d])."""
        x_bits = _c(x_bits, np.uint16)
        B, T, d = x_bits.shape
        assert w_in.shape == (3 * d, d) and w_out.shape == (d, d)
        st = np.zeros((B, d), np.float64) if state is None else _c(state, np.float64).copy()
        y = np.empty((B, T, d), np.float64)
        p = np.empty((B, T, d), np.uint16)
        self.h.orc_mlgru_ternary(_ptr(x_bits), _ptr(_c(g_in, np.float32)), _ptr(_c(w_in, np.int8)),
                                 float(gamma_in), _ptr(_c(g_out, np.float32)), _ptr(_c(w_out, np.int8)),
                                 float(gamma_out), B, T, d, float(eps), _ptr(st), _ptr(y), _ptr(p))
        return dict(y=y, p=p, state=st)

    def mlgru(self, x_bits, g_in, W_in, g_out, W_out, state=None, eps=1e-6):
        x_bits = _c(x_bits, np.uint16)
        B, T, d = x_bits.shape
        assert W_in.shape == (3 * d, d) and W_out.shape == (d, d)
        st = np.zeros((B, d), np.float64) if state is None else _c(state, np.float64).copy()
        y = np.empty((B, T, d), np.float64)
        p = np.empty((B, T, d), np.uint16)
        self.h.orc_mlgru(_ptr(x_bits), _ptr(_c(g_in, np.float32)), _ptr(_c(W_in, np.float32)),
                         _ptr(_c(g_out, np.float32)), _ptr(_c(W_out, np.float32)), B, T, d, float(eps),
                         _ptr(st), _ptr(y), _ptr(p))
        return dict(y=y, p=p, state=st)

    def lm_layer_ternary(self, x_bits, mlgru_w, glu_w, state=None, eps=1e-6):
        """One layer, u = bf16(x + MLGRU(x)), out = bf16(u + GLU(u)).
        mlgru_w = (g_in, w_in, gamma_in, g_out, w_out, gamma_out), glu_w =
        (g_gu, w_gu, gamma_gu, g_down, w_down, gamma_down), ternary.  x bf16
        [B, T, d] -> dict(out bf16 [B, T, d], u bf16 [B, T, d], state)."""
        x_bits = _c(x_bits, np.uint16)
        B, T, d = x_bits.shape
        g_in, w_in, gamma_in, g_out, w_out, gamma_out = mlgru_w
        g_gu, w_gu, gamma_gu, g_dn, w_dn, gamma_dn = glu_w
        F = w_dn.shape[1]
        assert w_in.shape == (3 * d, d) and w_out.shape == (d, d)
        assert w_gu.shape == (2 * F, d) and w_dn.shape == (d, F)
        st = np.zeros((B, d), np.float64) if state is None else _c(state, np.float64).copy()
        out = np.empty((B, T, d), np.uint16)
        u = np.empty((B, T, d), np.uint16)
        self.h.orc_lm_layer_ternary(
            _ptr(x_bits), _ptr(_c(g_in, np.float32)), _ptr(_c(w_in, np.int8)), float(gamma_in),
            _ptr(_c(g_out, np.float32)), _ptr(_c(w_out, np.int8)), float(gamma_out),
            _ptr(_c(g_gu, np.float32)), _ptr(_c(w_gu, np.int8)), float(gamma_gu),
            _ptr(_c(g_dn, np.float32)), _ptr(_c(w_dn, np.int8)), float(gamma_dn),
            B, T, d, F, float(eps), _ptr(st), _ptr(out), _ptr(u))
        return dict(out=out, u=u, state=st)

    def backward(self, x_bits, g, w, gamma, dy, eps=1e-6):
        """Straight-through backward of the layer (w ternary [N, K], dy fp32
        [M, N]) -> dict(dx [M, K], dg [K], dW [N, K]), fp64."""
        x_bits = _c(x_bits, np.uint16)
        w = _c(w, np.int8)
        dy = _c(dy, np.float32)
        M, K = x_bits.shape
        N = w.shape[0]
        assert w.shape == (N, K) and dy.shape == (M, N)
        dx = np.empty((M, K), np.float64)
        dg = np.empty(K, np.float64)
        dW = np.empty((N, K), np.float64)
        self.h.orc_bitlinear_backward(_ptr(x_bits), _ptr(_c(g, np.float32)), _ptr(w), float(gamma),
                                      _ptr(dy), M, N, K, float(eps), _ptr(dx), _ptr(dg), _ptr(dW))
        return dict(dx=dx, dg=dg, dW=dW)
