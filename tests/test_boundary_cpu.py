"""The C-ABI library without a GPU: it loads, exports every symbol that
include/bitlinear.h declares, sizes buffers as documented and rejects bad
arguments before any launch (every call here fails validation or is an empty
call, so no HIP work is ever enqueued)."""
import ctypes
import os
import re

import pytest

import bitlinear_layer_amd as bl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

FAKE = ctypes.c_void_p(0x10000)       # 16- and 256-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = bl.lib()
    decl = declared_functions()
    assert len(decl) >= 15
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(bl.exported_symbols()) == decl


def test_abi_version():
    assert bl.bitlinear_abi_version() == 1


def test_sizes():
    assert bl.bitlinear_packed_bytes(2048, 2048) == 2048 * 512
    assert bl.bitlinear_packed_bytes(7, 48) == 7 * 12
    assert bl.bitlinear_packed_bytes(7, 12) == 0
    assert bl.bitlinear_packed_bytes(-1, 16) == 0
    fw = bl.bitlinear_forward_workspace_bytes(8192, 2048, 2048)
    assert fw >= 8192 * 2048 + 2 * 8192 * 4 and fw % 256 == 0
    assert bl.bitlinear_forward_workspace_bytes(0, 16, 16) == 0
    assert bl.bitlinear_forward_batched_workspace_bytes(4, 1, 64, 64) == bl.bitlinear_forward_workspace_bytes(4, 64, 64)
    assert bl.bitlinear_glu_batched_workspace_bytes(4, 1, 64, 96) == bl.bitlinear_glu_workspace_bytes(4, 64, 96)
    assert bl.bitlinear_glu_batched_workspace_bytes(0, 1, 64, 96) == 0
    gw = bl.bitlinear_glu_workspace_bytes(4096, 2048, 5632)
    assert gw >= 4096 * 2048 + 4096 * 5632 * 2 + 4096 * 5632
    assert bl.bitlinear_pack_workspace_bytes(2048, 2048) % 256 == 0
    assert bl.bitlinear_pack_batched_workspace_bytes(1, 2048, 2048) == bl.bitlinear_pack_workspace_bytes(2048, 2048)
    assert bl.bitlinear_pack_batched_workspace_bytes(64, 2048, 2048) >= 64 * 8 * 2
    assert bl.bitlinear_pack_batched_workspace_bytes(0, 2048, 2048) == 0
    assert bl.bitlinear_pack_batched_workspace_bytes(70000, 64, 64) == 0


def _fwd(x=FAKE, g=FAKE, p=FAKE, gamma=FAKE, M=4, N=64, K=64, eps=1e-6, y=FAKE, ws=FAKE,
         ws_bytes=1 << 20, kernel=0):
    return bl.lib().bitlinear_forward_ex(x, g, p, gamma, M, N, K, eps, y, ws, ws_bytes, None, kernel)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(y=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(gamma=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(x=MISALIGNED), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(K=12), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(K=0), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(M=-1), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(N=-5), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(M=1 << 31), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(K=(1 << 24) + 16, M=1, N=1), bl.BITLINEAR_ERR_INVALID_ARG),  # past BITLINEAR_MAX_K
    (dict(eps=0.0), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(eps=float("nan")), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(ws=None), bl.BITLINEAR_ERR_WORKSPACE),
    (dict(ws_bytes=100), bl.BITLINEAR_ERR_WORKSPACE),
    (dict(ws=MISALIGNED), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(kernel=7), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(kernel=1, M=9), bl.BITLINEAR_ERR_INVALID_ARG),
])
def test_forward_rejects(kwargs, status):
    assert _fwd(**kwargs) == status
    assert bl.bitlinear_last_error() != ""


def test_forward_empty_is_ok():
    assert _fwd(M=0, x=None, y=None, ws=None) == bl.BITLINEAR_OK
    assert _fwd(N=0, x=None, y=None, ws=None) == bl.BITLINEAR_OK


def test_other_entry_points_reject():
    L = bl.lib()
    assert L.bitlinear_pack_weights(FAKE, 64, 12, FAKE, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_pack_weights(FAKE, 0, 16, FAKE, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_pack_weights(FAKE, 64, 64, FAKE, FAKE, None, 0, None) == bl.BITLINEAR_ERR_WORKSPACE
    assert L.bitlinear_unpack_weights(None, 4, 64, FAKE, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_pack_weights_batched(FAKE, 0, 64, 64, FAKE, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_pack_weights_batched(FAKE, 70000, 64, 64, FAKE, FAKE, FAKE, 1 << 30, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_pack_weights_batched(FAKE, 2, 64, 12, FAKE, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_pack_weights_batched(FAKE, 2, 64, 64, FAKE, None, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_pack_weights_batched(FAKE, 2, 64, 64, FAKE, FAKE, FAKE, 8, None) == bl.BITLINEAR_ERR_WORKSPACE
    assert L.bitlinear_forward_batched(FAKE, FAKE, FAKE, FAKE, 0, 1, 64, 64, 1e-6, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_forward_batched(FAKE, FAKE, FAKE, FAKE, 70000, 1, 64, 64, 1e-6, FAKE, FAKE, 1 << 30, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_glu_forward_batched(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 64, 64, 1e-6, FAKE,
                                           FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_glu_forward_batched(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 64, 72, 1e-6, FAKE,
                                           FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_glu_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 40, 1e-6, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_glu_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 64, 1e-6, FAKE, FAKE, 16, None) == bl.BITLINEAR_ERR_WORKSPACE
    assert L.bitlinear_glu_hidden(FAKE, FAKE, FAKE, FAKE, 4, 64, 64, 1e-6, FAKE, FAKE, 16, None, 0) == bl.BITLINEAR_ERR_WORKSPACE
    assert L.bitlinear_quantize(FAKE, FAKE, 4, 30, 1e-6, FAKE, FAKE, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_quantize(FAKE, FAKE, 4, 32, -1.0, FAKE, FAKE, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_ternary_matmul_i32(FAKE, FAKE, 4, 64, 64, FAKE, FAKE, 8, None, 0) == bl.BITLINEAR_ERR_WORKSPACE
    assert L.bitlinear_ternary_matmul_i32(FAKE, None, 4, 64, 64, FAKE, FAKE, 1 << 20, None, 0) == bl.BITLINEAR_ERR_INVALID_ARG
    # reduction lengths past BITLINEAR_MAX_K (int32 sums could no longer be exact)
    big = (1 << 24) + 16
    assert L.bitlinear_ternary_matmul_i32(FAKE, FAKE, 1, 1, big, FAKE, FAKE, 1 << 30, None, 0) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_quantize(FAKE, FAKE, 1, big, 1e-6, FAKE, FAKE, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_glu_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, big, 1e-6, FAKE, FAKE, 1 << 30,
                                   None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_decode_supported(1, big) == 0
    assert L.bitlinear_ternary_matmul_i32(FAKE, FAKE, 1, 1, 1 << 24, FAKE, FAKE, 0, None, 0) == bl.BITLINEAR_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(bl, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(bl, "_lib", None)
    with pytest.raises(RuntimeError):
        bl.lib()


def _bwd(x=FAKE, g=FAKE, p=FAKE, gamma=FAKE, dy=FAKE, M=4, N=64, K=64, eps=1e-6, dx=FAKE, dg=FAKE, dW=FAKE,
         ws=FAKE, ws_bytes=1 << 30):
    return bl.lib().bitlinear_backward(x, g, p, gamma, dy, M, N, K, eps, dx, dg, dW, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(dy=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(dx=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(dg=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(dW=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(p=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(gamma=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(dy=MISALIGNED), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(K=24), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(K=(1 << 24) + 16, M=1, N=1), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(M=-1), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(eps=float("inf")), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(ws=None), bl.BITLINEAR_ERR_WORKSPACE),
    (dict(ws_bytes=1024), bl.BITLINEAR_ERR_WORKSPACE),
])
def test_backward_rejects(kwargs, status):
    assert _bwd(**kwargs) == status


def test_backward_workspace_query():
    L = bl.lib()
    assert L.bitlinear_backward_workspace_bytes(4, 64, 12) == 0
    assert L.bitlinear_backward_workspace_bytes(-1, 64, 64) == 0
    small = L.bitlinear_backward_workspace_bytes(1, 16, 16)
    big = L.bitlinear_backward_workspace_bytes(8192, 2048, 2048)
    assert 0 < small < big and big % 256 == 0


# --------------------------------------------------------------------------
# The binding checks every caller-supplied output before a pointer reaches the
# library.  The checks run dtype -> shape -> contiguity -> device, so CPU
# tensors exercise every rejection except the device one, and the last case
# shows a well-formed CPU tensor is still refused (it is not on the GPU).
# --------------------------------------------------------------------------

import torch  # noqa: E402


def test_output_check_rejects_wrong_dtype():
    like = torch.empty(4, 8)
    with pytest.raises(TypeError):
        bl._out(torch.empty(4, 8, dtype=torch.bfloat16), "y", (torch.float32,), (4, 8), like)
    with pytest.raises(TypeError):
        bl._out(None, "y", (torch.float32,), (4, 8), like)


@pytest.mark.parametrize("shape", [(4, 7), (8, 4), (32,), (4, 8, 1), (5, 8)])
def test_output_check_rejects_wrong_shape(shape):
    like = torch.empty(4, 8)
    with pytest.raises(ValueError, match="shape"):
        bl._out(torch.empty(shape), "y", (torch.float32,), (4, 8), like)


def test_output_check_rejects_non_contiguous():
    like = torch.empty(4, 8)
    t = torch.empty(8, 4).t()
    assert t.shape == (4, 8) and not t.is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        bl._out(t, "y", (torch.float32,), (4, 8), like)


def test_output_check_rejects_host_tensor():
    like = torch.empty(4, 8)
    with pytest.raises(ValueError, match="must be on"):
        bl._out(torch.empty(4, 8), "y", (torch.float32,), (4, 8), like)
    with pytest.raises(ValueError, match="must be on"):
        bl._new_or_out(torch.empty(4, 8), "y", torch.float32, (4, 8), like)
    # a caller's workspace goes through the same device check
    with pytest.raises(ValueError, match="must be on"):
        bl._workspace(64, torch.empty(64, dtype=torch.uint8), like)


def test_gamma_must_hold_one_value_per_matrix():
    with pytest.raises(ValueError):  # a host tensor fails the device check first
        bl._scalar(torch.ones(1), "gamma")


# --------------------------------------------------------------------------
# MLGRU token mixer and the layer: validation before any launch
# --------------------------------------------------------------------------

def test_mlgru_scan_rejects():
    L = bl.lib()
    assert L.bitlinear_mlgru_scan(FAKE, 1, 4, 24, FAKE, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_mlgru_scan(None, 1, 4, 32, FAKE, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_mlgru_scan(FAKE, 1, 4, 32, None, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_mlgru_scan(FAKE, 1, 4, 32, FAKE, MISALIGNED, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_mlgru_scan(FAKE, -1, 4, 32, FAKE, FAKE, FAKE, 1 << 20, None) == bl.BITLINEAR_ERR_INVALID_ARG
    # a long single sequence needs chunk summaries: refused without them
    need = L.bitlinear_mlgru_scan_workspace_bytes(1, 2048, 2048)
    assert need > 0
    assert L.bitlinear_mlgru_scan(FAKE, 1, 2048, 2048, FAKE, FAKE, None, 0, None) == bl.BITLINEAR_ERR_WORKSPACE
    assert L.bitlinear_mlgru_scan(FAKE, 1, 2048, 2048, FAKE, FAKE, FAKE, need - 1, None) == bl.BITLINEAR_ERR_WORKSPACE
    # empty sequences are valid no-ops
    assert L.bitlinear_mlgru_scan(None, 3, 0, 32, None, None, None, 0, None) == bl.BITLINEAR_OK
    assert L.bitlinear_mlgru_scan(None, 0, 5, 32, None, None, None, 0, None) == bl.BITLINEAR_OK


def test_mlgru_and_layer_workspace_queries():
    L = bl.lib()
    assert L.bitlinear_mlgru_scan_workspace_bytes(1, 1, 2048) == 0          # one token: one pass
    assert L.bitlinear_mlgru_scan_workspace_bytes(64, 5, 2048) == 0         # many channels: one pass
    assert L.bitlinear_mlgru_scan_workspace_bytes(1, 2048, 24) == 0         # d % 16 != 0: invalid
    m = L.bitlinear_mlgru_workspace_bytes(1, 2048, 2048)
    assert m >= 2048 * 3 * 2048 * 4 + 2048 * 2048 * 3 and m % 256 == 0
    assert L.bitlinear_mlgru_workspace_bytes(0, 5, 32) == 0
    lw = L.bitlinear_layer_workspace_bytes(1, 2048, 2048, 5632)
    assert lw >= max(m, L.bitlinear_glu_workspace_bytes(2048, 2048, 5632)) + 2048 * 2048 * 6
    assert L.bitlinear_layer_workspace_bytes(1, 8, 2048, 100) == 0


def _mlgru_call(x=FAKE, w=FAKE, B=1, T=4, d=64, eps=1e-6, state=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return bl.lib().bitlinear_mlgru_forward(x, w, w, w, w, w, w, B, T, d, eps, state, y, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(w=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(state=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(y=None), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(d=40), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(d=(1 << 24) + 16), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(T=-2), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(eps=0.0), bl.BITLINEAR_ERR_INVALID_ARG),
    (dict(ws=None), bl.BITLINEAR_ERR_WORKSPACE),
    (dict(ws_bytes=4096), bl.BITLINEAR_ERR_WORKSPACE),
])
def test_mlgru_forward_rejects(kwargs, status):
    assert _mlgru_call(**kwargs) == status
    assert bl.bitlinear_last_error() != ""


def test_layer_forward_rejects():
    L = bl.lib()
    args = [FAKE] * 13

    def call(a=args, B=1, T=4, d=64, F=96, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return L.bitlinear_layer_forward(*a, B, T, d, F, 1e-6, FAKE, out, ws, ws_bytes, None)

    assert call(F=100) == bl.BITLINEAR_ERR_INVALID_ARG
    assert call(out=None) == bl.BITLINEAR_ERR_INVALID_ARG
    for i in range(13):
        bad = list(args)
        bad[i] = None
        assert call(a=bad) == bl.BITLINEAR_ERR_INVALID_ARG, i
    assert call(ws_bytes=64) == bl.BITLINEAR_ERR_WORKSPACE
    assert call(T=0, out=None, ws=None) == bl.BITLINEAR_OK


def test_noalloc_rejects_before_touching_the_gpu():
    """bitlinear_forward_noalloc refuses a stage larger than its fixed
    scratch (and bad sizes) before any HIP call."""
    L = bl.lib()
    big_m = (48 << 20) // 2048 + 1
    assert L.bitlinear_forward_noalloc(FAKE, FAKE, FAKE, FAKE, big_m, 64, 2048, 1e-6, FAKE, None) == \
        bl.BITLINEAR_ERR_INVALID_ARG
    assert "scratch" in bl.bitlinear_last_error()
    assert L.bitlinear_forward_noalloc(FAKE, FAKE, FAKE, FAKE, 4, 64, 24, 1e-6, FAKE, None) == \
        bl.BITLINEAR_ERR_INVALID_ARG
    assert L.bitlinear_forward_noalloc(None, None, None, None, 0, 64, 64, 1e-6, None, None) == bl.BITLINEAR_OK
