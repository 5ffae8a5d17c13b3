"""Backward pass (straight-through estimator) on the GPU against the oracle.

The two gradient products run in bf16 with fp32 accumulation; every other
step is fp32 or exact.  The bar per element is derived from that arithmetic.
bf16 keeps 8 significant bits, so rounding a term's operand dy (or
dy * (1 / s), itself two fp32 roundings of dy / s) to nearest bf16 moves the
term by at most 2^-8 (plus 2^-22) of its size, and fp32 accumulation of
R <= 2^15 terms adds at most R * 2^-24 <= 2^-9 of the sum of their sizes:
    |dxn - dxn_ref| <= U * gamma * sum_n |dy[m][n]| |w[n][k]|             (E)
    |dW - dW_ref|   <= U * sum_m |dy[m][n] / s[m]| |q[m][k]|
with U = 2^-8 + 2^-9 + 2^-22; dx and dg inherit E through the RMSNorm
backward (linear in dxn), plus 1e-5 of their own terms for the fp32
arithmetic there.  Exact zeros are required where the method has them
(M = 0, N = 0), and one token's dW, a single product per element, is
checked bit for bit.
"""
import numpy as np
import pytest
import torch

import bitlinear_layer_amd as bl
import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

EPS = 1e-6
U = 2.0 ** -8 + 2.0 ** -9 + 2.0 ** -22


def _case(M, N, K, seed, outliers=True):
    x = wl.x_normal(M, K, seed=seed, outlier_frac=0.01 if outliers else 0.0, outlier_scale=20.0)
    g = wl.rms_weight(K, "random", seed=seed)
    W = wl.w_normal(N, K, seed=seed)
    dy = wl.dy_normal(M, N, seed=seed)
    return x, g, W, dy


def _run_gpu(x, g, packed, gamma, dy):
    dx, dg, dW = bl.bitlinear_backward(gu.to_dev_bf16(x), gu.to_dev(g), packed, gamma, gu.to_dev(dy), eps=EPS)
    torch.cuda.synchronize()
    return dx.cpu().numpy(), dg.cpu().numpy(), dW.cpu().numpy()


def _bounds(x, g, w, gamma, dy, q, s):
    """Per-element bounds for dx, dg and dW (see the module docstring)."""
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    gf = g.astype(np.float64)
    K = x.shape[1]
    aw = np.abs(w).astype(np.float64)
    E = U * float(gamma) * (np.abs(dy).astype(np.float64) @ aw)            # [M, K]
    r = 1.0 / np.sqrt((xf ** 2).mean(axis=1) + float(np.float32(EPS)))      # [M]
    dxn_abs = float(gamma) * (np.abs(dy).astype(np.float64) @ aw)           # >= |dxn|
    row_e = (E * np.abs(gf) * np.abs(xf)).sum(axis=1)
    row_t = (dxn_abs * np.abs(gf) * np.abs(xf)).sum(axis=1)
    b_dx = (r[:, None] * np.abs(gf) * E + np.abs(xf) * (r ** 3 / K * row_e)[:, None]
            + 1e-5 * (r[:, None] * np.abs(gf) * dxn_abs + np.abs(xf) * (r ** 3 / K * row_t)[:, None]))
    b_dg = (E * np.abs(xf) * r[:, None]).sum(axis=0) + 1e-5 * (dxn_abs * np.abs(xf) * r[:, None]).sum(axis=0)
    dq = np.abs(dy).astype(np.float64) / s.astype(np.float64)[:, None]      # [M, N]
    b_dW = U * (dq.T @ np.abs(q).astype(np.float64))
    return b_dx, b_dg, b_dW


def _check(got, ref, bound, name):
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > bound + 1e-30
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} outside the bound; worst "
                           f"err {err[bad].max():.3e} vs bound {bound[bad][np.argmax(err[bad])]:.3e}")


def _parity(M, N, K, seed, outliers=True):
    x, g, W, dy = _case(M, N, K, seed, outliers)
    packed, gamma = gu.pack_on_gpu(W)
    orc = gu.orc()
    gm = float(gamma.item())
    w = orc.ternarize(W, gm)
    ref = orc.backward(x, g, w, gm, dy, EPS)
    dx, dg, dW = _run_gpu(x, g, packed, gamma, dy)
    q, s = orc.rmsnorm_quant(x, g, EPS)
    b_dx, b_dg, b_dW = _bounds(x, g, w, gm, dy, q, s)
    _check(dx, ref["dx"], b_dx, "dx")
    _check(dg, ref["dg"], b_dg, "dg")
    _check(dW, ref["dW"], b_dW, "dW")
    # and in aggregate the results sit within bf16 precision of the oracle
    # (a transposed or misplaced result would be off by its own size)
    for got, r in ((dx, ref["dx"]), (dW, ref["dW"])):
        assert np.linalg.norm(got - r) <= U * np.linalg.norm(r) + 1e-30


# (M, N, K): one tile, ragged tiles on every edge (M, N, K not multiples of
# the 64-row operand padding or of the 128-wide product tiles), several
# tiles with a ragged tail, and tall/wide shapes.
SHAPES = [
    (1, 16, 16), (5, 40, 48), (64, 64, 64), (130, 200, 272), (257, 129, 320),
    (600, 300, 1024), (33, 1000, 96), (1000, 24, 160),
    # RMSNorm backward: rows held in registers up to K = 4096 (full and
    # ragged last chunk), the two-pass form above
    (37, 64, 4096), (21, 40, 3856), (40, 50, 4160),
    # dg from more than 64 partial sums, so the reduction over partials runs
    # its chained steps: 128 partials on the register form, 138 on the
    # two-pass form
    (2048, 64, 256), (1100, 40, 4160),
    # 64 rows and more: re-quantisation inside the RMSNorm backward up to
    # K = 2048 (here a ragged fourth chunk per lane), the separate quantiser
    # and the register form above
    (200, 100, 2000), (96, 48, 3072),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_backward_matches_oracle(M, N, K):
    _parity(M, N, K, seed=M * 7 + N * 3 + K)


@pytest.mark.parametrize("N,K", [(300, 784), (37, 272), (64, 16)])
def test_backward_one_token_dW_exact(N, K):
    """M = 1: dW[n][k] = bf16(dy[n] * (1 / s)) * q[k], one product of a bf16
    and an int8 value, exact in fp32.  q and s are the forward's (the
    quantisation kernel the backward reruns); the rest is worked out here
    with fp32 arithmetic and round-to-nearest-even bf16."""
    x, g, W, dy = _case(1, N, K, seed=N + K)
    packed, gamma = gu.pack_on_gpu(W)
    q, s = bl.bitlinear_quantize(gu.to_dev_bf16(x), gu.to_dev(g), eps=EPS)
    _, _, dW = _run_gpu(x, g, packed, gamma, dy)
    q = q.cpu().numpy().astype(np.float64)
    s = s.cpu().numpy().astype(np.float32)
    a = dy[0].astype(np.float32) * (np.float32(1.0) / s[0])
    a = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(a)).astype(np.float64)
    want = a[:, None] * q[0][None, :]
    assert np.array_equal(dW.astype(np.float64), want), np.abs(dW - want).max()


@pytest.mark.parametrize("M,N,K,row", [(100, 300, 272, 63), (100, 64, 1024, 0), (130, 37, 1040, 129),
                                       (64, 200, 2048, 17)])
def test_backward_one_row_dW_exact(M, N, K, row):
    """dy zero except one token row: dW[n][k] = bf16(dy[row][n] * (1 / s)) * q[k]
    exactly, the other rows adding exact zeros.  At 64 rows and more the
    backward re-quantises x inside its RMSNorm backward kernel; q and s must
    still be the forward quantiser's bits (ragged and whole chunk counts)."""
    x, g, W, dy = _case(M, N, K, seed=M + N + K)
    keep = dy[row].copy()
    dy[:] = 0
    dy[row] = keep
    packed, gamma = gu.pack_on_gpu(W)
    q, s = bl.bitlinear_quantize(gu.to_dev_bf16(x), gu.to_dev(g), eps=EPS)
    _, _, dW = _run_gpu(x, g, packed, gamma, dy)
    q = q.cpu().numpy()[row].astype(np.float64)
    s = s.cpu().numpy().astype(np.float32)[row]
    a = keep.astype(np.float32) * (np.float32(1.0) / s)
    a = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(a)).astype(np.float64)
    want = a[:, None] * q[None, :]
    assert np.array_equal(dW.astype(np.float64), want), np.abs(dW - want).max()


def test_backward_without_outliers_and_unit_gain():
    M, N, K = 96, 80, 256
    x, _, W, dy = _case(M, N, K, seed=5, outliers=False)
    g = np.ones(K, np.float32)
    packed, gamma = gu.pack_on_gpu(W)
    orc = gu.orc()
    gm = float(gamma.item())
    w = orc.ternarize(W, gm)
    ref = orc.backward(x, g, w, gm, dy, EPS)
    dx, dg, dW = _run_gpu(x, g, packed, gamma, dy)
    q, s = orc.rmsnorm_quant(x, g, EPS)
    b = _bounds(x, g, w, gm, dy, q, s)
    for got, r, bb, n in zip((dx, dg, dW), (ref["dx"], ref["dg"], ref["dW"]), b, ("dx", "dg", "dW")):
        _check(got, r, bb, n)


def test_backward_empty_dims():
    K = 64
    x, g, W, dy = _case(3, 20, K, seed=9)
    packed, gamma = gu.pack_on_gpu(W)
    dev = gu.DEV
    # M = 0: dg and dW are sums over no tokens
    dx, dg, dW = bl.bitlinear_backward(torch.empty((0, K), dtype=torch.bfloat16, device=dev), gu.to_dev(g),
                                       packed, gamma, torch.empty((0, 20), dtype=torch.float32, device=dev))
    dg0 = torch.full((K,), 7.0, device=dev)
    dW0 = torch.full((20, K), 7.0, device=dev)
    bl.bitlinear_backward(torch.empty((0, K), dtype=torch.bfloat16, device=dev), gu.to_dev(g), packed, gamma,
                          torch.empty((0, 20), dtype=torch.float32, device=dev), dg=dg0, dW=dW0)
    torch.cuda.synchronize()
    assert dx.shape == (0, K) and torch.all(dg0 == 0) and torch.all(dW0 == 0)
    # N = 0: no output, so dx = 0 and dg = 0
    dx1 = torch.full((3, K), 7.0, device=dev)
    dg1 = torch.full((K,), 7.0, device=dev)
    bl.bitlinear_backward(gu.to_dev_bf16(x), gu.to_dev(g), torch.empty((0, K // 4), dtype=torch.uint8, device=dev),
                          gamma, torch.empty((3, 0), dtype=torch.float32, device=dev), dx=dx1, dg=dg1)
    torch.cuda.synchronize()
    assert torch.all(dx1 == 0) and torch.all(dg1 == 0)


def test_backward_deterministic_and_zero_weights():
    M, N, K = 200, 96, 512
    x, g, W, dy = _case(M, N, K, seed=11)
    packed, gamma = gu.pack_on_gpu(W)
    a = _run_gpu(x, g, packed, gamma, dy)
    b = _run_gpu(x, g, packed, gamma, dy)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    # all-zero weights (gamma = 0): dx = 0 and dg = 0 exactly; dW is still dy^T xq
    p0, g0 = gu.pack_on_gpu(np.zeros((N, K), np.float32))
    dx, dg, dW = _run_gpu(x, g, p0, g0, dy)
    assert np.all(dx == 0) and np.all(dg == 0)
    assert np.array_equal(dW, a[2])


def test_backward_full_size_sampled():
    """8192 tokens, 2048 x 2048: dx on sampled rows (rows are independent)
    and dW on sampled output rows (each depends on its own column of dy)."""
    M, N, K = 8192, 2048, 2048
    x = wl.make_x(M, K, "student_t3", seed=0)
    g = wl.rms_weight(K)
    W = wl.w_normal(N, K, seed=0)
    dy = wl.dy_normal(M, N, seed=0)
    packed, gamma = gu.pack_on_gpu(W)
    dx, dg, dW = _run_gpu(x, g, packed, gamma, dy)
    orc = gu.orc()
    gm = float(gamma.item())
    w = orc.ternarize(W, gm)
    rows = np.array([0, 1, 127, 128, 4095, 6000, 8190, 8191])
    ref = orc.backward(x[rows], g, w, gm, dy[rows], EPS)
    q, s = orc.rmsnorm_quant(x[rows], g, EPS)
    b_dx, _, _ = _bounds(x[rows], g, w, gm, dy[rows], q, s)
    _check(dx[rows], ref["dx"], b_dx, "dx rows")
    ns = np.array([0, 5, 127, 128, 1000, 2047])
    ref = orc.backward(x, g, w[ns], gm, dy[:, ns], EPS)
    q, s = orc.rmsnorm_quant(x, g, EPS)
    dq = np.abs(dy[:, ns]).astype(np.float64) / s.astype(np.float64)[:, None]
    b_dW = U * (dq.T @ np.abs(q).astype(np.float64))
    _check(dW[ns], ref["dW"], b_dW, "dW rows")
    assert np.all(np.isfinite(dg))


def test_backward_rows_longer_than_65535_tiles():
    """K = 4194368: 65537 tiles of 64 along K, one past what a second grid
    dimension could hold; two tokens, three outputs."""
    M, N, K = 2, 3, 4194368
    _parity(M, N, K, seed=13, outliers=False)
