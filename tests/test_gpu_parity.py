"""Parity of the HIP library with the CPU oracle, element by element, on the
same seeded inputs.  Every call goes through the C ABI (ctypes binding).

Bars: packed bytes, gamma, int8 codes and int32 accumulations bit-exact
(codes: at most 0.1% of elements one step off where an fp32 reduction-order
tie flips); fp32 outputs within 1e-2 of the row maximum (and within the fp32
rescale's 2^-22 relative on rows whose codes match); GLU hidden bf16 equal
except rare one-ulp rounding flips.
"""
import numpy as np
import pytest
import torch

import bitlinear_layer_amd as bl
import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GEMV, MFMA, DECODE = bl.BITLINEAR_KERNEL_GEMV, bl.BITLINEAR_KERNEL_MFMA, bl.BITLINEAR_KERNEL_DECODE


def kernels_for(M, K):
    """Every kernel that takes this shape: AUTO, MFMA, the GEMV (M <= 8) and
    the fused decode kernel where it applies."""
    ks = [bl.BITLINEAR_KERNEL_AUTO, MFMA]
    if M <= 8:
        ks.append(GEMV)
    if bl.bitlinear_decode_supported(M, K):
        ks.append(DECODE)
    return ks


def _say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(7, 48), (256, 256), (300, 2064), (2048, 2048), (11264, 2048),
                                 (2048, 5632), (2560, 6912)])
def test_pack_matches_oracle(N, K):
    _say("pack", N, K)
    W = wl.w_normal(N, K, seed=N + K)
    packed, gamma = gu.pack_on_gpu(W)
    g_ref = gu.orc().gamma(W)
    w_ref = gu.orc().ternarize(W, g_ref)
    assert gamma.cpu().numpy()[0] == g_ref
    assert np.array_equal(packed.cpu().numpy(), gu.orc().pack(w_ref))
    assert np.array_equal(bl.bitlinear_unpack_weights(packed, K).cpu().numpy(), w_ref)


def test_pack_edge_cases():
    _say("pack edge cases")
    W = np.zeros((3, 32), np.float32)
    packed, gamma = gu.pack_on_gpu(W)
    assert gamma.item() == 0.0 and np.all(packed.cpu().numpy() == 0x55)
    a = np.float32(0.25)
    W = np.full((4, 64), a, np.float32)
    W[1::2] *= -1
    packed, gamma = gu.pack_on_gpu(W)
    assert gamma.item() == a
    w = bl.bitlinear_unpack_weights(packed, 64).cpu().numpy()
    assert np.all(w[0::2] == 1) and np.all(w[1::2] == -1)
    # exact rounding ties W/d = +-0.5 -> 0 and +-1.5 -> 2 -> 1 (ties to even)
    W = wl.w_normal(16, 64, seed=9)
    g_ref = gu.orc().gamma(W)
    d = np.float32(g_ref + np.float32(1e-5))
    W[0, :4] = [np.float32(0.5) * d, np.float32(-0.5) * d, np.float32(1.5) * d, np.float32(2.5) * d]
    g_ref = gu.orc().gamma(W)
    packed, gamma = gu.pack_on_gpu(W)
    assert gamma.item() == g_ref
    w_ref = gu.orc().ternarize(W, g_ref)
    assert np.array_equal(bl.bitlinear_unpack_weights(packed, 64).cpu().numpy(), w_ref)


@pytest.mark.parametrize("N,K", [(300, 2064), (2048, 2048)])
def test_pack_batched(N, K):
    """Three matrices in one call (normal, all zero, normal x 40): each gets
    the oracle's bytes and gamma, the same as from a call of its own."""
    _say("pack batched", N, K)
    Ws = [wl.w_normal(N, K, seed=N + 1), np.zeros((N, K), np.float32),
          (wl.w_normal(N, K, seed=N + 2) * np.float32(40.0)).astype(np.float32)]
    packed, gamma = bl.bitlinear_pack_weights_batched(torch.stack([gu.to_dev(W) for W in Ws]))
    packed, gamma = packed.cpu().numpy(), gamma.cpu().numpy()
    for b, W in enumerate(Ws):
        g_ref = gu.orc().gamma(W)
        assert gamma[b] == g_ref, b
        assert np.array_equal(packed[b], gu.orc().pack(gu.orc().ternarize(W, g_ref))), b
        p1, g1 = gu.pack_on_gpu(W)
        assert g1.item() == gamma[b] and np.array_equal(p1.cpu().numpy(), packed[b]), b


def test_pack_batched_large():
    """Five 4096 x 4096 matrices (320 MB of fp32, more than the chip's last-
    level cache) in one call, one of them all zero: every matrix gets the
    bytes and gamma of a call of its own, and the last one the oracle's."""
    N = K = 4096
    _say("pack batched large", 5, N, K)
    W = torch.stack([wl.w_normal_device(N, K, seed=7, layer=b, device=gu.DEV) for b in range(5)])
    W[1].zero_()
    packed, gamma = bl.bitlinear_pack_weights_batched(W)
    for b in range(5):
        p1, g1 = bl.bitlinear_pack_weights(W[b].contiguous())
        assert g1.item() == gamma[b].item() and torch.equal(p1, packed[b]), b
    Wl = W[4].cpu().numpy()
    g_ref = gu.orc().gamma(Wl)
    assert gamma[4].item() == g_ref
    assert np.array_equal(packed[4].cpu().numpy(), gu.orc().pack(gu.orc().ternarize(Wl, g_ref)))


def test_unpack_marks_unused_code():
    p = torch.full((2, 4), 0xFF, dtype=torch.uint8, device=gu.DEV)
    w = bl.bitlinear_unpack_weights(p, 16).cpu().numpy()
    assert np.all(w == 2)


# --------------------------------------------------------------------------
# RMSNorm + absmax quantisation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,recipe", [(1, 16, "normal"), (16, 256, "normal"), (5, 2048, "student_t3"),
                                        (3, 5632, "normal"), (2, 6912, "normal"),
                                        (4, 20000, "normal"), (300, 2048, "normal")])
def test_quantize(M, K, recipe):
    _say("quantize", M, K, recipe)
    x = wl.make_x(M, K, recipe, seed=M * 7 + K, outlier_frac=0.01, outlier_scale=20.0)
    g = wl.rms_weight(K, "random", seed=K)
    q_ref, s_ref = gu.orc().rmsnorm_quant(x, g)
    q, s = bl.bitlinear_quantize(gu.to_dev_bf16(x), gu.to_dev(g))
    gu.assert_q_parity(q.cpu().numpy(), q_ref, s.cpu().numpy(), s_ref)


# Many rows take the streaming layout (a wave per row); K picks the chunks
# per lane (1..16), exact multiples of 512 skip the bounds tests, and K above
# 8192 falls back to a block per row.
@pytest.mark.parametrize("K", [16, 512, 528, 2080, 4096, 5632, 6912, 8192, 8208])
def test_quantize_many_rows(K):
    M = 96
    _say("quantize many rows", M, K)
    x = wl.make_x(M, K, "student_t3", seed=K, outlier_frac=0.01, outlier_scale=20.0)
    x[7] = 0                                    # zero row inside the stream
    g = wl.rms_weight(K, "random", seed=K + 1)
    q_ref, s_ref = gu.orc().rmsnorm_quant(x, g)
    q, s = bl.bitlinear_quantize(gu.to_dev_bf16(x), gu.to_dev(g))
    gu.assert_q_parity(q.cpu().numpy(), q_ref, s.cpu().numpy(), s_ref)


def test_quantize_edge_rows():
    _say("quantize edge rows")
    K = 64
    x = wl.x_normal(6, K, seed=3)
    x[0] = 0                                    # zero row
    x[1] = 0x3FC0                               # constant 1.5
    x[2] = wl.f32_to_bf16_bits(np.full(K, 3e-4, np.float32))  # eps-dominated
    x[3, 5] = 0x4B00                            # one huge outlier
    x[4] = x[3] ^ np.uint16(0x8000)             # negated row
    g = wl.rms_weight(K, "random", seed=1)
    q_ref, s_ref = gu.orc().rmsnorm_quant(x, g, 1e-6)
    q, s = bl.bitlinear_quantize(gu.to_dev_bf16(x), gu.to_dev(g), 1e-6)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)


def _extreme_rows(M, K, seed):
    """M token rows cycling through magnitudes at the edges of the format:
    normal rows scaled to 1e15 and 1e18 (squares near the fp32 range), 1e30
    (the fp32 mean square overflows, so the row quantises to zero on both
    sides by the same reading), 1e-20 (eps dominates), bf16 subnormals, and
    an ordinary row."""
    base = wl.bf16_bits_to_f32(wl.x_normal(M, K, seed=seed)).astype(np.float64)
    scales = (1e15, 1e18, 1e30, 1e-20, None, 1.0)
    rng = wl.rng(seed, 7)
    x = np.empty((M, K), np.uint16)
    for m in range(M):
        sc = scales[m % len(scales)]
        if sc is None:  # subnormal bf16 patterns with random signs
            mant = rng.integers(1, 128, size=K).astype(np.uint16)
            x[m] = mant | (rng.integers(0, 2, size=K).astype(np.uint16) << 15)
        else:
            x[m] = wl.f32_to_bf16_bits((base[m] * sc).astype(np.float32))
    return x


@pytest.mark.parametrize("M,K", [(6, 256), (72, 256), (4, 2048), (12, 1280)])
def test_quantize_extreme_magnitudes(M, K):
    """Every quantisation path (block per row, streaming, and through the
    fused kernels below) on rows at the edges of bf16 and fp32."""
    _say("quantize extreme magnitudes", M, K)
    x = _extreme_rows(M, K, seed=M + K)
    g = wl.rms_weight(K, "random", seed=2)
    q_ref, s_ref = gu.orc().rmsnorm_quant(x, g, 1e-6)
    q, s = bl.bitlinear_quantize(gu.to_dev_bf16(x), gu.to_dev(g), 1e-6)
    gu.assert_q_parity(q.cpu().numpy(), q_ref, s.cpu().numpy(), s_ref)


@pytest.mark.parametrize("M,N,K", [(4, 64, 2048), (8, 64, 2048), (1, 40, 6912), (130, 64, 512)])
def test_forward_extreme_magnitudes(M, N, K):
    """The same rows through the fused decode kernel (1-4 tokens, register
    and three-pass prologues), the fused few-token kernel (8 tokens) and the
    quantisation pass + MFMA tiles (130 tokens), against the oracle."""
    _say("forward extreme magnitudes", M, N, K)
    x = _extreme_rows(M, K, seed=M + N + K)
    if M == 1:
        x[0] = _extreme_rows(2, K, seed=5)[1]  # the 1e18 row
    W = wl.w_normal(N, K, seed=3)
    g = wl.rms_weight(K, "random", seed=3)
    ref = gu.orc().bitlinear(x, g, W)
    packed, gamma = gu.pack_on_gpu(W)
    y = bl.bitlinear_forward(gu.to_dev_bf16(x), gu.to_dev(g), packed, gamma).cpu().numpy()
    q, _ = bl.bitlinear_quantize(gu.to_dev_bf16(x), gu.to_dev(g), 1e-6)
    gu.assert_y_parity(y, ref["y"], np.all(q.cpu().numpy() == ref["q"], axis=1))


# --------------------------------------------------------------------------
# ternary accumulation (int32, bit-exact)
# --------------------------------------------------------------------------

MATMUL = [(M, N, K) for M in (1, 3, 8, 130, 257) for (N, K) in ((7, 16), (129, 48), (300, 2064))]
# K % 128 == 0 with M > 128 runs the 32x32x32 MFMA kernel: 128-row tiles
# when 256-row tiles would be few (first two), 256-row tiles otherwise; all
# with ragged M and N, and even and odd numbers of LDS stages (one, three,
# four, five, eight).
MATMUL += [(300, 520, 1024), (129, 256, 128), (2900, 3000, 512), (300, 520, 384), (2900, 3000, 640)]
# M <= 16 with K % 256 == 0 runs the few-token MFMA kernels: K % 512 == 0 up
# to 2048 the run-loading one (two to eight chunks), else the quarter-loading
# one (one to three load groups); ragged N, 1 to 16 tokens.
MATMUL += [(1, 300, 512), (5, 130, 768), (8, 2100, 2048), (16, 77, 1280), (12, 64, 3328),
           (3, 90, 1024), (16, 200, 1536)]
# K = 2048 and 4096 with 5..16 tokens run the K-split few-token kernel: one
# batch of four groups, a ragged group past several batches, a problem
# smaller than one group, all 16 token rows.
MATMUL += [(5, 64, 2048), (16, 1000, 2048), (7, 17, 4096), (13, 333, 4096)]


@pytest.mark.parametrize("M,N,K", MATMUL)
def test_ternary_matmul_bit_exact(M, N, K):
    r = wl.rng(M * 1000 + N, 0)
    q = r.integers(-128, 128, size=(M, K)).astype(np.int8)
    w = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    # large cases: the oracle computes 48 sampled rows (first and last tiles included)
    rows = np.arange(M) if M * N * K <= 3e8 else np.unique(np.concatenate(
        [[0, 1, 255, 256, M - 2, M - 1], r.choice(M, size=42, replace=False)]))
    acc_ref = gu.orc().accumulate(q[rows], w)
    packed = gu.to_dev(gu.orc().pack(w))
    kernels = [MFMA] + ([GEMV] if M <= 8 else [])
    for kern in kernels:
        _say("matmul", M, N, K, "kernel", kern)
        acc = bl.bitlinear_ternary_matmul_i32(gu.to_dev(q), packed, kernel=kern).cpu().numpy()[rows]
        assert np.array_equal(acc, acc_ref), (kern, int(np.abs(acc - acc_ref).max()))


def test_ternary_matmul_extremes():
    """All -128 codes against all -1 / all +1 weights at the largest K of the
    workloads: the accumulator reaches +-128*6912 exactly."""
    K, M, N = 6912, 8, 32
    q = np.full((M, K), -128, np.int8)
    w = np.ones((N, K), np.int8)
    w[::2] = -1
    acc_ref = gu.orc().accumulate(q, w)
    packed = gu.to_dev(gu.orc().pack(w))
    for kern in (GEMV, MFMA):
        acc = bl.bitlinear_ternary_matmul_i32(gu.to_dev(q), packed, kernel=kern).cpu().numpy()
        assert np.array_equal(acc, acc_ref)


@pytest.mark.parametrize("M,N,K", [(4224, 2304, 512), (8192, 4096, 1024), (4096, 2560, 2560)])
def test_ternary_matmul_many_tiles(M, N, K):
    """The 256 x 256 tile kernel over more tiles than CUs (153, 512 and 160
    tiles), K of 4, 8 and 20 stages: int32 bit-exact on rows sampled across
    the tiles, including the first and last rows of tiles."""
    _say("many tiles", M, N, K)
    r = wl.rng(M + N + K, wl.STREAM_X)
    q = r.integers(-127, 128, size=(M, K), dtype=np.int8)
    w = (r.integers(0, 3, size=(N, K)) - 1).astype(np.int8)
    packed = gu.to_dev(gu.orc().pack(w))
    acc = bl.bitlinear_ternary_matmul_i32(gu.to_dev(q), packed, kernel=MFMA).cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, M, 127), [1, 126, 127, 128, 129, 255, 256, M - 129, M - 2, M - 1]]))
    rows = rows[(rows >= 0) & (rows < M)]
    ref = gu.orc().accumulate(q[rows], w)
    assert np.array_equal(acc[rows], ref)


def test_ternary_matmul_tile_path_long_rows():
    """The 256-row tile kernel at K = 8421632, where the byte offset of a
    tile's last row, 255 * K, passes 2^31: 129 tiles of 256 x 256 (so the
    256-row tiles are chosen), 256 x 33024 outputs.  The operands repeat a
    seeded pattern -- q row m repeats its own 128 codes along k, weight row n
    repeats pattern row n % 64 -- so acc[m][n] = (K / 128) * (the oracle's
    product of the patterns)[m][n % 64], every one of the 8.5 M outputs
    known.  About 72 GB of device memory."""
    P, REP, M, NREP = 128, 65794, 256, 516
    K, N = P * REP, 64 * NREP
    assert 255 * K > 2 ** 31 and (N // 256) * (M // 256) > 128
    r = wl.rng(11, wl.STREAM_X)
    q_pat = r.integers(-127, 128, size=(M, P), dtype=np.int8)
    w_pat = (r.integers(0, 3, size=(64, P)) - 1).astype(np.int8)
    acc_pat = gu.orc().accumulate(q_pat, w_pat).astype(np.int64)
    expect = (acc_pat * REP)[:, np.arange(N) % 64]
    assert np.abs(expect).max() < 2 ** 31
    _say("tile path, long rows: filling", M, N, K)
    q = torch.empty((M, K), dtype=torch.int8, device=gu.DEV)
    q.view(M, REP, P).copy_(gu.to_dev(q_pat).view(M, 1, P).expand(M, REP, P))
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=gu.DEV)
    p_pat = gu.to_dev(gu.orc().pack(w_pat))  # [64, 32]: one 128-weight period per row
    packed.view(NREP, 64, REP, P // 4).copy_(p_pat.view(1, 64, 1, P // 4).expand(NREP, 64, REP, P // 4))
    acc = bl.bitlinear_ternary_matmul_i32(q, packed, kernel=MFMA).cpu().numpy()
    del q, packed
    torch.cuda.empty_cache()
    assert np.array_equal(acc, expect.astype(np.int32))


# --------------------------------------------------------------------------
# end-to-end forward
# --------------------------------------------------------------------------

FORWARD = [
    (16, 256, 256, "normal", 0.01, 20.0),   # single layer, 1% outliers x20
    (1, 2048, 2048, "normal", 0.0, 1.0),    # decode, hidden 2048
    (8, 2048, 2048, "normal", 0.0, 1.0),
    (3, 129, 48, "student_t3", 0.0, 1.0),
    (130, 300, 2064, "normal", 0.005, 50.0),
    (257, 7, 16, "normal", 0.0, 1.0),
    (2, 300, 6912, "normal", 0.005, 50.0),   # decode, two 16-byte steps per lane
    (1, 129, 5632, "normal", 0.0, 1.0),      # decode, three steps per lane
    (4, 65, 4096, "student_t3", 0.0, 1.0),
    (1, 1000, 16384, "normal", 0.0, 1.0),    # decode, four steps per lane
    (3, 77, 192, "normal", 0.0, 1.0),
    (1, 70, 2176, "normal", 0.0, 1.0),       # decode, 8 lanes a row, five steps per lane
    (1, 33, 3008, "student_t3", 0.0, 1.0),   # decode, six steps per lane
    (1, 65, 3520, "normal", 0.005, 50.0),    # decode, seven steps per lane
    (13, 333, 2048, "student_t3", 0.01, 20.0),  # fused few-token kernel, ragged groups
    (6, 200, 4096, "normal", 0.0, 1.0),      # fused few-token kernel, K = 4096
    (16, 130, 4096, "normal", 0.0, 1.0),     # 16 x 4096 codes exceed its LDS: two launches
    (1, 65, 8192, "normal", 0.005, 50.0),    # widest decode row quantised from registers
    (4, 33, 8192, "student_t3", 0.0, 1.0),   # the same, four tokens
    (1, 40, 28672, "normal", 0.0, 1.0),      # widest row the fused decode kernel takes
    (2, 24, 28736, "normal", 0.0, 1.0),      # one chunk past it: quantisation pass + product
]


def _forward_case(M, N, K, recipe, of, os_, kernel, g_kind="random", seed=0):
    x, W, g = gu.oracle_inputs(M, N, K, seed, recipe, of, os_, g_kind)
    ref = gu.orc().bitlinear(x, g, W)
    packed, gamma = gu.pack_on_gpu(W)
    xd, gd = gu.to_dev_bf16(x), gu.to_dev(g)
    y = bl.bitlinear_forward(xd, gd, packed, gamma, kernel=kernel).cpu().numpy()
    q, s = bl.bitlinear_quantize(xd, gd)
    q = q.cpu().numpy()
    gu.assert_q_parity(q, ref["q"], s.cpu().numpy(), ref["s"])
    rows_eq = np.all(q == ref["q"], axis=1)
    return gu.assert_y_parity(y, ref["y"], rows_eq)


@pytest.mark.parametrize("M,N,K,recipe,of,os_", FORWARD)
def test_forward(M, N, K, recipe, of, os_):
    for kern in kernels_for(M, K):
        _say("forward", M, N, K, recipe, "kernel", kern)
        _forward_case(M, N, K, recipe, of, os_, kern)


def _random_shapes(n, seed):
    """Seeded (M, N, K) draws across the dispatch bands (1-4 tokens, 5-16,
    17-128, 129-700) and row lengths that select different kernels (K % 64,
    % 128, % 256, % 512 or 1024, 2048 and 4096 exactly, long rows), with N
    ragged; sizes kept so the oracle stays fast."""
    r = wl.rng(seed, 11)
    ks = [16, 48, 64, 128, 256, 384, 512, 528, 1024, 1536, 2048, 2064, 2560, 3008, 4096, 5632, 6912, 8192]
    bands = [(1, 5), (5, 17), (17, 129), (129, 701)]
    out = []
    for i in range(n):
        lo, hi = bands[i % 4]
        M, K, N = int(r.integers(lo, hi)), int(r.choice(ks)), int(r.integers(1, 3001))
        while M * N * K > 4e7 and N > 1:
            N = max(1, N // 2)
        out.append((M, N, K))
    return out


RANDOM_SHAPES = _random_shapes(96, 2024)


@pytest.mark.parametrize("case", range(len(RANDOM_SHAPES)))
def test_forward_random_shapes(case):
    """Every kernel that takes a seeded random shape against the oracle."""
    M, N, K = RANDOM_SHAPES[case]
    recipe, of, os_ = ("student_t3", 0.0, 1.0) if case % 3 == 0 else ("normal", 0.01 * (case % 2), 20.0)
    x, W, g = gu.oracle_inputs(M, N, K, case, recipe, of, os_, "random")
    ref = gu.orc().bitlinear(x, g, W)
    packed, gamma = gu.pack_on_gpu(W)
    xd, gd = gu.to_dev_bf16(x), gu.to_dev(g)
    q, s = bl.bitlinear_quantize(xd, gd)
    q = q.cpu().numpy()
    gu.assert_q_parity(q, ref["q"], s.cpu().numpy(), ref["s"])
    rows_eq = np.all(q == ref["q"], axis=1)
    for kern in kernels_for(M, K):
        _say("random shape", case, M, N, K, recipe, "kernel", kern)
        y = bl.bitlinear_forward(xd, gd, packed, gamma, kernel=kern).cpu().numpy()
        gu.assert_y_parity(y, ref["y"], rows_eq)


def test_forward_parity_config_ones_gain():
    """The single-layer workload exactly as stated: gain 1, seed 0."""
    _say("forward parity config")
    _forward_case(16, 256, 256, "normal", 0.01, 20.0, bl.BITLINEAR_KERNEL_AUTO, g_kind="ones")


@pytest.mark.parametrize("K", [512, 528])
def test_forward_batched(K):
    B, N = 5, 256
    for M in (1, 3, 20):
        _say("batched", B, M, N, K)
        xs = [wl.x_normal(M, K, seed=10 + b) for b in range(B)]
        Ws = [wl.w_normal(N, K, seed=20 + b) for b in range(B)]
        gs = [wl.rms_weight(K, "random", seed=30 + b) for b in range(B)]
        packs = [gu.pack_on_gpu(W) for W in Ws]
        x = torch.stack([gu.to_dev_bf16(a) for a in xs])
        g = torch.stack([gu.to_dev(a) for a in gs])
        packed = torch.stack([p for p, _ in packs])
        gamma = torch.cat([gm for _, gm in packs])
        y = bl.bitlinear_forward_batched(x, g, packed, gamma).cpu().numpy()
        for b in range(B):
            ref = gu.orc().bitlinear(xs[b], gs[b], Ws[b])
            gu.assert_y_parity(y[b], ref["y"])


# Batched few-token problems on the K-split kernel (K = 2048, 4096): each
# slice has its own codes, scales and weights; N = 200 leaves a ragged group.
@pytest.mark.parametrize("K", [2048, 4096])
def test_forward_batched_few_tokens(K):
    B, N = 3, 200
    for M in (5, 8, 16):
        _say("batched few tokens", B, M, N, K)
        xs = [wl.x_normal(M, K, seed=70 + b) for b in range(B)]
        Ws = [wl.w_normal(N, K, seed=80 + b) for b in range(B)]
        gs = [wl.rms_weight(K, "random", seed=90 + b) for b in range(B)]
        packs = [gu.pack_on_gpu(W) for W in Ws]
        x = torch.stack([gu.to_dev_bf16(a) for a in xs])
        g = torch.stack([gu.to_dev(a) for a in gs])
        packed = torch.stack([p for p, _ in packs])
        gamma = torch.cat([gm for _, gm in packs])
        y = bl.bitlinear_forward_batched(x, g, packed, gamma).cpu().numpy()
        for b in range(B):
            ref = gu.orc().bitlinear(xs[b], gs[b], Ws[b])
            gu.assert_y_parity(y[b], ref["y"])


# Batched with a weight per slice and enough rows for the streaming layout:
# long exact rows, long ragged rows and ragged rows past the register budget.
@pytest.mark.parametrize("K", [4160, 5632, 6912])
def test_forward_batched_long_rows(K):
    B, M, N = 4, 20, 64
    _say("batched long rows", B, M, N, K)
    xs = [wl.x_normal(M, K, seed=40 + b) for b in range(B)]
    Ws = [wl.w_normal(N, K, seed=50 + b) for b in range(B)]
    gs = [wl.rms_weight(K, "random", seed=60 + b) for b in range(B)]
    packs = [gu.pack_on_gpu(W) for W in Ws]
    x = torch.stack([gu.to_dev_bf16(a) for a in xs])
    g = torch.stack([gu.to_dev(a) for a in gs])
    packed = torch.stack([p for p, _ in packs])
    gamma = torch.cat([gm for _, gm in packs])
    y = bl.bitlinear_forward_batched(x, g, packed, gamma).cpu().numpy()
    for b in range(B):
        ref = gu.orc().bitlinear(xs[b], gs[b], Ws[b])
        gu.assert_y_parity(y[b], ref["y"])


def test_forward_structural_zeros():
    """A zero activation row gives a zero output row; a zero weight row gives
    a zero output column; an all-zero matrix (gamma = 0) gives zeros."""
    M, N, K = 12, 96, 128
    x, W, g = gu.oracle_inputs(M, N, K, seed=4)
    x[3] = 0
    W[5] = 0
    packed, gamma = gu.pack_on_gpu(W)
    for kern in (GEMV, MFMA, DECODE):
        xs = x[:8] if kern == GEMV else (x[:4] if kern == DECODE else x)
        y = bl.bitlinear_forward(gu.to_dev_bf16(xs), gu.to_dev(g), packed, gamma, kernel=kern).cpu().numpy()
        assert np.all(y[3] == 0) and np.all(y[:, 5] == 0)
    packed0, gamma0 = gu.pack_on_gpu(np.zeros((N, K), np.float32))
    y = bl.bitlinear_forward(gu.to_dev_bf16(x), gu.to_dev(g), packed0, gamma0).cpu().numpy()
    assert np.all(y == 0)


def _near_tie_rows(M, K, seed):
    """Token rows whose two largest |x g| tie exactly with swapped factors,
    x = 6, g = 10 at one position and x = 10, g = 6 at another: which of
    the two is larger after the fp32 scaling (x r) g depends on each row's
    r, so some rows' absmax comes from the one and some from the other."""
    r = wl.rng(seed, 21)
    x = (r.standard_normal((M, K)) * 0.5).astype(np.float32)
    g = (0.5 + r.random(K)).astype(np.float32)
    i1, i2 = int(r.integers(0, K // 2)), int(r.integers(K // 2, K))
    x[:, i1], g[i1] = 6.0, 10.0
    x[:, i2], g[i2] = 10.0, 6.0
    x[M // 2:, [i1, i2]] *= -1.0
    return wl.f32_to_bf16_bits(x), g


@pytest.mark.parametrize("M,K", [(1, 64), (1, 2048), (2, 1024), (4, 4096), (1, 8192), (3, 2176), (1, 16384)])
def test_decode_quantisation_matches_stand_alone(M, K):
    """The fused decode kernel quantises its token rows itself; its codes and
    scales must equal those of the stand-alone quantiser, so its output must
    equal, bit for bit, the GEMV path's (stand-alone quantisation, then the
    GEMV: the same integer sums and the same rescale), here on rows built so
    that the two largest |x g| tie, and on plain rows."""
    N = 96
    W = wl.w_normal(N, K, seed=K)
    packed, gamma = gu.pack_on_gpu(W)
    for seed in range(6):
        if seed < 4:
            x, g = _near_tie_rows(M, K, seed + 10 * K)
        else:
            x, g = wl.x_normal(M, K, seed=seed), wl.rms_weight(K, "random", seed=seed)
        _say("decode vs stand-alone quantisation", M, K, "seed", seed)
        xd, gd = gu.to_dev_bf16(x), gu.to_dev(g)
        y_dec = bl.bitlinear_forward(xd, gd, packed, gamma, kernel=DECODE).cpu().numpy()
        y_gemv = bl.bitlinear_forward(xd, gd, packed, gamma, kernel=GEMV).cpu().numpy()
        assert np.array_equal(y_dec.view(np.uint32), y_gemv.view(np.uint32)), seed
        q, s = bl.bitlinear_quantize(xd, gd)
        ref = gu.orc().rmsnorm_quant(x, g, 1e-6)
        gu.assert_q_parity(q.cpu().numpy(), ref[0], s.cpu().numpy(), ref[1])


def test_forward_empty_and_deterministic():
    N, K = 64, 128
    x, W, g = gu.oracle_inputs(40, N, K, seed=5)
    packed, gamma = gu.pack_on_gpu(W)
    xe = torch.empty((0, K), dtype=torch.int16, device=gu.DEV)
    y = bl.bitlinear_forward(xe, gu.to_dev(g), packed, gamma)
    assert y.shape == (0, N)
    xd, gd = gu.to_dev_bf16(x), gu.to_dev(g)
    y1 = bl.bitlinear_forward(xd, gd, packed, gamma).cpu().numpy()
    y2 = bl.bitlinear_forward(xd, gd, packed, gamma).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_forward_rejects_bad_workspace():
    N, K = 64, 128
    x, W, g = gu.oracle_inputs(4, N, K, seed=6)
    packed, gamma = gu.pack_on_gpu(W)
    small = torch.empty(64, dtype=torch.uint8, device=gu.DEV)
    with pytest.raises(bl.BitlinearError) as e:
        bl.bitlinear_forward(gu.to_dev_bf16(x), gu.to_dev(g), packed, gamma, ws=small)
    assert e.value.status == bl.BITLINEAR_ERR_WORKSPACE


# --------------------------------------------------------------------------
# GLU channel mixer
# --------------------------------------------------------------------------

def _glu_inputs(M, D, F, seed=0):
    x = wl.x_normal(M, D, seed=seed)
    g_gu = wl.rms_weight(D, "random", seed=seed + 1)
    g_dn = wl.rms_weight(F, "random", seed=seed + 2)
    W_gu = wl.w_normal(2 * F, D, seed=seed)
    W_dn = wl.w_normal(D, F, seed=seed, stream=wl.STREAM_W2)
    return x, g_gu, W_gu, g_dn, W_dn


def assert_h_parity(h_gpu, h_ref):
    """bf16 hidden: equal except rare one-ulp rounding flips (the oracle forms
    SiLU(gate)*up in fp64, the kernel in fp32)."""
    diff = np.abs(h_gpu.view(np.int16).astype(np.int32) - h_ref.view(np.int16).astype(np.int32))
    assert diff.max(initial=0) <= 1 and np.mean(diff != 0) <= 1e-3, (diff.max(), np.mean(diff != 0))


# (768, 64, 11008): 258 tiles of 256 x 256 (two rounds of 256 blocks), so the
# gate|up product takes 128 x 256 tiles (three rounds of half the work).
@pytest.mark.parametrize("M,D,F", [(1, 256, 320), (5, 256, 320), (130, 256, 320), (1, 3008, 64), (3, 2048, 5632),
                                   (2, 208, 96), (768, 64, 11008)])
def test_glu_hidden(M, D, F):
    x, g_gu, W_gu, g_dn, W_dn = _glu_inputs(M, D, F, seed=M)
    ref = gu.orc().glu(x, g_gu, W_gu, g_dn, W_dn)
    packed, gamma = gu.pack_on_gpu(W_gu)
    for kern in kernels_for(M, D):
        _say("glu hidden", M, D, F, "kernel", kern)
        h = bl.bitlinear_glu_hidden(gu.to_dev_bf16(x), gu.to_dev(g_gu), packed, gamma, kernel=kern)
        assert_h_parity(gu.from_dev_bf16(h), ref["h"])


@pytest.mark.parametrize("M,D,F", [(1, 256, 320), (7, 256, 320), (200, 256, 320), (4, 512, 1024)])
def test_glu_forward(M, D, F):
    _say("glu forward", M, D, F)
    x, g_gu, W_gu, g_dn, W_dn = _glu_inputs(M, D, F, seed=M + 100)
    ref = gu.orc().glu(x, g_gu, W_gu, g_dn, W_dn)
    pgu, ggu = gu.pack_on_gpu(W_gu)
    pdn, gdn = gu.pack_on_gpu(W_dn)
    y = bl.bitlinear_glu_forward(gu.to_dev_bf16(x), gu.to_dev(g_gu), pgu, ggu, gu.to_dev(g_dn), pdn,
                                 gdn).cpu().numpy()
    gu.assert_y_parity(y, ref["y"])


# Batched mixers: one-token problems take the fused kernel for both
# projections, five tokens the quantisation pass and few-token product, 130
# the tiled MFMA product; each mixer has its own weights and RMSNorm gains.
@pytest.mark.parametrize("M", [1, 5, 130])
def test_glu_forward_batched(M):
    B, D, F = 3, 256, 320
    _say("glu forward batched", B, M, D, F)
    cases = [_glu_inputs(M, D, F, seed=M + 200 + b) for b in range(B)]
    packs = [(gu.pack_on_gpu(c[2]), gu.pack_on_gpu(c[4])) for c in cases]
    x = torch.stack([gu.to_dev_bf16(c[0]) for c in cases])
    g_gu = torch.stack([gu.to_dev(c[1]) for c in cases])
    g_dn = torch.stack([gu.to_dev(c[3]) for c in cases])
    pgu = torch.stack([p[0][0] for p in packs])
    ggu = torch.cat([p[0][1] for p in packs])
    pdn = torch.stack([p[1][0] for p in packs])
    gdn = torch.cat([p[1][1] for p in packs])
    y = bl.bitlinear_glu_forward_batched(x, g_gu, pgu, ggu, g_dn, pdn, gdn).cpu().numpy()
    for b, c in enumerate(cases):
        ref = gu.orc().glu(*c)
        gu.assert_y_parity(y[b], ref["y"])


@pytest.mark.parametrize("M,D,F", [(1, 64, 96), (2, 2048, 5632), (3, 512, 1040), (6, 256, 2048),
                                   (11, 2048, 1024), (40, 128, 320), (300, 256, 96), (130, 1024, 2048)])
def test_glu_forward_more_shapes(M, D, F):
    """GLU mixers across the dispatch bands of both projections (fused
    decode, few-token, small and large MFMA tiles), D and F ragged against
    the tile widths."""
    _say("glu shapes", M, D, F)
    c = _glu_inputs(M, D, F, seed=M + D + F)
    pgu, ggu = gu.pack_on_gpu(c[2])
    pdn, gdn = gu.pack_on_gpu(c[4])
    xd = gu.to_dev_bf16(c[0])
    y = bl.bitlinear_glu_forward(xd, gu.to_dev(c[1]), pgu, ggu, gu.to_dev(c[3]), pdn, gdn).cpu().numpy()
    h = gu.from_dev_bf16(bl.bitlinear_glu_hidden(xd, gu.to_dev(c[1]), pgu, ggu))
    ref = gu.orc().glu(*c)
    assert_h_parity(h, ref["h"])
    gu.assert_y_parity(y, ref["y"])


# --------------------------------------------------------------------------
# workloads at full size (oracle on sampled rows; rows are independent)
# --------------------------------------------------------------------------

def _sample_rows(M, n, seed):
    r = wl.rng(seed, 9)
    rows = set(r.choice(M, size=min(n, M), replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(rows))


@pytest.mark.parametrize("M", [1, 8])
def test_full_decode_2048(M):
    _say("full decode", M)
    x, W, g = gu.oracle_inputs(M, 2048, 2048, seed=0, g_kind="ones")
    ref = gu.orc().bitlinear(x, g, W)
    packed, gamma = gu.pack_on_gpu(W)
    y = bl.bitlinear_forward(gu.to_dev_bf16(x), gu.to_dev(g), packed, gamma).cpu().numpy()
    gu.assert_y_parity(y, ref["y"], np.ones(M, bool))


def _check_layer_stack(L, M, N, K, nrows):
    """L independent layers in one batched call: sampled rows of sampled
    layers match the oracle, and each sampled layer matches a single-layer
    call bit for bit (the same arithmetic per row under a different
    blocking)."""
    x = wl.x_normal(L * M, K, seed=0).reshape(L, M, K)
    g = np.ones(K, np.float32)
    packed = torch.empty((L, N, K // 4), dtype=torch.uint8, device=gu.DEV)
    gamma = torch.empty(L, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(bl.bitlinear_pack_workspace_bytes(N, K), dtype=torch.uint8, device=gu.DEV)
    for layer in range(L):
        W = wl.w_normal_device(N, K, seed=0, layer=layer, device=gu.DEV)
        bl.bitlinear_pack_weights(W, packed=packed[layer], gamma=gamma[layer:layer + 1], ws=ws)
    xd = gu.to_dev_bf16(x.reshape(L * M, K)).view(L, M, K)
    gd = torch.ones((L, K), dtype=torch.float32, device=gu.DEV)
    y = bl.bitlinear_forward_batched(xd, gd, packed, gamma).cpu().numpy()
    for layer in (0, 1, L // 3, L - 2, L - 1):
        W = wl.w_normal_device(N, K, seed=0, layer=layer, device=gu.DEV).cpu().numpy()
        rows = _sample_rows(M, nrows, layer)
        ref = gu.orc().bitlinear(x[layer][rows], g, W)
        gu.assert_y_parity(y[layer][rows], ref["y"])
        y1 = bl.bitlinear_forward(xd[layer], gd[layer], packed[layer], gamma[layer:layer + 1]).cpu().numpy()
        assert np.array_equal(y1, y[layer]), layer
    del packed
    torch.cuda.empty_cache()


# The timed decode steps exactly as launched: L layers in one batched call,
# with the layer counts that make about 1 GiB of weights.
@pytest.mark.parametrize("L,M,N,K", [(1024, 1, 2048, 2048), (1024, 8, 2048, 2048), (645, 1, 2560, 2560),
                                     (240, 1, 6912, 2560), (239, 1, 2560, 6912)])
def test_full_decode_layers(L, M, N, K):
    _say("full decode, layers", L, M, N, K)
    _check_layer_stack(L, M, N, K, M)


# The timed 64- and 512-token steps of the 2560/6912 shapes exactly as
# launched: about 1 GiB of layers in one batched call on the MFMA tiles.
@pytest.mark.parametrize("L,M,N,K", [(408, 64, 2560, 2560), (164, 64, 6912, 2560), (179, 64, 2560, 6912),
                                     (112, 512, 2560, 2560), (50, 512, 6912, 2560), (64, 512, 2560, 6912)])
def test_full_sweep_layers(L, M, N, K):
    _say("full sweep, layers", L, M, N, K)
    _check_layer_stack(L, M, N, K, 8)


def test_full_glu_128_mixers():
    """The timed one-token GLU step exactly as launched: 128 mixers of
    2048/5632 in one batched call; sampled mixers against the oracle and
    against single-mixer calls, bit for bit."""
    L, D, F = 128, 2048, 5632
    _say("full glu, 128 mixers")
    x = wl.x_normal(L, D, seed=2).reshape(L, 1, D)
    pgu = torch.empty((L, 2 * F, D // 4), dtype=torch.uint8, device=gu.DEV)
    pdn = torch.empty((L, D, F // 4), dtype=torch.uint8, device=gu.DEV)
    ggu = torch.empty(L, dtype=torch.float32, device=gu.DEV)
    gdn = torch.empty(L, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(max(bl.bitlinear_pack_workspace_bytes(2 * F, D), bl.bitlinear_pack_workspace_bytes(D, F)),
                     dtype=torch.uint8, device=gu.DEV)
    w_gu = lambda layer: wl.w_normal_device(2 * F, D, seed=2, layer=2 * layer, device=gu.DEV)
    w_dn = lambda layer: wl.w_normal_device(D, F, seed=2, layer=2 * layer + 1, device=gu.DEV)
    for layer in range(L):
        bl.bitlinear_pack_weights(w_gu(layer), packed=pgu[layer], gamma=ggu[layer:layer + 1], ws=ws)
        bl.bitlinear_pack_weights(w_dn(layer), packed=pdn[layer], gamma=gdn[layer:layer + 1], ws=ws)
    xd = gu.to_dev_bf16(x.reshape(L, D)).view(L, 1, D)
    g_gu = torch.ones((L, D), dtype=torch.float32, device=gu.DEV)
    g_dn = torch.ones((L, F), dtype=torch.float32, device=gu.DEV)
    y = bl.bitlinear_glu_forward_batched(xd, g_gu, pgu, ggu, g_dn, pdn, gdn).cpu().numpy()
    ones_d, ones_f = np.ones(D, np.float32), np.ones(F, np.float32)
    for layer in (0, 1, 77, L - 1):
        ref = gu.orc().glu(x[layer], ones_d, w_gu(layer).cpu().numpy(), ones_f, w_dn(layer).cpu().numpy())
        gu.assert_y_parity(y[layer], ref["y"])
        y1 = bl.bitlinear_glu_forward(xd[layer], g_gu[layer], pgu[layer], ggu[layer:layer + 1], g_dn[layer],
                                      pdn[layer], gdn[layer:layer + 1]).cpu().numpy()
        assert np.array_equal(y1, y[layer]), layer
    del pgu, pdn
    torch.cuda.empty_cache()


def _full_sampled(M, N, K, recipe, of, os_, nrows, kernel=bl.BITLINEAR_KERNEL_AUTO):
    x, W, g = gu.oracle_inputs(M, N, K, seed=0, recipe=recipe, outlier_frac=of, outlier_scale=os_,
                               g_kind="ones")
    packed, gamma = gu.pack_on_gpu(W)
    xd, gd = gu.to_dev_bf16(x), gu.to_dev(g)
    y = bl.bitlinear_forward(xd, gd, packed, gamma, kernel=kernel).cpu().numpy()
    q, s = bl.bitlinear_quantize(xd, gd)
    rows = _sample_rows(M, nrows, M + N + K)
    ref = gu.orc().bitlinear(x[rows], g, W)
    assert gamma.item() == ref["gamma"]
    qr = q.cpu().numpy()[rows]
    gu.assert_q_parity(qr, ref["q"], s.cpu().numpy()[rows], ref["s"])
    gu.assert_y_parity(y[rows], ref["y"], np.all(qr == ref["q"], axis=1))


def test_full_prefill_8192():
    _say("full prefill 8192x2048x2048")
    _full_sampled(8192, 2048, 2048, "student_t3", 0.0, 1.0, 48)


@pytest.mark.parametrize("M", [1, 64, 512, 4096, 16384])
@pytest.mark.parametrize("K,N", [(2560, 2560), (2560, 6912), (6912, 2560)])
def test_full_sweep_2560(M, K, N):
    _say("sweep", M, K, N)
    _full_sampled(M, N, K, "normal", 0.005, 50.0, 12)


@pytest.mark.parametrize("M", [1, 4096])
def test_full_glu_2048_5632(M):
    _say("full glu", M)
    D, F = 2048, 5632
    x, g_gu, W_gu, g_dn, W_dn = _glu_inputs(M, D, F, seed=0)
    g_gu = np.ones(D, np.float32)
    g_dn = np.ones(F, np.float32)
    pgu, ggu = gu.pack_on_gpu(W_gu)
    pdn, gdn = gu.pack_on_gpu(W_dn)
    xd = gu.to_dev_bf16(x)
    y = bl.bitlinear_glu_forward(xd, gu.to_dev(g_gu), pgu, ggu, gu.to_dev(g_dn), pdn, gdn).cpu().numpy()
    h = gu.from_dev_bf16(bl.bitlinear_glu_hidden(xd, gu.to_dev(g_gu), pgu, ggu))
    rows = _sample_rows(M, 8, 77)
    ref = gu.orc().glu(x[rows], g_gu, W_gu, g_dn, W_dn)
    assert_h_parity(h[rows], ref["h"])
    gu.assert_y_parity(y[rows], ref["y"])
