"""Pins of the CPU oracle to facts fixed outside it.

Each pin_* function takes an oracle.Oracle and raises AssertionError when
the oracle disagrees with something the pages or the mathematics fix: a
closed form, an invariant, brute force in exact rational arithmetic, a
library routine that computes the same plain definition, or the
quantisation error bound.  test_oracle_pins.py runs them on the oracle;
test_oracle_mutants.py runs them on deliberately altered builds of the
oracle and checks that every alteration is caught by at least one pin.
"""
import math
import os
import sys
from fractions import Fraction

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import workloads as wl  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# bf16 conversions
# --------------------------------------------------------------------------

def pin_bf16_widening(orc):
    """bf16 is the top half of an fp32 pattern: 0x3F80 = 1, 0xC040 = -3,
    0x0001 = 2^-133 (smallest subnormal), 0x7F7F = largest finite."""
    assert orc.bf16_to_float(0x3F80) == 1.0
    assert orc.bf16_to_float(0xC040) == -3.0
    assert orc.bf16_to_float(0x0001) == np.float32(2.0 ** -133)
    assert orc.bf16_to_float(0x7F7F) == np.float32((2 - 2 ** -7) * 2.0 ** 127)


def pin_bf16_rounding(orc):
    """Nearest bf16, ties to even: worked ties around 1.0 (spacing 2^-7),
    then brute force on random doubles: the result is no farther than either
    neighbouring bf16 value."""
    one = 0x3F80
    assert orc.double_to_bf16(1.0) == one
    assert orc.double_to_bf16(1.0 + 2.0 ** -8) == one          # tie -> even (…80)
    assert orc.double_to_bf16(1.0 + 3 * 2.0 ** -8) == one + 2  # tie -> even (…82)
    assert orc.double_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == one + 1
    assert orc.double_to_bf16(-1.0) == 0x8000 | one
    assert orc.double_to_bf16(0.0) == 0
    r = wl.rng(11, 0)
    vals = r.standard_normal(400) * np.exp(r.uniform(-30, 30, 400))
    for v in vals:
        b = orc.double_to_bf16(v)
        got = float(orc.bf16_to_float(b))
        assert math.copysign(1.0, got) == math.copysign(1.0, v)
        for nb in ((b + 1) & 0xFFFF, (b - 1) & 0xFFFF):
            other = float(orc.bf16_to_float(nb))
            if math.isfinite(other) and (nb & 0x7FFF) != 0x7F80:
                assert abs(got - v) <= abs(other - v), (v, b, nb)


# --------------------------------------------------------------------------
# absmean weight scale and ternarisation
# --------------------------------------------------------------------------

def pin_gamma_closed_forms(orc):
    """gamma of +-a everywhere is a; of zeros is 0; of N(0, sigma^2) is
    sigma*sqrt(2/pi) within sampling error; equals NumPy's fp64 mean of |W|."""
    a = np.float32(0.0371)
    W = np.full((7, 48), a, np.float32)
    W[::2, 1::3] *= -1
    assert orc.gamma(W) == a
    assert orc.gamma(np.zeros((3, 16), np.float32)) == 0.0
    W = wl.w_normal(256, 512, 0.02, seed=5)
    g = float(orc.gamma(W))
    expect = 0.02 * math.sqrt(2 / math.pi)
    sd = 0.02 * math.sqrt(1 - 2 / math.pi) / math.sqrt(W.size)
    assert abs(g - expect) < 6 * sd, (g, expect)
    assert orc.gamma(W) == np.float32(np.abs(W.astype(np.float64)).mean())


def pin_ternarize_closed_forms(orc):
    """Codes are in {-1,0,1}; +-a with a >> 1e-5 maps to +-1; 0 maps to 0;
    thresholds at half the divisor; ties round to even (0.5 -> 0, 1.5 -> 2 ->
    clipped 1); odd symmetry."""
    gamma = np.float32(0.02)
    d = np.float32(gamma + np.float32(1e-5))
    cases = {
        0.0: 0, 0.49: 0, 0.51: 1, -0.51: -1, 0.99: 1, 1.49: 1, 1.51: 1, 2.6: 1,
        -7.0: -1, 0.5: 0, -0.5: 0, 1.5: 1,
    }
    vals = np.array([list(cases)], np.float64)
    W = (vals * np.float64(d)).astype(np.float32)
    # nudge the exact ties so that W / d is exactly the tie in fp32
    for j, c in enumerate(cases):
        if abs(c) in (0.5, 1.5):
            W[0, j] = np.float32(np.float32(c) * d)
            assert np.float32(W[0, j] / d) == np.float32(c)
    w = orc.ternarize(W, gamma)
    assert list(w[0]) == list(cases.values()), (list(w[0]), list(cases.values()))
    a = np.float32(0.3)
    W = np.array([[a, -a, a, 0]], np.float32)
    assert list(orc.ternarize(W, orc.gamma(W))[0]) == [1, -1, 1, 0]
    W = wl.w_normal(64, 128, seed=3)
    g = orc.gamma(W)
    assert np.array_equal(orc.ternarize(-W, g), -orc.ternarize(W, g))


def pin_ternarize_statistics(orc):
    """For N(0, sigma^2) weights the zero fraction is P(|Z| < sqrt(2/pi)/2)
    = 0.3101 and the +1/-1 fractions are equal, within sampling error."""
    W = wl.w_normal(512, 512, seed=7)
    w = orc.ternarize(W, orc.gamma(W))
    assert set(np.unique(w)) <= {-1, 0, 1}
    z = float(np.mean(w == 0))
    p0 = math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2))
    sd = math.sqrt(p0 * (1 - p0) / w.size)
    assert abs(z - p0) < 6 * sd, (z, p0)
    pos, neg = float(np.mean(w == 1)), float(np.mean(w == -1))
    assert abs(pos - neg) < 6 * math.sqrt(0.35 / w.size)


# --------------------------------------------------------------------------
# packed storage
# --------------------------------------------------------------------------

def _golden_pack():
    with open(os.path.join(GOLDEN, "pack_example.txt")) as f:
        lines = [ln for ln in f if not ln.startswith("#") and ln.strip()]
    kv = dict(ln.split(":", 1) for ln in lines)
    w = np.array([int(t) for t in kv["weights"].split()], np.int8)[None, :]
    b = np.array([int(t, 16) for t in kv["bytes"].split()], np.uint8)[None, :]
    return w, b


def pin_pack_golden(orc):
    """The hand-worked row in tests/golden/pack_example.txt packs to its
    bytes and unpacks back."""
    w, b = _golden_pack()
    assert np.array_equal(orc.pack(w), b), orc.pack(w)
    assert np.array_equal(orc.unpack(b, 16), w)


def pin_pack_roundtrip(orc):
    """unpack(pack(w)) == w for random codes over several groups and rows;
    the code 3 and K % 16 != 0 are rejected; a zero row packs to 0x55."""
    r = wl.rng(21, 0)
    w = r.integers(-1, 2, size=(9, 80)).astype(np.int8)
    p = orc.pack(w)
    assert p.shape == (9, 20)
    assert np.array_equal(orc.unpack(p, 80), w)
    assert np.all(orc.pack(np.zeros((2, 32), np.int8)) == 0x55)
    bad = p.copy()
    bad[4, 7] |= 0xC0
    try:
        orc.unpack(bad, 80)
        raise AssertionError("code 3 accepted")
    except ValueError:
        pass
    try:
        orc.pack(np.zeros((1, 12), np.int8))
        raise AssertionError("K=12 accepted")
    except ValueError:
        pass


# --------------------------------------------------------------------------
# RMSNorm + absmax quantisation
# --------------------------------------------------------------------------

def _round_half_even(fr):
    fl = math.floor(fr)
    d = fr - fl
    if d > Fraction(1, 2):
        return fl + 1
    if d < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def pin_quant_exact_rational(orc):
    """r cancels: q_k = round(127 * x_k g_k / max_j |x_j g_j|) exactly.
    Brute force in rationals on small rows with a non-trivial gain; elements
    within 1e-3 of a rounding tie are skipped (fp32 may fall either side)."""
    M, K = 6, 48
    x = wl.x_normal(M, K, seed=31, outlier_frac=0.05, outlier_scale=20.0)
    g = wl.rms_weight(K, "random", seed=31)
    q, s = orc.rmsnorm_quant(x, g)
    xf = wl.bf16_bits_to_f32(x)
    checked = 0
    for m in range(M):
        prod = [Fraction(float(xf[m, k])) * Fraction(float(g[k])) for k in range(K)]
        amax = max(abs(p) for p in prod)
        for k in range(K):
            exact = 127 * prod[k] / amax
            if abs(abs(exact - math.floor(exact)) - Fraction(1, 2)) < Fraction(1, 1000):
                continue
            assert q[m, k] == _round_half_even(exact), (m, k, float(exact), q[m, k])
            checked += 1
    assert checked > M * K * 0.95


def pin_quant_scale_formula(orc):
    """s = 127 / (max_k |x_k| * g_k * r), r = 1/sqrt(mean(x^2) + eps), eps
    inside the root: checked in fp64 to 1e-6 on ordinary rows and on tiny
    rows where mean(x^2) is comparable to eps."""
    K = 64
    x = wl.x_normal(4, K, seed=41)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    xf[2] *= 1e-3
    xf[3] *= 3e-4
    x = wl.f32_to_bf16_bits(xf.astype(np.float32))
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    g = wl.rms_weight(K, "random", seed=41).astype(np.float64)
    for eps in (1e-6, 1e-3):
        _, s = orc.rmsnorm_quant(x, g.astype(np.float32), eps)
        for m in range(4):
            r = 1.0 / math.sqrt(np.mean(xf[m] ** 2) + eps)
            expect = 127.0 / np.max(np.abs(xf[m] * g) * r)
            assert abs(s[m] / expect - 1) < 1e-6, (m, eps, s[m], expect)


def pin_quant_invariants(orc):
    """q in [-127, 127]; the row maximum maps to +-127; q(-x) = -q(x); a
    zero row gives q = 0 and s = 127/1e-5; a constant row gives +-127."""
    M, K = 8, 96
    x = wl.x_student_t(M, K, seed=51)
    g = wl.rms_weight(K, "random", seed=51)
    q, s = orc.rmsnorm_quant(x, g)
    assert q.min() >= -127 and q.max() <= 127
    xg = np.abs(wl.bf16_bits_to_f32(x) * g)
    for m in range(M):
        assert abs(int(q[m, int(np.argmax(xg[m]))])) == 127
    qn, sn = orc.rmsnorm_quant(x ^ np.uint16(0x8000), g)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    z = np.zeros((2, K), np.uint16)
    z[1, :] = 0xBF80  # -1.0
    qz, sz = orc.rmsnorm_quant(z, np.ones(K, np.float32))
    assert np.all(qz[0] == 0) and sz[0] == np.float32(127.0) / np.float32(1e-5)
    assert np.all(qz[1] == -127)


# --------------------------------------------------------------------------
# ternary accumulation and rescale
# --------------------------------------------------------------------------

def pin_accumulate_vs_integer_matmul(orc):
    """The add/subtract loop equals the integer product sum_k q w in int64
    (NumPy), bit for bit, on a non-square case."""
    r = wl.rng(61, 0)
    q = r.integers(-128, 128, size=(5, 96)).astype(np.int8)
    w = r.integers(-1, 2, size=(7, 96)).astype(np.int8)
    ref = q.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(orc.accumulate(q, w), ref)


def pin_accumulate_structure(orc):
    """Identity weights return q; a single +1 at (n, k) copies column k; a
    zero row gives a zero column; acc(-w) = -acc(w); permuting k in both
    operands leaves acc unchanged."""
    r = wl.rng(62, 0)
    K = 32
    q = r.integers(-127, 128, size=(4, K)).astype(np.int8)
    assert np.array_equal(orc.accumulate(q, np.eye(K, dtype=np.int8)), q.astype(np.int32))
    w = np.zeros((3, K), np.int8)
    w[1, 5] = 1
    w[2, 9] = -1
    acc = orc.accumulate(q, w)
    assert np.all(acc[:, 0] == 0)
    assert np.array_equal(acc[:, 1], q[:, 5].astype(np.int32))
    assert np.array_equal(acc[:, 2], -q[:, 9].astype(np.int32))
    w = r.integers(-1, 2, size=(6, K)).astype(np.int8)
    assert np.array_equal(orc.accumulate(q, -w), -orc.accumulate(q, w))
    perm = r.permutation(K)
    assert np.array_equal(orc.accumulate(q[:, perm], w[:, perm]), orc.accumulate(q, w))


def pin_rescale_vs_dequantised_matmul(orc):
    """y equals the fp64 product of the dequantised operands,
    (q / s) @ (gamma * w)^T, to 1e-12 relative."""
    M, N, K = 5, 11, 64
    x = wl.x_normal(M, K, seed=71, outlier_frac=0.02, outlier_scale=20.0)
    g = wl.rms_weight(K, "random", seed=71)
    W = wl.w_normal(N, K, seed=71)
    out = orc.bitlinear(x, g, W)
    deq_x = out["q"].astype(np.float64) / out["s"].astype(np.float64)[:, None]
    deq_w = out["w"].astype(np.float64) * float(out["gamma"])
    ref = deq_x @ deq_w.T
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # zero weight row -> zero output column
    W2 = W.copy()
    W2[3] = 0
    y2 = orc.bitlinear(x, g, W2)["y"]
    assert np.all(y2[:, 3] == 0.0)


def pin_bitlinear_error_bound(orc):
    """The quantised layer stays within the int8 rounding bound of the
    unquantised one: with xn the fp64 RMSNorm output and W~ = gamma * w,
    |y - xn W~^T| <= gamma * sum_k |w_nk| * (0.5 / s + 1e-6 |xn_k|) per element.
    Checked on a non-square layer with a non-trivial gain."""
    M, N, K = 6, 40, 128
    x = wl.x_normal(M, K, seed=81, outlier_frac=0.01, outlier_scale=20.0)
    g = wl.rms_weight(K, "random", seed=81)
    W = wl.w_normal(N, K, seed=81)
    out = orc.bitlinear(x, g, W)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(xf ** 2, axis=1, keepdims=True) + 1e-6)
    xn = xf * r * g.astype(np.float64)
    wt = out["w"].astype(np.float64) * float(out["gamma"])
    y_cont = xn @ wt.T
    s = out["s"].astype(np.float64)
    bound = (np.abs(wt) @ (0.5 / s[:, None] + 1e-6 * np.abs(xn)).T).T
    err = np.abs(out["y"] - y_cont)
    assert np.all(err <= bound * 1.0001 + 1e-30), float((err / (bound + 1e-30)).max())
    # the bound is not vacuous: it sits well below the outputs, and the
    # typical error (rounding errors average out) is a small fraction of them
    assert np.median(np.abs(y_cont)) > 2 * np.median(bound)
    assert np.median(err) < 0.05 * np.median(np.abs(y_cont))


# --------------------------------------------------------------------------
# GLU channel mixer
# --------------------------------------------------------------------------

def pin_glu_step(orc):
    """h = bf16(SiLU(gate) * up) with gate the first F rows of the fused
    projection, SiLU(v) = v * sigmoid(v) evaluated independently in NumPy,
    and y = the down BitLinear of h.  Zero gate rows give h = 0 (SiLU(0) = 0)."""
    M, D, F = 3, 64, 48
    x = wl.x_normal(M, D, seed=91)
    g_gu = wl.rms_weight(D, "random", seed=91)
    g_dn = wl.rms_weight(F, "random", seed=92)
    W_gu = wl.w_normal(2 * F, D, seed=91)
    W_dn = wl.w_normal(D, F, seed=92)
    out = orc.glu(x, g_gu, W_gu, g_dn, W_dn)
    z = orc.bitlinear(x, g_gu, W_gu)["y"]
    gate, up = z[:, :F], z[:, F:]
    h_val = gate / (1.0 + np.exp(-gate)) * up
    h_bits = np.array([[orc.double_to_bf16(v) for v in row] for row in h_val], np.uint16)
    hf = wl.bf16_bits_to_f32(h_bits).astype(np.float64)
    # NumPy's and libm's exp agree to an ulp or so: bf16 ties aside, equal
    close = np.abs(wl.bf16_bits_to_f32(out["h"]) - hf) <= 2.0 ** -7 * np.abs(hf)
    assert close.all()
    assert np.mean(out["h"] == h_bits) > 0.999
    y_ref = orc.bitlinear(out["h"], g_dn, W_dn)["y"]
    assert np.array_equal(out["y"], y_ref)
    W0 = W_gu.copy()
    W0[:F] = 0
    out0 = orc.glu(x, g_gu, W0, g_dn, W_dn)
    assert np.all(wl.bf16_bits_to_f32(out0["h"]) == 0.0)
    assert np.all(out0["y"] == 0.0)


def pin_glu_silu_invariants(orc):
    """SiLU and the gate/up split pinned by properties rather than by the
    formula: since sigmoid(v) + sigmoid(-v) = 1, SiLU(v) - SiLU(-v) = v, so
    negating the gate rows of W (which negates gate exactly and leaves up)
    must change h by gate * up, up to bf16 rounding; far out on either side
    SiLU(v) -> v and SiLU(v) -> 0.  Scaling the RMSNorm weight by 2^12
    scales z = [gate, up] by exactly 2^12 (the per-token scale absorbs it),
    which pushes most gates past |30|."""
    M, D, F = 4, 64, 40
    x = wl.x_normal(M, D, seed=93)
    g_gu = wl.rms_weight(D, "random", seed=93)
    g_dn = wl.rms_weight(F, "random", seed=94)
    W_gu = wl.w_normal(2 * F, D, seed=93)
    W_dn = wl.w_normal(D, F, seed=94)
    W_neg = W_gu.copy()
    W_neg[:F] = -W_neg[:F]
    z1 = orc.bitlinear(x, g_gu, W_gu)["y"]
    for c in (1.0, 4096.0):
        gc = (g_gu * np.float32(c)).astype(np.float32)
        z = orc.bitlinear(x, gc, W_gu)["y"]
        assert np.array_equal(z, z1 * c)
        gate, up = z[:, :F], z[:, F:]
        zn = orc.bitlinear(x, gc, W_neg)["y"]
        assert np.array_equal(zn[:, :F], -gate) and np.array_equal(zn[:, F:], up)
        hp = wl.bf16_bits_to_f32(orc.glu(x, gc, W_gu, g_dn, W_dn)["h"]).astype(np.float64)
        hm = wl.bf16_bits_to_f32(orc.glu(x, gc, W_neg, g_dn, W_dn)["h"]).astype(np.float64)
        assert np.all(np.abs(hp - hm - gate * up) <= 2.0 ** -8 * (np.abs(hp) + np.abs(hm)) + 1e-30)
        if c > 1.0:
            pos, neg = gate > 30.0, gate < -30.0
            assert pos.sum() >= 10 and neg.sum() >= 10
            prod = np.array([orc.double_to_bf16(v) for v in (gate * up)[pos]], np.uint16)
            assert np.array_equal(wl.bf16_bits_to_f32(prod).astype(np.float64), hp[pos])
            assert np.all(np.abs(hp[neg]) <= 1e-11 * np.abs(up[neg]))


# --------------------------------------------------------------------------
# backward pass (straight-through estimator)
# --------------------------------------------------------------------------

def _backward_case(orc, M, N, K, seed, eps=1e-6):
    x = wl.x_normal(M, K, seed=seed, outlier_frac=0.03, outlier_scale=20.0)
    g = wl.rms_weight(K, "random", seed=seed)
    W = wl.w_normal(N, K, seed=seed)
    gamma = orc.gamma(W)
    w = orc.ternarize(W, gamma)
    dy = wl.dy_normal(M, N, seed=seed)
    return x, g, W, gamma, w, dy, orc.backward(x, g, w, gamma, dy, eps)


def pin_backward_vs_autograd(orc):
    """The gradients equal torch.autograd (fp64, CPU) of the forward written
    with both quantisers passed straight through:
    xq = xn + (q/s - xn).detach(), W~ = W + (gamma w - W).detach(),
    loss = sum((xq @ W~^T) * dy), xn = x r g, r = (mean(x^2) + eps)^-1/2."""
    import torch

    eps = 1e-6
    for M, N, K, seed in ((6, 40, 48, 81), (3, 17, 5, 82), (9, 8, 33, 83)):
        x, g, W, gamma, w, dy, got = _backward_case(orc, M, N, K, seed, eps)
        q, s = orc.rmsnorm_quant(x, g, eps)
        f64 = torch.float64
        xt = torch.tensor(wl.bf16_bits_to_f32(x), dtype=f64, requires_grad=True)
        gt = torch.tensor(g, dtype=f64, requires_grad=True)
        Wt = torch.tensor(W, dtype=f64, requires_grad=True)
        r = torch.rsqrt(xt.pow(2).mean(dim=1, keepdim=True) + float(np.float32(eps)))
        xn = xt * r * gt
        xdq = torch.tensor(q.astype(np.float64) / s.astype(np.float64)[:, None])
        xq = xn + (xdq - xn).detach()
        Wq = Wt + (float(gamma) * torch.tensor(w, dtype=f64) - Wt).detach()
        loss = ((xq @ Wq.T) * torch.tensor(dy, dtype=f64)).sum()
        loss.backward()
        for name, ref in (("dx", xt.grad), ("dg", gt.grad), ("dW", Wt.grad)):
            ref = ref.numpy()
            tol = 1e-11 * max(np.abs(ref).max(), 1e-300)
            assert np.abs(got[name] - ref).max() <= tol, (name, M, N, K)


def pin_backward_scale_invariance(orc):
    """RMSNorm is invariant to scaling its input (up to eps): doubling x
    halves dx and leaves dg unchanged, and sum_k x_k dx_k ~ 0 for every row
    (the gradient is orthogonal to the direction that does not change xn).
    A one-hot dy[m][n] reaches dxn only through row n of gamma * w."""
    M, N, K = 5, 24, 64
    x, g, W, gamma, w, dy, out = _backward_case(orc, M, N, K, 91)
    x2 = wl.f32_to_bf16_bits(2.0 * wl.bf16_bits_to_f32(x))  # exact
    out2 = orc.backward(x2, g, w, gamma, dy)
    assert np.allclose(out2["dx"], 0.5 * out["dx"], rtol=1e-5, atol=1e-5 * np.abs(out["dx"]).max())
    assert np.allclose(out2["dg"], out["dg"], rtol=1e-5, atol=1e-5 * np.abs(out["dg"]).max())
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    proj = (xf * out["dx"]).sum(axis=1)
    assert np.all(np.abs(proj) <= 1e-5 * (np.abs(xf * out["dx"]).sum(axis=1) + 1e-300))
    # one-hot output gradient: with g = 1 and r the row's norm factor,
    # r * dxn[m] minus its projection on x[m] is dx[m]; the projection
    # vanishes against x, so dx[m] . v = r gamma w[n] . v for v orthogonal to x[m]
    m, n = 2, 7
    e = np.zeros((M, N), np.float32)
    e[m, n] = 1.0
    ones = np.ones(K, np.float32)
    o = orc.backward(x, ones, w, gamma, e)
    assert np.all(o["dx"][np.arange(M) != m] == 0.0)
    assert np.all(o["dW"][np.arange(N) != n] == 0.0)
    v = w[n].astype(np.float64)
    v = v - (v @ xf[m]) / (xf[m] @ xf[m]) * xf[m]
    r = 1.0 / math.sqrt((xf[m] ** 2).mean() + float(np.float32(1e-6)))
    assert math.isclose(o["dx"][m] @ v, r * float(gamma) * (w[n].astype(np.float64) @ v), rel_tol=1e-9)


def pin_backward_weight_gradient(orc):
    """dW is the outer-product sum of dy and the dequantised activations:
    for a single token it is dy[0][n] * q[0][k] / s[0] exactly (one term);
    for two tokens it is the sum of the one-token results."""
    N, K = 12, 32
    x, g, W, gamma, w, dy, out = _backward_case(orc, 2, N, K, 95)
    parts = []
    for m in range(2):
        o = orc.backward(x[m:m + 1], g, w, gamma, dy[m:m + 1])
        q, s = orc.rmsnorm_quant(x[m:m + 1], g)
        one = dy[m].astype(np.float64)[:, None] * (q[0].astype(np.float64) / float(s[0]))[None, :]
        assert np.array_equal(o["dW"], one)
        parts.append(one)
    assert np.allclose(out["dW"], parts[0] + parts[1], rtol=0, atol=1e-15 * np.abs(out["dW"]).max())


def pin_backward_single_feature_closed_form(orc):
    """K = 1: xn = g x / sqrt(x^2 + eps), so d xn / d x = g eps r^3 with
    r = (x^2 + eps)^-1/2, and dx = g dxn eps r^3, dg = dxn x r, where
    dxn = gamma sum_n dy[n] w[n][0]."""
    eps = float(np.float32(1e-3))  # large enough that eps r^3 is far from rounding noise
    x = wl.f32_to_bf16_bits(np.array([[0.75], [-0.125], [2.0]], np.float32))
    g = np.array([1.5], np.float32)
    w = np.array([[1], [-1], [0], [1]], np.int8)
    gamma = 0.25
    dy = np.array([[1.0, 2.0, 4.0, -0.5], [0.0, 1.0, 0.0, 0.0], [3.0, 0.0, 1.0, 1.0]], np.float32)
    out = orc.backward(x, g, w, gamma, dy, eps)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)[:, 0]
    dxn = gamma * (dy.astype(np.float64) @ w.astype(np.float64))[:, 0]
    r = 1.0 / np.sqrt(xf ** 2 + eps)
    assert np.allclose(out["dx"][:, 0], 1.5 * dxn * eps * r ** 3, rtol=1e-9, atol=0)
    assert math.isclose(out["dg"][0], float((dxn * xf * r).sum()), rel_tol=1e-12)


# --------------------------------------------------------------------------
# MLGRU token mixer and the layer
# --------------------------------------------------------------------------

def _np_gates(z):
    """f, c, g from z [..., 3d] straight from the definitions (numpy, fp64)."""
    d = z.shape[-1] // 3
    zf, zc, zg = z[..., :d], z[..., d:2 * d], z[..., 2 * d:]
    return 1.0 / (1.0 + np.exp(-zf)), zc / (1.0 + np.exp(-zc)), 1.0 / (1.0 + np.exp(-zg))


def _bf16_half_ulp(v):
    """Half the bf16 spacing at |v| (8 significant bits)."""
    _, e = np.frexp(np.abs(v))
    return np.ldexp(1.0, e - 9)


def pin_mlgru_scan_unrolled_sum(orc):
    """The recurrence h_t = f_t h_{t-1} + (1 - f_t) c_t unrolled:
    h_t = (prod_{r<=t} f_r) h_0 + sum_{s<=t} (prod_{s<r<=t} f_r)(1 - f_s) c_s,
    evaluated term by term; p_t is g_t h_t rounded to the nearest bf16."""
    r = wl.rng(21, 0)
    B, T, d = 2, 13, 8
    z = r.standard_normal((B, T, 3 * d)) * 2.0
    h0 = r.standard_normal((B, d))
    out = orc.mlgru_scan(z, h0)
    f, c, g = _np_gates(z)
    for b in range(B):
        for t in range(T):
            h = np.prod(f[b, :t + 1], axis=0) * h0[b]
            for s_ in range(t + 1):
                h = h + np.prod(f[b, s_ + 1:t + 1], axis=0) * (1.0 - f[b, s_]) * c[b, s_]
            v = g[b, t] * h
            pv = wl.bf16_bits_to_f32(out["p"][b, t]).astype(np.float64)
            assert np.all(np.abs(pv - v) <= _bf16_half_ulp(v) * (1 + 1e-9) + 1e-300), (b, t)
            if t == T - 1:
                assert np.allclose(out["state"][b], h, rtol=1e-12, atol=1e-14)


def pin_mlgru_constant_gates_closed_form(orc):
    """Constant pre-activations: h_t = f^t h_0 + (1 - f^t) c (a geometric
    approach to the candidate)."""
    B, T, d = 1, 40, 4
    zf, zc = np.array([-1.0, 0.3, 2.0, 0.0]), np.array([0.7, -2.0, 1.5, 3.0])
    z = np.zeros((B, T, 3 * d))
    z[..., :d], z[..., d:2 * d] = zf, zc
    h0 = np.array([[1.0, -0.5, 0.25, 2.0]])
    out = orc.mlgru_scan(z, h0)
    f = 1.0 / (1.0 + np.exp(-zf))
    c = zc / (1.0 + np.exp(-zc))
    assert np.allclose(out["state"][0], f ** T * h0[0] + (1 - f ** T) * c, rtol=1e-12, atol=1e-15)


def pin_mlgru_steps_convex_and_split(orc):
    """Gates lie in (0, 1), so each new state lies between the previous state
    and the candidate; and running the tokens one call at a time, carrying
    the state, gives exactly the state of one call over the whole sequence."""
    r = wl.rng(22, 0)
    B, T, d = 3, 17, 12
    z = r.standard_normal((B, T, 3 * d)) * 3.0
    h = r.standard_normal((B, d))
    whole = orc.mlgru_scan(z, h)
    _, c, _ = _np_gates(z)
    for t in range(T):
        step = orc.mlgru_scan(z[:, t:t + 1], h)
        lo, hi = np.minimum(h, c[:, t]), np.maximum(h, c[:, t])
        assert np.all(step["state"] >= lo - 1e-15) and np.all(step["state"] <= hi + 1e-15)
        assert np.array_equal(step["p"][:, 0], whole["p"][:, t])
        h = step["state"]
    assert np.array_equal(h, whole["state"])


def _mlgru_case(r, d, gain=True):
    g_in = (0.5 + r.random(d)).astype(np.float32) if gain else np.ones(d, np.float32)
    g_out = (0.5 + r.random(d)).astype(np.float32) if gain else np.ones(d, np.float32)
    W_in = (r.standard_normal((3 * d, d)) * 0.02).astype(np.float32)
    W_out = (r.standard_normal((d, d)) * 0.02).astype(np.float32)
    return g_in, W_in, g_out, W_out


def pin_mlgru_zero_input(orc):
    """x = 0: every code is 0, so z = 0, f = g = 1/2 and c = 0; the state
    halves each step (exact powers of two) and p_t = 2^-(t+2) h_0 exactly."""
    r = wl.rng(23, 0)
    B, T, d = 2, 6, 32
    g_in, W_in, g_out, W_out = _mlgru_case(r, d)
    h0 = r.standard_normal((B, d))
    out = orc.mlgru(np.zeros((B, T, d), np.uint16), g_in, W_in, g_out, W_out, h0)
    assert np.array_equal(out["state"], h0 * 0.5 ** T)
    for t in range(T):
        v = h0 * 0.5 ** (t + 2)
        pv = wl.bf16_bits_to_f32(out["p"][:, t]).astype(np.float64)
        assert np.all(np.abs(pv - v) <= _bf16_half_ulp(v) * (1 + 1e-9))
    h0z = orc.mlgru(np.zeros((B, T, d), np.uint16), g_in, W_in, g_out, W_out)
    assert np.all(h0z["y"] == 0) and np.all(h0z["state"] == 0)


def pin_mlgru_is_bitlinear_scan_bitlinear(orc):
    """The token mixer maps every token of every sequence through the pinned
    BitLinear with the input matrix (gain g_in), runs the pinned recurrence
    along each sequence, and maps p through BitLinear with the output matrix
    (gain g_out); from master weights it ternarises each matrix with its own
    gamma."""
    r = wl.rng(24, 0)
    B, T, d = 2, 5, 48
    g_in, W_in, g_out, W_out = _mlgru_case(r, d)
    x = wl.x_normal(B * T, d, seed=24).reshape(B, T, d)
    h0 = r.standard_normal((B, d))
    out = orc.mlgru(x, g_in, W_in, g_out, W_out, h0)
    gi, go = orc.gamma(W_in), orc.gamma(W_out)
    wi, wo = orc.ternarize(W_in, gi), orc.ternarize(W_out, go)
    z = orc.bitlinear_ternary(x.reshape(B * T, d), g_in, wi, gi)["y"].reshape(B, T, 3 * d)
    sc = orc.mlgru_scan(z, h0)
    assert np.array_equal(sc["p"], out["p"]) and np.array_equal(sc["state"], out["state"])
    y = orc.bitlinear_ternary(sc["p"].reshape(B * T, d), g_out, wo, go)["y"].reshape(B, T, d)
    assert np.array_equal(y, out["y"])
    tern = orc.mlgru_ternary(x, g_in, wi, gi, g_out, wo, go, h0)
    assert np.array_equal(tern["y"], out["y"])


def _layer_weights(orc, r, d, F, zero_in=False, zero_gu=False):
    g_in, W_in, g_out, W_out = _mlgru_case(r, d)
    if zero_in:
        W_in[:] = 0
    g_gu = (0.5 + r.random(d)).astype(np.float32)
    g_dn = (0.5 + r.random(F)).astype(np.float32)
    W_gu = (r.standard_normal((2 * F, d)) * 0.02).astype(np.float32)
    if zero_gu:
        W_gu[:] = 0
    W_dn = (r.standard_normal((d, F)) * 0.02).astype(np.float32)
    t = []
    for gain, W in ((g_in, W_in), (g_out, W_out), (g_gu, W_gu), (g_dn, W_dn)):
        gm = orc.gamma(W)
        t.append((gain, orc.ternarize(W, gm), gm))
    return (t[0] + t[1]), (t[2] + t[3])


def pin_layer_residual_identity(orc):
    """With all-zero input and gate|up matrices both mixers output exactly 0
    (z = 0 gives c = 0, hence p = 0, and SiLU(0) * 0 = 0), so the layer is
    the identity on x, bit for bit, whatever the other matrices hold."""
    r = wl.rng(25, 0)
    B, T, d, F = 2, 4, 32, 48
    mw, gw = _layer_weights(orc, r, d, F, zero_in=True, zero_gu=True)
    x = wl.x_normal(B * T, d, seed=25).reshape(B, T, d)
    out = orc.lm_layer_ternary(x, mw, gw)
    assert np.array_equal(out["out"], x) and np.array_equal(out["u"], x)


def pin_layer_is_token_then_channel_mixer(orc):
    """u = bf16(x + MLGRU(x)) and out = bf16(u + GLU(u)), each sum rounded
    once to the nearest bf16 (checked as within half a bf16 spacing), with
    the pinned mixers; the state is the MLGRU's."""
    r = wl.rng(26, 0)
    B, T, d, F = 2, 3, 32, 64
    mw, gw = _layer_weights(orc, r, d, F)
    x = wl.x_normal(B * T, d, seed=26).reshape(B, T, d)
    h0 = r.standard_normal((B, d))
    out = orc.lm_layer_ternary(x, mw, gw, h0)
    m = orc.mlgru_ternary(x, *mw, state=h0)
    assert np.array_equal(out["state"], m["state"])
    v = wl.bf16_bits_to_f32(x).astype(np.float64) + m["y"]
    uf = wl.bf16_bits_to_f32(out["u"]).astype(np.float64)
    assert np.all(np.abs(uf - v) <= _bf16_half_ulp(v) * (1 + 1e-9) + 1e-300)
    gl = orc.glu_ternary(out["u"].reshape(B * T, d), *gw)["y"].reshape(B, T, d)
    v2 = uf + gl
    of = wl.bf16_bits_to_f32(out["out"]).astype(np.float64)
    assert np.all(np.abs(of - v2) <= _bf16_half_ulp(v2) * (1 + 1e-9) + 1e-300)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def run_all(lib_path=None):
    """Run every pin against the library at lib_path; exit status 1 on the
    first failure (used on altered oracle builds)."""
    import oracle
    orc = oracle.Oracle(oracle.lib(lib_path) if lib_path else None)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001  (a raise is a failed pin too)
            failed.append((pin.__name__, str(e)[:200]))
    for name, msg in failed:
        print(f"FAILED {name}: {msg}")
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(run_all(sys.argv[1] if len(sys.argv) > 1 else None))
