"""The MLGRU token mixer and the layer (token mixer, then GLU channel mixer)
on the GPU against the oracle.

The recurrence stage takes the same fp32 pre-activations z on both sides,
so its bar is derived from the fp32 arithmetic of the kernels (u = 2^-24):
sigmoid and SiLU come from 2^x and a reciprocal (about one ulp each) of an
argument whose rounding moves them by up to |z| u, so f, 1 - f, c and g are
each within (6 + |z|) u relative; each step h = fma(f, h, (1 - f) c) adds
two roundings; the chunked order adds one multiply-add per chunk boundary.
The state error then obeys
    e_t <= f_t e_{t-1} + |f_t h_{t-1}| (df + u) + |(1 - f_t) c_t| (df + dc + 2u) + 2u |h_t|
(oracle values, fp64), and the test allows twice that.  The GPU's
exponential flushes results below the smallest normal fp32 value 2^-126 to
zero, so a gate or candidate that small may come out as 0: each step also
allows 2^-126 (|h_{t-1}| + 100) absolute (|z| <= 90 here, so |c| < 100
2^-126 when it flushes), and p allows 2^-126 (|h_t| + 1).  p_t = bf16(g h_t)
must be within half a bf16 spacing of a value within the propagated error
of g h_t.  End to end (BitLinear projections with their int8 codes) the bar
is the stated one: per row, max |dy| <= 1e-2 max |y_ref|.
"""
import numpy as np
import pytest
import torch

import bitlinear_layer_amd as bl
import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
TINY = 2.0 ** -126  # smallest normal fp32


def _say(*a):
    print(*a, flush=True)


def _scan_inputs(B, T, d, seed, scale=2.0, extremes=True):
    r = wl.rng(seed, wl.STREAM_X)
    z = (r.standard_normal((B, T, 3 * d)) * scale).astype(np.float32)
    if extremes and z.size >= 64:
        idx = r.choice(z.size, size=max(1, z.size // 200), replace=False)
        z.reshape(-1)[idx] = r.choice(np.array([-90.0, -30.0, -8.0, 8.0, 30.0, 90.0], np.float32), idx.size)
    h0 = r.standard_normal((B, d)).astype(np.float32)
    return z, h0


def _oracle_states(z64, h0):
    """Oracle p and the state after every token (one-token calls carrying the
    state equal the whole-sequence call exactly; an oracle pin checks it)."""
    B, T, _ = z64.shape
    orc = gu.orc()
    hs = np.empty((B, T, h0.shape[1]))
    ps = np.empty((B, T, h0.shape[1]), np.uint16)
    h = h0.astype(np.float64)
    for t in range(T):
        r = orc.mlgru_scan(z64[:, t:t + 1], h)
        h = r["state"]
        hs[:, t], ps[:, t] = h, r["p"][:, 0]
    return ps, hs


def _scan_bounds(z64, h0, hs):
    d = h0.shape[1]
    zf, zc, zg = z64[..., :d], z64[..., d:2 * d], z64[..., 2 * d:]
    f = 1.0 / (1.0 + np.exp(-zf))
    omf = 1.0 / (1.0 + np.exp(zf))
    c = zc / (1.0 + np.exp(-zc))
    g = 1.0 / (1.0 + np.exp(-zg))
    df, dc, dg = (6 + np.abs(zf)) * U, (6 + np.abs(zc)) * U, (6 + np.abs(zg)) * U
    e = np.zeros_like(hs)
    prev_e = np.zeros_like(h0, dtype=np.float64)
    prev_h = h0.astype(np.float64)
    for t in range(hs.shape[1]):
        cur = (f[:, t] * prev_e + np.abs(f[:, t] * prev_h) * (df[:, t] + U)
               + np.abs(omf[:, t] * c[:, t]) * (df[:, t] + dc[:, t] + 2 * U) + 2 * U * np.abs(hs[:, t])
               + TINY * (np.abs(prev_h) + 100.0))
        e[:, t] = cur
        prev_e, prev_h = cur, hs[:, t]
    e = 2.0 * e
    v = g * hs
    ev = np.abs(g) * e + np.abs(v) * (dg + 2 * U) + TINY * (np.abs(hs) + 1.0)
    return e, v, ev


def _check_p(p_gpu, v, ev):
    pf = wl.bf16_bits_to_f32(p_gpu.astype(np.uint16)).astype(np.float64)
    m = np.maximum(np.abs(pf), np.abs(v))
    _, ex = np.frexp(m)
    half = np.ldexp(1.0, ex - 9)
    bad = np.abs(pf - v) > half + ev + 1e-300
    assert not bad.any(), f"{int(bad.sum())} p values off; e.g. {pf[bad][:3]} vs {v[bad][:3]}"


# (B, T, d): one token; single chunk; many chunks of one to several tokens;
# a ragged last chunk; many channels (one pass); the widths of the layer.
SCAN_SHAPES = [(1, 1, 16), (2, 1, 16), (1, 7, 32), (2, 33, 64), (3, 100, 48), (1, 130, 2048),
               (1, 2048, 256), (64, 5, 2048), (1, 97, 1024)]


@pytest.mark.parametrize("B,T,d", SCAN_SHAPES)
def test_mlgru_scan_matches_oracle(B, T, d):
    _say("mlgru scan", B, T, d)
    z, h0 = _scan_inputs(B, T, d, seed=B * 1000 + T * 7 + d)
    z64 = z.astype(np.float64)
    ps, hs = _oracle_states(z64, h0)
    state = gu.to_dev(h0.copy())
    p = bl.bitlinear_mlgru_scan(gu.to_dev(z), state)
    torch.cuda.synchronize()
    p_gpu = p.cpu().numpy().view(np.uint16)
    st = state.cpu().numpy().astype(np.float64)
    e, v, ev = _scan_bounds(z64, h0, hs)
    err = np.abs(st - hs[:, -1])
    assert np.all(err <= e[:, -1] + 1e-300), f"state: worst {err.max():.3e}, bound {e[:, -1][np.argmax(err)]:.3e}"
    _check_p(p_gpu, v, ev)
    assert np.mean(p_gpu != ps) <= 1e-2


def test_mlgru_scan_full_size_sampled_channels():
    """The pages' inference setting, one sequence of 2048 tokens at d = 2048
    (64 chunks of 32 tokens): every channel is independent in the
    recurrence, so the oracle runs on 24 sampled channels."""
    B, T, d = 1, 2048, 2048
    z, h0 = _scan_inputs(B, T, d, seed=77)
    state = gu.to_dev(h0.copy())
    p = bl.bitlinear_mlgru_scan(gu.to_dev(z), state)
    torch.cuda.synchronize()
    sel = np.array([0, 1, 63, 64, 255, 256, 511, 700, 1023, 1024, 1500, 2000, 2040, 2046, 2047,
                    5, 17, 333, 901, 1111, 1234, 1777, 1888, 1999])
    zs = np.concatenate([z[..., sel], z[..., d + sel], z[..., 2 * d + sel]], axis=-1).astype(np.float64)
    ps, hs = _oracle_states(zs, h0[:, sel])
    e, v, ev = _scan_bounds(zs, h0[:, sel], hs)
    st = state.cpu().numpy().astype(np.float64)[:, sel]
    assert np.all(np.abs(st - hs[:, -1]) <= e[:, -1])
    _check_p(p.cpu().numpy().view(np.uint16)[..., sel], v, ev)


def test_mlgru_scan_state_carried_across_calls():
    """Two calls over the halves of a sequence, carrying the state, against
    one call over the whole sequence (different chunkings)."""
    B, T, d = 2, 300, 512
    z, h0 = _scan_inputs(B, T, d, seed=5)
    zd = gu.to_dev(z)
    s1 = gu.to_dev(h0.copy())
    p1 = bl.bitlinear_mlgru_scan(zd, s1)
    s2 = gu.to_dev(h0.copy())
    pa = bl.bitlinear_mlgru_scan(zd[:, :120].contiguous(), s2)
    pb = bl.bitlinear_mlgru_scan(zd[:, 120:].contiguous(), s2)
    torch.cuda.synchronize()
    z64 = z.astype(np.float64)
    _, hs = _oracle_states(z64, h0)
    e, _, _ = _scan_bounds(z64, h0, hs)
    for s in (s1, s2):
        assert np.all(np.abs(s.cpu().numpy() - hs[:, -1]) <= e[:, -1])
    two = torch.cat([pa, pb], dim=1).cpu().numpy().view(np.uint16)
    assert np.mean(two != p1.cpu().numpy().view(np.uint16)) <= 1e-2


def test_mlgru_scan_empty_and_zero():
    d = 32
    st = torch.ones((2, d), dtype=torch.float32, device=gu.DEV)
    bl.bitlinear_mlgru_scan(torch.empty((2, 0, 3 * d), dtype=torch.float32, device=gu.DEV), st)
    torch.cuda.synchronize()
    assert torch.all(st == 1)
    # z = 0: f = g = 1/2 and c = 0, so the state halves each token, exactly
    T = 10
    st = torch.full((2, d), 3.0, dtype=torch.float32, device=gu.DEV)
    p = bl.bitlinear_mlgru_scan(torch.zeros((2, T, 3 * d), dtype=torch.float32, device=gu.DEV), st)
    torch.cuda.synchronize()
    assert torch.all(st == 3.0 * 0.5 ** T)
    pf = wl.bf16_bits_to_f32(p.cpu().numpy().view(np.uint16))
    for t in range(T):
        assert np.all(pf[:, t] == np.float32(3.0 * 0.5 ** (t + 2)))


# --------------------------------------------------------------------------
# the token mixer end to end
# --------------------------------------------------------------------------

def _mlgru_weights(d, seed):
    r = wl.rng(seed, wl.STREAM_G)
    g_in = (0.5 + r.random(d)).astype(np.float32)
    g_out = (0.5 + r.random(d)).astype(np.float32)
    W_in = wl.w_normal(3 * d, d, seed=seed)
    W_out = wl.w_normal(d, d, seed=seed, stream=wl.STREAM_W2)
    return g_in, W_in, g_out, W_out


def _dev_mlgru(g_in, W_in, g_out, W_out):
    pin, gin = gu.pack_on_gpu(W_in)
    pout, gout = gu.pack_on_gpu(W_out)
    return (gu.to_dev(g_in), pin, gin, gu.to_dev(g_out), pout, gout)


# (B, T, d): one token (fused decode kernels), two sequences of one token,
# 16 tokens (few-token kernels), 120 and 300 tokens (MFMA tiles), the layer
# width at 130 tokens.
MIXER_SHAPES = [(1, 1, 64), (2, 1, 128), (1, 16, 256), (3, 40, 128), (1, 300, 256), (1, 130, 2048)]


@pytest.mark.parametrize("B,T,d", MIXER_SHAPES)
def test_mlgru_forward_matches_oracle(B, T, d):
    _say("mlgru forward", B, T, d)
    seed = B * 100 + T + d
    g_in, W_in, g_out, W_out = _mlgru_weights(d, seed)
    x = wl.x_normal(B * T, d, seed=seed, outlier_frac=0.005, outlier_scale=20.0).reshape(B, T, d)
    h0 = wl.rng(seed, 9).standard_normal((B, d)).astype(np.float32)
    ref = gu.orc().mlgru(x, g_in, W_in, g_out, W_out, h0)
    w = _dev_mlgru(g_in, W_in, g_out, W_out)
    state = gu.to_dev(h0.copy())
    y = bl.bitlinear_mlgru_forward(gu.to_dev_bf16(x), *w, state)
    torch.cuda.synchronize()
    gu.assert_y_parity(y.cpu().numpy().reshape(B * T, d), ref["y"].reshape(B * T, d))
    st = state.cpu().numpy()
    scale = np.abs(ref["state"]).max(axis=1, keepdims=True)
    assert np.all(np.abs(st - ref["state"]) <= 1e-3 * scale), float(np.abs(st - ref["state"]).max())


def test_mlgru_decode_steps_match_sequence():
    """Token-by-token decoding (T = 1 per call, the state carried, one fused
    kernel per projection) against the oracle over the whole sequence."""
    B, T, d = 1, 12, 2048
    g_in, W_in, g_out, W_out = _mlgru_weights(d, 31)
    x = wl.x_normal(B * T, d, seed=31).reshape(B, T, d)
    ref = gu.orc().mlgru(x, g_in, W_in, g_out, W_out)
    w = _dev_mlgru(g_in, W_in, g_out, W_out)
    state = torch.zeros((B, d), dtype=torch.float32, device=gu.DEV)
    xd = gu.to_dev_bf16(x)
    ys = [bl.bitlinear_mlgru_forward(xd[:, t:t + 1].contiguous(), *w, state) for t in range(T)]
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=1).cpu().numpy()
    gu.assert_y_parity(y.reshape(B * T, d), ref["y"].reshape(B * T, d))
    scale = np.abs(ref["state"]).max()
    assert np.all(np.abs(state.cpu().numpy() - ref["state"]) <= 1e-3 * scale)


def test_mlgru_zero_weights_and_empty():
    B, T, d = 2, 9, 64
    x = wl.x_normal(B * T, d, seed=3).reshape(B, T, d)
    z0 = np.zeros((3 * d, d), np.float32)
    g = np.ones(d, np.float32)
    w = _dev_mlgru(g, z0, g, wl.w_normal(d, d, seed=3))
    state = torch.full((B, d), 2.0, dtype=torch.float32, device=gu.DEV)
    y = bl.bitlinear_mlgru_forward(gu.to_dev_bf16(x), *w, state)
    torch.cuda.synchronize()
    # W_in = 0: z = 0, the state halves each token; p = 2^-(t+2) * 2 is exact
    assert torch.all(state == 2.0 * 0.5 ** T)
    ref = gu.orc().mlgru(x, g, z0, g, wl.w_normal(d, d, seed=3), np.full((B, d), 2.0))
    gu.assert_y_parity(y.cpu().numpy().reshape(B * T, d), ref["y"].reshape(B * T, d))
    empty = torch.empty((B, 0, d), dtype=torch.int16, device=gu.DEV)
    y0 = bl.bitlinear_mlgru_forward(empty, *w, state)
    assert y0.shape == (B, 0, d)


# --------------------------------------------------------------------------
# one layer: token mixer, then channel mixer
# --------------------------------------------------------------------------

def _layer(d, F, seed):
    g_in, W_in, g_out, W_out = _mlgru_weights(d, seed)
    r = wl.rng(seed, wl.STREAM_G + 10)
    g_gu = (0.5 + r.random(d)).astype(np.float32)
    g_dn = (0.5 + r.random(F)).astype(np.float32)
    W_gu = wl.w_normal(2 * F, d, seed=seed + 1)
    W_dn = wl.w_normal(d, F, seed=seed + 1, stream=wl.STREAM_W2)
    orc = gu.orc()
    tern = []
    for gain, W in ((g_in, W_in), (g_out, W_out), (g_gu, W_gu), (g_dn, W_dn)):
        gm = orc.gamma(W)
        tern.append((gain, orc.ternarize(W, gm), gm))
    dev = []
    for gain, W in ((g_in, W_in), (g_out, W_out), (g_gu, W_gu), (g_dn, W_dn)):
        pk, gm = gu.pack_on_gpu(W)
        assert gm.item() == orc.gamma(W)
        dev.append((gu.to_dev(gain), pk, gm))
    return (tern[0] + tern[1], tern[2] + tern[3]), (dev[0] + dev[1], dev[2] + dev[3])


def _assert_bf16_rows(out_gpu, out_ref, rel=1e-2):
    a = wl.bf16_bits_to_f32(out_gpu.astype(np.uint16)).astype(np.float64)
    b = wl.bf16_bits_to_f32(out_ref.astype(np.uint16)).astype(np.float64)
    a, b = a.reshape(-1, a.shape[-1]), b.reshape(-1, b.shape[-1])
    scale = np.abs(b).max(axis=1)
    assert np.all(np.abs(a - b).max(axis=1) <= rel * scale)
    assert np.mean(a != b) <= 2e-2


# (B, T, d, F): one token (every projection on the fused decode kernels),
# 8 tokens, 128 and 200 tokens (MFMA tiles), the layer's full width at 32
# tokens.
LAYER_SHAPES = [(1, 1, 64, 96), (1, 8, 128, 192), (2, 64, 256, 384), (1, 200, 256, 512), (1, 32, 2048, 5632)]


@pytest.mark.parametrize("B,T,d,F", LAYER_SHAPES)
def test_layer_forward_matches_oracle(B, T, d, F):
    _say("layer", B, T, d, F)
    (mw, gw), (mdev, gdev) = _layer(d, F, seed=B + T + d + F)
    x = wl.x_normal(B * T, d, seed=T + d).reshape(B, T, d)
    h0 = wl.rng(T, 8).standard_normal((B, d)).astype(np.float32)
    ref = gu.orc().lm_layer_ternary(x, mw, gw, h0)
    state = gu.to_dev(h0.copy())
    out = bl.bitlinear_layer_forward(gu.to_dev_bf16(x), mdev, gdev, state)
    torch.cuda.synchronize()
    _assert_bf16_rows(out.cpu().numpy().view(np.uint16), ref["out"])
    scale = np.abs(ref["state"]).max(axis=1, keepdims=True)
    assert np.all(np.abs(state.cpu().numpy() - ref["state"]) <= 1e-3 * scale)


def test_layer_decode_steps_full_width():
    """Decoding 6 tokens one call at a time through a full-width layer
    (d = 2048, F = 5632), the state carried, against the oracle's layer over
    the whole sequence."""
    B, T, d, F = 1, 6, 2048, 5632
    (mw, gw), (mdev, gdev) = _layer(d, F, seed=41)
    x = wl.x_normal(B * T, d, seed=41).reshape(B, T, d)
    ref = gu.orc().lm_layer_ternary(x, mw, gw)
    state = torch.zeros((B, d), dtype=torch.float32, device=gu.DEV)
    xd = gu.to_dev_bf16(x)
    outs = [bl.bitlinear_layer_forward(xd[:, t:t + 1].contiguous(), mdev, gdev, state) for t in range(T)]
    torch.cuda.synchronize()
    out = torch.cat(outs, dim=1).cpu().numpy().view(np.uint16)
    _assert_bf16_rows(out, ref["out"])


def test_layer_full_sequence_properties():
    """The pages' setting, one sequence of 2048 tokens through a layer of
    width 2048 / 5632: deterministic, and the state after the sequence
    equals the state after its two halves run one after the other."""
    B, T, d, F = 1, 2048, 2048, 5632
    (_, _), (mdev, gdev) = _layer(d, F, seed=51)
    x = gu.to_dev_bf16(wl.x_normal(B * T, d, seed=51).reshape(B, T, d))
    s1 = torch.zeros((B, d), dtype=torch.float32, device=gu.DEV)
    o1 = bl.bitlinear_layer_forward(x, mdev, gdev, s1)
    s2 = torch.zeros((B, d), dtype=torch.float32, device=gu.DEV)
    o2 = bl.bitlinear_layer_forward(x, mdev, gdev, s2)
    s3 = torch.zeros((B, d), dtype=torch.float32, device=gu.DEV)
    bl.bitlinear_layer_forward(x[:, :1024].contiguous(), mdev, gdev, s3)
    bl.bitlinear_layer_forward(x[:, 1024:].contiguous(), mdev, gdev, s3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.isfinite(o1.view(torch.bfloat16).float()).all()
    scale = s1.abs().max().item()
    assert (s1 - s3).abs().max().item() <= 1e-4 * scale


def _bf16_add(a_bits, y):
    """bf16(a + y) in fp32, rounded to nearest even (torch's conversion)."""
    return (a_bits.view(torch.bfloat16).float() + y).to(torch.bfloat16).view(torch.int16)


# (B, d, F): one token per sequence, so every projection runs on the fused
# decode kernel with the recurrence step or a residual add in its epilogue.
ONE_TOKEN = [(1, 64, 96), (3, 128, 192), (4, 256, 384), (1, 2048, 5632), (2, 2048, 5632)]


@pytest.mark.parametrize("B,d,F", ONE_TOKEN)
def test_layer_one_token_fused_equals_composed(B, d, F):
    """A one-token step of the layer fuses the recurrence step into the
    input projection and the two residual adds into the output and down
    projections.  Each epilogue uses the arithmetic of the kernel it
    replaces, so the layer's output and state must equal, bit for bit, the
    same step composed from the separate entry points (projection, scan,
    projection, bf16(x + y), GLU, bf16(u + y))."""
    _say("one-token fused vs composed", B, d, F)
    (_, _), (mdev, gdev) = _layer(d, F, seed=7 * B + d)
    x = gu.to_dev_bf16(wl.x_normal(B, d, seed=B + d).reshape(B, 1, d))
    h0 = wl.rng(B + d, 8).standard_normal((B, d)).astype(np.float32)
    s_fused = gu.to_dev(h0.copy())
    out = bl.bitlinear_layer_forward(x, mdev, gdev, s_fused)
    y_mix = bl.bitlinear_mlgru_forward(x, *mdev, gu.to_dev(h0.copy()))

    s_comp = gu.to_dev(h0.copy())
    g_in, p_in, gm_in, g_out, p_out, gm_out = mdev
    z = bl.bitlinear_forward(x.reshape(B, d), g_in, p_in, gm_in)
    p = bl.bitlinear_mlgru_scan(z.reshape(B, 1, 3 * d), s_comp)
    y = bl.bitlinear_forward(p.reshape(B, d), g_out, p_out, gm_out)
    u = _bf16_add(x.reshape(B, d), y)
    yg = bl.bitlinear_glu_forward(u, *gdev)
    ref = _bf16_add(u, yg)
    torch.cuda.synchronize()
    assert torch.equal(y_mix.reshape(B, d), y)
    assert torch.equal(out.reshape(B, d), ref)
    assert torch.equal(s_fused, s_comp)


# (B, T, d, F): more than 128 tokens, so the output and down projections run
# on the large-tile product, which adds the residual in its epilogue (on
# 128 x 128 tiles up to 2048 tokens at d = 2048, on 128 x 256 tiles above;
# d = 192 leaves the last 128-column tile half full).
MANY_TOKENS = [(1, 300, 256, 384), (2, 160, 128, 256), (1, 200, 192, 256), (1, 1024, 2048, 5632),
               (1, 2200, 2048, 512)]


@pytest.mark.parametrize("B,T,d,F", MANY_TOKENS)
def test_layer_many_tokens_fused_equals_composed(B, T, d, F):
    """Above 128 tokens the output projection and the GLU down projection
    add the residual in the large-tile product's epilogue, with the fp32
    arithmetic of the separate residual pass, so the layer's output and state
    must equal, bit for bit, the same layer composed from the separate entry
    points (token mixer, bf16(x + y), channel mixer, bf16(u + y))."""
    _say("many-token fused vs composed", B, T, d, F)
    (_, _), (mdev, gdev) = _layer(d, F, seed=3 * B + T)
    x = gu.to_dev_bf16(wl.x_normal(B * T, d, seed=B + T).reshape(B, T, d))
    h0 = wl.rng(B + T, 8).standard_normal((B, d)).astype(np.float32)
    s_fused = gu.to_dev(h0.copy())
    out = bl.bitlinear_layer_forward(x, mdev, gdev, s_fused)

    s_comp = gu.to_dev(h0.copy())
    y = bl.bitlinear_mlgru_forward(x, *mdev, s_comp)
    u = _bf16_add(x, y)
    yg = bl.bitlinear_glu_forward(u.reshape(B * T, d), *gdev)
    ref = _bf16_add(u.reshape(B * T, d), yg)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(B * T, d), ref)
    assert torch.equal(s_fused, s_comp)
