#!/usr/bin/env python3
"""Benchmark of the fused BitLinear layer on one MI355X.

Headline ("HBM GB/s at M=1"): one decode step through `--layers`
independent BitLinear layers of the decode shape (M = 1 token, K = N = 2048,
x bf16 ~ N(0,1), W ~ N(0, 0.02^2) ternarised and packed), issued as one
bitlinear_forward_batched call.  1024 layers hold 1 GiB of packed weights,
four times the 256 MB Infinity Cache, so the weights stream from HBM.
value = algorithmic bytes moved per step / wall time per step, where the
algorithmic bytes of one layer are N*K/4 (packed W) + 2*M*K (x) + 4*K (RMSNorm
weight) + 4*M*N (y) + 4 (gamma).

Also reported (`secondary`): the literal single-layer call at M=1, the same
calls over the 1024 layers replayed from one HIP graph, the M=8
decode step, the one-token decode step of the 2560/6912 layer shapes (each
over about 1 GiB of cold weights) and the same shapes at 64 and 512 tokens
(over about 1 GiB, with HBM, int8 and combined-bound fractions) and at 4096
and 16384 tokens, the 8192-token prefill (int8 TOPS of the MFMA product
kernel, timed apart from the quantisation kernel), the GLU
mixer at M=1 (one call, and one step through 128 mixers) and M=4096, the
batched re-ternarisation of 64 fp32 master matrices of 2048 x 2048, the
straight-through backward of one layer at 8192 x 2048 x 2048 (TFLOP/s of its
two bf16 products; `--only backward` runs the headline and this leg alone),
and, as context, a plain 2 GiB device copy and, beside each product of 4096
tokens or more, the vendor's dense int8 GEMM on the same shape.  `roofline` is for the
headline's dominant kernel, timed with one HIP event pair on the stream it
runs on, around a second pass of the timed steps; `cpu_baseline` times the
CPU oracle on a bounded sample of the headline workload on this host.

One GPU only: `--gpus N` with N > 1 exits with a message.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12        # B/s, MI355X HBM3E
I8_PEAK = 5.0e15         # dense int8 MFMA ops/s, MI355X
BF16_PEAK = 2.5e15       # dense bf16 MFMA flops/s, MI355X
DEV = "cuda:0"


def layer_bytes(M, N, K):
    return N * K // 4 + 2 * M * K + 4 * K + 4 * M * N + 4


def glu_bytes(M, D, F):
    return layer_bytes(M, 2 * F, D) - 4 * M * 2 * F + layer_bytes(M, D, F) - 2 * M * F


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class EventTimer:
    """HIP events around each call, on the stream the library launches on."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        self.pairs = []

    def __enter__(self):
        self.start = self.torch.cuda.Event(enable_timing=True)
        self.end = self.torch.cuda.Event(enable_timing=True)
        self.start.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.end.record(self.stream)
        self.pairs.append((self.start, self.end))

    def mean_ms(self):
        self.torch.cuda.synchronize()
        return sum(s.elapsed_time(e) for s, e in self.pairs) / max(1, len(self.pairs))


def timed_loop(torch, fn, steps, warmup, stream, per_call_events=False):
    """Run fn warmup times, then exactly `steps` times between device
    synchronisations.  Returns (wall ms per step, event ms per call).

    By default the wall time covers exactly `steps` calls between two device
    synchronisations, and a second pass of `steps` calls gives the event
    time: one HIP event pair on the library's stream brackets them, recorded
    behind one untimed call, so the device is already busy when the span
    opens and the span holds the calls' own device time, not the host's
    latency to issue the first of them.  Nothing is inserted between calls.
    With per_call_events each call gets its own pair (for single-call
    latency)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if per_call_events:
        timer = EventTimer(torch, stream)
        t0 = time.perf_counter()
        for _ in range(steps):
            with timer:
                fn()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return wall, timer.mean_ms()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    fn()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return wall, start.elapsed_time(end) / steps


# sources the headline kernel is compiled from (its counters go stale when any changes)
DECODE_SOURCES = ("decode.hip", "device_common.h", "epilogue.h", "launch.h")


def _code_only(text):
    """Source text without comments and blank space, so that editing a
    comment does not mark stored counters stale (any code change does)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bitlinear_layer_amd", "csrc", n), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel_file, digest, algorithmic_bytes):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none, the kernel source changed since it was taken, or it was
    taken on another workload (its algorithmic bytes per launch differ)."""
    path = os.path.join(ROOT, "profiles", "traffic_" + kernel_file.replace(".hip", "") + ".txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != digest:
        return None
    try:
        if int(vals["algorithmic_bytes_per_launch"]) != int(algorithmic_bytes):
            return None
        return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def make_decode_layers(torch, bl, wl, L, M, N, K, seed=0):
    x = torch.from_numpy(wl.x_normal(L * M, K, seed=seed).view("int16")).to(DEV).view(L, M, K)
    g = torch.ones((L, K), dtype=torch.float32, device=DEV)
    packed = torch.empty((L, N, K // 4), dtype=torch.uint8, device=DEV)
    gamma = torch.empty(L, dtype=torch.float32, device=DEV)
    ws = torch.empty(bl.bitlinear_pack_workspace_bytes(N, K), dtype=torch.uint8, device=DEV)
    for layer in range(L):
        W = wl.w_normal_device(N, K, seed=seed, layer=layer, device=DEV)
        bl.bitlinear_pack_weights(W, packed=packed[layer], gamma=gamma[layer:layer + 1], ws=ws)
        del W
    y = torch.empty((L, M, N), dtype=torch.float32, device=DEV)
    wsf = torch.empty(bl.bitlinear_forward_batched_workspace_bytes(L, M, N, K), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    return x, g, packed, gamma, y, wsf


def bench_decode(torch, bl, wl, L, M, N, K, steps, warmup, stream):
    x, g, packed, gamma, y, ws = make_decode_layers(torch, bl, wl, L, M, N, K)

    def step():
        bl.bitlinear_forward_batched(x, g, packed, gamma, y=y, ws=ws)

    wall, ev = timed_loop(torch, step, steps, warmup, stream)
    nbytes = L * layer_bytes(M, N, K)
    del x, g, packed, gamma, y, ws
    torch.cuda.empty_cache()
    return dict(layers=L, M=M, N=N, K=K, bytes_per_step=nbytes, wall_ms=wall, event_ms=ev,
                gbps=nbytes / (wall * 1e-3) / 1e9, kernel_gbps=nbytes / (ev * 1e-3) / 1e9)


def bench_sweep_layers(torch, bl, wl, M, N, K, steps, warmup, stream):
    """A layer shape at M tokens over about 1 GiB of algorithmic bytes (L
    independent layers in one batched call), with both roofline fractions:
    HBM (bytes / 8 TB/s) and int8 MFMA (2 M N K / 5.0 POPS), and the fraction
    of the combined bound max(bytes / BW, ops / peak)."""
    L = max(1, (1 << 30) // layer_bytes(M, N, K))
    r = bench_decode(torch, bl, wl, L, M, N, K, steps, warmup, stream)
    t = r["event_ms"] * 1e-3
    ops = 2.0 * L * M * N * K
    t_min = max(r["bytes_per_step"] / HBM_PEAK, ops / I8_PEAK)
    r.update(int8_ops_per_step=ops, tops=ops / t / 1e12, frac_hbm=r["bytes_per_step"] / t / HBM_PEAK,
             frac_i8=ops / t / I8_PEAK, frac_combined_bound=t_min / t)
    return r


def bench_single_layer(torch, bl, wl, M, N, K, steps, stream):
    x, g, packed, gamma, y, ws = make_decode_layers(torch, bl, wl, 1, M, N, K, seed=1)
    x, g, y = x[0], g[0], y[0]

    def step():
        bl.bitlinear_forward(x, g, packed[0], gamma[:1], y=y, ws=ws)

    wall, ev = timed_loop(torch, step, steps, 20, stream, per_call_events=True)
    nbytes = layer_bytes(M, N, K)
    return dict(M=M, N=N, K=K, us_per_call_wall=wall * 1e3, us_per_call_event=ev * 1e3,
                implied_gbps=nbytes / (ev * 1e-3) / 1e9)


def bench_graph_calls(torch, bl, wl, L, M, N, K, steps, warmup, stream):
    """L single-layer bitlinear_forward calls, one per layer of an L-layer
    stack, captured once into a HIP graph and replayed: the time per call
    that a caller issuing layer by layer sees without host launch overhead
    (the batched call runs the same stack as one launch)."""
    x, g, packed, gamma, y, _ = make_decode_layers(torch, bl, wl, L, M, N, K, seed=2)
    ws = torch.empty(bl.bitlinear_forward_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)

    def calls():
        for layer in range(L):
            bl.bitlinear_forward(x[layer], g[layer], packed[layer], gamma[layer:layer + 1], y=y[layer], ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    wall, ev = timed_loop(torch, graph.replay, steps, warmup, stream)
    nbytes = L * layer_bytes(M, N, K)
    del graph, x, g, packed, gamma, y, ws
    torch.cuda.empty_cache()
    return dict(calls=L, M=M, N=N, K=K, us_per_call_event=ev * 1e3 / L, us_per_call_wall=wall * 1e3 / L,
                gbps=nbytes / (ev * 1e-3) / 1e9)


def bench_prefill(torch, bl, wl, M, N, K, steps, warmup, stream):
    x = torch.from_numpy(wl.x_student_t(M, K, seed=0).view("int16")).to(DEV)
    g = torch.ones(K, dtype=torch.float32, device=DEV)
    packed, gamma = bl.bitlinear_pack_weights(torch.from_numpy(wl.w_normal(N, K, seed=0)).to(DEV))
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ws = torch.empty(bl.bitlinear_forward_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
    ops = 2.0 * M * N * K
    wall_q, ev_q = timed_loop(torch, lambda: bl.bitlinear_prepare_activations(x, g, ws=ws), steps, warmup, stream)
    wall_p, ev_p = timed_loop(torch, lambda: bl.bitlinear_forward_prepared(ws, packed, gamma, M, y=y),
                              steps, warmup, stream)
    wall_f, ev_f = timed_loop(torch, lambda: bl.bitlinear_forward(x, g, packed, gamma, y=y, ws=ws),
                              steps, warmup, stream)
    vendor_us = vendor_int8_gemm_us(torch, M, N, K, steps, warmup, stream)
    return dict(M=M, N=N, K=K, int8_ops=ops, quant_us=ev_q * 1e3, product_us=ev_p * 1e3,
                product_tops=ops / (ev_p * 1e-3) / 1e12, product_frac_i8_peak=ops / (ev_p * 1e-3) / I8_PEAK,
                context_vendor_int8_gemm_us=vendor_us,
                forward_us=ev_f * 1e3, forward_tops=ops / (ev_f * 1e-3) / 1e12,
                forward_us_wall=wall_f * 1e3, forward_bytes=layer_bytes(M, N, K))


def bench_backward(torch, bl, wl, M, N, K, steps, warmup, stream):
    """Straight-through backward of one layer (dx, dg, dW from x, the packed
    weights and dy).  Its two gradient products are bf16 contractions of
    2*M*N*K flops each; the algorithmic bytes are x, dy, g, the packed
    weights and gamma read once and dx, dg, dW written once."""
    x = torch.from_numpy(wl.x_student_t(M, K, seed=0).view("int16")).to(DEV)
    g = torch.ones(K, dtype=torch.float32, device=DEV)
    packed, gamma = bl.bitlinear_pack_weights(torch.from_numpy(wl.w_normal(N, K, seed=0)).to(DEV))
    dy = torch.from_numpy(wl.dy_normal(M, N, seed=0)).to(DEV)
    dx = torch.empty((M, K), dtype=torch.float32, device=DEV)
    dg = torch.empty(K, dtype=torch.float32, device=DEV)
    dW = torch.empty((N, K), dtype=torch.float32, device=DEV)
    ws = torch.empty(bl.bitlinear_backward_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
    wall, ev = timed_loop(torch, lambda: bl.bitlinear_backward(x, g, packed, gamma, dy, dx=dx, dg=dg, dW=dW, ws=ws),
                          steps, warmup, stream)
    flops = 4.0 * M * N * K
    nbytes = 2 * M * K + 4 * M * N + 4 * K + N * K // 4 + 4 + 4 * M * K + 4 * K + 4 * N * K
    del x, g, packed, gamma, dy, dx, dg, dW, ws
    torch.cuda.empty_cache()
    return dict(M=M, N=N, K=K, flops=flops, algorithmic_bytes=nbytes, backward_us=ev * 1e3,
                backward_us_wall=wall * 1e3, tflops=flops / (ev * 1e-3) / 1e12,
                frac_bf16_peak=flops / (ev * 1e-3) / BF16_PEAK,
                roofline_us=max(flops / BF16_PEAK, nbytes / HBM_PEAK) * 1e6)


def bench_glu(torch, bl, wl, M, D, F, steps, warmup, stream):
    x = torch.from_numpy(wl.x_normal(M, D, seed=0).view("int16")).to(DEV)
    g_gu = torch.ones(D, dtype=torch.float32, device=DEV)
    g_dn = torch.ones(F, dtype=torch.float32, device=DEV)
    pgu, ggu = bl.bitlinear_pack_weights(wl.w_normal_device(2 * F, D, seed=0, layer=0, device=DEV))
    pdn, gdn = bl.bitlinear_pack_weights(wl.w_normal_device(D, F, seed=0, layer=1, device=DEV))
    y = torch.empty((M, D), dtype=torch.float32, device=DEV)
    ws = torch.empty(bl.bitlinear_glu_workspace_bytes(M, D, F), dtype=torch.uint8, device=DEV)
    wall, ev = timed_loop(torch, lambda: bl.bitlinear_glu_forward(x, g_gu, pgu, ggu, g_dn, pdn, gdn, y=y, ws=ws),
                          steps, warmup, stream)
    ops = 2.0 * M * D * F * 3
    nbytes = glu_bytes(M, D, F)
    return dict(M=M, D=D, F=F, us=ev * 1e3, us_wall=wall * 1e3, gbps=nbytes / (ev * 1e-3) / 1e9,
                tops=ops / (ev * 1e-3) / 1e12, bytes=nbytes, int8_ops=ops)


def bench_glu_layers(torch, bl, wl, L, M, D, F, steps, warmup, stream):
    """One decode step through L independent GLU mixers (one batched call)."""
    x = torch.from_numpy(wl.x_normal(L * M, D, seed=2).view("int16")).to(DEV).view(L, M, D)
    g_gu = torch.ones((L, D), dtype=torch.float32, device=DEV)
    g_dn = torch.ones((L, F), dtype=torch.float32, device=DEV)
    pgu = torch.empty((L, 2 * F, D // 4), dtype=torch.uint8, device=DEV)
    pdn = torch.empty((L, D, F // 4), dtype=torch.uint8, device=DEV)
    ggu = torch.empty(L, dtype=torch.float32, device=DEV)
    gdn = torch.empty(L, dtype=torch.float32, device=DEV)
    ws_p = torch.empty(max(bl.bitlinear_pack_workspace_bytes(2 * F, D), bl.bitlinear_pack_workspace_bytes(D, F)),
                       dtype=torch.uint8, device=DEV)
    for layer in range(L):
        W = wl.w_normal_device(2 * F, D, seed=2, layer=2 * layer, device=DEV)
        bl.bitlinear_pack_weights(W, packed=pgu[layer], gamma=ggu[layer:layer + 1], ws=ws_p)
        W = wl.w_normal_device(D, F, seed=2, layer=2 * layer + 1, device=DEV)
        bl.bitlinear_pack_weights(W, packed=pdn[layer], gamma=gdn[layer:layer + 1], ws=ws_p)
        del W
    y = torch.empty((L, M, D), dtype=torch.float32, device=DEV)
    ws = torch.empty(bl.bitlinear_glu_batched_workspace_bytes(L, M, D, F), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    wall, ev = timed_loop(torch, lambda: bl.bitlinear_glu_forward_batched(x, g_gu, pgu, ggu, g_dn, pdn, gdn,
                                                                          y=y, ws=ws), steps, warmup, stream)
    nbytes = L * glu_bytes(M, D, F)
    del x, g_gu, g_dn, pgu, pdn, ggu, gdn, y, ws
    torch.cuda.empty_cache()
    return dict(layers=L, M=M, D=D, F=F, bytes_per_step=nbytes, wall_ms=wall, event_ms=ev,
                gbps=nbytes / (wall * 1e-3) / 1e9, kernel_gbps=nbytes / (ev * 1e-3) / 1e9)


def bench_repack(torch, bl, wl, L, N, K, steps, warmup, stream):
    """Re-ternarisation of L fp32 master matrices [N, K] in one batched pack
    call (a training step's re-pack of a layer stack).  The algorithmic bytes
    are one read of W and the packed write; the two-pass kernels read W
    twice (gamma, then the codes)."""
    W = torch.empty((L, N, K), dtype=torch.float32, device=DEV)
    for layer in range(L):
        W[layer] = wl.w_normal_device(N, K, seed=0, layer=layer, device=DEV)
    packed = torch.empty((L, N, K // 4), dtype=torch.uint8, device=DEV)
    gamma = torch.empty(L, dtype=torch.float32, device=DEV)
    ws = torch.empty(bl.bitlinear_pack_batched_workspace_bytes(L, N, K), dtype=torch.uint8, device=DEV)
    wall, ev = timed_loop(torch, lambda: bl.bitlinear_pack_weights_batched(W, packed=packed, gamma=gamma, ws=ws),
                          steps, warmup, stream)
    alg = L * (4 * N * K + N * K // 4 + 4)
    two_pass = L * (8 * N * K + N * K // 4 + 4)
    del W, packed, gamma, ws
    torch.cuda.empty_cache()
    return dict(layers=L, N=N, K=K, wall_ms=wall, event_ms=ev, algorithmic_bytes=alg,
                gbps_algorithmic=alg / (ev * 1e-3) / 1e9, gbps_two_pass=two_pass / (ev * 1e-3) / 1e9,
                weights_per_s=L * N * K / (ev * 1e-3))


def bench_hbm_copy(torch, nbytes, steps):
    """Context: a plain device-to-device copy of buffers far larger than the
    256 MB Infinity Cache (read + write bytes per second)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    del a, b
    torch.cuda.empty_cache()
    return dict(bytes_each_way=nbytes, gbps_read_plus_write=2.0 * nbytes * steps / el / 1e9)


def vendor_int8_gemm_us(torch, M, N, K, steps, warmup, stream):
    """Context, not this library's path: device time of the vendor's dense
    int8 GEMM (torch._int_mm, int8 [M, K] x int8 [K, N] -> int32 [M, N]) on
    the same shape, with random int8 operands and B column-major (its faster
    layout here).  It does no quantisation, no 2-bit unpacking and no
    rescale.  None where the call is not available."""
    if not hasattr(torch, "_int_mm"):
        return None
    gen = torch.Generator(device=DEV)
    gen.manual_seed(0)
    a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=DEV, generator=gen)
    b = torch.randint(-1, 2, (N, K), dtype=torch.int8, device=DEV, generator=gen).t()
    try:
        _, ev = timed_loop(torch, lambda: torch._int_mm(a, b), steps, warmup, stream)
    except (RuntimeError, NotImplementedError):
        return None
    del a, b
    return ev * 1e3


def bench_mlgru_scan(torch, bl, wl, B, T, d, steps, warmup, stream):
    """The MLGRU recurrence alone (bitlinear_mlgru_scan) from fp32
    pre-activations z [B, T, 3d]: algorithmic bytes are z read once (12 per
    token and channel), p written once (2) and the state read and written
    (8 per channel)."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    z = torch.randn((B, T, 3 * d), generator=gen, device=DEV, dtype=torch.float32) * 2.0
    state = torch.zeros((B, d), dtype=torch.float32, device=DEV)
    p = torch.empty((B, T, d), dtype=torch.int16, device=DEV)
    ws = torch.empty(max(1, bl.bitlinear_mlgru_scan_workspace_bytes(B, T, d)), dtype=torch.uint8, device=DEV)
    wall, ev = timed_loop(torch, lambda: bl.bitlinear_mlgru_scan(z, state, p=p, ws=ws), steps, warmup, stream)
    nbytes = 14 * B * T * d + 8 * B * d
    del z, state, p, ws
    torch.cuda.empty_cache()
    return dict(B=B, T=T, d=d, us=ev * 1e3, us_wall=wall * 1e3, algorithmic_bytes=nbytes,
                gbps=nbytes / (ev * 1e-3) / 1e9, frac_hbm=nbytes / (ev * 1e-3) / HBM_PEAK)


def make_layer(torch, bl, wl, d, F, seed=0):
    """One layer's weights, packed on the device: MLGRU in [3d, d] and out
    [d, d], GLU gate|up [2F, d] and down [d, F]; RMSNorm gains of 1."""
    def packed(N, K, layer):
        return bl.bitlinear_pack_weights(wl.w_normal_device(N, K, seed=seed, layer=layer, device=DEV))

    ones = lambda n: torch.ones(n, dtype=torch.float32, device=DEV)  # noqa: E731
    pin, gin = packed(3 * d, d, 0)
    pout, gout = packed(d, d, 1)
    pgu, ggu = packed(2 * F, d, 2)
    pdn, gdn = packed(d, F, 3)
    mw = (ones(d), pin, gin, ones(d), pout, gout)
    gw = (ones(d), pgu, ggu, ones(F), pdn, gdn)
    weight_bytes = sum(t.numel() * t.element_size() for t in mw + gw)
    return mw, gw, weight_bytes


def bench_layer_prefill(torch, bl, wl, B, T, d, F, steps, warmup, stream):
    """One layer (MLGRU token mixer, then GLU channel mixer, residuals in
    bf16) over B sequences of T tokens, the pages' inference setting at B =
    1, T = 2048: latency per layer and the device memory one layer holds
    (packed weights and gains, input, output, state and workspace)."""
    mw, gw, wbytes = make_layer(torch, bl, wl, d, F)
    x = torch.from_numpy(wl.x_normal(B * T, d, seed=3).view("int16")).to(DEV).view(B, T, d)
    state = torch.zeros((B, d), dtype=torch.float32, device=DEV)
    out = torch.empty((B, T, d), dtype=torch.int16, device=DEV)
    wsb = bl.bitlinear_layer_workspace_bytes(B, T, d, F)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)

    def step():
        state.zero_()
        bl.bitlinear_layer_forward(x, mw, gw, state, out=out, ws=ws)

    wall, ev = timed_loop(torch, step, steps, warmup, stream)
    ops = 2.0 * B * T * d * (3 * d + d + 3 * F)
    act = 2 * x.numel() * 2 + 4 * state.numel()
    del x, state, out, ws, mw, gw
    torch.cuda.empty_cache()
    return dict(B=B, T=T, d=d, F=F, us=ev * 1e3, us_wall=wall * 1e3, ms=ev, tokens_per_s=B * T / (ev * 1e-3),
                int8_ops=ops, tops=ops / (ev * 1e-3) / 1e12, weight_bytes=wbytes, activation_bytes=act,
                workspace_bytes=wsb, memory_gb=(wbytes + act + wsb) / 1e9)


def bench_layer_decode(torch, bl, wl, d, F, tokens, steps, warmup, stream):
    """Decoding one sequence through one layer, one token per call with the
    state carried (T = 1, B = 1): `tokens` consecutive calls captured into
    one HIP graph and replayed, and the same calls issued eagerly."""
    mw, gw, wbytes = make_layer(torch, bl, wl, d, F, seed=1)
    x = torch.from_numpy(wl.x_normal(tokens, d, seed=4).view("int16")).to(DEV).view(1, tokens, d)
    xs = [x[:, t:t + 1].contiguous() for t in range(tokens)]
    state = torch.zeros((1, d), dtype=torch.float32, device=DEV)
    outs = [torch.empty((1, 1, d), dtype=torch.int16, device=DEV) for _ in range(tokens)]
    ws = torch.empty(bl.bitlinear_layer_workspace_bytes(1, 1, d, F), dtype=torch.uint8, device=DEV)

    def calls():
        for t in range(tokens):
            bl.bitlinear_layer_forward(xs[t], mw, gw, state, out=outs[t], ws=ws)

    wall_e, ev_e = timed_loop(torch, calls, 3, 1, stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    wall, ev = timed_loop(torch, graph.replay, steps, warmup, stream)
    del graph, x, xs, state, outs, ws, mw, gw
    torch.cuda.empty_cache()
    return dict(d=d, F=F, tokens=tokens, us_per_token_graph=ev * 1e3 / tokens,
                us_per_token_eager=ev_e * 1e3 / tokens, weight_bytes=wbytes,
                weight_gbps_graph=wbytes / (ev * 1e-3 / tokens) / 1e9,
                ms_per_2048_tokens_graph=ev / tokens * 2048)


def bench_crossover(torch, bl, wl, K, N, Ms, steps, warmup, stream):
    """Each kernel choice of bitlinear_forward_ex at M tokens of one layer
    shape: about 1 GiB of cold weights, one call per layer captured into a
    HIP graph and replayed; microseconds per call.  The crossover is the
    smallest M at which the int8 MFMA path beats the best streaming path
    (the fused decode kernel or the GEMV)."""
    L = max(32, (1 << 30) // (N * K // 4))
    packed = torch.empty((L, N, K // 4), dtype=torch.uint8, device=DEV)
    gamma = torch.empty(L, dtype=torch.float32, device=DEV)
    wsp = torch.empty(bl.bitlinear_pack_workspace_bytes(N, K), dtype=torch.uint8, device=DEV)
    for layer in range(L):
        W = wl.w_normal_device(N, K, seed=5, layer=layer, device=DEV)
        bl.bitlinear_pack_weights(W, packed=packed[layer], gamma=gamma[layer:layer + 1], ws=wsp)
        del W
    g = torch.ones(K, dtype=torch.float32, device=DEV)
    names = {bl.BITLINEAR_KERNEL_AUTO: "auto", bl.BITLINEAR_KERNEL_DECODE: "decode",
             bl.BITLINEAR_KERNEL_GEMV: "gemv", bl.BITLINEAR_KERNEL_MFMA: "mfma"}
    table = {}
    for M in Ms:
        log(f"[bench]   M={M}")
        x = torch.from_numpy(wl.x_normal(M, K, seed=M).view("int16")).to(DEV)
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        ws = torch.empty(bl.bitlinear_forward_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
        kernels = [bl.BITLINEAR_KERNEL_AUTO, bl.BITLINEAR_KERNEL_MFMA]
        if M <= 8:
            kernels.append(bl.BITLINEAR_KERNEL_GEMV)
        if bl.bitlinear_decode_supported(M, K):
            kernels.append(bl.BITLINEAR_KERNEL_DECODE)
        row = {}
        for kern in kernels:
            def calls(kern=kern):
                for layer in range(L):
                    bl.bitlinear_forward(x, g, packed[layer], gamma[layer:layer + 1], y=y, ws=ws, kernel=kern)

            calls()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                calls()
            torch.cuda.synchronize()
            _, ev = timed_loop(torch, graph.replay, steps, warmup, stream)
            row[names[kern]] = round(ev * 1e3 / L, 3)
            del graph
        stream_best = min([row[k] for k in ("decode", "gemv") if k in row], default=None)
        row["fastest"] = min((v, k) for k, v in row.items() if k != "auto")[1]
        row["auto_vs_fastest"] = round(row["auto"] / row[row["fastest"]], 3)
        row["mfma_beats_streaming"] = None if stream_best is None else bool(row["mfma"] < stream_best)
        table[M] = row
        del x, y, ws
    crossover = next((M for M in Ms if table[M]["mfma_beats_streaming"]), None)
    del packed, gamma, wsp
    torch.cuda.empty_cache()
    return dict(K=K, N=N, layers=L, us_per_call=table, crossover_m=crossover)


# --------------------------------------------------------------------------
# CPU oracle baseline
# --------------------------------------------------------------------------

def host_cpu():
    """This host's CPU model, logical CPU count and the CPUs this process may
    run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return dict(cpu_model=model, nproc=os.cpu_count(), usable_cpus=usable)


def _oracle_threads(threads, work, seconds, min_items):
    """Run work(i) for i = 0, 1, ... on `threads` Python threads until
    `seconds` have passed and at least `min_items` items are done; the oracle
    is C behind ctypes, which releases the interpreter lock during each call,
    so the threads run in parallel.  Returns (items done, elapsed s)."""
    import threading

    lock = threading.Lock()
    state = dict(next=0, done=0)
    t0 = time.perf_counter()

    def worker():
        while True:
            with lock:
                if time.perf_counter() - t0 >= seconds and state["next"] >= min_items:
                    return
                i = state["next"]
                state["next"] += 1
            work(i)
            with lock:
                state["done"] += 1

    ts = [threading.Thread(target=worker) for _ in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return state["done"], time.perf_counter() - t0


def cpu_baseline(wl, M, N, K, seconds, threads):
    """The CPU oracle (plain C, -O2, one add/subtract per weight) on this
    host, unchanged: the headline's decode layers on one thread and on
    `threads` threads (independent layers per thread), and a row sample of
    the 8192 x 2048 x 2048 prefill on as many threads, scaled to all 8192
    rows (the oracle's cost is linear in the rows).  `value` is the
    all-threads decode rate in the headline's unit."""
    import numpy as np
    import oracle

    orc = oracle.Oracle()
    pool = []
    for i in range(4):
        x = wl.x_normal(M, K, seed=100 + i)
        W = wl.w_normal(N, K, seed=100 + i)
        gm = orc.gamma(W)
        pool.append((x, orc.ternarize(W, gm), gm))
    g = np.ones(K, np.float32)

    def decode(i):
        x, w, gm = pool[i % len(pool)]
        orc.bitlinear_ternary(x, g, w, gm)

    n1, el1 = _oracle_threads(1, decode, seconds / 2, 4)
    nt, elt = _oracle_threads(threads, decode, seconds / 4, 4 * threads)
    one = dict(value=n1 * layer_bytes(M, N, K) / el1 / 1e9, unit="GB/s", cores=1,
               sample=f"{n1} layers of the decode workload, {el1:.1f} s")

    # prefill: 8192 x 2048 x 2048, Student-t x; blocks of 32 token rows
    PM, PN, PK, rows = 8192, 2048, 2048, 32
    Wp = wl.w_normal(PN, PK, seed=0)
    gp = orc.gamma(Wp)
    wp = orc.ternarize(Wp, gp)
    xp = wl.x_student_t(PM, PK, seed=0)
    gpk = np.ones(PK, np.float32)

    def prefill(i):
        r0 = (i * rows) % PM
        orc.bitlinear_ternary(xp[r0:r0 + rows], gpk, wp, gp)

    blocks, elp = _oracle_threads(threads, prefill, seconds / 4, max(8, threads))
    done_rows = blocks * rows
    ops = 2.0 * done_rows * PN * PK
    prefill = dict(value=ops / elp / 1e12, unit="int8 TOPS", cores=threads,
                   extrapolated_ms_per_8192_rows=elp * 1e3 * PM / done_rows,
                   sample=f"{done_rows} of the 8192 token rows of the prefill (blocks of {rows} rows over "
                          f"{threads} threads), {elp:.1f} s; the full layer's time extrapolated linearly "
                          f"in rows (extrapolated)")
    return dict(value=nt * layer_bytes(M, N, K) / elt / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"{nt} layers of the M={M} K={K} N={N} decode workload (4 seeded layers cycled) on "
                       f"{threads} threads, {elt:.1f} s",
                single_thread=one, prefill_8192=prefill, host=host_cpu(),
                seconds=el1 + elt + elp)


# --------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=1024)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="total seconds of oracle work for cpu_baseline (split over its three samples)")
    ap.add_argument("--cpu-threads", type=int, default=16,
                    help="threads for the all-cores oracle samples (capped at the CPUs this process may use)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="",
                    help="run only these secondary workloads after the headline (comma-separated; "
                         "available: backward, layer, crossover, prefill, repack)")
    ap.add_argument("--skip", default="",
                    help="skip these secondary workloads in a full run (comma-separated: layer, crossover, "
                         "backward); for profiling runs, where counter collection serialises every dispatch")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay line (its 1024-node graphs are slow under counter collection)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the layer is measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bitlinear_layer_amd as bl
    import workloads as wl

    torch.cuda.set_device(0)
    bl.lib()
    stream = torch.cuda.current_stream()

    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=DEV)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    M, N, K = 1, 2048, 2048
    log(f"[bench] decode M={M} K={K} N={N} x {args.layers} layers: {args.steps} steps")
    head = bench_decode(torch, bl, wl, args.layers, M, N, K, args.steps, args.warmup, stream)
    log(f"[bench] decode: {head['gbps']:.1f} GB/s wall, {head['kernel_gbps']:.1f} GB/s by events")

    secondary = {}
    only = [w for w in args.only.split(",") if w]
    skip = [w for w in args.skip.split(",") if w]
    if not args.no_secondary and not only:
        log("[bench] single layer M=1")
        secondary["decode_m1_single_layer"] = bench_single_layer(torch, bl, wl, 1, N, K, 200, stream)
        if not args.no_graph:
            log("[bench] single-layer calls over 1024 layers, replayed from a HIP graph")
            secondary["decode_m1_graph_1024_calls"] = bench_graph_calls(torch, bl, wl, args.layers, 1, N, K, 5,
                                                                        2, stream)
        log("[bench] decode M=8")
        secondary["decode_m8_layers"] = bench_decode(torch, bl, wl, args.layers, 8, N, K, max(5, args.steps // 2),
                                                     args.warmup, stream)
        log("[bench] prefill 8192")
        secondary["prefill_8192"] = bench_prefill(torch, bl, wl, 8192, 2048, 2048, max(10, args.steps // 2),
                                                  args.warmup, stream)
        for K2, N2 in ((2560, 2560), (2560, 6912), (6912, 2560)):
            L2 = max(64, (1 << 30) // layer_bytes(1, N2, K2))  # about 1 GiB of weights, cold
            log(f"[bench] decode M=1 K={K2} N={N2} x {L2} layers")
            secondary[f"decode_m1_k{K2}_n{N2}_layers"] = bench_decode(
                torch, bl, wl, L2, 1, N2, K2, max(5, args.steps // 2), args.warmup, stream)
        for K2, N2 in ((2560, 2560), (2560, 6912), (6912, 2560)):
            for M2 in (64, 512):
                log(f"[bench] sweep M={M2} K={K2} N={N2} over ~1 GiB")
                secondary[f"sweep_m{M2}_k{K2}_n{N2}_layers"] = bench_sweep_layers(
                    torch, bl, wl, M2, N2, K2, max(5, args.steps // 5), args.warmup, stream)
            for M2 in (4096, 16384):
                log(f"[bench] sweep M={M2} K={K2} N={N2}")
                secondary[f"sweep_m{M2}_k{K2}_n{N2}"] = bench_prefill(torch, bl, wl, M2, N2, K2, max(5, args.steps // 5),
                                                                      args.warmup, stream)
        log("[bench] glu")
        secondary["glu_m1_layers"] = bench_glu_layers(torch, bl, wl, 128, 1, 2048, 5632, max(5, args.steps // 2),
                                                      args.warmup, stream)
        secondary["glu_m1"] = bench_glu(torch, bl, wl, 1, 2048, 5632, 100, args.warmup, stream)
        log("[bench] re-ternarisation of 64 x 2048 x 2048 fp32 master weights")
        secondary["repack_64x2048x2048"] = bench_repack(torch, bl, wl, 64, 2048, 2048, 10, 2, stream)
        secondary["context_hbm_copy_2gib"] = bench_hbm_copy(torch, 2 << 30, 10)
        secondary["glu_m4096"] = bench_glu(torch, bl, wl, 4096, 2048, 5632, max(10, args.steps // 2),
                                           args.warmup, stream)

    if only and "repack" in only:
        log("[bench] re-ternarisation of 64 x 2048 x 2048 fp32 master weights")
        secondary["repack_64x2048x2048"] = bench_repack(torch, bl, wl, 64, 2048, 2048, 10, 2, stream)
        secondary["context_hbm_copy_2gib"] = bench_hbm_copy(torch, 2 << 30, 10)

    if only and "prefill" in only:
        log("[bench] prefill 8192 and the MFMA-tile sweep shapes")
        secondary["prefill_8192"] = bench_prefill(torch, bl, wl, 8192, 2048, 2048, max(10, args.steps // 2),
                                                  args.warmup, stream)
        for K2, N2 in ((2560, 2560), (2560, 6912), (6912, 2560)):
            for M2 in (4096, 16384):
                secondary[f"sweep_m{M2}_k{K2}_n{N2}"] = bench_prefill(torch, bl, wl, M2, N2, K2,
                                                                      max(5, args.steps // 5), args.warmup, stream)
        secondary["glu_m4096"] = bench_glu(torch, bl, wl, 4096, 2048, 5632, max(10, args.steps // 2),
                                           args.warmup, stream)

    if (not args.no_secondary and not only and "layer" not in skip) or "layer" in only:
        log("[bench] MLGRU scan, one sequence of 2048 tokens, d = 2048")
        secondary["mlgru_scan_b1_t2048_d2048"] = bench_mlgru_scan(torch, bl, wl, 1, 2048, 2048, 20, 3, stream)
        secondary["mlgru_scan_b64_t256_d2048"] = bench_mlgru_scan(torch, bl, wl, 64, 256, 2048, 10, 2, stream)
        log("[bench] one layer (MLGRU + GLU), batch 1, 2048 tokens")
        secondary["layer_prefill_b1_t2048"] = bench_layer_prefill(torch, bl, wl, 1, 2048, 2048, 5632, 10, 2, stream)
        log("[bench] one layer, decoding 64 tokens one call each")
        secondary["layer_decode_b1"] = bench_layer_decode(torch, bl, wl, 2048, 5632, 64, 10, 2, stream)

    if (not args.no_secondary and not only and "crossover" not in skip) or "crossover" in only:
        for K2, N2 in ((2560, 2560), (2560, 6912), (6912, 2560)):
            log(f"[bench] kernel crossover K={K2} N={N2}")
            secondary[f"crossover_k{K2}_n{N2}"] = bench_crossover(torch, bl, wl, K2, N2,
                                                                  (1, 2, 4, 8, 16, 32, 64, 128), 5, 1, stream)

    if (not args.no_secondary and not only and "backward" not in skip) or "backward" in only:
        log("[bench] backward (straight-through) 8192 x 2048 x 2048")
        secondary["backward_8192x2048x2048"] = bench_backward(torch, bl, wl, 8192, 2048, 2048,
                                                              max(10, args.steps // 2), args.warmup, stream)

    cpu = None
    if not args.no_cpu:
        log(f"[bench] cpu oracle for ~{args.cpu_seconds:.0f} s")
        usable = host_cpu()["usable_cpus"] or 1
        threads = max(1, min(args.cpu_threads or usable, usable))
        cpu = cpu_baseline(wl, M, N, K, args.cpu_seconds, threads)
        cpu.pop("seconds")

    digest = source_digest(*DECODE_SOURCES)
    traffic = read_traffic("decode.hip", digest, head["bytes_per_step"])
    achieved = head["bytes_per_step"] / (head["event_ms"] * 1e-3) / 1e9
    out = {
        "metric": "fused BitLinear: HBM GB/s at M=1 and int8 TOPS at M=8192 (% of roofline)",
        "value": round(head["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"decode step M=1 K=2048 N=2048 through {args.layers} independent layers",
                   "M": M, "K": K, "N": N, "layers": args.layers,
                   "bytes_per_step": head["bytes_per_step"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved / (HBM_PEAK / 1e9), 4),
                     "traffic": None if traffic is None else traffic * 1.0,
                     "kernel": "bl::decode_kernel (fused quantise + GEMV, one launch per step)", "source_sha256_16": digest},
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
