"""HIP graph capture of the library's calls.

Every entry point only launches kernels on the caller's stream: no
allocation, memset, copy or synchronisation, with scratch taken from the
caller's workspace.  A caller can therefore capture a sequence of calls into
one graph and replay it.  Each replay here runs on new inputs copied into the
captured tensors, with eager library calls and synchronisations in between,
and must equal eager calls on the same inputs bit for bit.
"""
import numpy as np
import pytest
import torch

import bitlinear_layer_amd as bl
import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    dev = gu.DEV
    K, N = 2048, 2048
    packed, gamma = gu.pack_on_gpu(wl.w_normal(N, K, seed=3))
    g = gu.to_dev(wl.rms_weight(K, kind="uniform", seed=3))
    D, F = 256, 320
    pgu, ggu = gu.pack_on_gpu(wl.w_normal(2 * F, D, seed=4))
    pdn, gdn = gu.pack_on_gpu(wl.w_normal(D, F, seed=4, stream=wl.STREAM_W2))
    g_gu, g_dn = gu.to_dev(wl.rms_weight(D)), gu.to_dev(wl.rms_weight(F))

    # one token (fused decode kernel), 8 tokens (fused K-split kernel),
    # 64 tokens (quantisation pass, then the MFMA tiles); GLU at 1 and 70
    dense_m = (1, 8, 64)
    glu_m = (1, 70)

    def inputs(rep):
        xs = [gu.to_dev_bf16(wl.x_normal(m, K, seed=100 + 10 * rep + m)) for m in dense_m]
        xg = [gu.to_dev_bf16(wl.x_normal(m, D, seed=200 + 10 * rep + m)) for m in glu_m]
        return xs, xg

    def new_outputs():
        return ([torch.empty((m, N), dtype=torch.float32, device=dev) for m in dense_m],
                [torch.empty((m, D), dtype=torch.float32, device=dev) for m in glu_m])

    ws_d = [torch.empty(bl.bitlinear_forward_workspace_bytes(m, N, K), dtype=torch.uint8, device=dev)
            for m in dense_m]
    ws_g = [torch.empty(bl.bitlinear_glu_workspace_bytes(m, D, F), dtype=torch.uint8, device=dev)
            for m in glu_m]

    def run(xs, xg, ys, yg, wsd, wsg):
        for x, y, ws in zip(xs, ys, wsd):
            bl.bitlinear_forward(x, g, packed, gamma, y=y, ws=ws)
        for x, y, ws in zip(xg, yg, wsg):
            bl.bitlinear_glu_forward(x, g_gu, pgu, ggu, g_dn, pdn, gdn, y=y, ws=ws)

    # captured tensors: inputs, outputs and workspaces stay at fixed addresses
    cap_x, cap_xg = inputs(0)
    cap_y, cap_yg = new_outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(cap_x, cap_xg, cap_y, cap_yg, ws_d, ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(cap_x, cap_xg, cap_y, cap_yg, ws_d, ws_g)
    torch.cuda.synchronize()

    eager_ws_d = [torch.empty_like(w) for w in ws_d]
    eager_ws_g = [torch.empty_like(w) for w in ws_g]
    prev = None
    for rep in range(1, 4):
        xs, xg = inputs(rep)
        for dst, src in zip(cap_x + cap_xg, xs + xg):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu().numpy() for t in cap_y + cap_yg]
        ye, yge = new_outputs()
        run(xs, xg, ye, yge, eager_ws_d, eager_ws_g)
        torch.cuda.synchronize()
        want = [t.cpu().numpy() for t in ye + yge]
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), f"replay {rep}, output {i}"
        # each replay reads the inputs copied in before it
        if prev is not None:
            assert not np.array_equal(got[0], prev)
        prev = got[0]


def test_graph_replay_backward_matches_eager():
    """The backward pass captured into a graph (seven launches, both split
    reductions included) and replayed on new x and dy equals eager calls."""
    dev = gu.DEV
    M, N, K = 300, 2048, 512  # dW has 16 tiles, so its reduction is split
    packed, gamma = gu.pack_on_gpu(wl.w_normal(N, K, seed=21))
    g = gu.to_dev(wl.rms_weight(K, kind="uniform", seed=21))

    def inputs(rep):
        return (gu.to_dev_bf16(wl.x_normal(M, K, seed=300 + rep)), gu.to_dev(wl.dy_normal(M, N, seed=300 + rep)))

    def outs():
        return (torch.empty((M, K), dtype=torch.float32, device=dev), torch.empty(K, dtype=torch.float32, device=dev),
                torch.empty((N, K), dtype=torch.float32, device=dev))

    ws = torch.empty(bl.bitlinear_backward_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
    cx, cdy = inputs(0)
    co = outs()

    def run(x, dy, o, w):
        bl.bitlinear_backward(x, g, packed, gamma, dy, dx=o[0], dg=o[1], dW=o[2], ws=w)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(cx, cdy, co, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(cx, cdy, co, ws)
    torch.cuda.synchronize()
    ews = torch.empty_like(ws)
    for rep in range(1, 4):
        x, dy = inputs(rep)
        cx.copy_(x)
        cdy.copy_(dy)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu().numpy() for t in co]
        eo = outs()
        run(x, dy, eo, ews)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, [t.cpu().numpy() for t in eo])):
            assert np.array_equal(a, b), f"replay {rep}, output {i}"
