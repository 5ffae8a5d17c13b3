"""bitlinear_forward_noalloc (the entry point that allocates nothing) against
bitlinear_forward and the oracle, through the C ABI.

Two calls in a row on the MFMA path (the second with fewer tokens and a
shorter row, so the shared scratch still holds the first call's larger
stage), one on the fused one-token path, a HIP-graph capture of the call
(capture fails if the call allocates) replayed on new inputs with eager work
in between, and the rejection of a size beyond the scratch.  Outputs must be
bit-identical to bitlinear_forward's (same kernels) and within the oracle
bar (per-row 1e-2 of the row maximum)."""
import numpy as np
import pytest
import torch

import bitlinear_layer_amd as bl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _one(M, N, K, seed):
    print("noalloc", M, N, K, flush=True)
    x, W, g = gu.oracle_inputs(M, N, K, seed=seed, outlier_frac=0.005, outlier_scale=50.0)
    packed, gamma = gu.pack_on_gpu(W)
    xd, gd = gu.to_dev_bf16(x), gu.to_dev(g)
    y_ref = bl.bitlinear_forward(xd, gd, packed, gamma)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=gu.DEV)
    bl.bitlinear_forward_noalloc(xd, gd, packed, gamma, y)
    torch.cuda.synchronize()
    a, b = y.cpu().numpy(), y_ref.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ref = gu.orc().bitlinear(x, g, W)
    gu.assert_y_parity(a, ref["y"])


def test_noalloc_two_calls_second_smaller():
    _one(300, 520, 2048, seed=1)   # 256-row tiles, stage of 300 x 2048 codes
    _one(40, 264, 1024, seed=2)    # 64-row tiles, a smaller stage over the same scratch


def test_noalloc_one_token_fused_path():
    _one(1, 2048, 2048, seed=3)


def test_noalloc_rejects_beyond_scratch():
    M, K = 32768, 2048  # 64 MiB of codes > 48 MiB
    x = torch.zeros((M, K), dtype=torch.int16, device=gu.DEV)
    g = torch.ones(K, dtype=torch.float32, device=gu.DEV)
    packed = torch.zeros((16, K // 4), dtype=torch.uint8, device=gu.DEV)
    gamma = torch.ones(1, dtype=torch.float32, device=gu.DEV)
    y = torch.empty((M, 16), dtype=torch.float32, device=gu.DEV)
    with pytest.raises(bl.BitlinearError) as e:
        bl.bitlinear_forward_noalloc(x, g, packed, gamma, y)
    assert e.value.status == bl.BITLINEAR_ERR_INVALID_ARG and "scratch" in str(e.value)


def test_noalloc_captured_in_a_graph():
    M, N, K = 200, 512, 2048
    x0, W, g = gu.oracle_inputs(M, N, K, seed=4)
    packed, gamma = gu.pack_on_gpu(W)
    xd, gd = gu.to_dev_bf16(x0), gu.to_dev(g)
    y = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
    bl.bitlinear_forward_noalloc(xd, gd, packed, gamma, y)  # first call on the device: before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bl.bitlinear_forward_noalloc(xd, gd, packed, gamma, y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bl.bitlinear_forward_noalloc(xd, gd, packed, gamma, y)
    torch.cuda.synchronize()
    for rep in range(3):
        xr, _, _ = gu.oracle_inputs(M, N, K, seed=10 + rep)
        xd.copy_(gu.to_dev_bf16(xr))
        graph.replay()
        torch.cuda.synchronize()
        eager = bl.bitlinear_forward(xd, gd, packed, gamma)  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), eager.cpu().numpy().view(np.uint32)), rep
