"""Helpers for the GPU parity tests: moving seeded inputs to the device and
comparing library results with the oracle."""
import numpy as np
import torch

import bitlinear_layer_amd as bl
import oracle
import workloads as wl

DEV = "cuda:0"


def to_dev_bf16(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def from_dev_bf16(t):
    return t.cpu().numpy().view(np.uint16)


def pack_on_gpu(W):
    """Pack fp32 W with the library; returns (packed device tensor, gamma device tensor)."""
    return bl.bitlinear_pack_weights(to_dev(W))


def q_flip_stats(q_gpu, q_ref):
    """(fraction of elements that differ, largest difference)."""
    d = np.abs(q_gpu.astype(np.int32) - q_ref.astype(np.int32))
    return float(np.mean(d != 0)), int(d.max()) if d.size else 0


def assert_q_parity(q_gpu, q_ref, s_gpu=None, s_ref=None):
    """int8 codes: equal except at most 0.1% of elements, each off by exactly
    one step (a reduction-order tie flip); scales equal on rows whose codes are
    equal and within 2 ulp elsewhere."""
    frac, dmax = q_flip_stats(q_gpu, q_ref)
    assert dmax <= 1 and frac <= 1e-3, (frac, dmax)
    if s_gpu is not None:
        same_rows = np.all(q_gpu == q_ref, axis=1)
        assert np.array_equal(s_gpu[same_rows], s_ref[same_rows])
        ulp = np.abs(s_gpu.view(np.int32).astype(np.int64) - s_ref.view(np.int32).astype(np.int64))
        assert ulp.max(initial=0) <= 2
    return frac


def assert_y_parity(y_gpu, y_ref, q_rows_equal=None, rel_row=1e-2):
    """fp32 outputs: per row, max |dy| <= rel_row * max |y_ref| (the stated
    end-to-end bound); on rows whose int8 codes matched exactly, also the
    element-wise bound of the fp32 rescale: |dy| <= 2^-22 |y_ref|."""
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    scale = np.abs(y_ref).max(axis=1, keepdims=True)
    row_rel = (err / np.where(scale > 0, scale, 1.0)).max(axis=1) if err.size else np.zeros(0)
    assert np.all(row_rel <= rel_row), float(row_rel.max())
    zero_rows = scale[:, 0] == 0
    assert np.all(err[zero_rows] == 0)
    if q_rows_equal is not None:
        rows = np.asarray(q_rows_equal)
        bound = 2.0 ** -22 * np.abs(y_ref[rows])
        assert np.all(err[rows] <= bound), float((err[rows] - bound).max())
    return float(row_rel.max()) if row_rel.size else 0.0


def oracle_inputs(M, N, K, seed=0, recipe="normal", outlier_frac=0.0, outlier_scale=1.0,
                  g_kind="random"):
    x = wl.make_x(M, K, recipe, seed, outlier_frac, outlier_scale)
    W = wl.w_normal(N, K, seed=seed)
    g = wl.rms_weight(K, g_kind, seed=seed)
    return x, W, g


ORC = None


def orc():
    global ORC
    if ORC is None:
        ORC = oracle.Oracle()
    return ORC
