"""Seeded synthetic inputs for the BitLinear layer and its GLU mixer.

Shared by the tests, the smoke check and the benchmark, for both the HIP
library and the CPU oracle.  This module draws random numbers and rounds
them to the storage types; it holds none of the method's arithmetic.

Generator: NumPy's PCG64 seeded with SeedSequence([seed, stream]), one
stream per tensor (x = 0, outlier positions = 1, W = 2, second W = 3, RMSNorm
weights = 4, output gradient = 5), so every tensor is reproducible on its own.  The pages train on
a text corpus that is not available; these draws stand in for the layer
activations and master weights at the pages' model widths.
"""
import numpy as np

STREAM_X, STREAM_OUTLIER, STREAM_W, STREAM_W2, STREAM_G, STREAM_DY = 0, 1, 2, 3, 4, 5


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the uint16
    bit patterns.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def x_normal(M, K, seed=0, outlier_frac=0.0, outlier_scale=1.0):
    """bf16 [M, K] ~ N(0, 1).  With outlier_frac > 0, exactly
    round(outlier_frac * M * K) distinct entries (drawn without replacement)
    are multiplied by outlier_scale before rounding to bf16."""
    x = rng(seed, STREAM_X).standard_normal((M, K)).astype(np.float32)
    n_out = int(round(outlier_frac * M * K))
    if n_out > 0:
        idx = rng(seed, STREAM_OUTLIER).choice(M * K, size=n_out, replace=False)
        flat = x.reshape(-1)
        flat[idx] = flat[idx] * np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


def x_student_t(M, K, df=3, seed=0):
    """bf16 [M, K] drawn from Student's t with df degrees of freedom."""
    x = rng(seed, STREAM_X).standard_t(df, size=(M, K)).astype(np.float32)
    return f32_to_bf16_bits(x)


def w_normal(N, K, sigma=0.02, seed=0, stream=STREAM_W):
    """fp32 [N, K] master weights ~ N(0, sigma^2)."""
    return (rng(seed, stream).standard_normal((N, K)) * sigma).astype(np.float32)


def dy_normal(M, N, seed=0, scale=1.0):
    """fp32 [M, N] ~ N(0, scale^2): the gradient of a loss with respect to
    the layer output, for the backward pass."""
    return (rng(seed, STREAM_DY).standard_normal((M, N)) * scale).astype(np.float32)


def rms_weight(K, kind="ones", seed=0):
    """RMSNorm gain [K]: all ones (the pages' setting), or uniform in
    [0.5, 1.5) so that a dropped or misplaced gain shows in tests."""
    if kind == "ones":
        return np.ones(K, np.float32)
    return (0.5 + rng(seed, STREAM_G).random(K)).astype(np.float32)


# Workload shapes: a single layer at hidden 256 (parity), decode at hidden
# 2048, prefill at 8192 tokens, the GLU channel mixer at d=2048 / inner 5632,
# and a 2560-wide sweep.  x recipe per workload as named in "x".
WORKLOADS = {
    "parity_16x256x256": dict(M=16, K=256, N=256, x="normal", outlier_frac=0.01,
                              outlier_scale=20.0),
    "decode_2048": dict(Ms=(1, 8), K=2048, N=2048, x="normal"),
    "prefill_8192x2048x2048": dict(M=8192, K=2048, N=2048, x="student_t3"),
    "glu_2048_5632": dict(Ms=(1, 4096), D=2048, F=5632, x="normal"),
    "sweep_2560": dict(Ms=(1, 64, 512, 4096, 16384), KN=((2560, 2560), (2560, 6912), (6912, 2560)),
                       x="normal", outlier_frac=0.005, outlier_scale=50.0),
}


def make_x(M, K, recipe="normal", seed=0, outlier_frac=0.0, outlier_scale=1.0):
    if recipe == "normal":
        return x_normal(M, K, seed, outlier_frac, outlier_scale)
    if recipe == "student_t3":
        return x_student_t(M, K, 3, seed)
    raise ValueError(recipe)


def w_normal_device(N, K, sigma=0.02, seed=0, layer=0, device="cuda"):
    """fp32 [N, K] ~ N(0, sigma^2) drawn on the GPU with torch's seeded
    generator (Philox), for benchmarks that need many distinct layers; layer
    selects an independent stream."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1_000_003 + int(layer) * 7919 + STREAM_W)
    return torch.randn((N, K), generator=gen, device=device, dtype=torch.float32) * sigma
