// device_common.h -- device helpers shared by the BitLinear kernels (gfx950).
//
// Wave size is 64 on CDNA; every block-level helper assumes blockDim.x is a
// multiple of 64 and at most 1024.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Packed ternary decode.  A 32-bit packed word holds one group of 16 weights:
// weight j = 4*i + t in byte t, bits 2i+1..2i, as code = w + 1.  Shifting by
// 2i and masking each byte to 2 bits yields the codes of weights 4i..4i+3 as
// four int8 lanes in order, so the four words below are the 16 codes of the
// group in k order (byte b of the 16-byte result = weight b).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void decode_codes(uint32_t w, int32_t& c0, int32_t& c1,
                                             int32_t& c2, int32_t& c3) {
    c0 = (int32_t)(w & 0x03030303u);
    c1 = (int32_t)((w >> 2) & 0x03030303u);
    c2 = (int32_t)((w >> 4) & 0x03030303u);
    c3 = (int32_t)((w >> 6) & 0x03030303u);
}

// Signed 4 x int8 dot product accumulated into an int32 (v_dot4c_i32_i8).
__device__ __forceinline__ int32_t dot4(int32_t a, int32_t b, int32_t acc) {
    return __builtin_amdgcn_sdot4(a, b, acc, false);
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Nearest bf16 (ties to even) of a finite fp32 value, as a bit pattern.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---------------------------------------------------------------------------
// Wave and block reductions (fixed order, so results are deterministic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}
__device__ __forceinline__ int32_t wave_sum(int32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Block reductions: every thread returns the block-wide result.  `scratch`
// holds at least blockDim.x / 64 elements; the helper synchronises before
// reusing it, so consecutive calls may share one scratch array.
template <typename T, typename WaveOp, typename Combine>
__device__ __forceinline__ T block_reduce(T v, T* scratch, WaveOp wave_op, Combine combine) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    v = wave_op(v);
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    T r = scratch[0];
    for (int i = 1; i < nwaves; ++i) r = combine(r, scratch[i]);
    return r;
}

__device__ __forceinline__ double block_sum(double v, double* scratch) {
    return block_reduce<double>(
        v, scratch, [](double a) { return wave_sum(a); }, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ int32_t block_sum(int32_t v, int32_t* scratch) {
    return block_reduce<int32_t>(
        v, scratch, [](int32_t a) { return wave_sum(a); },
        [](int32_t a, int32_t b) { return a + b; });
}
__device__ __forceinline__ float block_max(float v, float* scratch) {
    return block_reduce<float>(
        v, scratch, [](float a) { return wave_max(a); }, [](float a, float b) { return fmaxf(a, b); });
}

}  // namespace bl
