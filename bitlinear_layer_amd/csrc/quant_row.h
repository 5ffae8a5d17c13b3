// quant_row.h -- RMSNorm + absmax int8 quantisation of one token row held
// in a wave's registers (library internal; used by the streaming quantiser
// and the fused few-token kernel).
//
// [ld246, "融合 BitLinear 层的创新"]: RMSNorm and quantisation as one fused
// step, the activations read once; [datacamp, "Các thành phần lõi: MLGRU và
// GLU"]: RMS normalisation before the per-token absmax quantisation.
// Lane l owns the 8-element chunks l, l + 64, ... of the row; the fp64 sum of
// squares, the fp32 max and the int32 code sum are wave-wide reductions over
// permlane/DPP (no LDS, no barrier).  The arithmetic is written to need about
// nine VALU operations per element while staying bit-identical to
//   r = 1 / sqrt(fp32(sum x^2 / K) + eps),  xn = (x * r) * g,
//   s = 127 / max(max|xn|, 1e-5),  q = clip(rint(xn * s), -128, 127):
//   * x^2 of a bf16 value is exact in fp64, so fma(x, x, ss) equals ss + x*x;
//   * |xn * s| <= 127 * (1 + 2^-22) by construction (|xn| <= amax, s is the
//     correctly rounded 127 / max(amax, 1e-5)), so the clip never binds;
//   * for |y| < 2^22, fl(y + 1.5 * 2^23) = 1.5 * 2^23 + rint(y) (ties to
//     even), so the bit pattern of that sum minus 0x4B400000 is the integer
//     code: its low byte is the int8 code and integer sums of the patterns
//     give the code sum.
#pragma once

#include "device_common.h"

namespace bl {

constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23
constexpr uint32_t kRoundMagicBits = 0x4B400000u;

// FULL: the row is exactly CPL * 64 chunks, so no lane needs a bounds test.
template <int CPL, bool FULL>
__device__ __forceinline__ void load_x_row(const uint16_t* __restrict__ xr, uint32_t lane, int nchunks,
                                           uint4 (&dst)[CPL]) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const uint32_t idx = lane + (uint32_t)c * kWave;
        if (FULL) {
            dst[c] = load_stream16(reinterpret_cast<const uint32_t*>(xr + 8 * idx));
        } else {
            dst[c] = make_uint4(0u, 0u, 0u, 0u);
            if (idx < (uint32_t)nchunks)
                dst[c] = load_stream16(reinterpret_cast<const uint32_t*>(xr + 8 * idx));
        }
    }
}

template <int CPL, bool FULL>
__device__ __forceinline__ void load_g_row(const float* __restrict__ gr, uint32_t lane, int nchunks,
                                           float4 (&dst)[CPL][2]) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const uint32_t idx = lane + (uint32_t)c * kWave;
        if (FULL || idx < (uint32_t)nchunks) {
            dst[c][0] = *reinterpret_cast<const float4*>(gr + 8 * idx);
            dst[c][1] = *reinterpret_cast<const float4*>(gr + 8 * idx + 4);
        } else {
            dst[c][0] = dst[c][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

// RMSNorm + quantisation of one row held in registers (xc: bf16 pairs);
// gfetch(c, lo, hi) yields the RMSNorm weight of this lane's chunk c (zero
// past the row end).  Lane 0 writes s and the code sum.
template <int CPL, bool FULL, typename GFetch>
__device__ __forceinline__ void quant_row_regs(const uint4 (&xc)[CPL], GFetch gfetch, int64_t row,
                                               uint32_t lane, int K, float eps,
                                               int8_t* __restrict__ q, float* __restrict__ s,
                                               int32_t* __restrict__ sumq) {
    const int nchunks = K / 8;
    float v[CPL][8];
    double ss0 = 0.0, ss1 = 0.0;  // two chains halve the fma latency stall
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const uint32_t p[4] = {xc[c].x, xc[c].y, xc[c].z, xc[c].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[c][2 * j] = bf16_lo(p[j]);
            v[c][2 * j + 1] = bf16_hi(p[j]);
            ss0 = fma((double)v[c][2 * j], (double)v[c][2 * j], ss0);
            ss1 = fma((double)v[c][2 * j + 1], (double)v[c][2 * j + 1], ss1);
        }
    }
    const double ss = wave_sum_dpp(ss0 + ss1);
    const float ms = (float)(ss / (double)K);
    const float r = 1.0f / sqrtf(ms + eps);

    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        // Compiler-only fence: keeps the weight reads of each group of four
        // chunks next to their use instead of all hoisted up front (which
        // spills for long rows).
        if (CPL > 8 && c % 4 == 0) asm volatile("" ::: "memory");
        float4 g0, g1;
        gfetch(c, g0, g1);
        const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[c][j] = (v[c][j] * r) * gg[j];
            amax = fmaxf(amax, fabsf(v[c][j]));
        }
    }
    amax = wave_max_dpp(amax);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);

    uint32_t bits_sum = 0;
    int8_t* qr = q + row * K;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        uint32_t b[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            b[j] = __float_as_uint(v[c][j] * scale + kRoundMagic);
            bits_sum += b[j];
        }
        // low bytes of b[0..3] and b[4..7] -> two words of int8 codes
        const uint32_t w0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u),
                                                  0x05040100u);
        const uint32_t w1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u),
                                                  0x05040100u);
        const uint32_t idx = lane + (uint32_t)c * kWave;
        if (FULL || idx < (uint32_t)nchunks)
            *reinterpret_cast<uint2*>(qr + 8 * idx) = make_uint2(w0, w1);
    }
    if (sumq) {
        // each lane summed CPL * 8 patterns (zeros past the row end give
        // exactly the offset), so subtract that many offsets, mod 2^32
        const int32_t lane_sum = (int32_t)(bits_sum - (uint32_t)(CPL * 8) * kRoundMagicBits);
        const int32_t total = wave_sum_dpp(lane_sum);
        if (lane == 0) sumq[row] = total;
    }
    if (lane == 0) s[row] = scale;
}

}  // namespace bl
