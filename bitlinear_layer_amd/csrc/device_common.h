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

// The same codes, each scaled by 4^i instead of shifted down, for i = 0..2
// (byte values 0..32, still valid int8), plus the fourth word shifted:
// 5 VALU ops per 16 weights instead of 7.  Products against q must then be
// accumulated separately per scale and recombined as a1 + a4/4 + a16/16;
// each partial sum is an exact multiple of its scale.
__device__ __forceinline__ void decode_codes_scaled(uint32_t w, int32_t& c0, int32_t& c1x4,
                                                    int32_t& c2x16, int32_t& c3) {
    c0 = (int32_t)(w & 0x03030303u);
    c1x4 = (int32_t)(w & 0x0C0C0C0Cu);
    c2x16 = (int32_t)(w & 0x30303030u);
    c3 = (int32_t)((w >> 6) & 0x03030303u);
}

// 16-byte load of data read once (non-temporal hint: do not keep in cache).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const uint32_t* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
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

// ---------------------------------------------------------------------------
// Row sums over groups of LPR lanes without LDS.  Each exchange level pairs
// every lane with one partner that differs in bit log2(O) of the lane index:
//   O = 32, 16 -> v_permlane32_swap / v_permlane16_swap (gfx950);
//   O = 8, 4   -> DPP row_mirror / row_half_mirror (partner lane ^ 15, ^ 7);
//   O = 2, 1   -> DPP quad_perm (partner lane ^ 2, ^ 1).
// The XOR masks 32, 16, 15, 7, 2, 1 span all lane bits, so the levels form a
// hypercube and every group total counts each lane exactly once.
// ---------------------------------------------------------------------------
template <int O>
__device__ __forceinline__ int32_t dpp_partner(int32_t v) {
    constexpr int ctrl = O == 8 ? 0x140 : (O == 4 ? 0x141 : (O == 2 ? 0x4E : 0xB1));
    return __builtin_amdgcn_update_dpp(0, v, ctrl, 0xF, 0xF, false);
}

// Reduce-scatter step: lanes with bit log2(O) clear keep lo + partner's lo,
// lanes with it set keep hi + partner's hi.
template <int O>
__device__ __forceinline__ int32_t scatter_level(int32_t lo, int32_t hi, int lane) {
    if constexpr (O == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
        return (int32_t)r[0] + (int32_t)r[1];
    } else if constexpr (O == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(lo, hi, false, false);
        return (int32_t)r[0] + (int32_t)r[1];
    } else {
        const bool up = (lane & O) != 0;
        const int32_t keep = up ? hi : lo;
        const int32_t send = up ? lo : hi;
        return keep + dpp_partner<O>(send);
    }
}

// All-reduce step over the same pairs.
template <int O>
__device__ __forceinline__ int32_t allreduce_level(int32_t v) {
    if constexpr (O == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (int32_t)r[0] + (int32_t)r[1];
    } else if constexpr (O == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (int32_t)r[0] + (int32_t)r[1];
    } else {
        return v + dpp_partner<O>(v);
    }
}

// v[0..U) are this lane's partial sums for U rows; lanes in aligned groups
// of LPR share the rows.  Returns the full sum of row
// (lane % LPR) >> log2(LPR / U); it is complete in every lane, and lanes with
// (lane % LPR) % (LPR / U) == 0 hold distinct rows.
template <int LPR, int U, int O = LPR / 2>
__device__ __forceinline__ int32_t group_row_sums(int32_t (&v)[U], int lane) {
    static_assert(U >= 1 && U <= LPR && (U & (U - 1)) == 0, "U must be a power of two <= LPR");
    if constexpr (O == 0) {
        return v[0];
    } else if constexpr (U > 1) {
        int32_t h[U / 2];
#pragma unroll
        for (int i = 0; i < U / 2; ++i) h[i] = scatter_level<O>(v[i], v[i + U / 2], lane);
        return group_row_sums<LPR, U / 2, O / 2>(h, lane);
    } else {
        int32_t r[1] = {allreduce_level<O>(v[0])};
        return group_row_sums<LPR, 1, O / 2>(r, lane);
    }
}

// Wave-wide all-reduce over the same hypercube, without LDS: every lane
// returns the total.  At each level a lane combines its value with its
// partner's.  A permlane swap of a register with itself leaves the lane's own
// value in one result and the partner's in the other, so combining the two
// results needs no lane test; the combine is commutative, so both lanes of a
// pair hold the same bits and the total is identical in all 64 lanes.
template <int O>
__device__ __forceinline__ void xor_pair_u32(uint32_t v, uint32_t& a, uint32_t& b) {
    if constexpr (O == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        a = (uint32_t)r[0];
        b = (uint32_t)r[1];
    } else if constexpr (O == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        a = (uint32_t)r[0];
        b = (uint32_t)r[1];
    } else {
        a = v;
        b = (uint32_t)dpp_partner<O>((int32_t)v);
    }
}

template <typename T, typename Combine, int O = 32>
__device__ __forceinline__ T wave_allreduce(T v, Combine combine) {
    if constexpr (O == 0) {
        return v;
    } else {
        T a, b;
        if constexpr (sizeof(T) == 8) {
            const uint64_t u = __builtin_bit_cast(uint64_t, v);
            uint32_t alo, blo, ahi, bhi;
            xor_pair_u32<O>((uint32_t)u, alo, blo);
            xor_pair_u32<O>((uint32_t)(u >> 32), ahi, bhi);
            a = __builtin_bit_cast(T, ((uint64_t)ahi << 32) | alo);
            b = __builtin_bit_cast(T, ((uint64_t)bhi << 32) | blo);
        } else {
            uint32_t ua, ub;
            xor_pair_u32<O>(__builtin_bit_cast(uint32_t, v), ua, ub);
            a = __builtin_bit_cast(T, ua);
            b = __builtin_bit_cast(T, ub);
        }
        constexpr int next = O == 32 ? 16 : (O == 16 ? 8 : (O == 8 ? 4 : (O == 4 ? 2 : (O == 2 ? 1 : 0))));
        return wave_allreduce<T, Combine, next>(combine(a, b), combine);
    }
}

__device__ __forceinline__ double wave_sum_dpp(double v) {
    return wave_allreduce(v, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ float wave_max_dpp(float v) {
    return wave_allreduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ int32_t wave_sum_dpp(int32_t v) {
    return wave_allreduce(v, [](int32_t a, int32_t b) { return a + b; });
}

// Block reductions: every thread returns the block-wide result.  Each wave
// reduces over the register hypercube above (no LDS round trips), lane 0
// leaves the wave's total in scratch[wave], and every thread combines the
// wave totals in wave order, so all threads and all kernels using these
// helpers get the same bits for the same data layout.  `scratch` holds at
// least blockDim.x / 64 elements.  The default form synchronises before
// writing, so consecutive calls may share one scratch array; with
// kFresh = true the caller guarantees that no thread still reads this
// scratch (a slot used once per launch) and the leading barrier is skipped.
// kNW > 0 fixes the number of waves at compile time (the block size the
// kernel is launched with), so the combine is unrolled.
template <bool kFresh = false, int kNW = 0, typename T, typename WaveOp, typename Combine>
__device__ __forceinline__ T block_reduce(T v, T* scratch, WaveOp wave_op, Combine combine) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = kNW > 0 ? kNW : (int)(blockDim.x / kWave);
    v = wave_op(v);
    if constexpr (!kFresh) __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int i = 1; i < nwaves; ++i) r = combine(r, scratch[i]);
    return r;
}

template <bool kFresh = false, int kNW = 0>
__device__ __forceinline__ double block_sum(double v, double* scratch) {
    return block_reduce<kFresh, kNW>(
        v, scratch, [](double a) { return wave_sum_dpp(a); }, [](double a, double b) { return a + b; });
}
template <bool kFresh = false, int kNW = 0>
__device__ __forceinline__ int32_t block_sum(int32_t v, int32_t* scratch) {
    return block_reduce<kFresh, kNW>(
        v, scratch, [](int32_t a) { return wave_sum_dpp(a); },
        [](int32_t a, int32_t b) { return a + b; });
}
template <bool kFresh = false, int kNW = 0>
__device__ __forceinline__ float block_max(float v, float* scratch) {
    return block_reduce<kFresh, kNW>(
        v, scratch, [](float a) { return wave_max_dpp(a); }, [](float a, float b) { return fmaxf(a, b); });
}

}  // namespace bl
