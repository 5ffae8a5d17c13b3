// quant.hip -- fused RMSNorm + per-token absmax int8 quantisation.
//
// [ld246, "融合 BitLinear 层的创新"] and [jiqizhixin, "具有三值权重的 MatMul-free
// 密集层", Algorithm 1]: RMSNorm and quantisation are one fused step in front
// of the ternary product, reading the activations from HBM once;
// [datacamp, "Các thành phần lõi: MLGRU và GLU", panel "RMS norm"]: the
// activations are RMS-normalised before quantisation.  Readings:
//   r = 1 / sqrt(fp32(sum x^2 / K) + eps)   (sum of squares in fp64)
//   xn = (x * r) * g,  s = 127 / max(max|xn|, 1e-5),  q = clip(rint(xn * s))
// with every fp32 operation correctly rounded (no fast-math, no contraction).
//
// Two layouts, same arithmetic: waves streaming over many rows (wave-wide
// reductions, no barriers), one 256-thread block per row for few rows.  Each
// thread keeps its slice of the row in registers (8 bf16 per 16-byte load),
// so x is read from HBM once and q written once.  Three reductions: fp64
// sum of squares (fixed tree order, deterministic), fp32 max, int32 sum of
// the codes (the sum the offset-coded product subtracts).
#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "quant_row.h"

namespace bl {
namespace {

constexpr int kQuantThreads = 256;

template <int CPT>  // 8-element chunks per thread
__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ g,
                                                              int64_t rows_per_g, int K, float eps,
                                                              int8_t* __restrict__ q,
                                                              float* __restrict__ s,
                                                              int32_t* __restrict__ sumq) {
    __shared__ double dscratch[kQuantThreads / kWave];
    __shared__ float fscratch[kQuantThreads / kWave];
    __shared__ int32_t iscratch[kQuantThreads / kWave];

    const int64_t row = blockIdx.x;
    const uint16_t* xr = x + row * K;
    const float* gr = g + (row / rows_per_g) * K;
    const int nchunks = K / 8;

    float v[CPT][8];
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int idx = threadIdx.x + c * kQuantThreads;
        if (idx < nchunks) {
            const uint4 raw = *reinterpret_cast<const uint4*>(xr + 8 * idx);
            const uint32_t p[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[c][2 * j] = bf16_lo(p[j]);
                v[c][2 * j + 1] = bf16_hi(p[j]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) ss += (double)v[c][j] * (double)v[c][j];
        }
    }
    ss = block_sum(ss, dscratch);
    const float ms = (float)(ss / (double)K);
    const float r = 1.0f / sqrtf(ms + eps);

    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int idx = threadIdx.x + c * kQuantThreads;
        if (idx < nchunks) {
            const float4 g0 = *reinterpret_cast<const float4*>(gr + 8 * idx);
            const float4 g1 = *reinterpret_cast<const float4*>(gr + 8 * idx + 4);
            const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[c][j] = (v[c][j] * r) * gv[j];
                amax = fmaxf(amax, fabsf(v[c][j]));
            }
        }
    }
    amax = block_max(amax, fscratch);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);

    int32_t qsum = 0;
    int8_t* qr = q + row * K;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int idx = threadIdx.x + c * kQuantThreads;
        if (idx < nchunks) {
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float t = fminf(fmaxf(rintf(v[c][j] * scale), -128.0f), 127.0f);
                const int32_t qi = (int32_t)t;
                qsum += qi;
                packed[j >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (j & 3));
            }
            *reinterpret_cast<uint2*>(qr + 8 * idx) = make_uint2(packed[0], packed[1]);
        }
    }
    qsum = block_sum(qsum, iscratch);
    if (threadIdx.x == 0) {
        s[row] = scale;
        if (sumq) sumq[row] = qsum;
    }
}

// Streaming layout for many rows: each wave walks the rows
// wave_id, wave_id + W, ... (W = waves in the grid) and loads the next row's
// x while it reduces and stores the current one, so HBM reads and writes
// overlap across the whole pass.  Lane l owns the 8-element chunks
// l, l + 64, ... of a row; the three reductions are wave-wide over
// permlane/DPP (no LDS, no barrier).  The row index is wave-uniform, so
// addressing runs on the scalar unit.
//
// The pass is VALU-bound unless each element costs few instructions (a
// wave64 VALU op takes 4 cycles on a 16-lane SIMD); the per-row arithmetic
// (quant_row.h) needs about nine per element and stays bit-identical to the
// definition above.

// Rows of at most 8 chunks per lane prefetch the next row's x (two buffers,
// alternating, so no copies); longer rows skip the prefetch to stay within
// the register file, leaving the other resident waves to cover the load
// latency.  When one RMSNorm weight serves every row, each block stages it
// once in LDS (low and high halves of each 8-element chunk in separate
// arrays, so a wave's 16-byte reads are contiguous and bank-conflict free);
// re-reading it from L2 per wave and row would move more bytes than x itself.
// With a weight per group of rows it is loaded from memory per row.
constexpr int kStreamThreads = 256;
constexpr int64_t kStreamBlocks = 1024;  // 4 blocks (16 waves) per CU on 256 CUs

template <int CPL>
constexpr size_t stream_lds_bytes() { return 2 * CPL * kWave * sizeof(float4); }

// SHARED_G: one weight for all rows (staged in LDS); otherwise a weight per
// group of rows_per_g rows, loaded per row.
template <int CPL, bool FULL, bool SHARED_G, bool PREFETCH = (SHARED_G && CPL <= 8)>
__global__ __launch_bounds__(kStreamThreads) void quant_stream_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ g, int64_t rows_per_g, int64_t rows,
    int K, float eps, int8_t* __restrict__ q, float* __restrict__ s, int32_t* __restrict__ sumq) {
    extern __shared__ float4 g_lds[];  // [2][CPL * 64]: low halves, then high halves
    constexpr int kSpan = CPL * kWave;
    constexpr int kWavesPerBlock = kStreamThreads / kWave;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
    const int nchunks = K / 8;

    if constexpr (SHARED_G) {
        // grid y: groups of `rows` rows with a weight each (a stack of
        // layers); group blockIdx.y is a problem of its own from here on.
        const int64_t group = blockIdx.y;
        x += group * rows * K;
        g += group * K;
        q += group * rows * K;
        s += group * rows;
        if (sumq) sumq += group * rows;
        for (int i = threadIdx.x; i < kSpan; i += kStreamThreads) {
            float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
            if (FULL || i < nchunks) {
                lo = *reinterpret_cast<const float4*>(g + 8 * i);
                hi = *reinterpret_cast<const float4*>(g + 8 * i + 4);
            }
            g_lds[i] = lo;
            g_lds[kSpan + i] = hi;
        }
        __syncthreads();
    }
    int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (row >= rows) return;

    if constexpr (SHARED_G) {
        auto from_lds = [&](int c, float4& lo, float4& hi) {
            const uint32_t idx = lane + (uint32_t)c * kWave;
            lo = g_lds[idx];
            hi = g_lds[kSpan + idx];
        };
        if constexpr (PREFETCH) {
            uint4 xa[CPL], xb[CPL];
            auto step = [&](const uint4 (&cur)[CPL], uint4 (&nxt)[CPL]) {
                if (row + stride < rows) load_x_row<CPL, FULL>(x + (row + stride) * K, lane, nchunks, nxt);
                quant_row_regs<CPL, FULL>(cur, from_lds, row, lane, K, eps, q, s, sumq);
                row += stride;
            };
            load_x_row<CPL, FULL>(x + row * K, lane, nchunks, xa);
            for (;;) {
                step(xa, xb);
                if (row >= rows) break;
                step(xb, xa);
                if (row >= rows) break;
            }
        } else {
            uint4 xc[CPL];
            for (; row < rows; row += stride) {
                load_x_row<CPL, FULL>(x + row * K, lane, nchunks, xc);
                quant_row_regs<CPL, FULL>(xc, from_lds, row, lane, K, eps, q, s, sumq);
            }
        }
    } else if constexpr (CPL <= 8) {
        uint4 xc[CPL];
        float4 gv[CPL][2];
        auto from_regs = [&](int c, float4& lo, float4& hi) {
            lo = gv[c][0];
            hi = gv[c][1];
        };
        for (; row < rows; row += stride) {
            load_x_row<CPL, FULL>(x + row * K, lane, nchunks, xc);
            load_g_row<CPL, FULL>(g + (row / rows_per_g) * K, lane, nchunks, gv);
            quant_row_regs<CPL, FULL>(xc, from_regs, row, lane, K, eps, q, s, sumq);
        }
    } else {
        // long rows: read the weight where it is used, four chunks at a time
        uint4 xc[CPL];
        for (; row < rows; row += stride) {
            const float* gr = g + (row / rows_per_g) * K;
            auto from_global = [&](int c, float4& lo, float4& hi) {
                const uint32_t idx = lane + (uint32_t)c * kWave;
                lo = hi = make_float4(0.f, 0.f, 0.f, 0.f);
                if (FULL || idx < (uint32_t)nchunks) {
                    lo = *reinterpret_cast<const float4*>(gr + 8 * idx);
                    hi = *reinterpret_cast<const float4*>(gr + 8 * idx + 4);
                }
            };
            load_x_row<CPL, FULL>(x + row * K, lane, nchunks, xc);
            quant_row_regs<CPL, FULL>(xc, from_global, row, lane, K, eps, q, s, sumq);
        }
    }
}

// Ragged long rows with a weight per group of rows do not fit the register
// file in the streaming layout; they take the block-per-row kernels.
constexpr bool stream_per_row_g_ok(int cpl, bool full) { return full || cpl <= 12; }

template <int CPL, bool FULL>
void launch_stream_g(dim3 grid, hipStream_t stream, const uint16_t* x, const float* g,
                     int64_t rows_per_g, int64_t rows, int K, float eps, const ActStage& out) {
    if (rows_per_g >= rows) {
        quant_stream_kernel<CPL, FULL, true><<<grid, kStreamThreads, stream_lds_bytes<CPL>(), stream>>>(
            x, g, rows_per_g, rows, K, eps, out.q, out.s, out.sumq);
    } else if (rows % rows_per_g == 0 && rows / rows_per_g <= 65535) {
        // A weight per group of rows (a stack of layers): one launch with the
        // groups along grid y, each block staging its group's weight in LDS
        // once and walking that group's rows (up to 4 per wave, prefetched)
        // -- rather than each wave re-reading a weight row per x row.
        const int64_t groups = rows / rows_per_g;
        const int64_t per_block = (int64_t)(kStreamThreads / kWave) * 4;
        const dim3 ggrid((unsigned)((rows_per_g + per_block - 1) / per_block), (unsigned)groups);
        quant_stream_kernel<CPL, FULL, true><<<ggrid, kStreamThreads, stream_lds_bytes<CPL>(), stream>>>(
            x, g, rows_per_g, rows_per_g, K, eps, out.q, out.s, out.sumq);
    } else if constexpr (stream_per_row_g_ok(CPL, FULL)) {
        quant_stream_kernel<CPL, FULL, false><<<grid, kStreamThreads, 0, stream>>>(
            x, g, rows_per_g, rows, K, eps, out.q, out.s, out.sumq);
    }
}

template <int CPL>
void launch_stream(dim3 grid, hipStream_t stream, const uint16_t* x, const float* g, int64_t rows_per_g,
                   int64_t rows, int K, float eps, const ActStage& out) {
    if (K == CPL * kWave * 8)
        launch_stream_g<CPL, true>(grid, stream, x, g, rows_per_g, rows, K, eps, out);
    else
        launch_stream_g<CPL, false>(grid, stream, x, g, rows_per_g, rows, K, eps, out);
}

// Rows longer than 8 * 8 * 256 elements: same arithmetic, re-reading x and g
// from memory (L2) in each of the three passes instead of holding the row.
__global__ __launch_bounds__(kQuantThreads) void quant_long_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ g, int64_t rows_per_g, int K,
    float eps, int8_t* __restrict__ q, float* __restrict__ s, int32_t* __restrict__ sumq) {
    __shared__ double dscratch[kQuantThreads / kWave];
    __shared__ float fscratch[kQuantThreads / kWave];
    __shared__ int32_t iscratch[kQuantThreads / kWave];
    const int64_t row = blockIdx.x;
    const uint16_t* xr = x + row * K;
    const float* gr = g + (row / rows_per_g) * K;
    double ss = 0.0;
    for (int k = threadIdx.x; k < K; k += kQuantThreads) {
        const double xv = (double)__uint_as_float((uint32_t)xr[k] << 16);
        ss += xv * xv;
    }
    ss = block_sum(ss, dscratch);
    const float ms = (float)(ss / (double)K);
    const float r = 1.0f / sqrtf(ms + eps);
    float amax = 0.0f;
    for (int k = threadIdx.x; k < K; k += kQuantThreads) {
        const float xn = (__uint_as_float((uint32_t)xr[k] << 16) * r) * gr[k];
        amax = fmaxf(amax, fabsf(xn));
    }
    amax = block_max(amax, fscratch);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);
    int32_t qsum = 0;
    for (int k = threadIdx.x; k < K; k += kQuantThreads) {
        const float xn = (__uint_as_float((uint32_t)xr[k] << 16) * r) * gr[k];
        const int32_t qi = (int32_t)fminf(fmaxf(rintf(xn * scale), -128.0f), 127.0f);
        qsum += qi;
        q[row * K + k] = (int8_t)qi;
    }
    qsum = block_sum(qsum, iscratch);
    if (threadIdx.x == 0) {
        s[row] = scale;
        if (sumq) sumq[row] = qsum;
    }
}

__global__ __launch_bounds__(kQuantThreads) void row_sums_kernel(const int8_t* __restrict__ q, int K,
                                                                 int32_t* __restrict__ sumq) {
    __shared__ int32_t iscratch[kQuantThreads / kWave];
    const int64_t row = blockIdx.x;
    int32_t acc = 0;
    for (int k = threadIdx.x; k < K; k += kQuantThreads) acc += q[row * K + k];
    acc = block_sum(acc, iscratch);
    if (threadIdx.x == 0) sumq[row] = acc;
}

}  // namespace

size_t act_stage_bytes(int64_t rows, int64_t K) {
    return (size_t)(round_up(rows * K, 256) + 2 * round_up(rows * 4, 256));
}

ActStage act_stage_carve(void* base, int64_t rows, int64_t K) {
    char* p = static_cast<char*>(base);
    ActStage a;
    a.q = reinterpret_cast<int8_t*>(p);
    p += round_up(rows * K, 256);
    a.s = reinterpret_cast<float*>(p);
    p += round_up(rows * 4, 256);
    a.sumq = reinterpret_cast<int32_t*>(p);
    return a;
}

hipError_t launch_quant(const uint16_t* x, const float* g, int64_t rows, int64_t rows_per_g, int K,
                        float eps, ActStage out, hipStream_t stream) {
    const int nchunks = K / 8;
    const int cpl = (nchunks + kWave - 1) / kWave;  // chunks per lane, one wave per row
    const bool full = K == cpl * kWave * 8;
    const bool grouped_g = rows % rows_per_g == 0 && rows / rows_per_g <= 65535;
    if (rows >= 64 && cpl <= 16 && (rows_per_g >= rows || grouped_g || stream_per_row_g_ok(cpl, full))) {
        const int64_t waves_per_block = kStreamThreads / kWave;
        const dim3 grid((unsigned)std::min<int64_t>((rows + waves_per_block - 1) / waves_per_block,
                                                    kStreamBlocks));
        switch (cpl) {
            case 1: launch_stream<1>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 2: launch_stream<2>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 3: launch_stream<3>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 4: launch_stream<4>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 5: launch_stream<5>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 6: launch_stream<6>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 7: launch_stream<7>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 8: launch_stream<8>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 9: launch_stream<9>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 10: launch_stream<10>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 11: launch_stream<11>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 12: launch_stream<12>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 13: launch_stream<13>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 14: launch_stream<14>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            case 15: launch_stream<15>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
            default: launch_stream<16>(grid, stream, x, g, rows_per_g, rows, K, eps, out); break;
        }
        return hipGetLastError();
    }
    // Few rows: one block per row spreads each row over more lanes.
    const int cpt = (nchunks + kQuantThreads - 1) / kQuantThreads;
    const dim3 grid((unsigned)rows);
    if (cpt <= 1)
        quant_kernel<1><<<grid, kQuantThreads, 0, stream>>>(x, g, rows_per_g, K, eps, out.q, out.s, out.sumq);
    else if (cpt <= 2)
        quant_kernel<2><<<grid, kQuantThreads, 0, stream>>>(x, g, rows_per_g, K, eps, out.q, out.s, out.sumq);
    else if (cpt <= 4)
        quant_kernel<4><<<grid, kQuantThreads, 0, stream>>>(x, g, rows_per_g, K, eps, out.q, out.s, out.sumq);
    else if (cpt <= 8)
        quant_kernel<8><<<grid, kQuantThreads, 0, stream>>>(x, g, rows_per_g, K, eps, out.q, out.s, out.sumq);
    else
        quant_long_kernel<<<grid, kQuantThreads, 0, stream>>>(x, g, rows_per_g, K, eps, out.q, out.s, out.sumq);
    return hipGetLastError();
}

hipError_t launch_row_sums(const int8_t* q, int64_t rows, int K, int32_t* sumq, hipStream_t stream) {
    row_sums_kernel<<<(unsigned)rows, kQuantThreads, 0, stream>>>(q, K, sumq);
    return hipGetLastError();
}

}  // namespace bl
