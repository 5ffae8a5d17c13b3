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
// One 256-thread block per token row; each thread keeps its slice of the
// row in registers (8 bf16 per 16-byte load), so x is read from HBM once and
// q written once.  Three block reductions: fp64 sum of squares (fixed tree
// order, deterministic), fp32 max, int32 sum of the codes (the sum the
// offset-coded product subtracts).
#include "device_common.h"
#include "launch.h"

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
    const int cpt = (K / 8 + kQuantThreads - 1) / kQuantThreads;
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
