// gemv.hip -- decode-shaped ternary product (few tokens, weights streamed).
//
// For M <= 8 tokens the product is bound by reading the packed weights from
// HBM (N*K/4 bytes against 2*M*N*K int8 operations).  One wave owns one
// output row n at a time; its 64 lanes stride along K one packed 32-bit word
// (16 weights) at a time, expand each word into four int8 code words with
// shifts and masks, and accumulate against the int8 activations with
// v_dot4 (4 products per instruction).  A wave reduction gives the row sum.
#include "epilogue.h"

namespace bl {
namespace {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

template <int MAXM, Epilogue EP>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(ProductArgs a, int rows_per_block) {
    constexpr bool kGlu = EP == Epilogue::kGluBf16;
    const int b = blockIdx.y;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int M = a.M, N = a.N, K = a.K;
    const int nwords = K / 16;
    const int64_t nrows = kGlu ? 2 * (int64_t)N : (int64_t)N;
    const uint32_t* P = reinterpret_cast<const uint32_t*>(a.packed) + (int64_t)b * nrows * nwords;
    const int8_t* Q = a.q + (int64_t)b * M * K;
    const int64_t tok0 = (int64_t)b * M;

    const int n_begin = blockIdx.x * rows_per_block;
    const int n_end = min(N, n_begin + rows_per_block);
    for (int n = n_begin + wave; n < n_end; n += kGemvWaves) {
        int32_t acc[MAXM], acc2[MAXM];
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc[m] = acc2[m] = 0;
        const uint32_t* prow = P + (int64_t)n * nwords;
        const uint32_t* prow2 = P + ((int64_t)N + n) * nwords;  // up row (GLU only)
        for (int w = lane; w < nwords; w += kWave) {
            int32_t c[4], u[4];
            decode_codes(prow[w], c[0], c[1], c[2], c[3]);
            if (kGlu) decode_codes(prow2[w], u[0], u[1], u[2], u[3]);
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                if (m < M) {
                    const int4 qv = *reinterpret_cast<const int4*>(Q + (int64_t)m * K + 16 * w);
                    acc[m] = dot4(c[0], qv.x, acc[m]);
                    acc[m] = dot4(c[1], qv.y, acc[m]);
                    acc[m] = dot4(c[2], qv.z, acc[m]);
                    acc[m] = dot4(c[3], qv.w, acc[m]);
                    if (kGlu) {
                        acc2[m] = dot4(u[0], qv.x, acc2[m]);
                        acc2[m] = dot4(u[1], qv.y, acc2[m]);
                        acc2[m] = dot4(u[2], qv.z, acc2[m]);
                        acc2[m] = dot4(u[3], qv.w, acc2[m]);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            if (m < M) {
                acc[m] = wave_sum(acc[m]);
                if (kGlu) acc2[m] = wave_sum(acc2[m]);
            }
        }
        if (lane == 0) {
            const float gamma = a.gamma ? a.gamma[b] : 0.0f;
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                if (m >= M) continue;
                const int64_t t = tok0 + m;
                const int32_t v = acc[m] - a.sumq[t];
                if (EP == Epilogue::kI32) {
                    static_cast<int32_t*>(a.out)[t * N + n] = v;
                } else {
                    const float cs = gamma / a.s[t];
                    if (EP == Epilogue::kF32) {
                        static_cast<float*>(a.out)[t * N + n] = rescale(v, cs);
                    } else {
                        const int32_t vu = acc2[m] - a.sumq[t];
                        static_cast<uint16_t*>(a.out)[t * N + n] = glu_bf16(rescale(v, cs), rescale(vu, cs));
                    }
                }
            }
        }
    }
}

template <Epilogue EP>
hipError_t launch_gemv_ep(const ProductArgs& a, hipStream_t stream) {
    // Aim for about 2048 blocks in total, at least 4 and at most 256 rows each.
    int64_t total_rows = (int64_t)a.N * a.batch;
    int64_t rpb = (total_rows + 2047) / 2048;
    rpb = rpb < 4 ? 4 : (rpb > 256 ? 256 : rpb);
    rpb = round_up(rpb, kGemvWaves);
    const dim3 grid((unsigned)((a.N + rpb - 1) / rpb), (unsigned)a.batch);
    if (a.M <= 1)
        gemv_kernel<1, EP><<<grid, kGemvThreads, 0, stream>>>(a, (int)rpb);
    else if (a.M <= 2)
        gemv_kernel<2, EP><<<grid, kGemvThreads, 0, stream>>>(a, (int)rpb);
    else if (a.M <= 4)
        gemv_kernel<4, EP><<<grid, kGemvThreads, 0, stream>>>(a, (int)rpb);
    else
        gemv_kernel<8, EP><<<grid, kGemvThreads, 0, stream>>>(a, (int)rpb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const ProductArgs& a, Epilogue ep, hipStream_t stream) {
    if (a.M > kGemvMaxM) return hipErrorInvalidValue;
    switch (ep) {
        case Epilogue::kF32: return launch_gemv_ep<Epilogue::kF32>(a, stream);
        case Epilogue::kI32: return launch_gemv_ep<Epilogue::kI32>(a, stream);
        case Epilogue::kGluBf16: return launch_gemv_ep<Epilogue::kGluBf16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace bl
