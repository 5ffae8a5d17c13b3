// gemm_mfma.hip -- prefill-shaped ternary product on the int8 matrix cores.
//
// At large token counts the ternary product is a dense contraction
// (2*M*N*K int8 operations against (M+N/4)*K bytes), so it runs on
// v_mfma_i32_16x16x64_i8.  The packed weights are the B operand: one packed
// 32-bit word holds the 16 codes of one 16-weight group, and a lane's
// 16-byte B fragment of a 16x16x64 step is exactly one such group, so each
// lane loads one word per step and expands it in registers (shift + mask,
// 7 VALU ops per 16 weights).  The int8 activations (A operand) are staged
// through LDS and shared by the waves of the block.
//
// Operand pairing: lane l of A supplies row l%16, k = 16*(l/16) + 0..15 of
// the 64-wide step; lane l of B supplies column l%16 at the same k.  The
// accumulator holds D[4*(l/16) + v][l%16] in element v.
#include "epilogue.h"

namespace bl {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves as 2 x 2
constexpr int kBM = 128;       // tokens per block
constexpr int kBN = 128;       // packed weight rows per block (64 f for the GLU)
constexpr int kBK = 64;        // k per MFMA step
constexpr int kLdsPitch = kBK + 16;

template <Epilogue EP>
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(ProductArgs a) {
    constexpr bool kGlu = EP == Epilogue::kGluBf16;
    __shared__ __attribute__((aligned(16))) int8_t As[kBM * kLdsPitch];

    const int b = blockIdx.y;
    const int cols_per_block = kGlu ? kBN / 2 : kBN;
    const int ntiles_n = (a.N + cols_per_block - 1) / cols_per_block;
    const int tile_n = blockIdx.x % ntiles_n;
    const int tile_m = blockIdx.x / ntiles_n;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wm = wave >> 1, wn = wave & 1;
    const int M = a.M, N = a.N, K = a.K;
    const int nwords = K / 16;
    const int64_t nrows = kGlu ? 2 * (int64_t)N : (int64_t)N;
    const int8_t* Q = a.q + (int64_t)b * M * K;
    const uint32_t* P = reinterpret_cast<const uint32_t*>(a.packed) + (int64_t)b * nrows * nwords;
    const int m0 = tile_m * kBM;

    // Packed row feeding N-block bj of this lane (clamped in range; results
    // for clamped rows are never stored).
    const uint32_t* brow[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        int64_t row;
        if (kGlu) {
            const int f = tile_n * (kBN / 2) + wn * 32 + (bj & 1) * 16 + (lane & 15);
            row = (bj < 2 ? 0 : (int64_t)N) + min(f, N - 1);
        } else {
            const int n = tile_n * kBN + wn * 64 + bj * 16 + (lane & 15);
            row = min(n, N - 1);
        }
        brow[bj] = P + row * nwords;
    }

    i32x4 acc[4][4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = i32x4{0, 0, 0, 0};

    const int lrow = threadIdx.x >> 1;          // A tile row this thread loads
    const int lcol = (threadIdx.x & 1) * 32;    // and its 32-byte half
    const int64_t grow = min(m0 + lrow, M - 1);
    for (int k0 = 0; k0 < K; k0 += kBK) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kk = k0 + lcol + 16 * j;
            int4 v = make_int4(0, 0, 0, 0);
            if (kk < K) v = *reinterpret_cast<const int4*>(Q + grow * K + kk);
            *reinterpret_cast<int4*>(&As[lrow * kLdsPitch + lcol + 16 * j]) = v;
        }
        __syncthreads();

        const int kw = k0 / 16 + (lane >> 4);
        i32x4 bfrag[4];
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const uint32_t pw = kw < nwords ? brow[bj][kw] : 0u;
            int32_t c0, c1, c2, c3;
            decode_codes(pw, c0, c1, c2, c3);
            bfrag[bj] = i32x4{c0, c1, c2, c3};
        }
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
            const i32x4 afrag = *reinterpret_cast<const i32x4*>(
                &As[(wm * 64 + bi * 16 + (lane & 15)) * kLdsPitch + 16 * (lane >> 4)]);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                acc[bi][bj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afrag, bfrag[bj], acc[bi][bj], 0, 0, 0);
        }
    }

    // Epilogue: subtract sum_k q, rescale (or form the GLU product), store.
    const float gamma = a.gamma ? a.gamma[b] : 0.0f;
    const int64_t tok0 = (int64_t)b * M;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = m0 + wm * 64 + bi * 16 + 4 * (lane >> 4) + v;
            if (m >= M) continue;
            const int64_t t = tok0 + m;
            const int32_t sq = a.sumq[t];
            const float cs = EP == Epilogue::kI32 ? 0.0f : gamma / a.s[t];
            if (kGlu) {
#pragma unroll
                for (int bj = 0; bj < 2; ++bj) {
                    const int f = tile_n * (kBN / 2) + wn * 32 + bj * 16 + (lane & 15);
                    if (f < N) {
                        const float zg = rescale(acc[bi][bj][v] - sq, cs);
                        const float zu = rescale(acc[bi][bj + 2][v] - sq, cs);
                        static_cast<uint16_t*>(a.out)[t * N + f] = glu_bf16(zg, zu);
                    }
                }
            } else {
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) {
                    const int n = tile_n * kBN + wn * 64 + bj * 16 + (lane & 15);
                    if (n < N) {
                        const int32_t val = acc[bi][bj][v] - sq;
                        if (EP == Epilogue::kI32)
                            static_cast<int32_t*>(a.out)[t * N + n] = val;
                        else
                            static_cast<float*>(a.out)[t * N + n] = rescale(val, cs);
                    }
                }
            }
        }
    }
}

template <Epilogue EP>
hipError_t launch_ep(const ProductArgs& a, hipStream_t stream) {
    const int cols_per_block = EP == Epilogue::kGluBf16 ? kBN / 2 : kBN;
    const int64_t tiles = (int64_t)((a.N + cols_per_block - 1) / cols_per_block) *
                          ((a.M + kBM - 1) / kBM);
    const dim3 grid((unsigned)tiles, (unsigned)a.batch);
    gemm_mfma_kernel<EP><<<grid, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(const ProductArgs& a, Epilogue ep, hipStream_t stream) {
    switch (ep) {
        case Epilogue::kF32: return launch_ep<Epilogue::kF32>(a, stream);
        case Epilogue::kI32: return launch_ep<Epilogue::kI32>(a, stream);
        case Epilogue::kGluBf16: return launch_ep<Epilogue::kGluBf16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace bl
