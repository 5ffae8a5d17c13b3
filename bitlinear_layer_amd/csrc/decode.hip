// decode.hip -- fused decode-shaped BitLinear: one launch per call.
//
// For a handful of tokens (M <= 4) the layer is bound by streaming the
// packed weights from HBM (N*K/4 bytes against 2*M*N*K int8 operations), so
// everything else is folded into the one kernel that streams them:
//   1. each block quantises the M token rows itself ([ld246, "融合 BitLinear
//      层的创新"]: activations read once, normalised and quantised on chip):
//      fp64 sum of squares, fp32 absmax and the int8 codes go to LDS; the
//      block's reductions use a fixed order, so every block computes the
//      same codes, bit for bit, as the block-per-row quantisation kernel
//      (the layout the stand-alone pass uses below 64 rows);
//   2. each lane copies the codes of the k-columns it owns into registers;
//   3. the block streams its share of the weight rows: LPR lanes share a
//      row, each loading 16 bytes (64 weights) per step with U rows in
//      flight per wave, expanding the 2-bit codes with shifts and masks and
//      accumulating with v_dot4 ([ld246, "三值权重的应用"]: +1 adds, -1
//      subtracts, 0 skips -- here as sum q*(w+1) - sum q);
//   4. a butterfly over the LPR lanes gives each row's sum; one lane per row
//      rescales ([datacamp, "Các thành phần lõi: MLGRU và GLU"]: scaled
//      ternary accumulation) or, for the GLU, forms bf16(SiLU(gate) * up).
// B independent problems of the same shape run in one launch (grid.y).
#include <algorithm>
#include <atomic>

#include "epilogue.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxDevices = 64;
constexpr int kDefaultCus = 256;
constexpr int kMaxRowChunks = 4;  // rows up to 4 * 8 * kThreads = 8192 wide stay in registers

// Sum q of the row is needed only in the epilogue: each wave leaves its
// partial sum in qpart[wave] (made visible by the barrier that follows the
// quantisation), instead of a block reduction with two more barriers here.
// The integer sum does not depend on the order.
__device__ __forceinline__ void put_wave_sum(int32_t v, int32_t* qpart) {
    v = wave_sum_dpp(v);
    if ((threadIdx.x & (kWave - 1)) == 0) qpart[threadIdx.x / kWave] = v;
}

// The mean of the squares, ss / K rounded to fp32.  For K a power of two
// the quotient is the exact scaling ldexp(ss, -log2 K) (the same bits as the
// division, which is also exact there), one instruction instead of the fp64
// division sequence on the prologue's critical path.
__device__ __forceinline__ float mean_square(double ss, int K) {
    if ((K & (K - 1)) == 0) return (float)ldexp(ss, -__builtin_ctz((unsigned)K));
    return (float)(ss / (double)K);
}

// Codes in LDS are grouped by 16-byte unit: unit j (k in [64c + 16j,
// 64c + 16j + 16)) of every 64-wide chunk c lies at (j * nchunks + c) * 16,
// so the lanes reading unit j of consecutive chunks read consecutive
// 16-byte words (no bank conflicts).  Element block i (k in [8i, 8i + 8)) is
// the low or high half of unit (i / 2) % 4 of chunk i / 8.
__device__ __forceinline__ int code_offset(int i, int nchunks) {
    return (((i >> 1) & 3) * nchunks + (i >> 3)) * 16 + (i & 1) * 8;
}

// Block-cooperative RMSNorm + absmax int8 of one token row into LDS; the
// same arithmetic and reduction order as the block-per-row quant_kernel, so
// the codes agree with it.  dscr and fscr are this row's own scratch slots
// (used once per launch), so the reductions skip their leading barrier.
__device__ __forceinline__ void quantise_row_to_lds(const uint16_t* __restrict__ xr,
                                                    const float* __restrict__ gr, int K, float eps,
                                                    int8_t* __restrict__ qrow, double* dscr,
                                                    float* fscr, int32_t* qpart, float& scale_out) {
    const int nchunks = K / 8;
    double ss = 0.0;
    for (int i = threadIdx.x; i < nchunks; i += kThreads) {
        const uint4 raw = *reinterpret_cast<const uint4*>(xr + 8 * i);
        const uint32_t p[4] = {raw.x, raw.y, raw.z, raw.w};
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_lo(p[j]);
            v[2 * j + 1] = bf16_hi(p[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) ss += (double)v[j] * (double)v[j];
    }
    ss = block_sum<true, kWaves>(ss, dscr);
    const float ms = mean_square(ss, K);
    const float r = 1.0f / sqrtf(ms + eps);
    float amax = 0.0f;
    for (int i = threadIdx.x; i < nchunks; i += kThreads) {
        const uint4 raw = *reinterpret_cast<const uint4*>(xr + 8 * i);
        const uint32_t p[4] = {raw.x, raw.y, raw.z, raw.w};
        const float4 g0 = *reinterpret_cast<const float4*>(gr + 8 * i);
        const float4 g1 = *reinterpret_cast<const float4*>(gr + 8 * i + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float xv = (j & 1) ? bf16_hi(p[j >> 1]) : bf16_lo(p[j >> 1]);
            amax = fmaxf(amax, fabsf((xv * r) * gv[j]));
        }
    }
    amax = block_max<true, kWaves>(amax, fscr);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);
    int32_t qsum = 0;
    for (int i = threadIdx.x; i < nchunks; i += kThreads) {
        const uint4 raw = *reinterpret_cast<const uint4*>(xr + 8 * i);
        const uint32_t p[4] = {raw.x, raw.y, raw.z, raw.w};
        const float4 g0 = *reinterpret_cast<const float4*>(gr + 8 * i);
        const float4 g1 = *reinterpret_cast<const float4*>(gr + 8 * i + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float xv = (j & 1) ? bf16_hi(p[j >> 1]) : bf16_lo(p[j >> 1]);
            const float t = fminf(fmaxf(rintf(((xv * r) * gv[j]) * scale), -128.0f), 127.0f);
            const int32_t qi = (int32_t)t;
            qsum += qi;
            packed[j >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (j & 3));
        }
        *reinterpret_cast<uint2*>(qrow + code_offset(i, K / 64)) = make_uint2(packed[0], packed[1]);
    }
    put_wave_sum(qsum, qpart);
    scale_out = scale;
}

// The same for rows of at most CPT * kThreads chunks of 8 elements: each
// thread loads its chunks of x and of the RMSNorm weight once, up front, and
// keeps them in registers for all three passes, so the prologue waits on
// memory once instead of once per pass.  Every sum runs in the order of
// quantise_row_to_lds (chunk by chunk, element by element, then the block
// reduction), so the codes are the same bit for bit.
template <int CPT>
__device__ __forceinline__ void quantise_row_regs(const uint16_t* __restrict__ xr,
                                                  const float* __restrict__ gr, int K, float eps,
                                                  int8_t* __restrict__ qrow, double* dscr, float* fscr,
                                                  int32_t* qpart, float& scale_out) {
    const int nchunks = K / 8;
    uint32_t p[CPT][4];
    float gv[CPT][8];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int i = threadIdx.x + c * kThreads;
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        float4 g0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), g1 = g0;
        if (i < nchunks) {
            raw = *reinterpret_cast<const uint4*>(xr + 8 * i);
            g0 = *reinterpret_cast<const float4*>(gr + 8 * i);
            g1 = *reinterpret_cast<const float4*>(gr + 8 * i + 4);
        }
        p[c][0] = raw.x;
        p[c][1] = raw.y;
        p[c][2] = raw.z;
        p[c][3] = raw.w;
        gv[c][0] = g0.x;
        gv[c][1] = g0.y;
        gv[c][2] = g0.z;
        gv[c][3] = g0.w;
        gv[c][4] = g1.x;
        gv[c][5] = g1.y;
        gv[c][6] = g1.z;
        gv[c][7] = g1.w;
    }
    auto xval = [&](int c, int j) { return (j & 1) ? bf16_hi(p[c][j >> 1]) : bf16_lo(p[c][j >> 1]); };
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        if (threadIdx.x + c * kThreads >= nchunks) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float v = xval(c, j);
            ss += (double)v * (double)v;
        }
    }
    ss = block_sum<true, kWaves>(ss, dscr);
    const float ms = mean_square(ss, K);
    const float r = 1.0f / sqrtf(ms + eps);
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        if (threadIdx.x + c * kThreads >= nchunks) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((xval(c, j) * r) * gv[c][j]));
    }
    amax = block_max<true, kWaves>(amax, fscr);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);
    int32_t qsum = 0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int i = threadIdx.x + c * kThreads;
        if (i >= nchunks) continue;
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float t = fminf(fmaxf(rintf(((xval(c, j) * r) * gv[c][j]) * scale), -128.0f), 127.0f);
            const int32_t qi = (int32_t)t;
            qsum += qi;
            packed[j >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (j & 3));
        }
        *reinterpret_cast<uint2*>(qrow + code_offset(i, K / 64)) = make_uint2(packed[0], packed[1]);
    }
    put_wave_sum(qsum, qpart);
    scale_out = scale;
}

// One wave quantises a whole token row by itself, for blocks that hold
// several token rows: each wave takes its own row and no barrier is needed
// until the codes are published.  Lane l stands in for the block's threads
// l, l + 64, l + 128 and l + 192 (the "virtual threads" of
// quantise_row_regs), each summing its chunks in the same order, and the
// four wave sums are added in the same order as the block reduction's, so
// r, the scale and the codes are the same bit for bit.  Each pass reloads
// the row (from L1/L2 after the first) instead of holding kWaves * CPT
// chunks in registers.  Lane 0 writes Σq to qpart[0] and lanes 1..3 clear
// qpart[1..3], so the block-form sum over qpart stays the row's Σq.
template <int CPT>
__device__ __forceinline__ float quantise_row_wave(const uint16_t* __restrict__ xr,
                                                   const float* __restrict__ gr, int K, float eps,
                                                   int8_t* __restrict__ qrow, int32_t* qpart) {
    constexpr int V = kWaves;  // virtual threads per lane
    const int nchunks = K / 8;
    const int lane = threadIdx.x & (kWave - 1);
    auto chunk_of = [&](int v, int c) { return lane + kWave * v + kThreads * c; };
    auto load_x = [&](int i) {
        return i < nchunks ? *reinterpret_cast<const uint4*>(xr + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
    };
    auto load_g = [&](int i, float (&gv)[8]) {
        float4 g0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), g1 = g0;
        if (i < nchunks) {
            g0 = *reinterpret_cast<const float4*>(gr + 8 * i);
            g1 = *reinterpret_cast<const float4*>(gr + 8 * i + 4);
        }
        gv[0] = g0.x; gv[1] = g0.y; gv[2] = g0.z; gv[3] = g0.w;
        gv[4] = g1.x; gv[5] = g1.y; gv[6] = g1.z; gv[7] = g1.w;
    };
    auto xv = [](const uint4& raw, int j) {
        const uint32_t w = j < 2 ? raw.x : (j < 4 ? raw.y : (j < 6 ? raw.z : raw.w));
        return (j & 1) ? bf16_hi(w) : bf16_lo(w);
    };
    // pass 1: sum of squares, per virtual thread in chunk and element order
    uint4 raw[V][CPT];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int c = 0; c < CPT; ++c) raw[v][c] = load_x(chunk_of(v, c));
    double tot = 0.0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        double ss = 0.0;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            if (chunk_of(v, c) >= nchunks) continue;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = xv(raw[v][c], j);
                ss += (double)x * (double)x;
            }
        }
        ss = wave_sum_dpp(ss);
        tot = v == 0 ? ss : tot + ss;
    }
    const float ms = mean_square(tot, K);
    const float r = 1.0f / sqrtf(ms + eps);
    // pass 2: absmax (order-free)
    float amax = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int i = chunk_of(v, c);
            if (i >= nchunks) continue;
            float gv[8];
            load_g(i, gv);
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((xv(raw[v][c], j) * r) * gv[j]));
        }
    amax = wave_max_dpp(amax);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);
    // pass 3: codes
    int32_t qsum = 0;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int i = chunk_of(v, c);
            if (i >= nchunks) continue;
            float gv[8];
            load_g(i, gv);
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float t = fminf(fmaxf(rintf(((xv(raw[v][c], j) * r) * gv[j]) * scale), -128.0f), 127.0f);
                const int32_t qi = (int32_t)t;
                qsum += qi;
                packed[j >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (j & 3));
            }
            *reinterpret_cast<uint2*>(qrow + code_offset(i, K / 64)) = make_uint2(packed[0], packed[1]);
        }
    qsum = wave_sum_dpp(qsum);
    if (lane < kWaves) qpart[lane] = lane == 0 ? qsum : 0;
    return scale;
}

// Weight rows that feed one output: the GLU pairs gate row n with up row
// N + n; one MLGRU token gathers rows n, N + n and 2N + n (z_f, z_c, z_g).
template <Epilogue EP>
constexpr int rows_per_output() {
    return EP == Epilogue::kGluBf16 ? 2 : (EP == Epilogue::kMlgruStep ? 3 : 1);
}

template <int MAXM, int S, int U, int LPR, Epilogue EP>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a, int rows_per_block) {
    constexpr int kR = rows_per_output<EP>();
    constexpr int RW = kWave / LPR;     // rows per wave-wide load
    constexpr int kSpread = LPR / U;    // lanes holding one finished row sum
    extern __shared__ __attribute__((aligned(16))) int8_t qlds[];  // [M][K]
    __shared__ double dscr[MAXM][kWaves];
    __shared__ float fscr[MAXM][kWaves];
    __shared__ int32_t s_qpart[MAXM][kWaves];

    const int b = blockIdx.y;
    const int M = a.M, N = a.N, K = a.K;
    const int nwords = K / 16;
    const int nchunks = K / 64;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int lr = lane & (LPR - 1);
    const int grp = lane / LPR;

    const int64_t nrows = kR * (int64_t)N;
    const uint32_t* P = reinterpret_cast<const uint32_t*>(a.packed) + (int64_t)b * nrows * nwords;
    const int n0 = blockIdx.x * rows_per_block;
    const int n_end = min(N, n0 + rows_per_block);
    const int step = kWaves * U * RW;

    uint4 wa[kR][U][S], wb[kR][U][S];
    // Weights of rows base + u*RW + grp (and their partner rows N and 2N
    // further on), this lane's chunks.  Loads are unconditional from clamped
    // addresses: a row past the end is computed and never stored, and a
    // chunk past the end of K meets zero codes in qreg, so it adds nothing.
    auto load = [&](uint4 (&w)[kR][U][S], int base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t n = min(base + u * RW + grp, n_end - 1);
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int c = min(lr + s * LPR, nchunks - 1);
#pragma unroll
                for (int rr = 0; rr < kR; ++rr)
                    w[rr][u][s] = load_stream16(P + ((int64_t)rr * N + n) * nwords + 4 * c);
            }
        }
    };
    // Issue the first weight loads and the gain before quantising: they do
    // not depend on it, and each is one memory round trip.
    const int base0 = n0 + wave * U * RW;
    load(wa, base0);
    const float gamma = a.gamma[b];

    // 1. quantise the block's token rows into LDS
    const uint16_t* X = a.x + (int64_t)b * M * K;
    const float* G = a.g + (int64_t)b * a.g_stride;
    // Rows this instance takes are at most 64 * S * LPR wide (S chunks of 64
    // weights per lane, LPR lanes per row), so one form is compiled.
    constexpr int kRowChunks = (64 * S * LPR + 8 * kThreads - 1) / (8 * kThreads);
    // Three or four token rows with at most two chunks per thread (rows up
    // to 4096 wide): one wave per row, the rows side by side; each wave
    // publishes its row's scale in LDS.  (Measured per call over cold
    // 2560 x 2560 layers: 7.5 us at M = 4 against 9.4 for the rows one after
    // another; at M = 2 the per-wave work of the four stand-in threads costs
    // more than the barriers it saves, 6.3 against 5.9 us.)  Otherwise the
    // whole block takes the rows one after another, and every thread ends a
    // row holding its scale, so the rescale factor gamma / s is formed in
    // registers before the barrier.  The row loop is unrolled over MAXM so
    // cs stays in registers; M is the same for the whole block.
    constexpr bool kWaveRows = MAXM == kWaves && kRowChunks <= 2;
    __shared__ float s_scale[kWaveRows ? MAXM : 1];
    float cs[MAXM];
    if constexpr (kWaveRows) {
        if (wave < M) {
            const float sc = quantise_row_wave<kRowChunks>(X + (int64_t)wave * K, G, K, a.eps,
                                                           qlds + (int64_t)wave * K, s_qpart[wave]);
            if (lane == 0) s_scale[wave] = sc;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MAXM; ++m) cs[m] = m < M ? gamma / s_scale[m] : 0.0f;
    } else {
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            cs[m] = 0.0f;
            if (m >= M) continue;
            float sc;
            const uint16_t* xr = X + (int64_t)m * K;
            int8_t* qr = qlds + (int64_t)m * K;
            if constexpr (kRowChunks <= kMaxRowChunks)
                quantise_row_regs<kRowChunks>(xr, G, K, a.eps, qr, dscr[m], fscr[m], s_qpart[m], sc);
            else
                quantise_row_to_lds(xr, G, K, a.eps, qr, dscr[m], fscr[m], s_qpart[m], sc);
            cs[m] = gamma / sc;
        }
        __syncthreads();
    }

    // 2. this lane's codes: chunk c = lr + s*LPR covers k in [64c, 64c + 64)
    int4 qreg[MAXM][S][4];
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int c = lr + s * LPR;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qreg[m][s][j] = make_int4(0, 0, 0, 0);
                if (m < M && c < nchunks)
                    qreg[m][s][j] = *reinterpret_cast<const int4*>(qlds + (int64_t)m * K + (j * nchunks + c) * 16);
            }
        }
    int32_t sumq[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        sumq[m] = 0;
        if (m < M) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) sumq[m] += s_qpart[m][w];
        }
    }

    // 3. products of one buffered set of rows, 4. row sums and epilogue
    auto dot_rows = [&](const uint4 (&w)[U][S], int32_t (&out)[MAXM][U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int32_t a1[MAXM], a4[MAXM], a16[MAXM];
#pragma unroll
            for (int m = 0; m < MAXM; ++m) a1[m] = a4[m] = a16[m] = 0;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const uint32_t ww[4] = {w[u][s].x, w[u][s].y, w[u][s].z, w[u][s].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    int32_t c0, c1, c2, c3;
                    decode_codes_scaled(ww[j], c0, c1, c2, c3);
#pragma unroll
                    for (int m = 0; m < MAXM; ++m) {
                        a1[m] = dot4(c0, qreg[m][s][j].x, a1[m]);
                        a4[m] = dot4(c1, qreg[m][s][j].y, a4[m]);
                        a16[m] = dot4(c2, qreg[m][s][j].z, a16[m]);
                        a1[m] = dot4(c3, qreg[m][s][j].w, a1[m]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MAXM; ++m) out[m][u] = a1[m] + (a4[m] >> 2) + (a16[m] >> 4);
        }
    };
    const int u_out = lr / kSpread;
    const bool writer = (lr % kSpread) == 0;
    auto finish = [&](const uint4 (&w)[kR][U][S], int base) {
        int32_t tot[kR][MAXM];
#pragma unroll
        for (int rr = 0; rr < kR; ++rr) {
            int32_t part[MAXM][U];
            dot_rows(w[rr], part);
#pragma unroll
            for (int m = 0; m < MAXM; ++m) tot[rr][m] = group_row_sums<LPR, U>(part[m], lane);
        }
        const int n = base + u_out * RW + grp;
        if (writer && n < n_end) {
#pragma unroll
            for (int m = 0; m < MAXM; ++m) {
                if (m >= M) continue;
                const int64_t o = ((int64_t)b * M + m) * N + n;
                const float z0 = rescale(tot[0][m] - sumq[m], cs[m]);
                if constexpr (EP == Epilogue::kGluBf16) {
                    static_cast<uint16_t*>(a.out)[o] = glu_bf16(z0, rescale(tot[1][m] - sumq[m], cs[m]));
                } else if constexpr (EP == Epilogue::kResBf16) {
                    // the residual stream: u = bf16(res + y), as the stand-alone
                    // residual pass forms it
                    static_cast<uint16_t*>(a.out)[o] =
                        (uint16_t)f32_to_bf16_bits(__uint_as_float((uint32_t)a.res[o] << 16) + z0);
                } else if constexpr (EP == Epilogue::kMlgruStep) {
                    // one token of its own sequence: state in and out
                    float h = a.state[o];
                    const uint32_t p = mlgru_token(z0, rescale(tot[1][m] - sumq[m], cs[m]),
                                                   rescale(tot[2][m] - sumq[m], cs[m]), h);
                    a.state[o] = h;
                    static_cast<uint16_t*>(a.out)[o] = (uint16_t)p;
                } else {
                    static_cast<float*>(a.out)[o] = z0;
                }
            }
        }
    };

    // Software pipeline: the loads of the next set are in flight while the
    // current set is decoded and reduced.
    for (int base = base0; base < n_end; base += 2 * step) {
        load(wb, base + step);
        finish(wa, base);
        if (base + step >= n_end) break;
        load(wa, base + 2 * step);
        finish(wb, base + step);
    }
}

struct Plan {
    int lpr_log2 = -1;
    int S = 0;
};

// Lanes per row (LPR) and 16-byte steps per lane (S) for a row of `nchunks`
// 64-weight chunks: fewest idle lanes with at most 4 / MAXM code chunks
// held per lane (64 registers) -- 7 for one token, whose codes leave room --
// preferring wider rows on ties.
constexpr int kMaxStepsOneToken = 7;
Plan plan_for(int nchunks, int maxm) {
    Plan best;
    double best_idle = 2.0;
    for (int l2 = 6; l2 >= 3; --l2) {
        const int lpr = 1 << l2;
        const int s = (nchunks + lpr - 1) / lpr;
        if (s < 1 || s * maxm > (maxm == 1 ? kMaxStepsOneToken : 4)) continue;
        const double idle = 1.0 - (double)nchunks / (double)(s * lpr);
        if (idle < best_idle - 1e-9) {
            best_idle = idle;
            best.lpr_log2 = l2;
            best.S = s;
        }
    }
    return best;
}

template <int MAXM, int S, int LPR, Epilogue EP>
hipError_t launch_msl(const DecodeArgs& a, hipStream_t stream) {
    // Loads in flight per lane, double buffered: U row sets of S 16-byte
    // chunks, U = 8 / S for S <= 2 and 2 beyond (divided by the rows per
    // output: the GLU loads a gate and an up row per set, an MLGRU token
    // three rows).
    constexpr int kBufRows = 8 / rows_per_output<EP>() / (S >= 3 ? 4 : S);
    constexpr int U = kBufRows < 1 ? 1 : (kBufRows > LPR ? LPR : kBufRows);
    constexpr int RW = kWave / LPR;
    const int64_t rpb = balanced_rows_per_block(a.N, a.batch, (int64_t)kWaves * RW);
    const dim3 grid((unsigned)((a.N + rpb - 1) / rpb), (unsigned)a.batch);
    const size_t lds = (size_t)a.M * a.K;
    // A block whose rows do not fill one set of U rows in every wave (a
    // single small layer spread over all CUs) takes one row per wave-wide
    // load instead: its rows then spread over the four waves, rather than
    // one wave decoding them all while the others idle.
    if constexpr (U > 1) {
        if (rpb < (int64_t)kWaves * U * RW) {
            decode_kernel<MAXM, S, 1, LPR, EP><<<grid, kThreads, lds, stream>>>(a, (int)rpb);
            return hipGetLastError();
        }
    }
    decode_kernel<MAXM, S, U, LPR, EP><<<grid, kThreads, lds, stream>>>(a, (int)rpb);
    return hipGetLastError();
}

template <int MAXM, int S, Epilogue EP>
hipError_t launch_ms(const DecodeArgs& a, const Plan& p, hipStream_t stream) {
    switch (p.lpr_log2) {
        case 3: return launch_msl<MAXM, S, 8, EP>(a, stream);
        case 4: return launch_msl<MAXM, S, 16, EP>(a, stream);
        case 5: return launch_msl<MAXM, S, 32, EP>(a, stream);
        case 6: return launch_msl<MAXM, S, 64, EP>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int MAXM, Epilogue EP>
hipError_t launch_m(const DecodeArgs& a, const Plan& p, hipStream_t stream) {
    // plan_for keeps S * MAXM <= 4 (S <= 7 for one token), so only those
    // instantiations exist.
    switch (p.S) {
        case 1: return launch_ms<MAXM, 1, EP>(a, p, stream);
        case 2: if constexpr (MAXM <= 2) return launch_ms<MAXM, 2, EP>(a, p, stream); break;
        case 3: if constexpr (MAXM == 1) return launch_ms<MAXM, 3, EP>(a, p, stream); break;
        case 4: if constexpr (MAXM == 1) return launch_ms<MAXM, 4, EP>(a, p, stream); break;
        case 5: if constexpr (MAXM == 1) return launch_ms<MAXM, 5, EP>(a, p, stream); break;
        case 6: if constexpr (MAXM == 1) return launch_ms<MAXM, 6, EP>(a, p, stream); break;
        case 7: if constexpr (MAXM == 1) return launch_ms<MAXM, 7, EP>(a, p, stream); break;
    }
    return hipErrorInvalidValue;
}

template <Epilogue EP>
hipError_t launch_ep(const DecodeArgs& a, hipStream_t stream) {
    const int maxm = a.M <= 1 ? 1 : (a.M <= 2 ? 2 : 4);
    const Plan p = plan_for(a.K / 64, maxm);
    if (maxm == 1) return launch_m<1, EP>(a, p, stream);
    if (maxm == 2) return launch_m<2, EP>(a, p, stream);
    return launch_m<4, EP>(a, p, stream);
}

}  // namespace

int device_cu_count() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCus;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = kDefaultCus;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Rows per block (a multiple of `gran`) for `batch` problems of N rows.
// Blocks stay inside one problem, so the rows of a problem are split into nb
// equal blocks. The split minimises the rows of the busiest CU when the
// nb * batch blocks are dealt out evenly over the device's CUs, counting one
// granule of set-up per block. Unequal blocks (a full block beside a sliver,
// or one block more on a few CUs) otherwise cost up to a quarter of the rate.
// Candidates are nb = 1..16 and the nb that make nb * batch a small multiple
// of the CU count, so the search stays cheap beside a launch.
int64_t balanced_rows_per_block(int64_t N, int64_t batch, int64_t gran) {
    const int64_t ncu = device_cu_count();
    const int64_t nb_max = (N + gran - 1) / gran;
    int64_t best_r = round_up(N, gran);
    double best = -1.0;
    auto consider = [&](int64_t nb) {
        nb = std::min(std::max<int64_t>(nb, 1), nb_max);
        const int64_t r = round_up((N + nb - 1) / nb, gran);
        const int64_t blocks = (N + r - 1) / r * batch;
        const double cost = (double)((blocks + ncu - 1) / ncu) * (double)(r + gran);
        if (best < 0.0 || cost < best || (cost == best && r > best_r)) {
            best = cost;
            best_r = r;
        }
    };
    for (int64_t nb = 1; nb <= 16; ++nb) consider(nb);
    for (int64_t k = 1; k <= 32; ++k) {
        consider(k * ncu / batch);
        consider((k * ncu + batch - 1) / batch);
    }
    return best_r;
}

bool decode_supported(int M, int K) {
    if (M < 1 || M > kDecodeMaxM || K % 64 != 0) return false;
    const int maxm = M <= 1 ? 1 : (M <= 2 ? 2 : 4);
    return plan_for(K / 64, maxm).S > 0;
}

hipError_t launch_decode(const DecodeArgs& a, Epilogue ep, hipStream_t stream) {
    if (!decode_supported(a.M, a.K)) return hipErrorInvalidValue;
    switch (ep) {
        case Epilogue::kF32: return launch_ep<Epilogue::kF32>(a, stream);
        case Epilogue::kGluBf16: return launch_ep<Epilogue::kGluBf16>(a, stream);
        case Epilogue::kResBf16:
            if (a.res == nullptr) return hipErrorInvalidValue;
            return launch_ep<Epilogue::kResBf16>(a, stream);
        case Epilogue::kMlgruStep:
            if (a.state == nullptr) return hipErrorInvalidValue;
            return launch_ep<Epilogue::kMlgruStep>(a, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace bl
