// backward.hip -- gradients of the BitLinear layer (straight-through estimator).
//
// [ld246, "训练与优化：新的策略"]: training passes gradients straight through
// the ternary weights and the activation quantiser; [ld246, "融合 BitLinear
// 层的创新"]: the training-time layer fuses RMSNorm with the quantisation.
// Reading: both quantisers are the identity in the backward pass, gamma and s
// held constant.  For the forward value y = (q / s) (gamma w)^T and the
// output gradient dy:
//   dxn = gamma * dy w,        dW = dy^T (q / s),
//   dg[k]    = sum_m dxn[m][k] x[m][k] r[m],
//   dx[m][k] = r g[k] dxn[m][k] - x[m][k] r^3 / K * sum_j dxn[m][j] g[j] x[m][j],
// with r = (mean(x^2) + eps)^-1/2.  Nothing is kept from the forward call: q
// and s are recomputed by the forward's own quantisation kernel (the same
// bits), r from x.
//
// Both products are dense floating-point contractions and run on the bf16
// matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  Their
// operands are laid out with the reduction index contiguous and zero-padded
// to a multiple of 64:
//   dxn [M][K] = gamma * A1 [M][Np] . wT [K][Np]^T,   A1 = bf16(dy),  wT = w^T
//   dW  [N][K] =         A2 [N][Mp] . qT [K][Mp]^T,   A2 = bf16(dy / s)^T, qT = q^T
// w and q are exact in bf16, so the only roundings besides the fp32
// accumulation are those of dy and dy / s to bf16.  The second operands
// stay compact until they reach registers: wT as 2-bit codes (16 reduction
// indices per word) and qT as int8, each expanded to bf16 fragments right
// before its MFMAs, which keeps the LDS traffic of a stage well below what
// two bf16 operands take.
//
// Kernels: dy_prep (A1 and A2 from one read of dy), q_transpose (int8),
// w_transpose (2-bit codes, transposed), the NT GEMM, norm_backward (dx in
// place over dxn, per-block dg partials) and dg_reduce (fixed order, fp64).
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

constexpr int kT = 64;          // transpose tile edge
constexpr int kPrepThreads = 256;

// ---------------------------------------------------------------------------
// Operand preparation
// ---------------------------------------------------------------------------

// One 64 x 64 tile of dy: A1[m][n] = bf16(dy[m][n]) for m < M, n < Np (zero
// past N); A2[n][m] = bf16(dy[m][n] / s[m]) for n < N, m < Mp (zero past M).
// Rows of dy are read 16 bytes at a time when N % 4 == 0 (VEC), and both
// outputs are written four bf16 (8 bytes) at a time.
template <bool VEC>
__global__ __launch_bounds__(kPrepThreads) void dy_prep_kernel(const float* __restrict__ dy,
                                                               const float* __restrict__ s, int M, int N,
                                                               int Mp, int Np, uint2* __restrict__ A1,
                                                               uint2* __restrict__ A2) {
    __shared__ float tile[kT][kT + 1];
    __shared__ float sv[kT];
    const int64_t mt = Mp / kT;  // tiles along m; the grid is flat (m fastest)
    const int m0 = (int)(blockIdx.x % mt) * kT, n0 = (int)(blockIdx.x / mt) * kT;
    const int t = threadIdx.x;
    if (t < kT) sv[t] = (m0 + t < M) ? s[m0 + t] : 1.0f;
    // 64 rows x 16 groups of four columns
#pragma unroll
    for (int i = 0; i < kT / 16; ++i) {
        const int r = t / 16 + 16 * i, c = 4 * (t % 16);
        const int m = m0 + r, n = n0 + c;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m < M) {
            const float* src = dy + (int64_t)m * N + n;
            if (VEC) {
                if (n < N) v = *reinterpret_cast<const float4*>(src);
            } else {
                v.x = n < N ? src[0] : 0.f;
                v.y = n + 1 < N ? src[1] : 0.f;
                v.z = n + 2 < N ? src[2] : 0.f;
                v.w = n + 3 < N ? src[3] : 0.f;
            }
        }
        tile[r][c] = v.x;
        tile[r][c + 1] = v.y;
        tile[r][c + 2] = v.z;
        tile[r][c + 3] = v.w;
    }
    __syncthreads();
    auto pack4 = [](float a, float b, float c, float d) {
        return make_uint2(f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16),
                          f32_to_bf16_bits(c) | (f32_to_bf16_bits(d) << 16));
    };
    // A1 rows m, four columns per thread
#pragma unroll
    for (int i = 0; i < kT / 16; ++i) {
        const int r = t / 16 + 16 * i, c = 4 * (t % 16);
        const int m = m0 + r;
        if (m < M) A1[((int64_t)m * Np + n0 + c) / 4] = pack4(tile[r][c], tile[r][c + 1], tile[r][c + 2], tile[r][c + 3]);
    }
    // A2 rows n, four tokens per thread; dy / s is an IEEE fp32 division
#pragma unroll
    for (int i = 0; i < kT / 16; ++i) {
        const int c = t / 16 + 16 * i, r = 4 * (t % 16);
        const int n = n0 + c;
        if (n < N)
            A2[((int64_t)n * Mp + m0 + r) / 4] = pack4(tile[r][c] / sv[r], tile[r + 1][c] / sv[r + 1],
                                                       tile[r + 2][c] / sv[r + 2], tile[r + 3][c] / sv[r + 3]);
    }
}

// qT[k][m] = q[m][k] (int8) for k < K, m < Mp (zero past M).  K % 16 == 0.
__global__ __launch_bounds__(kPrepThreads) void q_transpose_kernel(const int8_t* __restrict__ q, int M, int K,
                                                                   int Mp, int8_t* __restrict__ qT) {
    __shared__ int8_t tile[kT][kT + 4];
    const int64_t mt = Mp / kT;  // flat grid, m fastest
    const int m0 = (int)(blockIdx.x % mt) * kT, k0 = (int)(blockIdx.x / mt) * kT;
    const int t = threadIdx.x;
    {
        const int r = t / 4, ch = t % 4;  // 64 rows x 4 chunks of 16 codes
        const int m = m0 + r, k = k0 + 16 * ch;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (m < M && k < K) v = *reinterpret_cast<const uint4*>(q + (int64_t)m * K + k);
        uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[r][16 * ch]);
        dst[0] = v.x;
        dst[1] = v.y;
        dst[2] = v.z;
        dst[3] = v.w;
    }
    __syncthreads();
    // 64 columns x 4 runs of 16 tokens: one 16-byte store per thread
    const int c = t / 4, r0 = 16 * (t % 4);
    const int k = k0 + c;
    if (k < K) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)(uint8_t)tile[r0 + 4 * i][c] | ((uint32_t)(uint8_t)tile[r0 + 4 * i + 1][c] << 8) |
                   ((uint32_t)(uint8_t)tile[r0 + 4 * i + 2][c] << 16) | ((uint32_t)(uint8_t)tile[r0 + 4 * i + 3][c] << 24);
        *reinterpret_cast<uint4*>(qT + (int64_t)k * Mp + m0 + r0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// wT[k] holds w[n][k] for n < Np (zero past N) as 2-bit codes, 16 values of
// n per 32-bit word, from the packed rows [N][K/4] (weight j of a 16-weight
// group sits in byte j % 4 of the group's word, bits 2 (j / 4) + 1 .. 2 (j / 4),
// as code w + 1).  In a word of wT, value i = 2p + e (e = 0 or 1) has its
// "nonzero" flag at bit 16 e + p and its "negative" flag at bit 16 e + 8 + p:
// the two values of a bf16 pair (2p, 2p + 1) then sit 16 bits apart, which is
// what the expansion to a pair of bf16 needs (expand_ternary).
__global__ __launch_bounds__(kPrepThreads) void w_transpose_kernel(const uint32_t* __restrict__ packed, int N,
                                                                   int K, int Np, uint32_t* __restrict__ wT) {
    __shared__ uint8_t tile[kT][kT + 4];
    const int64_t nt = Np / kT;  // flat grid, n fastest
    const int n0 = (int)(blockIdx.x % nt) * kT, k0 = (int)(blockIdx.x / nt) * kT;
    const int t = threadIdx.x;
    {
        const int r = t / 4, wi = t % 4;  // 64 rows x 4 words of 16 weights
        const int n = n0 + r, k = k0 + 16 * wi;
        uint32_t word = 0x55555555u;      // code 1 everywhere: weight 0
        if (n < N && k < K) word = packed[(int64_t)n * (K / 16) + k / 16];
#pragma unroll
        for (int j = 0; j < 16; ++j) tile[r][16 * wi + j] = (uint8_t)((word >> (8 * (j & 3) + 2 * (j >> 2))) & 3u);
    }
    __syncthreads();
    // 64 columns x 4 words of 16 rows: one word per thread
    const int c = t / 4, g = t % 4;
    const int k = k0 + c;
    if (k < K) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t code = tile[16 * g + i][c];
            const int bit = 16 * (i & 1) + (i >> 1);
            word |= (uint32_t)(code != 1u) << bit;
            word |= (uint32_t)(code == 0u) << (bit + 8);
        }
        wT[(int64_t)k * (Np / 16) + n0 / 16 + g] = word;
    }
}

// ---------------------------------------------------------------------------
// C[rows][cols] = alpha * A[rows][R] . B[cols][R]^T on the bf16 matrix cores.
// Block tile 256 x 256, eight waves as 2 x 4, each a 128 x 64 tile of 32 x 32
// fragments (4 x 2): per 16-wide reduction step a wave reads four A
// fragments from LDS for eight MFMAs.  R advances in stages of 64,
// double-buffered in LDS through registers: the next stage's global loads
// are in flight while the current one is multiplied.  Operand pairing:
// lane l of A supplies row l % 32 and lane l of B column l % 32, both with
// the same eight reduction indices 8 (l / 32) + 0..7 of a 16-wide step;
// accumulator element v of lane l holds C[(v % 4) + 8 (v / 4) + 4 (l / 32)]
// [l % 32].  R % 64 == 0 (zero-padded operands); rows and cols are
// arbitrary (loads clamped, stores masked).
//
// A is bf16 [rows][R].  B comes in one of two compact forms (BKind):
//   kTern2 -- ternary values as 2-bit codes [cols][R / 16] words (the
//             layout of w_transpose_kernel); a lane reads its column's four
//             words of a stage once and expands half a word per step;
//   kInt8  -- int8 [cols][R]; a lane reads 8 bytes per step and converts.
// Compared with a bf16 B operand, the compact forms cut a stage's LDS
// traffic (the writes of the staged operand and the per-step fragment
// reads) from 256 KiB to 172 KiB (kTern2) and 190 KiB (kInt8) per 64-deep
// stage, and the staging registers and global reads with it.
//
// When the output has fewer tiles than the chip has compute units, the
// reduction is split over `splits` blocks per tile (whole stages each); split
// s writes its fp32 partial to P + s * rows * cols and split_reduce adds the
// partials in split order and scales by alpha.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGT = 256;          // block tile edge
constexpr int kGK = 64;           // reduction per stage (bf16 elements)
constexpr int kGPitch = kGK + 8;  // bf16 per LDS row: 144 bytes, 16-byte reads of 8 rows hit distinct banks
constexpr int kGWM = 2, kGWN = 4; // wave grid
constexpr int kGThreads = kGWM * kGWN * kWave;
constexpr int kGFM = kGT / kGWM / 32, kGFN = kGT / kGWN / 32;  // fragments per wave: 4 x 2
constexpr int kGLoads = kGT * kGK * 2 / 16 / kGThreads;          // 16-byte loads per thread of the bf16 A operand: 4
constexpr int kMaxSplits = 8;
constexpr int kI8Pitch = kGK + 8;  // bytes per int8 LDS row: 8-byte reads of 32 rows hit distinct bank pairs

enum class BKind { kTern2, kInt8 };

// Bytes of one B row of a stage in LDS.
template <BKind BK>
constexpr int b_lds_pitch() {
    return BK == BKind::kTern2 ? kGK / 4 : kI8Pitch;
}

struct GemmArgs {
    const uint16_t* A;
    const void* B;
    float* C;            // final output (splits == 1)
    float* P;            // split partials (splits > 1)
    const float* alpha;  // device scalar, or nullptr for 1
    int rows, cols, R, splits;
};

// Eight ternary values of a w_transpose word as bf16 (-1, 0, +1): the half
// h (values 8h .. 8h + 7), bf16 pair q = values 8h + 2q, 8h + 2q + 1.  The
// "nonzero" flags of a pair sit at bits q and 16 + q of word >> 4h, the
// "negative" flags 8 bits higher: the flags times 0x3F80 (the magnitude of
// bf16 1.0) give the two magnitudes, and the negative flags shifted to bits
// 15 and 31 give the signs.  A zero value has neither flag.
__device__ __forceinline__ bf16x8 expand_ternary(uint32_t word, int h) {
    const uint32_t w = word >> (4 * h);
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t mag = (w & (0x00010001u << q)) * (0x3F80u >> q);  // both under 2^24: v_mul_u32_u24
        d[q] = mag | ((w & (0x01000100u << q)) << (7 - q));
    }
    return __builtin_bit_cast(bf16x8, make_uint4(d[0], d[1], d[2], d[3]));
}

// Eight int8 values as bf16: int8 -> fp32 is exact and |q| <= 128 has at
// most 8 significant bits, so the top half of the fp32 pattern is the bf16
// value.
__device__ __forceinline__ bf16x8 expand_int8(uint2 v) {
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t word = q < 2 ? v.x : v.y;
        const int sh = 16 * (q & 1);
        const uint32_t lo = __float_as_uint((float)(int8_t)(word >> sh));
        const uint32_t hi = __float_as_uint((float)(int8_t)(word >> (sh + 8)));
        d[q] = (lo >> 16) | (hi & 0xFFFF0000u);
    }
    return __builtin_bit_cast(bf16x8, make_uint4(d[0], d[1], d[2], d[3]));
}

template <BKind BK>
__global__ __launch_bounds__(kGThreads) void bwd_gemm_kernel(GemmArgs g) {
    constexpr int kBPitch = b_lds_pitch<BK>();
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kGT * kGPitch];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kGT * kBPitch];
    const int ntc = (g.cols + kGT - 1) / kGT;
    const int tile = blockIdx.x / g.splits, split = blockIdx.x % g.splits;
    const int tr = tile / ntc, tc = tile % ntc;
    const int row0 = tr * kGT, col0 = tc * kGT;
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    const int wm = wave / kGWN, wn = wave % kGWN;

    // stages [st0, st1) of this split
    const int nst = g.R / kGK;
    const int per = (nst + g.splits - 1) / g.splits;
    const int st0 = min(split * per, nst), st1 = min(st0 + per, nst);

    // global -> register staging of A: rows t / 8 + 64 i, 16-byte chunk t % 8
    const int srow = t / 8, sch = t % 8;
    constexpr int kRowStep = kGThreads / 8;  // 64
    static_assert(kGLoads == 4, "four staged loads of A per thread");
    const int64_t aoff0 = (int64_t)min(row0 + srow, g.rows - 1) * g.R + 8 * sch;
    const int64_t aoff1 = (int64_t)min(row0 + srow + kRowStep, g.rows - 1) * g.R + 8 * sch;
    const int64_t aoff2 = (int64_t)min(row0 + srow + 2 * kRowStep, g.rows - 1) * g.R + 8 * sch;
    const int64_t aoff3 = (int64_t)min(row0 + srow + 3 * kRowStep, g.rows - 1) * g.R + 8 * sch;
    const int lds0 = srow * kGPitch + 8 * sch;
    constexpr int kLdsStep = kRowStep * kGPitch;

    // Staging of B, per form (offsets in the form's own elements):
    //   kTern2: threads t < 256 one 16-byte row (four words);
    //   kInt8: thread t two 16-byte pieces of row t / 2 (bytes 32 (t % 2) ..).
    const uint32_t* B2 = static_cast<const uint32_t*>(g.B);
    const int8_t* B8 = static_cast<const int8_t*>(g.B);
    int64_t boff0 = 0;
    if constexpr (BK == BKind::kTern2)
        boff0 = (int64_t)min(col0 + (t & (kGT - 1)), g.cols - 1) * (g.R / 16);
    else
        boff0 = (int64_t)min(col0 + t / 2, g.cols - 1) * g.R + 32 * (t % 2);
    const bool b_stager = BK != BKind::kTern2 || t < kGT;
    // Named registers (not arrays): the staged values stay in VGPRs.
    uint4 ra0, ra1, ra2, ra3, rb0, rb1;
    auto load_stage = [&](int st) {
        const int64_t o = (int64_t)st * kGK;
        ra0 = *reinterpret_cast<const uint4*>(g.A + aoff0 + o);
        ra1 = *reinterpret_cast<const uint4*>(g.A + aoff1 + o);
        ra2 = *reinterpret_cast<const uint4*>(g.A + aoff2 + o);
        ra3 = *reinterpret_cast<const uint4*>(g.A + aoff3 + o);
        if constexpr (BK == BKind::kTern2) {
            if (b_stager) rb0 = *reinterpret_cast<const uint4*>(B2 + boff0 + (int64_t)st * (kGK / 16));
        } else {
            rb0 = *reinterpret_cast<const uint4*>(B8 + boff0 + o);
            rb1 = *reinterpret_cast<const uint4*>(B8 + boff0 + o + 16);
        }
    };
    auto store_stage = [&](int buf) {
        *reinterpret_cast<uint4*>(&As[buf][lds0]) = ra0;
        *reinterpret_cast<uint4*>(&As[buf][lds0 + kLdsStep]) = ra1;
        *reinterpret_cast<uint4*>(&As[buf][lds0 + 2 * kLdsStep]) = ra2;
        *reinterpret_cast<uint4*>(&As[buf][lds0 + 3 * kLdsStep]) = ra3;
        uint8_t* bs = Bs[buf];
        if constexpr (BK == BKind::kTern2) {
            if (b_stager) *reinterpret_cast<uint4*>(bs + t * kBPitch) = rb0;
        } else {
            // 8-byte pieces: the 72-byte row pitch is 8-byte aligned only
            uint2* d = reinterpret_cast<uint2*>(bs + (t / 2) * kBPitch + 32 * (t % 2));
            d[0] = make_uint2(rb0.x, rb0.y);
            d[1] = make_uint2(rb0.z, rb0.w);
            d[2] = make_uint2(rb1.x, rb1.y);
            d[3] = make_uint2(rb1.z, rb1.w);
        }
    };

    f32x16 acc[kGFM][kGFN];
#pragma unroll
    for (int i = 0; i < kGFM; ++i)
#pragma unroll
        for (int j = 0; j < kGFN; ++j) acc[i][j] = f32x16{};

    const int afrag = (wm * (kGT / kGWM) + (lane & 31)) * kGPitch + 8 * (lane >> 5);
    const int bcol = wn * (kGT / kGWN) + (lane & 31);  // B row (output column) of fragment 0
    const int half = lane >> 5;
    // Stage st sits in buffer (st - st0) % 2.  The loads of stage st + 1 are
    // issued during stage st - 1 (or here); during stage st they are written
    // to the other buffer ahead of its last 16-deep step, and the loads of
    // stage st + 2 go out right after.  The last step's MFMAs then keep the
    // matrix core busy while the waves meet at the barrier that publishes
    // stage st + 1, instead of the core idling through the LDS writes, the
    // barrier and the next stage's first reads.  Loads still get a whole
    // stage to land.
    if (st0 < st1) {
        load_stage(st0);
        store_stage(0);
        if (st0 + 1 < st1) load_stage(st0 + 1);
        __syncthreads();
    }
    // Fragments of one 16-deep step.  The next step's LDS reads are issued
    // before this step's MFMAs, behind a scheduling barrier (the waves of a
    // block run in lockstep between barriers and cannot hide that latency
    // for each other), and the compact B forms are expanded between the
    // MFMAs: the ternary words are in registers already; the int8 bytes are
    // expanded after the step's later MFMAs, by when their read has landed.
    struct Frags {
        bf16x8 a[kGFM], b[kGFN];
    };
    uint4 bw[kGFN];    // kTern2: the lane's four words of each B row this stage
    uint2 b8[kGFN];    // kInt8: the next step's B bytes
    auto read_frags = [&](int buf, int ks, Frags& f) {
#pragma unroll
        for (int i = 0; i < kGFM; ++i)
            f.a[i] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4*>(&As[buf][afrag + i * 32 * kGPitch + 16 * ks]));
        if constexpr (BK == BKind::kInt8) {
#pragma unroll
            for (int j = 0; j < kGFN; ++j)
                b8[j] = *reinterpret_cast<const uint2*>(&Bs[buf][(bcol + j * 32) * kBPitch + 16 * ks + 8 * half]);
        }
    };
    auto expand_b = [&](int ks, Frags& f, int j) {
        if constexpr (BK == BKind::kTern2) {
            const uint32_t wd = ks == 0 ? bw[j].x : (ks == 1 ? bw[j].y : (ks == 2 ? bw[j].z : bw[j].w));
            f.b[j] = expand_ternary(wd, half);
        } else {
            f.b[j] = expand_int8(b8[j]);
        }
    };
    constexpr int KS = kGK / 16;
    constexpr int kMf = kGFM * kGFN;
    for (int st = st0; st < st1; ++st) {
        const int buf = (st - st0) & 1;
        const bool more = st + 1 < st1;
        Frags cur, nxt;
        if constexpr (BK == BKind::kTern2) {
#pragma unroll
            for (int j = 0; j < kGFN; ++j) bw[j] = *reinterpret_cast<const uint4*>(&Bs[buf][(bcol + j * 32) * kBPitch]);
        }
        read_frags(buf, 0, cur);
#pragma unroll
        for (int j = 0; j < kGFN; ++j) expand_b(0, cur, j);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bool ahead = ks + 1 < KS;
            if (ahead) read_frags(buf, ks + 1, nxt);
            if (ks == KS - 1 && more) {
                store_stage(buf ^ 1);
                if (st + 2 < st1) load_stage(st + 2);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int idx = 0; idx < kMf; ++idx) {
                const int i = idx / kGFN, j = idx % kGFN;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
                if (ahead && idx >= kMf - kGFN) expand_b(ks + 1, nxt, idx - (kMf - kGFN));
                __builtin_amdgcn_sched_barrier(0);
            }
            if (ahead) cur = nxt;
        }
        __syncthreads();
    }

    const bool direct = g.splits == 1;
    const float alpha = direct ? (g.alpha ? *g.alpha : 1.0f) : 1.0f;
    float* out = direct ? g.C : g.P + (int64_t)split * g.rows * g.cols;
#pragma unroll
    for (int i = 0; i < kGFM; ++i)
#pragma unroll
        for (int j = 0; j < kGFN; ++j) {
            const int col = col0 + wn * (kGT / kGWN) + j * 32 + (lane & 31);
            const int rbase = row0 + wm * (kGT / kGWM) + i * 32 + 4 * (lane >> 5);
            if (col < g.cols) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = rbase + (v % 4) + 8 * (v / 4);
                    if (row < g.rows) out[(int64_t)row * g.cols + col] = alpha * acc[i][j][v];
                }
            }
        }
}

// C[i] = alpha * sum_s P[s][i], s in order.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ P, int splits, int64_t n,
                                                           const float* __restrict__ alpha_p, float* __restrict__ C) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    const float alpha = alpha_p ? *alpha_p : 1.0f;
    float4 a = *reinterpret_cast<const float4*>(P + i);
    for (int sp = 1; sp < splits; ++sp) {
        const float4 b = *reinterpret_cast<const float4*>(P + (int64_t)sp * n + i);
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    *reinterpret_cast<float4*>(C + i) = make_float4(alpha * a.x, alpha * a.y, alpha * a.z, alpha * a.w);
}

// Splits of the reduction for a rows x cols output over R: enough blocks to
// give every compute unit a tile, at most kMaxSplits, at least one stage each.
int gemm_splits(int64_t rows, int64_t cols, int64_t R, int cus) {
    const int64_t tiles = ((rows + kGT - 1) / kGT) * ((cols + kGT - 1) / kGT);
    const int64_t nst = R / kGK;
    int64_t sp = (cus + tiles - 1) / tiles;
    if (sp > kMaxSplits) sp = kMaxSplits;
    if (sp > nst) sp = nst;
    return sp < 1 ? 1 : (int)sp;
}

// ---------------------------------------------------------------------------
// RMSNorm backward.  A block owns kNormRows rows (small, so that the grid
// holds several blocks per compute unit).  Phase 1 (a wave per row):
// ss = sum x^2 and S = sum dxn g x in fp64, r = (ss / K + eps)^-1/2 and
// c = r^3 S / K.  Phase 2 (threads over columns, four each): dx = r g dxn -
// x c written over dxn, and the block's partial dg[k] = sum_m dxn x r.
// ---------------------------------------------------------------------------
constexpr int kNormRows = 8;
constexpr int kNormThreads = 256;

__global__ __launch_bounds__(kNormThreads) void norm_backward_kernel(const uint16_t* __restrict__ x,
                                                                     const float* __restrict__ gw, int M, int K,
                                                                     float eps, float* __restrict__ dxio,
                                                                     float* __restrict__ partial) {
    __shared__ float s_r[kNormRows], s_c[kNormRows];
    const int m0 = blockIdx.x * kNormRows;
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    constexpr int kWaves = kNormThreads / kWave;
    for (int rr = wave; rr < kNormRows; rr += kWaves) {
        const int m = m0 + rr;
        if (m >= M) break;
        const uint16_t* xr = x + (int64_t)m * K;
        const float* dr = dxio + (int64_t)m * K;
        double ss = 0.0, S = 0.0;
        for (int k = 4 * lane; k < K; k += 4 * kWave) {
            const uint2 xv = *reinterpret_cast<const uint2*>(xr + k);
            const float4 d = *reinterpret_cast<const float4*>(dr + k);
            const float4 gv = *reinterpret_cast<const float4*>(gw + k);
            const float xs[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
            const float ds[4] = {d.x, d.y, d.z, d.w};
            const float gs[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ss += (double)xs[j] * (double)xs[j];
                S += (double)ds[j] * (double)gs[j] * (double)xs[j];
            }
        }
        ss = wave_sum(ss);
        S = wave_sum(S);
        if (lane == 0) {
            const double r = 1.0 / sqrt(ss / (double)K + (double)eps);
            s_r[rr] = (float)r;
            s_c[rr] = (float)(r * r * r * S / (double)K);
        }
    }
    __syncthreads();
    const int mend = min(M - m0, kNormRows);
    for (int k = 4 * t; k < K; k += 4 * kNormThreads) {
        const float4 gv = *reinterpret_cast<const float4*>(gw + k);
        float dg0 = 0.f, dg1 = 0.f, dg2 = 0.f, dg3 = 0.f;
        for (int rr = 0; rr < mend; ++rr) {
            const int64_t off = (int64_t)(m0 + rr) * K + k;
            const uint2 xv = *reinterpret_cast<const uint2*>(x + off);
            const float4 d = *reinterpret_cast<const float4*>(dxio + off);
            const float r = s_r[rr], c = s_c[rr];
            const float x0 = bf16_lo(xv.x), x1 = bf16_hi(xv.x), x2 = bf16_lo(xv.y), x3 = bf16_hi(xv.y);
            float4 o;
            o.x = r * gv.x * d.x - x0 * c;
            o.y = r * gv.y * d.y - x1 * c;
            o.z = r * gv.z * d.z - x2 * c;
            o.w = r * gv.w * d.w - x3 * c;
            *reinterpret_cast<float4*>(dxio + off) = o;
            dg0 += d.x * x0 * r;
            dg1 += d.y * x1 * r;
            dg2 += d.z * x2 * r;
            dg3 += d.w * x3 * r;
        }
        *reinterpret_cast<float4*>(partial + (int64_t)blockIdx.x * K + k) = make_float4(dg0, dg1, dg2, dg3);
    }
}

// The same RMSNorm backward for rows of at most CPL * 256 elements, held in
// registers: a wave owns one row at a time (lane l: columns 4 (l + 64 c),
// c < CPL), so x and dxn are read once and dx written once, with no second
// pass.  A block owns kNormRowsRegs rows (each wave every fourth); its dg
// partial is the four waves' sums added in wave order through LDS.
constexpr int kNormRowsRegs = 16;

template <int CPL>
__global__ __launch_bounds__(kNormThreads) void norm_backward_regs_kernel(const uint16_t* __restrict__ x,
                                                                          const float* __restrict__ gw, int M,
                                                                          int K, float eps,
                                                                          float* __restrict__ dxio,
                                                                          float* __restrict__ partial) {
    __shared__ float4 red[CPL * kWave];
    const int m0 = blockIdx.x * kNormRowsRegs;
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    constexpr int kWaves = kNormThreads / kWave;
    float4 gv[CPL], acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int k = 4 * (lane + kWave * c);
        gv[c] = k < K ? *reinterpret_cast<const float4*>(gw + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int rr = wave; rr < kNormRowsRegs; rr += kWaves) {
        const int m = m0 + rr;
        if (m >= M) break;
        const uint16_t* xr = x + (int64_t)m * K;
        float* dr = dxio + (int64_t)m * K;
        float4 d[CPL], xv[CPL];
        double ss = 0.0, S = 0.0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int k = 4 * (lane + kWave * c);
            uint2 xb = make_uint2(0u, 0u);
            d[c] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (k < K) {
                xb = *reinterpret_cast<const uint2*>(xr + k);
                d[c] = *reinterpret_cast<const float4*>(dr + k);
            }
            xv[c] = make_float4(bf16_lo(xb.x), bf16_hi(xb.x), bf16_lo(xb.y), bf16_hi(xb.y));
            ss += (double)xv[c].x * (double)xv[c].x + (double)xv[c].y * (double)xv[c].y +
                  (double)xv[c].z * (double)xv[c].z + (double)xv[c].w * (double)xv[c].w;
            S += (double)d[c].x * (double)gv[c].x * (double)xv[c].x + (double)d[c].y * (double)gv[c].y * (double)xv[c].y +
                 (double)d[c].z * (double)gv[c].z * (double)xv[c].z + (double)d[c].w * (double)gv[c].w * (double)xv[c].w;
        }
        ss = wave_sum(ss);
        S = wave_sum(S);
        const double rd = 1.0 / sqrt(ss / (double)K + (double)eps);
        const float r = (float)rd, cc = (float)(rd * rd * rd * S / (double)K);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int k = 4 * (lane + kWave * c);
            if (k < K) {
                float4 o;
                o.x = r * gv[c].x * d[c].x - xv[c].x * cc;
                o.y = r * gv[c].y * d[c].y - xv[c].y * cc;
                o.z = r * gv[c].z * d[c].z - xv[c].z * cc;
                o.w = r * gv[c].w * d[c].w - xv[c].w * cc;
                *reinterpret_cast<float4*>(dr + k) = o;
            }
            acc[c].x += d[c].x * xv[c].x * r;
            acc[c].y += d[c].y * xv[c].y * r;
            acc[c].z += d[c].z * xv[c].z * r;
            acc[c].w += d[c].w * xv[c].w * r;
        }
    }
    // dg partial of the block: waves 0, 1, 2, 3 added in that order
    for (int w = 0; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float4 v = acc[c];
                if (w > 0) {
                    const float4 p = red[c * kWave + lane];
                    v = make_float4(p.x + v.x, p.y + v.y, p.z + v.z, p.w + v.w);
                }
                red[c * kWave + lane] = v;
            }
        }
        __syncthreads();
    }
    for (int i = t; i < CPL * kWave; i += kNormThreads) {
        const int c = i / kWave, l = i % kWave;
        const int k = 4 * (l + kWave * c);
        if (k < K) *reinterpret_cast<float4*>(partial + (int64_t)blockIdx.x * K + k) = red[i];
    }
}

// dg[k] = sum over blocks of the partials in fp64.  A block takes 16
// columns; its 64 thread groups each sum every 64th partial (in order), and
// the 64 group sums are added in group order, so the result is
// deterministic.  Short chains over many blocks keep the loads in flight.
constexpr int kDgCols = 16, kDgSplit = 64;

__global__ __launch_bounds__(kDgCols * kDgSplit) void dg_reduce_kernel(const float* __restrict__ partial,
                                                                       int nparts, int K, float* __restrict__ dg) {
    __shared__ double part[kDgSplit][kDgCols];
    const int c = threadIdx.x % kDgCols, p = threadIdx.x / kDgCols;
    const int k = blockIdx.x * kDgCols + c;
    double a = 0.0;
    if (k < K)
        for (int b = p; b < nparts; b += kDgSplit) a += (double)partial[(int64_t)b * K + k];
    part[p][c] = a;
    __syncthreads();
    if (p == 0 && k < K) {
        double sum = 0.0;
#pragma unroll
        for (int i = 0; i < kDgSplit; ++i) sum += part[i][c];
        dg[k] = (float)sum;
    }
}

inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// The reduction split is sized for the 256 compute units of the target chip
// (a fixed count, so that the workspace size does not depend on the device).
constexpr int kTargetCUs = 256;

size_t split_bytes(int64_t M, int64_t N, int64_t K) {
    const int64_t Mp = round_up(M, kT), Np = round_up(N, kT);
    const int s1 = M > 0 ? gemm_splits(M, K, Np, kTargetCUs) : 1;
    const int s2 = N > 0 ? gemm_splits(N, K, Mp, kTargetCUs) : 1;
    const int64_t b1 = s1 > 1 ? s1 * M * K * 4 : 0, b2 = s2 > 1 ? s2 * N * K * 4 : 0;
    return (size_t)round_up(b1 > b2 ? b1 : b2, 256);
}

}  // namespace

size_t backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int64_t Mp = round_up(M, kT), Np = round_up(N, kT);
    const int64_t nparts = (M + kNormRows - 1) / kNormRows;
    return act_stage_bytes(M, K) + (size_t)round_up(M * Np * 2, 256) + (size_t)round_up(N * Mp * 2, 256) +
           (size_t)round_up(K * Mp, 256) + (size_t)round_up(K * (Np / 4), 256) +
           (size_t)round_up(nparts * K * 4, 256) + split_bytes(M, N, K);
}

namespace {
// Blocks of the RMSNorm backward (= dg partials): the register form for rows
// of at most 4096, the two-pass form above that.
int64_t norm_blocks(int64_t M, int64_t K) {
    return K <= 16 * 256 ? (M + kNormRowsRegs - 1) / kNormRowsRegs : (M + kNormRows - 1) / kNormRows;
}

hipError_t launch_norm_backward(const BackwardArgs& a, float* partial, int64_t nblocks, hipStream_t stream) {
    const int M = (int)a.M, K = (int)a.K;
    const unsigned grid = (unsigned)nblocks;
    if (K <= 256)
        norm_backward_regs_kernel<1><<<grid, kNormThreads, 0, stream>>>(a.x, a.g, M, K, a.eps, a.dx, partial);
    else if (K <= 512)
        norm_backward_regs_kernel<2><<<grid, kNormThreads, 0, stream>>>(a.x, a.g, M, K, a.eps, a.dx, partial);
    else if (K <= 1024)
        norm_backward_regs_kernel<4><<<grid, kNormThreads, 0, stream>>>(a.x, a.g, M, K, a.eps, a.dx, partial);
    else if (K <= 2048)
        norm_backward_regs_kernel<8><<<grid, kNormThreads, 0, stream>>>(a.x, a.g, M, K, a.eps, a.dx, partial);
    else if (K <= 4096)
        norm_backward_regs_kernel<16><<<grid, kNormThreads, 0, stream>>>(a.x, a.g, M, K, a.eps, a.dx, partial);
    else
        norm_backward_kernel<<<grid, kNormThreads, 0, stream>>>(a.x, a.g, M, K, a.eps, a.dx, partial);
    return hipGetLastError();
}

template <BKind BK>
hipError_t run_gemm(const uint16_t* A, const void* B, float* C, float* P, const float* alpha, int64_t rows,
                    int64_t cols, int64_t R, hipStream_t stream) {
    const int sp = gemm_splits(rows, cols, R, kTargetCUs);
    GemmArgs g{A, B, C, P, alpha, (int)rows, (int)cols, (int)R, sp};
    bwd_gemm_kernel<BK><<<cdiv(rows, kGT) * cdiv(cols, kGT) * sp, kGThreads, 0, stream>>>(g);
    if (sp > 1) {
        const int64_t n = rows * cols;
        split_reduce_kernel<<<cdiv(n / 4, 256), 256, 0, stream>>>(P, sp, n, alpha, C);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t Mp = round_up(M, kT), Np = round_up(N, kT);
    const int64_t nparts = (M + kNormRows - 1) / kNormRows;
    char* base = static_cast<char*>(a.ws);
    ActStage act = act_stage_carve(base, M, K);
    base += act_stage_bytes(M, K);
    uint16_t* A1 = reinterpret_cast<uint16_t*>(base);
    base += round_up(M * Np * 2, 256);
    uint16_t* A2 = reinterpret_cast<uint16_t*>(base);
    base += round_up(N * Mp * 2, 256);
    int8_t* qT = reinterpret_cast<int8_t*>(base);
    base += round_up(K * Mp, 256);
    uint32_t* wT = reinterpret_cast<uint32_t*>(base);
    base += round_up(K * (Np / 4), 256);
    float* partial = reinterpret_cast<float*>(base);
    base += round_up(nparts * K * 4, 256);
    float* splitbuf = reinterpret_cast<float*>(base);
    const int64_t nparts_used = M > 0 ? norm_blocks(M, K) : 0;  // <= nparts, the size reserved

    hipError_t e;
    if (M > 0) {
        e = launch_quant(a.x, a.g, M, M, (int)K, a.eps, act, stream);
        if (e != hipSuccess) return e;
        if (Np > 0) {
            // flat grids: one dimension of grid y would cap N (or K) at 65535 tiles
            const unsigned grid = cdiv(Mp, kT) * cdiv(Np, kT);
            if (N % 4 == 0)
                dy_prep_kernel<true><<<grid, kPrepThreads, 0, stream>>>(
                    a.dy, act.s, (int)M, (int)N, (int)Mp, (int)Np, reinterpret_cast<uint2*>(A1), reinterpret_cast<uint2*>(A2));
            else
                dy_prep_kernel<false><<<grid, kPrepThreads, 0, stream>>>(
                    a.dy, act.s, (int)M, (int)N, (int)Mp, (int)Np, reinterpret_cast<uint2*>(A1), reinterpret_cast<uint2*>(A2));
            w_transpose_kernel<<<cdiv(Np, kT) * cdiv(K, kT), kPrepThreads, 0, stream>>>(
                reinterpret_cast<const uint32_t*>(a.packed), (int)N, (int)K, (int)Np, wT);
        }
        q_transpose_kernel<<<cdiv(Mp, kT) * cdiv(K, kT), kPrepThreads, 0, stream>>>(
            act.q, (int)M, (int)K, (int)Mp, qT);
        e = run_gemm<BKind::kTern2>(A1, wT, a.dx, splitbuf, a.gamma, M, K, Np, stream);
        if (e != hipSuccess) return e;
        e = launch_norm_backward(a, partial, nparts_used, stream);
        if (e != hipSuccess) return e;
    }
    if (N > 0) {
        e = run_gemm<BKind::kInt8>(A2, qT, a.dW, splitbuf, nullptr, N, K, Mp, stream);
        if (e != hipSuccess) return e;
    }
    dg_reduce_kernel<<<cdiv(K, kDgCols), kDgCols * kDgSplit, 0, stream>>>(partial, (int)nparts_used, (int)K, a.dg);
    return hipGetLastError();
}

}  // namespace bl
