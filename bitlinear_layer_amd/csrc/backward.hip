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
// and s are recomputed with the forward's own quantisation arithmetic (the
// same bits) -- inside the RMSNorm backward kernel, which holds each row of
// x anyway, where the forward's streaming quantiser applies (64 rows and
// more, K <= 2048), else by that quantiser itself -- and r from x.
//
// Both products are dense floating-point contractions and run on the bf16
// matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation), with the
// reduction index contiguous in LDS and zero-padded to a multiple of 64:
//   dxn [M][K] = gamma * A1 [M][Np] . wT [K][Np]^T,   A1 = bf16(dy),  wT = w^T
//   dW  [N][K] =         A2 [N][Mp] . qT [K][Mp]^T,   A2 = bf16(dy (1 / s))^T, qT = q^T
// None of A1, A2 or qT is written to memory: the products read dy (fp32)
// and q (int8) where the forward left them and form their operands while
// staging a tile into LDS -- A1 by rounding rows of dy, A2 by scaling
// columns of dy with 1 / s and rounding, qT by transposing 8 x 4 blocks of
// q bytes in registers.  w and q are exact in bf16, so the only roundings
// besides the fp32 accumulation are those of dy and dy (1 / s) to bf16.
// The weight operand stays compact until it reaches registers: wT as 2-bit
// codes (16 reduction indices per word), expanded to bf16 fragments right
// before its MFMAs.
//
// Kernels: w_transpose (2-bit codes, transposed), the NT GEMM (dxn, then
// dW, each with split_reduce when its reduction is split), norm_backward
// (dx in place over dxn, per-block dg partials; one form also re-quantises
// x) and dg_reduce (fixed order, fp64).
#include "device_common.h"
#include "launch.h"
#include "quant_row.h"
#include "xcd.h"

namespace bl {
namespace {

constexpr int kT = 64;          // transpose tile edge
constexpr int kPrepThreads = 256;

// ---------------------------------------------------------------------------
// Operand preparation
// ---------------------------------------------------------------------------

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
// Both operands are formed while a stage is staged into LDS (global loads
// into registers, conversion, LDS writes).  A comes from dy [M][N] fp32
// (AKind):
//   kRows       -- A[m][n] = bf16(dy[m][n]), zero for n >= N (dxn: rows M,
//                  R = Np); a thread converts 8 consecutive n of 4 rows;
//   kColsScaled -- A[n][m] = bf16(dy[m][n] * (1 / s[m])), zero for m >= M
//                  (dW: rows N, R = Mp); a thread reads 4 consecutive n of
//                  8 rows m, so that each of its 4 LDS rows gets 8
//                  consecutive reduction indices from one 16-byte write.
// VEC: N % 4 == 0, so 16-byte loads of dy rows are aligned and a 4-wide
// chunk is wholly inside or outside the row; else loads are per element.
// B comes in one of two compact forms (BKind):
//   kTern2    -- ternary values as 2-bit codes [cols][R / 16] words (the
//                layout of w_transpose_kernel); a lane reads its column's
//                four words of a stage once and expands half a word per step;
//   kInt8Cols -- q [M][cols] int8 as the forward wrote it: a thread reads 4
//                bytes of 8 rows m and transposes the 8 x 4 block with byte
//                permutes into 8 reduction bytes for each of 4 columns; in
//                LDS each column holds its stage's 64 bytes, and a lane
//                reads 8 bytes per step and converts them exactly.
// Compared with a bf16 B operand, the compact forms cut a stage's LDS
// traffic (the writes of the staged operand and the per-step fragment
// reads) from 256 KiB to 172 KiB (kTern2) and 190 KiB (kInt8Cols) per
// 64-deep stage.
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
constexpr int kMaxSplits = 8;
constexpr int kI8Pitch = kGK + 8;  // bytes per int8 LDS row: 8-byte reads of 32 rows hit distinct bank pairs

enum class AKind { kRows, kColsScaled };
enum class BKind { kTern2, kInt8Cols };

// Bytes of one B row of a stage in LDS.
template <BKind BK>
constexpr int b_lds_pitch() {
    return BK == BKind::kTern2 ? kGK / 4 : kI8Pitch;
}

struct GemmArgs {
    const float* dy;     // [M][N]
    const float* s;      // [M]: the activation scales (kColsScaled)
    const void* B;       // kTern2: wT words [cols][R / 16]; kInt8Cols: q [M][cols]
    float* C;            // final output (splits == 1)
    float* P;            // split partials (splits > 1)
    const float* alpha;  // device scalar, or nullptr for 1
    int rows, cols, R, splits;
    int M, N;            // shape of dy
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

// Two fp32 values as a bf16 pair (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ float f4_get(const float4& v, int j) {
    return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Four consecutive floats of a dy row from column n: one 16-byte load when
// VEC (n % 4 == 0, N % 4 == 0), else per element; zero past the row's end.
template <bool VEC>
__device__ __forceinline__ float4 load_dy4(const float* row, int n, int N) {
    if constexpr (VEC) {
        return n < N ? *reinterpret_cast<const float4*>(row + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        return make_float4(n < N ? row[n] : 0.f, n + 1 < N ? row[n + 1] : 0.f, n + 2 < N ? row[n + 2] : 0.f,
                           n + 3 < N ? row[n + 3] : 0.f);
    }
}

template <AKind AK, BKind BK, bool VEC>
__global__ __launch_bounds__(kGThreads) void bwd_gemm_kernel(GemmArgs g) {
    constexpr int kBPitch = b_lds_pitch<BK>();
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kGT * kGPitch];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kGT * kBPitch];
    // Work item f = split * tiles + tile, output column tiles fastest, under
    // the XCD map: an XCD takes whole rows of tiles of one split, so each
    // A panel (a row of tiles' rows over the split's stages) is fetched into
    // one L2, and B panels into as many as there are splits.
    const int ntc = (g.cols + kGT - 1) / kGT;
    const int tiles = (int)(gridDim.x / g.splits);
    const int f = xcd_tile(blockIdx.x, gridDim.x);
    const int split = f / tiles, tile = f % tiles;
    const int tr = tile / ntc, tc = tile % ntc;
    const int row0 = tr * kGT, col0 = tc * kGT;
    const int t = threadIdx.x, lane = t & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int wm = wave / kGWN, wn = wave % kGWN;

    // stages [st0, st1) of this split
    const int nst = g.R / kGK;
    const int per = (nst + g.splits - 1) / g.splits;
    const int st0 = min(split * per, nst), st1 = min(st0 + per, nst);

    // Staging of A (eight 4-float pieces per thread and stage):
    //   kRows: rows srow + 64 p (p < 4), stage elements 8 sch .. 8 sch + 7,
    //          written as one 16-byte bf16 piece per row;
    //   kColsScaled: dy rows m = 64 st + 8 wave + i (i < 8), columns
    //          row0 + 4 lane .. + 3, written as 8 bf16 of reduction index
    //          8 wave .. 8 wave + 7 into each of the LDS rows 4 lane + j.
    const int srow = t / 8, sch = t % 8;
    constexpr int kRowStep = kGThreads / 8;  // 64
    constexpr int kLdsStep = kRowStep * kGPitch;
    const int lds0 = srow * kGPitch + 8 * sch;
    int64_t arow[4] = {0, 0, 0, 0};
    if constexpr (AK == AKind::kRows) {
#pragma unroll
        for (int p = 0; p < 4; ++p) arow[p] = (int64_t)min(row0 + srow + p * kRowStep, g.rows - 1) * g.N;
    }
    // kColsScaled: first of the thread's four dy columns (clamped into the
    // row when VEC; those output rows are not stored)
    const int ncol = AK == AKind::kColsScaled ? (VEC ? min(row0 + 4 * lane, g.N - 4) : row0 + 4 * lane) : 0;
    float4 ra[8];
    float sl = 1.0f;  // kColsScaled: lane l holds s of the stage's row 8 wave + l % 8

    // Staging of B:
    //   kTern2: threads t < 256 one 16-byte row (four words);
    //   kInt8Cols: q rows m = 64 st + 8 wave + i (i < 8), 4 bytes from column
    //          col0 + 4 lane (clamped into the row: cols % 16 == 0).
    const uint32_t* B2 = static_cast<const uint32_t*>(g.B);
    const int8_t* B8 = static_cast<const int8_t*>(g.B);
    const int64_t boff0 = BK == BKind::kTern2 ? (int64_t)min(col0 + (t & (kGT - 1)), g.cols - 1) * (g.R / 16) : 0;
    const int kcol = BK == BKind::kInt8Cols ? min(col0 + 4 * lane, g.cols - 4) : 0;
    const bool b_stager = BK != BKind::kTern2 || t < kGT;
    uint4 rb0;
    uint32_t rq[8];

    auto load_stage = [&](int st) {
        if constexpr (AK == AKind::kRows) {
            const int n = st * kGK + 8 * sch;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                ra[2 * p] = load_dy4<VEC>(g.dy + arow[p], n, g.N);
                ra[2 * p + 1] = load_dy4<VEC>(g.dy + arow[p], n + 4, g.N);
            }
        } else {
            // rows m >= M read as zero (the reduction padding); s is then
            // read at a valid index and does not matter.  s goes through a
            // vector load: a scalar load would share the LDS reads' counter
            // and, returning out of order, make every fragment wait for it.
            sl = g.s[min(st * kGK + 8 * wave + (lane & 7), g.M - 1)];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int m = st * kGK + 8 * wave + i;
                const int mc = min(m, g.M - 1);
                ra[i] = m < g.M ? load_dy4<VEC>(g.dy + (int64_t)mc * g.N, ncol, g.N) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        if constexpr (BK == BKind::kTern2) {
            if (b_stager) rb0 = *reinterpret_cast<const uint4*>(B2 + boff0 + (int64_t)st * (kGK / 16));
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int mc = min(st * kGK + 8 * wave + i, g.M - 1);
                rq[i] = *reinterpret_cast<const uint32_t*>(B8 + (int64_t)mc * g.cols + kcol);
            }
        }
    };
    // Conversion and LDS writes of the staged registers, in pieces that the
    // main loop spreads between the MFMAs of a stage's second-to-last
    // 16-deep step (a wave's VALU work then issues while its MFMAs run):
    //   kRows: pieces 0..3, one LDS row each;
    //   kColsScaled: piece 0 the reciprocals 1 / s of the stage's 8 rows (one
    //          division per lane, broadcast from lanes 0..7), pieces 1..4 one
    //          LDS row (dy column) each;
    //   kTern2: one piece;
    //   kInt8Cols: pieces 0 and 2 the row-pair byte interleaves of columns
    //          0, 1 and of columns 2, 3, pieces 1 and 3 the LDS rows of
    //          those columns.
    // The transposing forms write LDS rows 4 lane + j; with rows of 144
    // (A) or 72 (B) bytes that would put 4 lanes on each bank.  Their
    // 16-byte (A) and 8-byte (B) chunks are therefore XOR-swizzled by row:
    // chunk c of row r sits at c ^ ((r >> 4) & 3) (A) and c ^ ((r >> 5) & 3)
    // (B), which spreads the writes of any 16 (A) or 32 (B) lanes over all
    // banks and keeps the fragment reads conflict-free.
    constexpr bool kSwz = AK == AKind::kColsScaled;
    static_assert(kSwz == (BK == BKind::kInt8Cols), "the dW operand forms go together");
    constexpr int kPiecesA = AK == AKind::kRows ? 4 : 5;
    constexpr int kPiecesB = BK == BKind::kTern2 ? 1 : 4;
    constexpr int kPieces = kPiecesA + kPiecesB;
    float inv[8];
    uint32_t e[4];
    auto store_piece = [&](int buf, int pc) {
        if (pc < kPiecesA) {
            if constexpr (AK == AKind::kRows) {
                const float4 u = ra[2 * pc], v = ra[2 * pc + 1];
                *reinterpret_cast<uint4*>(&As[buf][lds0 + pc * kLdsStep]) =
                    make_uint4(bf16_pair(u.x, u.y), bf16_pair(u.z, u.w), bf16_pair(v.x, v.y), bf16_pair(v.z, v.w));
            } else if (pc == 0) {
                const float r = 1.0f / sl;
#pragma unroll
                for (int i = 0; i < 8; ++i) inv[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), i));
            } else {
                const int j = pc - 1;
                uint32_t d[4];
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    d[h] = bf16_pair(f4_get(ra[2 * h], j) * inv[2 * h], f4_get(ra[2 * h + 1], j) * inv[2 * h + 1]);
                *reinterpret_cast<uint4*>(&As[buf][(4 * lane + j) * kGPitch + 8 * (wave ^ ((lane >> 2) & 3))]) =
                    make_uint4(d[0], d[1], d[2], d[3]);
            }
            return;
        }
        const int pb = pc - kPiecesA;
        uint8_t* bs = Bs[buf];
        if constexpr (BK == BKind::kTern2) {
            if (b_stager) *reinterpret_cast<uint4*>(bs + t * kBPitch) = rb0;
        } else if ((pb & 1) == 0) {
            // 8 x 4 bytes (row i, column c) -> e[pr] = rows 2 pr, 2 pr + 1 of
            // columns 2 hc and 2 hc + 1, interleaved byte by byte
            const uint32_t sel = pb == 0 ? 0x05010400u : 0x07030602u;
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) e[pr] = __builtin_amdgcn_perm(rq[2 * pr + 1], rq[2 * pr], sel);
        } else {
            const int hc = pb >> 1;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint32_t sel = c ? 0x07060302u : 0x05040100u;
                const uint32_t lo = __builtin_amdgcn_perm(e[1], e[0], sel);  // rows 0..3
                const uint32_t hi = __builtin_amdgcn_perm(e[3], e[2], sel);  // rows 4..7
                *reinterpret_cast<uint2*>(bs + (4 * lane + 2 * hc + c) * kBPitch + 8 * (wave ^ ((lane >> 3) & 3))) =
                    make_uint2(lo, hi);
            }
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int pc = 0; pc < kPieces; ++pc) store_piece(buf, pc);
    };

    f32x16 acc[kGFM][kGFN];
#pragma unroll
    for (int i = 0; i < kGFM; ++i)
#pragma unroll
        for (int j = 0; j < kGFN; ++j) acc[i][j] = f32x16{};

    const int afrag = (wm * (kGT / kGWM) + (lane & 31)) * kGPitch + 8 * ((lane >> 5) ^ (kSwz ? (lane >> 4) & 1 : 0));
    const int bcol = wn * (kGT / kGWN) + (lane & 31);  // B row (output column) of fragment 0
    const int half = lane >> 5;
    // Stage st sits in buffer (st - st0) % 2.  The loads of stage st + 1 are
    // issued during stage st - 1 (or here).  During stage st they are
    // converted and written to the other buffer in pieces between the MFMAs
    // of its second-to-last 16-deep step, and the loads of stage st + 2 go
    // out right after, so they still get a whole stage to land.  The
    // conversion work then issues while the MFMAs run, and the last step
    // runs MFMAs only, up to the barrier that publishes stage st + 1.
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
                bf16x8, *reinterpret_cast<const uint4*>(&As[buf][afrag + i * 32 * kGPitch + 16 * (kSwz ? ks ^ (i & 1) : ks)]));
        if constexpr (BK == BKind::kInt8Cols) {
#pragma unroll
            for (int j = 0; j < kGFN; ++j)
                b8[j] = *reinterpret_cast<const uint2*>(
                    &Bs[buf][(bcol + j * 32) * kBPitch + 8 * ((2 * ks + half) ^ ((2 * wn + j) & 3))]);
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
    constexpr int kPerSlot = (kPieces + kMf - 2) / (kMf - 1);
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
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int idx = 0; idx < kMf; ++idx) {
                const int i = idx / kGFN, j = idx % kGFN;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
                if (ahead && idx >= kMf - kGFN) expand_b(ks + 1, nxt, idx - (kMf - kGFN));
                if (ks == KS - 2 && more) {
                    // pieces over the step's first kMf - 1 MFMAs
#pragma unroll
                    for (int q = 0; q < kPerSlot; ++q)
                        if (idx * kPerSlot + q < kPieces) store_piece(buf ^ 1, idx * kPerSlot + q);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (ks == KS - 2 && more && st + 2 < st1) load_stage(st + 2);
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

// The register-form RMSNorm backward fused with the re-quantisation of the
// same rows (q and s for the dW product), for rows of at most CPL * 512
// elements.  Lane l holds the 8-element chunks l + 64 c (c < CPL) of its
// wave's row -- the streaming quantiser's layout -- and quantises the row
// with that kernel's own row function, so q and s are its bits; x is read
// once for both.  The RMSNorm backward arithmetic is that of
// norm_backward_regs_kernel (fp64 row sums, dx in place over dxn, the
// block's dg partial added over its waves in wave order).
template <int CPL, bool FULL>
__global__ __launch_bounds__(kNormThreads) void norm_backward_quant_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gw, int M, int K, float eps,
    float* __restrict__ dxio, float* __restrict__ partial, int8_t* __restrict__ q, float* __restrict__ s) {
    __shared__ float4 red[2 * CPL * kWave];
    const int m0 = blockIdx.x * kNormRowsRegs;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    constexpr int kWaves = kNormThreads / kWave;
    const int nchunks = K / 8;
    float4 gv[CPL][2], acc[CPL][2];
    load_g_row<CPL, FULL>(gw, lane, nchunks, gv);
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c][0] = acc[c][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    auto valid = [&](int c) { return FULL || (int)(lane + c * kWave) < nchunks; };
    for (int rr = wave; rr < kNormRowsRegs; rr += kWaves) {
        const int m = m0 + rr;
        if (m >= M) break;
        float* dr = dxio + (int64_t)m * K;
        uint4 xc[CPL];
        load_x_row<CPL, FULL>(x + (int64_t)m * K, lane, nchunks, xc);
        float4 d[CPL][2];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int k = 8 * (int)(lane + c * kWave);
            d[c][0] = d[c][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (valid(c)) {
                d[c][0] = *reinterpret_cast<const float4*>(dr + k);
                d[c][1] = *reinterpret_cast<const float4*>(dr + k + 4);
            }
        }
        double ss = 0.0, S = 0.0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float xs[8] = {bf16_lo(xc[c].x), bf16_hi(xc[c].x), bf16_lo(xc[c].y), bf16_hi(xc[c].y),
                                 bf16_lo(xc[c].z), bf16_hi(xc[c].z), bf16_lo(xc[c].w), bf16_hi(xc[c].w)};
            const float ds[8] = {d[c][0].x, d[c][0].y, d[c][0].z, d[c][0].w, d[c][1].x, d[c][1].y, d[c][1].z, d[c][1].w};
            const float gs[8] = {gv[c][0].x, gv[c][0].y, gv[c][0].z, gv[c][0].w,
                                 gv[c][1].x, gv[c][1].y, gv[c][1].z, gv[c][1].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                ss += (double)xs[j] * (double)xs[j];
                S += (double)ds[j] * (double)gs[j] * (double)xs[j];
            }
        }
        ss = wave_sum(ss);
        S = wave_sum(S);
        const double rd = 1.0 / sqrt(ss / (double)K + (double)eps);
        const float r = (float)rd, cc = (float)(rd * rd * rd * S / (double)K);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float xs[8] = {bf16_lo(xc[c].x), bf16_hi(xc[c].x), bf16_lo(xc[c].y), bf16_hi(xc[c].y),
                                 bf16_lo(xc[c].z), bf16_hi(xc[c].z), bf16_lo(xc[c].w), bf16_hi(xc[c].w)};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float4 g4 = gv[c][h], d4 = d[c][h];
                const float x0 = xs[4 * h], x1 = xs[4 * h + 1], x2 = xs[4 * h + 2], x3 = xs[4 * h + 3];
                if (valid(c)) {
                    float4 o;
                    o.x = r * g4.x * d4.x - x0 * cc;
                    o.y = r * g4.y * d4.y - x1 * cc;
                    o.z = r * g4.z * d4.z - x2 * cc;
                    o.w = r * g4.w * d4.w - x3 * cc;
                    *reinterpret_cast<float4*>(dr + 8 * (int)(lane + c * kWave) + 4 * h) = o;
                }
                acc[c][h].x += d4.x * x0 * r;
                acc[c][h].y += d4.y * x1 * r;
                acc[c][h].z += d4.z * x2 * r;
                acc[c][h].w += d4.w * x3 * r;
            }
        }
        quant_row_regs<CPL, FULL>(
            xc, [&](int c, float4& lo, float4& hi) { lo = gv[c][0]; hi = gv[c][1]; }, m, lane, K, eps, q, s,
            nullptr);
    }
    // dg partial of the block: waves 0, 1, 2, 3 added in that order
    for (int w = 0; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float4 v = acc[c][h];
                    const int i = (2 * c + h) * kWave + lane;
                    if (w > 0) {
                        const float4 p = red[i];
                        v = make_float4(p.x + v.x, p.y + v.y, p.z + v.z, p.w + v.w);
                    }
                    red[i] = v;
                }
        }
        __syncthreads();
    }
    for (int i = threadIdx.x; i < 2 * CPL * kWave; i += kNormThreads) {
        const int ch = i / kWave, l = i % kWave;  // ch = 2 c + h
        const int chunk = l + (ch / 2) * kWave;
        if (FULL || chunk < nchunks)
            *reinterpret_cast<float4*>(partial + (int64_t)blockIdx.x * K + 8 * chunk + 4 * (ch % 2)) = red[i];
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
    const int64_t Np = round_up(N, kT);
    const int64_t nparts = (M + kNormRows - 1) / kNormRows;
    return act_stage_bytes(M, K) + (size_t)round_up(K * (Np / 4), 256) + (size_t)round_up(nparts * K * 4, 256) +
           split_bytes(M, N, K);
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

// The fused RMSNorm backward + re-quantisation applies where the forward's
// quantiser is the streaming kernel (at least 64 rows) with at most four
// 8-element chunks per lane (K <= 2048, so the row, dxn, g and the dg sums
// stay in registers).
bool norm_quant_fused(int64_t M, int64_t K) { return M >= 64 && K <= 4 * kWave * 8; }

template <int CPL>
void launch_norm_quant_cpl(const BackwardArgs& a, float* partial, unsigned grid, const ActStage& act,
                           hipStream_t stream) {
    const int M = (int)a.M, K = (int)a.K;
    if (K == CPL * kWave * 8)
        norm_backward_quant_kernel<CPL, true><<<grid, kNormThreads, 0, stream>>>(a.x, a.g, M, K, a.eps, a.dx, partial,
                                                                                 act.q, act.s);
    else
        norm_backward_quant_kernel<CPL, false><<<grid, kNormThreads, 0, stream>>>(a.x, a.g, M, K, a.eps, a.dx,
                                                                                  partial, act.q, act.s);
}

hipError_t launch_norm_quant(const BackwardArgs& a, float* partial, int64_t nblocks, const ActStage& act,
                             hipStream_t stream) {
    const int cpl = (int)((a.K / 8 + kWave - 1) / kWave);
    const unsigned grid = (unsigned)nblocks;
    switch (cpl) {
        case 1: launch_norm_quant_cpl<1>(a, partial, grid, act, stream); break;
        case 2: launch_norm_quant_cpl<2>(a, partial, grid, act, stream); break;
        case 3: launch_norm_quant_cpl<3>(a, partial, grid, act, stream); break;
        default: launch_norm_quant_cpl<4>(a, partial, grid, act, stream); break;
    }
    return hipGetLastError();
}

template <AKind AK, BKind BK>
hipError_t run_gemm(const GemmArgs& g0, hipStream_t stream) {
    GemmArgs g = g0;
    g.splits = gemm_splits(g.rows, g.cols, g.R, kTargetCUs);
    const unsigned grid = cdiv(g.rows, kGT) * cdiv(g.cols, kGT) * g.splits;
    if (g.N % 4 == 0)
        bwd_gemm_kernel<AK, BK, true><<<grid, kGThreads, 0, stream>>>(g);
    else
        bwd_gemm_kernel<AK, BK, false><<<grid, kGThreads, 0, stream>>>(g);
    if (g.splits > 1) {
        const int64_t n = (int64_t)g.rows * g.cols;
        split_reduce_kernel<<<cdiv(n / 4, 256), 256, 0, stream>>>(g.P, g.splits, n, g.alpha, g.C);
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
    uint32_t* wT = reinterpret_cast<uint32_t*>(base);
    base += round_up(K * (Np / 4), 256);
    float* partial = reinterpret_cast<float*>(base);
    base += round_up(nparts * K * 4, 256);
    float* splitbuf = reinterpret_cast<float*>(base);
    const int64_t nparts_used = M > 0 ? norm_blocks(M, K) : 0;  // <= nparts, the size reserved

    hipError_t e;
    const bool fused_q = norm_quant_fused(M, K);
    if (M > 0) {
        if (!fused_q) {
            e = launch_quant(a.x, a.g, M, M, (int)K, a.eps, act, stream);
            if (e != hipSuccess) return e;
        }
        if (Np > 0)  // flat grid: one dimension of grid y would cap K at 65535 tiles
            w_transpose_kernel<<<cdiv(Np, kT) * cdiv(K, kT), kPrepThreads, 0, stream>>>(
                reinterpret_cast<const uint32_t*>(a.packed), (int)N, (int)K, (int)Np, wT);
        // dxn [M][K] = gamma bf16(dy) [M][Np] . wT^T
        GemmArgs g{a.dy, act.s, wT, a.dx, splitbuf, a.gamma, (int)M, (int)K, (int)Np, 1, (int)M, (int)N};
        e = run_gemm<AKind::kRows, BKind::kTern2>(g, stream);
        if (e != hipSuccess) return e;
        e = fused_q ? launch_norm_quant(a, partial, nparts_used, act, stream)
                    : launch_norm_backward(a, partial, nparts_used, stream);
        if (e != hipSuccess) return e;
    }
    if (N > 0) {
        // dW [N][K] = bf16(dy (1 / s))^T [N][Mp] . q [Mp][K]
        GemmArgs g{a.dy, act.s, act.q, a.dW, splitbuf, nullptr, (int)N, (int)K, (int)Mp, 1, (int)M, (int)N};
        e = run_gemm<AKind::kColsScaled, BKind::kInt8Cols>(g, stream);
        if (e != hipSuccess) return e;
    }
    dg_reduce_kernel<<<cdiv(K, kDgCols), kDgCols * kDgSplit, 0, stream>>>(partial, (int)nparts_used, (int)K, a.dg);
    return hipGetLastError();
}

}  // namespace bl
