// gemm_mfma.hip -- prefill-shaped ternary product on the int8 matrix cores.
//
// At large token counts the ternary product is a dense contraction
// (2*M*N*K int8 operations against (M+N/4)*K bytes), so it runs on
// v_mfma_i32_16x16x64_i8 ([jiqizhixin, "具有三值权重的 MatMul-free 密集层"]: the
// ternary product is an add/subtract accumulation; on the matrix cores it
// is the same integer sum, exactly).
//
// Block tile BM x BN (tokens x packed rows), 8 waves as WM x WN, each wave
// owning a (BM/WM) x (BN/WN) tile of 16x16 accumulators.  K advances in
// stages of 128 (two MFMA steps of 64), double-buffered in LDS:
//   A: int8 codes q, BM rows x 128 bytes per stage (row pitch padded by 16
//      bytes so that the 16-byte fragment reads of 8 lanes hit distinct banks);
//   B: packed weights, BN rows x 32 bytes per stage -- a quarter of the
//      int8 operand -- expanded in registers: a lane's 16-byte B fragment of
//      one 16x16x64 step is one packed 32-bit word (16 weights), 7 VALU ops.
// Operand pairing: lane l of A supplies row l%16, k = 16*(l/16) + 0..15 of
// the step; lane l of B supplies column l%16 at the same k.  The
// accumulator element v of lane l holds D[4*(l/16) + v][l%16].
#include <type_traits>

#include "epilogue.h"
#include "xcd.h"

namespace bl {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;                 // k per LDS stage
constexpr int kAPitch = kBK + 16;        // bytes per A row in LDS
constexpr int kBWords = kBK / 16;        // packed words per B row per stage (8)
constexpr int kBPitch = kBWords + 4;     // words per B row in LDS (16-byte aligned)

template <int BM, int BN, int WM, int WN, Epilogue EP>
struct Tile {
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 fragments per wave
    static constexpr bool kGlu = EP == Epilogue::kGluBf16;
    static constexpr int kCols = kGlu ? BN / 2 : BN;  // output columns per block
    static constexpr int kAChunks = BM * (kBK / 16) / kThreads;  // 16-byte A loads per thread
    static constexpr int kBChunks = BN * (kBK / 64) / kThreads;  // 16-byte B loads per thread
    static_assert(kAChunks >= 1 && kBChunks >= 1, "tile too small for the block");
    static_assert(!kGlu || FN % 2 == 0, "GLU tiles pair gate and up fragments");
    static constexpr int kLdsA = BM * kAPitch;          // bytes per stage
    static constexpr int kLdsB = BN * kBPitch * 4;      // bytes per stage
};

// Packed row (of the Nrows x K/4 matrix) that local B-tile row r of output
// tile tn maps to.  Plain: rows tn*BN + r.  GLU: the first BN/2 local rows
// are gate rows f0 + r, the rest the up rows F + f0 + r - BN/2, clamped.
template <int BN, bool GLU>
__device__ __forceinline__ int64_t b_row(int tn, int r, int N) {
    if (GLU) {
        const int f = tn * (BN / 2) + (r % (BN / 2));
        return (r < BN / 2 ? 0 : (int64_t)N) + min(f, N - 1);
    }
    return min(tn * BN + r, N - 1);
}

template <int BM, int BN, int WM, int WN, Epilogue EP>
__global__ __launch_bounds__(WM * WN * kWave) void gemm_kernel(ProductArgs a) {
    using T = Tile<BM, BN, WM, WN, EP>;
    constexpr bool kGlu = T::kGlu;
    __shared__ __attribute__((aligned(16))) int8_t As[2][T::kLdsA];
    __shared__ __attribute__((aligned(16))) uint32_t Bs[2][T::kLdsB / 4];

    const int M = a.M, N = a.N, K = a.K;
    const int nwords = K / 16;
    const int ntn = (N + T::kCols - 1) / T::kCols;
    const int per_problem = ntn * ((M + BM - 1) / BM);  // grid x = batch * per_problem
    const int f = xcd_tile(blockIdx.x, gridDim.x);
    const int b = f / per_problem;
    const int t = f - b * per_problem;
    const int tn = t % ntn;
    const int tm = t / ntn;
    const int m0 = tm * BM;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;

    const int64_t nrows = kGlu ? 2 * (int64_t)N : (int64_t)N;
    const int8_t* Q = a.q + (int64_t)b * M * K;
    const uint32_t* P = reinterpret_cast<const uint32_t*>(a.packed) + (int64_t)b * nrows * nwords;

    // Global -> register staging of one stage (k0 .. k0 + 127).
    int4 ra[T::kAChunks];
    uint4 rb[T::kBChunks];
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < T::kAChunks; ++i) {
            const int id = tid + i * T::kThreads;
            const int r = id / (kBK / 16), c = id % (kBK / 16);
            const int kk = k0 + 16 * c;
            const int64_t row = min(m0 + r, M - 1);
            ra[i] = kk < K ? *reinterpret_cast<const int4*>(Q + row * K + kk) : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < T::kBChunks; ++i) {
            const int id = tid + i * T::kThreads;
            const int r = id / (kBK / 64), c = id % (kBK / 64);
            const int w0 = k0 / 16 + 4 * c;
            const uint32_t* src = P + b_row<BN, kGlu>(tn, r, N) * nwords + w0;
            if (w0 + 4 <= nwords) {
                rb[i] = *reinterpret_cast<const uint4*>(src);
            } else {  // tail of K: words past the row end meet zero codes in A
                rb[i] = make_uint4(w0 < nwords ? src[0] : 0u, w0 + 1 < nwords ? src[1] : 0u,
                                   w0 + 2 < nwords ? src[2] : 0u, 0u);
            }
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::kAChunks; ++i) {
            const int id = tid + i * T::kThreads;
            const int r = id / (kBK / 16), c = id % (kBK / 16);
            *reinterpret_cast<int4*>(&As[buf][r * kAPitch + 16 * c]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < T::kBChunks; ++i) {
            const int id = tid + i * T::kThreads;
            const int r = id / (kBK / 64), c = id % (kBK / 64);
            *reinterpret_cast<uint4*>(&Bs[buf][r * kBPitch + 4 * c]) = rb[i];
        }
    };

    i32x4 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    const int nstages = (K + kBK - 1) / kBK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int st = 0; st < nstages; ++st) {
        const int buf = st & 1;
        if (st + 1 < nstages) load_stage((st + 1) * kBK);
#pragma unroll
        for (int kk = 0; kk < kBK / 64; ++kk) {
            i32x4 bfrag[T::FN];
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                int r;
                if (kGlu)  // gate fragments first, then the up fragments of the same f
                    r = (j < T::FN / 2 ? 0 : BN / 2) + wn * (T::TN / 2) + (j % (T::FN / 2)) * 16 + (lane & 15);
                else
                    r = wn * T::TN + j * 16 + (lane & 15);
                const uint32_t pw = Bs[buf][r * kBPitch + kk * 4 + (lane >> 4)];
                int32_t c0, c1, c2, c3;
                decode_codes(pw, c0, c1, c2, c3);
                bfrag[j] = i32x4{c0, c1, c2, c3};
            }
#pragma unroll
            for (int i = 0; i < T::FM; ++i) {
                const int r = wm * T::TM + i * 16 + (lane & 15);
                const i32x4 afrag =
                    *reinterpret_cast<const i32x4*>(&As[buf][r * kAPitch + kk * 64 + 16 * (lane >> 4)]);
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afrag, bfrag[j], acc[i][j], 0, 0, 0);
            }
        }
        if (st + 1 < nstages) store_stage(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: subtract sum_k q, rescale (or form the GLU product), store.
    const float gamma = a.gamma ? a.gamma[b] : 0.0f;
    const int64_t tok0 = (int64_t)b * M;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = m0 + wm * T::TM + i * 16 + 4 * (lane >> 4) + v;
            if (m >= M) continue;
            const int64_t t = tok0 + m;
            const int32_t sq = a.sumq[t];
            const float cs = EP == Epilogue::kI32 ? 0.0f : gamma / a.s[t];
            if (kGlu) {
#pragma unroll
                for (int j = 0; j < T::FN / 2; ++j) {
                    const int f = tn * (BN / 2) + wn * (T::TN / 2) + j * 16 + (lane & 15);
                    if (f < N) {
                        const float zg = rescale(acc[i][j][v] - sq, cs);
                        const float zu = rescale(acc[i][j + T::FN / 2][v] - sq, cs);
                        static_cast<uint16_t*>(a.out)[t * N + f] = glu_bf16(zg, zu);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < T::FN; ++j) {
                    const int n = tn * BN + wn * T::TN + j * 16 + (lane & 15);
                    if (n < N) {
                        const int32_t val = acc[i][j][v] - sq;
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

// ---------------------------------------------------------------------------
// The same product with the operands copied from global memory straight into
// LDS (global_load_lds_dwordx4, no register staging), three stages deep, so
// that two stages of loads are in flight while one is multiplied.  Requires
// K % 128 == 0.  LDS rows are unpadded; bank conflicts are avoided by an XOR
// swizzle of the 16-byte chunks instead (A: chunk ^ (row & 7); B: half ^
// ((row >> 3) & 1)), which the DMA realises by choosing, per lane, which
// global chunk lands in that lane's fixed LDS slot.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// 16 bytes per lane from gbase + voff into LDS at lds_addr + 16 * lane
// (global_load_lds_dwordx4; the LDS address goes through M0).  Issued as
// inline asm so that the compiler does not track these writes into LDS: its
// conservative tracking would wait for every DMA in flight before each LDS
// read.  The kernels order all DMA reuse of LDS themselves with explicit
// s_waitcnt vmcnt(n) and barriers.  The instruction has no register outputs
// and takes its address operands and M0 at issue, so M0 is restored right
// after it (M0 is reserved to the compiler); one wait state separates the
// M0 write from the DMA that reads it.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "s"(lds_addr), "v"(voff), "s"(gbase)
        : "memory");
}
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}




// Swizzle of the 16-byte pieces of a B stage row (BK / 64 pieces): rows
// r and r + 8 (BK = 128) or r, r + 4, r + 8, r + 12 (BK = 256) share banks
// and differ in the piece, so a 16-row fragment read is conflict free.
template <int BK>
__device__ __forceinline__ int b_swizzle(int r) {
    return BK == 128 ? ((r >> 3) & 1) : ((r >> 2) & 3);
}

// BK: k per LDS stage (128 or 256).  A stage row is BK bytes of codes; a B
// stage row is BK / 4 packed bytes.  With BK = 256 each DMA instruction reads
// 64 contiguous bytes of each of 16 weight rows, where BK = 128 reads 32 of
// each of 32 rows: 32-byte runs stream at about 3.8 TB/s, 64-byte runs at
// 6.3-6.4 and 128-byte runs at 6.8 (copies of the pattern without arithmetic).
template <int BM, int BN, int WM, int WN, Epilogue EP, int BK>
__global__ __launch_bounds__(WM * WN * kWave) void gemm_dma_kernel(ProductArgs a) {
    using T = Tile<BM, BN, WM, WN, EP>;
    constexpr bool kGlu = T::kGlu;
    constexpr int kWavesPerBlock = WM * WN;
    constexpr int kAStage = BM * BK;          // bytes
    constexpr int kBStage = BN * (BK / 4);    // bytes
    constexpr int kALanes = BK / 16;          // lanes per A row in a DMA instruction (8 or 16)
    constexpr int kBLanes = BK / 64;          // lanes per B row (2 or 4)
    static_assert(BK == 128 || BK == 256, "stage of 128 or 256 k");
    // Stages in flight while one is multiplied: two of 16 KiB at BK = 128
    // (three buffers, 48 KiB: three blocks per CU), one of 32 KiB at BK = 256
    // (two buffers, 64 KiB: two blocks per CU; three buffers would leave one
    // block per CU, which measured slower).
    constexpr int kDist = BK == 256 ? 1 : 2;
    constexpr int kBufs = kDist + 1;
    constexpr int kADma = kAStage / 1024 / kWavesPerBlock;  // 1 KiB DMA instructions per wave
    constexpr int kBDma = kBStage / 1024 / kWavesPerBlock;
    static_assert(kADma >= 1 && kBDma >= 1 && kADma * 1024 * kWavesPerBlock == kAStage &&
                      kBDma * 1024 * kWavesPerBlock == kBStage,
                  "stage must split into whole 1 KiB DMA instructions per wave");
    __shared__ __attribute__((aligned(1024))) int8_t lds[kBufs * (kAStage + kBStage)];

    const int M = a.M, N = a.N, K = a.K;
    const int nwords = K / 16;
    const int ntn = (N + T::kCols - 1) / T::kCols;
    const int per_problem = ntn * ((M + BM - 1) / BM);  // grid x = batch * per_problem
    const int f = xcd_tile(blockIdx.x, gridDim.x);
    const int b = f / per_problem;
    const int t = f - b * per_problem;
    const int tn = t % ntn;
    const int tm = t / ntn;
    const int m0 = tm * BM;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;

    const int64_t nrows = kGlu ? 2 * (int64_t)N : (int64_t)N;
    const int8_t* Q = a.q + (int64_t)b * M * K;
    const uint32_t* P = reinterpret_cast<const uint32_t*>(a.packed) + (int64_t)b * nrows * nwords;

    // Per-lane global sources (stage 0) and LDS slots of this wave's DMAs.
    const int8_t* asrc[kADma];
    const uint32_t* bsrc[kBDma];
    // The DMA writes lane i's 16 bytes to LDS slot i of its 1 KiB block, so
    // the XOR swizzles of the LDS layout are applied to the global source:
    // LDS slot (row r, chunk c) holds global chunk c ^ swizzle(r).
#pragma unroll
    for (int i = 0; i < kADma; ++i) {
        const int r = (wave * kADma + i) * (kWave / kALanes) + lane / kALanes;
        const int chunk = (lane % kALanes) ^ (r % kALanes);
        asrc[i] = Q + (int64_t)min(m0 + r, M - 1) * K + 16 * chunk;
    }
#pragma unroll
    for (int i = 0; i < kBDma; ++i) {
        const int r = (wave * kBDma + i) * (kWave / kBLanes) + lane / kBLanes;
        const int piece = (lane % kBLanes) ^ b_swizzle<BK>(r);
        bsrc[i] = P + b_row<BN, kGlu>(tn, r, N) * nwords + 4 * piece;
    }
    auto issue_stage = [&](int st) {
        const int buf = st % kBufs;
        int8_t* abase = lds + buf * kAStage;
        int8_t* bbase = lds + kBufs * kAStage + buf * kBStage;
#pragma unroll
        for (int i = 0; i < kADma; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(asrc[i] + st * BK),
                                             (lds_void_t*)(abase + (wave * kADma + i) * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < kBDma; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(bsrc[i] + st * (BK / 16)),
                                             (lds_void_t*)(bbase + (wave * kBDma + i) * 1024), 16, 0, 0);
    };

    i32x4 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    const int nstages = K / BK;
    for (int d = 0; d < kDist && d < nstages; ++d) issue_stage(d);
    for (int st = 0; st < nstages; ++st) {
        // Stage st has landed once at most the stages after it are pending.
        if (kDist == 2 && st + 1 < nstages)
            __builtin_amdgcn_s_waitcnt((kADma + kBDma) | (7 << 4) | (15 << 8));
        else
            __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
        // Every wave's DMAs have landed and stage st-1's buffer is free.  A bare
        // s_barrier: __syncthreads() would add a release fence that waits for
        // all outstanding DMAs, including the stage still in flight.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (st + kDist < nstages) issue_stage(st + kDist);
        const int buf = st % kBufs;
        const int8_t* abase = lds + buf * kAStage;
        const uint32_t* bbase = reinterpret_cast<const uint32_t*>(lds + kBufs * kAStage + buf * kBStage);
#pragma unroll
        for (int kk = 0; kk < BK / 64; ++kk) {
            i32x4 bfrag[T::FN];
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                int r;
                if (kGlu)
                    r = (j < T::FN / 2 ? 0 : BN / 2) + wn * (T::TN / 2) + (j % (T::FN / 2)) * 16 + (lane & 15);
                else
                    r = wn * T::TN + j * 16 + (lane & 15);
                const int piece = kk ^ b_swizzle<BK>(r);
                const uint32_t pw = bbase[r * (BK / 16) + piece * 4 + (lane >> 4)];
                int32_t c0, c1, c2, c3;
                decode_codes(pw, c0, c1, c2, c3);
                bfrag[j] = i32x4{c0, c1, c2, c3};
            }
#pragma unroll
            for (int i = 0; i < T::FM; ++i) {
                const int r = wm * T::TM + i * 16 + (lane & 15);
                const int chunk = (kk * 4 + (lane >> 4)) ^ (r % kALanes);
                const i32x4 afrag = *reinterpret_cast<const i32x4*>(abase + r * BK + 16 * chunk);
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afrag, bfrag[j], acc[i][j], 0, 0, 0);
            }
        }
    }

    const float gamma = a.gamma ? a.gamma[b] : 0.0f;
    const int64_t tok0 = (int64_t)b * M;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = m0 + wm * T::TM + i * 16 + 4 * (lane >> 4) + v;
            if (m >= M) continue;
            const int64_t t = tok0 + m;
            const int32_t sq = a.sumq[t];
            const float cs = EP == Epilogue::kI32 ? 0.0f : gamma / a.s[t];
            if (kGlu) {
#pragma unroll
                for (int j = 0; j < T::FN / 2; ++j) {
                    const int f = tn * (BN / 2) + wn * (T::TN / 2) + j * 16 + (lane & 15);
                    if (f < N) {
                        const float zg = rescale(acc[i][j][v] - sq, cs);
                        const float zu = rescale(acc[i][j + T::FN / 2][v] - sq, cs);
                        static_cast<uint16_t*>(a.out)[t * N + f] = glu_bf16(zg, zu);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < T::FN; ++j) {
                    const int n = tn * BN + wn * T::TN + j * 16 + (lane & 15);
                    if (n < N) {
                        const int32_t val = acc[i][j][v] - sq;
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

// ---------------------------------------------------------------------------
// Large-tile kernel on v_mfma_i32_32x32x32_i8.  On gfx950 this instruction
// sustains the int8 peak with a few independent accumulators per wave,
// while the 16x16x64 form needs many more chains than a tile can hold.
//   block 256 x 256, 8 waves as WM x WN, wave tile (256/WM) x (256/WN) of
//   32 x 32 fragments; lane l of A supplies row l%32, k = 16*(l/32)+0..15 of
//   a 32-wide k step; lane l of B supplies column l%32 at the same k, which
//   is exactly one packed 32-bit word; accumulator element v of lane l holds
//   D[(v%4) + 8*(v/4) + 4*(l/32)][l%32].
// K advances in 128-wide stages through four LDS buffers (all 160 KiB of
// the CU for 256 x 256 tiles), filled by DMA as above and taken in pairs
// with one barrier per pair.  Fragments are read and the packed words
// expanded one 32-wide step ahead of the MFMAs that use them; the barrier
// follows the MFMAs of the pair's last step, which run while the wave waits
// there.
// ---------------------------------------------------------------------------
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

template <int BM, int WM, int WN, Epilogue EP, int BN>
__global__ __launch_bounds__(WM * WN * kWave) void gemm_x32_kernel(ProductArgs a) {
    constexpr bool kGlu = EP == Epilogue::kGluBf16;
    constexpr bool kRes = EP == Epilogue::kResBf16;
    constexpr int kWavesPerBlock = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int kCols = kGlu ? BN / 2 : BN;
    static_assert(!kGlu || FN % 2 == 0, "GLU tiles pair gate and up fragments");
    constexpr int kAStage = BM * kBK;
    constexpr int kBStage = BN * (kBK / 4);
    constexpr int kADma = kAStage / 1024 / kWavesPerBlock;
    constexpr int kBDma = kBStage / 1024 / kWavesPerBlock;
    constexpr int kDma = kADma + kBDma;
    static_assert(kADma * 1024 * kWavesPerBlock == kAStage && kBDma * 1024 * kWavesPerBlock == kBStage,
                  "stage must split into whole 1 KiB DMA instructions per wave");
    constexpr int kXStages = 4;  // LDS buffers; stages run in pairs, one barrier per pair
    constexpr int KS = kBK / 32;  // 32-wide k steps per stage
    // One LDS object per stage buffer: with distinct objects the compiler can
    // tell that the DMA into one buffer does not feed the reads of another, so
    // it does not wait for every DMA in flight before each LDS read.
    __shared__ __attribute__((aligned(1024))) int8_t lds_a0[kAStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds_a1[kAStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds_a2[kAStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds_a3[kAStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds_b0[kBStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds_b1[kBStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds_b2[kBStage];
    __shared__ __attribute__((aligned(1024))) int8_t lds_b3[kBStage];

    const int M = a.M, N = a.N, K = a.K;
    const int nwords = K / 16;
    const int ntn = (N + kCols - 1) / kCols;
    const int per_problem = ntn * ((M + BM - 1) / BM);  // grid x = batch * per_problem
    const int f = xcd_tile(blockIdx.x, gridDim.x);
    const int b = f / per_problem;
    const int t = f - b * per_problem;
    const int tn = t % ntn;
    const int tm = t / ntn;
    const int m0 = tm * BM;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;

    const int64_t nrows = kGlu ? 2 * (int64_t)N : (int64_t)N;
    const int8_t* Q = a.q + (int64_t)b * M * K;
    const uint32_t* P = reinterpret_cast<const uint32_t*>(a.packed) + (int64_t)b * nrows * nwords;

    // DMA sources as 32-bit offsets from per-block bases.
    const int8_t* qbase = Q + (int64_t)m0 * K;
    uint32_t aoffs[kADma], boffs[kBDma];
#pragma unroll
    for (int i = 0; i < kADma; ++i) {
        const int r = (wave * kADma + i) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ (r & 7);
        // unsigned: (BM - 1) * K + 112 < 2^32 for K <= 2^24, where the
        // signed product would overflow from K > 2^31 / 255
        aoffs[i] = (uint32_t)(min(m0 + r, M - 1) - m0) * (uint32_t)K + 16u * (uint32_t)chunk;
    }
    const int64_t brow0 = b_row<BN, kGlu>(tn, 0, N);
#pragma unroll
    for (int i = 0; i < kBDma; ++i) {
        const int r = (wave * kBDma + i) * 32 + (lane >> 1);
        const int half = (lane & 1) ^ ((r >> 2) & 1);
        boffs[i] = (uint32_t)((b_row<BN, kGlu>(tn, r, N) - brow0) * nwords + 4 * half);
    }
    const uint32_t* pbase = P + brow0 * nwords;
    const int nstages = K / kBK;

    auto abuf = [&](auto bufc) -> int8_t* {
        constexpr int B_ = decltype(bufc)::value;
        return B_ == 0 ? lds_a0 : (B_ == 1 ? lds_a1 : (B_ == 2 ? lds_a2 : lds_a3));
    };
    auto bbuf = [&](auto bufc) -> int8_t* {
        constexpr int B_ = decltype(bufc)::value;
        return B_ == 0 ? lds_b0 : (B_ == 1 ? lds_b1 : (B_ == 2 ? lds_b2 : lds_b3));
    };
    // Byte offsets of B sources (relative to pbase) for the asm DMA.
#pragma unroll
    for (int i = 0; i < kBDma; ++i) boffs[i] *= 4;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // DMA d (0 <= d < kDma: first the A pieces, then the B pieces) of stage st.
    auto issue_dma = [&](auto bufc, int st, int d) {
        if (d < kADma) {
            const uint32_t abase = lds_address(abuf(bufc)) + wave_u * kADma * 1024;
            dma16(qbase + st * kBK, aoffs[d], abase + d * 1024);
        } else {
            const uint32_t bbase = lds_address(bbuf(bufc)) + wave_u * kBDma * 1024;
            dma16(reinterpret_cast<const int8_t*>(pbase) + st * (kBK / 4), boffs[d - kADma],
                  bbase + (d - kADma) * 1024);
        }
    };
    auto issue_stage = [&](auto bufc, int st) {
#pragma unroll
        for (int d = 0; d < kDma; ++d) issue_dma(bufc, st, d);
    };

    // Order of k inside a stage: step ks multiplies the 16-byte A chunks and
    // packed B words ks (lanes 0..31) and 4 + ks (lanes 32..63), so over a
    // stage a lane touches one 16-byte half of each B row only: it reads that
    // half once per stage (ds_read_b128) and expands one word per step.  The
    // integer sum does not depend on the order of k.
    // Fragment rows in LDS: A row wm*TM + i*32 + lane%32 (128 bytes a row;
    // chunk c stored at c ^ (row & 7)), B row per fragment j (32 bytes a row;
    // half h stored at h ^ ((row >> 2) & 1), so that the eight lanes of each
    // 128-byte read phase cover all 32 banks).
    const int arow0 = (wm * TM + (lane & 31)) * kBK;
    const int aswz = lane & 7;
    const int bhalf = ((lane >> 5) ^ ((lane >> 2) & 1)) * 16;
    int brow[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        if (kGlu)
            brow[j] = ((j < FN / 2 ? 0 : BN / 2) + wn * (TN / 2) + (j % (FN / 2)) * 32 + (lane & 31)) * 32;
        else
            brow[j] = (wn * TN + j * 32 + (lane & 31)) * 32;
    }

    struct Frags {
        i32x4 a[FM];
    };
    auto load_frags = [&](auto bufc, Frags& f, int ks) {
        const int8_t* abase = abuf(bufc);
        const int ach = ((ks + 4 * (lane >> 5)) ^ aswz) * 16;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f.a[i] = *reinterpret_cast<const i32x4*>(abase + arow0 + i * 32 * kBK + ach);
    };
    auto load_words = [&](auto bufc, uint4 (&wb)[FN]) {
        const int8_t* bbase = bbuf(bufc);
#pragma unroll
        for (int j = 0; j < FN; ++j) wb[j] = *reinterpret_cast<const uint4*>(bbase + brow[j] + bhalf);
    };
    auto word_of = [](const uint4& v, int ks) -> uint32_t {
        return ks == 0 ? v.x : (ks == 1 ? v.y : (ks == 2 ? v.z : v.w));
    };
    auto expand_one = [&](const uint4& v, int ks, i32x4& bq) {
        int32_t c0, c1, c2, c3;
        decode_codes(word_of(v, ks), c0, c1, c2, c3);
        // Pin the expanded codes in registers where they are computed: the
        // register allocator would otherwise recompute these cheap shifts
        // right before the MFMAs that read them, stalling their issue.
        asm volatile("" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
        bq = i32x4{c0, c1, c2, c3};
    };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = i32x16{};

    static_assert(BM <= WM * WN * kWave, "one row constant per thread");
    // Row constants are loaded first (they complete before the DMAs, which
    // the memory counter retires in order) and parked in LDS after the loop.
    int32_t my_sumq = 0;
    float my_s = 1.0f;
    if (tid < BM) {
        const int64_t tk = (int64_t)b * M + min(m0 + tid, M - 1);
        my_sumq = a.sumq[tk];
        if (EP != Epilogue::kI32) my_s = a.s[tk];
    }
    const float gamma = a.gamma ? a.gamma[b] : 0.0f;

    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    // Stages go in pairs (2j, 2j+1) with one barrier per pair, at the end of
    // the odd stage.  At that barrier both stages of the next pair have
    // landed; their DMAs are issued during the even stage of the current pair
    // into the two buffers the previous pair released, spread over its first
    // steps.  Stages 0 and 1 are loaded here.
    issue_stage(C0{}, 0);
    if (nstages > 1) issue_stage(C1{}, 1);
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    Frags cur, nxt;
    uint4 wb[FN];  // this stage's packed B words of the lane (one 16-byte half per row)
    i32x4 bcur[FN], bnxt[FN];
    load_words(C0{}, wb);
    load_frags(C0{}, cur, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) expand_one(wb[j], 0, bcur[j]);

    // One stage held in buffer BUF (= st % 4); BUF is even for the first
    // stage of a pair.
    auto run_stage = [&](auto bufc, int st) {
        constexpr int BUF = decltype(bufc)::value;
        constexpr bool kFirstOfPair = BUF % 2 == 0;
        using Next = std::integral_constant<int, (BUF + 1) % kXStages>;
        constexpr int kPairDma = 2 * kDma;
        constexpr int kPerStep = (kPairDma + KS - 2) / (KS - 1);
        // DMA d of the pair (stage st+2 for d < kDma, else st+3) into the
        // buffer two ahead of this one (released at the last barrier).
        auto pair_dma = [&](int d) {
            if (d < kDma) {
                if (st + 2 < nstages)
                    issue_dma(std::integral_constant<int, (BUF + 2) % kXStages>{}, st + 2, d);
            } else {
                if (st + 3 < nstages)
                    issue_dma(std::integral_constant<int, (BUF + 3) % kXStages>{}, st + 3, d - kDma);
            }
        };
        // The MFMAs of one step, with the expansion of the next step's B
        // words (words w of wsrc) slotted between them.
        auto mfma_step = [&](const uint4 (&wsrc)[FN], int w, bool expand_next) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int idx = 0; idx < FM * FN; ++idx) {
                const int i = idx / FN, j = idx % FN;
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[i], bcur[j], acc[i][j], 0, 0, 0);
                if (expand_next && idx < FN) expand_one(wsrc[idx], w, bnxt[idx]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks < KS - 1) {
                if (kFirstOfPair) {
#pragma unroll
                    for (int d = ks * kPerStep; d < (ks + 1) * kPerStep && d < kPairDma; ++d) pair_dma(d);
                }
                // the next step's A reads first, then this step's MFMAs
                load_frags(bufc, nxt, ks + 1);
                mfma_step(wb, ks + 1, true);
                cur = nxt;
#pragma unroll
                for (int j = 0; j < FN; ++j) bcur[j] = bnxt[j];
            } else if (kFirstOfPair) {
                // Last step of the first stage of a pair: stage st+1 landed
                // before the last barrier, so its first operands are read
                // ahead of this step's MFMAs, as within a stage (its B words
                // replace this stage's, which are all expanded by now).  When
                // st is the last stage these reads fetch a stale buffer that
                // nothing uses and no DMA writes; taking this path without a
                // test on st keeps the register allocation of the loop tight.
                load_words(Next{}, wb);
                load_frags(Next{}, nxt, 0);
                mfma_step(wb, 0, true);
                cur = nxt;
#pragma unroll
                for (int j = 0; j < FN; ++j) bcur[j] = bnxt[j];
            } else {
                // Last step of a pair: its MFMAs go first and keep the matrix
                // core busy while the wave waits at the barrier.  Once this
                // wave's DMAs and reads are done and every wave is there, the
                // next pair has landed and this pair's buffers are released;
                // then the first operands of stage st+1 are read and expanded.
                mfma_step(wb, 0, false);
                if (st + 1 < nstages) {
                    __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8));
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    load_words(Next{}, wb);
                    load_frags(Next{}, cur, 0);
#pragma unroll
                    for (int j = 0; j < FN; ++j) expand_one(wb[j], 0, bcur[j]);
                }
            }
        }
    };
    for (int st = 0; st < nstages; st += kXStages) {
        run_stage(C0{}, st);
        if (st + 1 < nstages) run_stage(C1{}, st + 1);
        if (st + 2 < nstages) run_stage(C2{}, st + 2);
        if (st + 3 < nstages) run_stage(C3{}, st + 3);
    }

    // Epilogue: subtract sum_k q, rescale (or form the GLU product), store.
    // The per-token constants of the block's rows (gamma / s, sum q) go to a
    // stage buffer that every wave has finished with, so that the epilogue
    // issues no global load between its stores (a load would wait for every
    // earlier store: one memory counter).
    __syncthreads();
    int32_t* row_sumq = reinterpret_cast<int32_t*>(lds_a0);
    float* row_scale = reinterpret_cast<float*>(lds_a0 + BM * sizeof(int32_t));
    if (tid < BM) {
        row_sumq[tid] = my_sumq;
        row_scale[tid] = EP == Epilogue::kI32 ? 0.0f : gamma / my_s;
    }
    __syncthreads();
    const int64_t tok0 = (int64_t)b * M;
    // Interior tiles (the common case) store without bounds tests, from a
    // block-uniform base plus a 32-bit lane offset; edge tiles test each row
    // and column.  Row r of the tile starts r * N elements after the base.
    const int col0 = tn * kCols;
    const bool interior = m0 + BM <= M && col0 + kCols <= N && (int64_t)BM * N <= ((int64_t)1 << 28);
    if (interior) {
        constexpr uint32_t kEsz = (kGlu || kRes) ? 2 : 4;  // bytes per output element
        char* const obase = static_cast<char*>(a.out) + ((tok0 + m0) * N + col0) * kEsz;
        const uint32_t lane_col = (kGlu ? wn * (TN / 2) : wn * TN) + (lane & 31);
        // The residual is loaded whole before the first store: loads and
        // stores share one in-order memory counter, so a load issued after
        // stores would wait for them.
        uint32_t resv[kRes ? FM : 1][kRes ? 16 : 1][kRes ? FN : 1];
        if constexpr (kRes) {
            const char* const rbase = reinterpret_cast<const char*>(a.res) + ((tok0 + m0) * N + col0) * kEsz;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = wm * TM + i * 32 + 4 * (lane >> 5) + (v & 3) + 8 * (v >> 2);
                    const uint32_t off = ((uint32_t)r * (uint32_t)N + lane_col) * kEsz;
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        resv[i][v][j] = *reinterpret_cast<const uint16_t*>(rbase + off + j * 32 * kEsz);
                }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r0 = wm * TM + i * 32 + 4 * (lane >> 5);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = r0 + (v & 3) + 8 * (v >> 2);
                const int32_t sq = row_sumq[r];
                const float cs = row_scale[r];
                // byte offset of this lane's first column in row r (< 2^31)
                const uint32_t off = ((uint32_t)r * (uint32_t)N + lane_col) * kEsz;
                if (kGlu) {
#pragma unroll
                    for (int j = 0; j < FN / 2; ++j) {
                        const float zg = rescale(acc[i][j][v] - sq, cs);
                        const float zu = rescale(acc[i][j + FN / 2][v] - sq, cs);
                        *reinterpret_cast<uint16_t*>(obase + off + j * 32 * kEsz) = glu_bf16(zg, zu);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int32_t val = acc[i][j][v] - sq;
                        if constexpr (EP == Epilogue::kI32) {
                            *reinterpret_cast<int32_t*>(obase + off + j * 32 * kEsz) = val;
                        } else if constexpr (kRes) {
                            // u = bf16(res + y), as the stand-alone residual pass forms it
                            *reinterpret_cast<uint16_t*>(obase + off + j * 32 * kEsz) = (uint16_t)f32_to_bf16_bits(
                                __uint_as_float(resv[i][v][j] << 16) + rescale(val, cs));
                        } else {
                            *reinterpret_cast<float*>(obase + off + j * 32 * kEsz) = rescale(val, cs);
                        }
                    }
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = wm * TM + i * 32 + (v & 3) + 8 * (v >> 2) + 4 * (lane >> 5);
            const int m = m0 + r;
            if (m >= M) continue;
            const int64_t tk = tok0 + m;
            const int32_t sq = row_sumq[r];
            const float cs = row_scale[r];
            if (kGlu) {
#pragma unroll
                for (int j = 0; j < FN / 2; ++j) {
                    const int f = tn * (BN / 2) + wn * (TN / 2) + j * 32 + (lane & 31);
                    if (f < N) {
                        const float zg = rescale(acc[i][j][v] - sq, cs);
                        const float zu = rescale(acc[i][j + FN / 2][v] - sq, cs);
                        static_cast<uint16_t*>(a.out)[tk * N + f] = glu_bf16(zg, zu);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = tn * BN + wn * TN + j * 32 + (lane & 31);
                    if (n < N) {
                        const int32_t val = acc[i][j][v] - sq;
                        if constexpr (EP == Epilogue::kI32)
                            static_cast<int32_t*>(a.out)[tk * N + n] = val;
                        else if constexpr (kRes)
                            static_cast<uint16_t*>(a.out)[tk * N + n] = (uint16_t)f32_to_bf16_bits(
                                __uint_as_float((uint32_t)a.res[tk * N + n] << 16) + rescale(val, cs));
                        else
                            static_cast<float*>(a.out)[tk * N + n] = rescale(val, cs);
                    }
                }
            }
        }
    }
}

template <int BM, int WM, int WN, Epilogue EP, int BN = 256>
hipError_t launch_x32(const ProductArgs& a, hipStream_t stream) {
    constexpr int kCols = EP == Epilogue::kGluBf16 ? BN / 2 : BN;
    const int64_t tiles = (int64_t)((a.N + kCols - 1) / kCols) * ((a.M + BM - 1) / BM);
    if (tiles * a.batch > 0x7fffffff) return hipErrorInvalidValue;  // one grid dimension
    const dim3 grid((unsigned)(tiles * a.batch));
    gemm_x32_kernel<BM, WM, WN, EP, BN><<<grid, WM * WN * kWave, 0, stream>>>(a);
    return hipGetLastError();
}

// Blocks of the x32 product with BM x BN tiles over all problems of the call.
template <int BM, int BN, Epilogue EP>
int64_t x32_tiles(const ProductArgs& a) {
    constexpr int kCols = EP == Epilogue::kGluBf16 ? BN / 2 : BN;
    return (int64_t)((a.N + kCols - 1) / kCols) * ((a.M + BM - 1) / BM) * a.batch;
}

// The x32 product with the largest tiles that still give more than 128
// blocks (half the compute units): 256 x 256 (8 waves of 64 x 128), else
// 128 x 256 (8 waves of 64 x 64), else 128 x 128 (4 waves of 64 x 64; two
// blocks fit a compute unit).  kResBf16 starts at 128 x 256: the 256-row
// tile's 128 residual values per lane would not fit beside its registers.
template <Epilogue EP>
hipError_t launch_x32_sized(const ProductArgs& a, hipStream_t stream) {
    if constexpr (EP != Epilogue::kResBf16) {
        // 256 x 256 tiles when they fill at least half the chip, unless
        // 128 x 256 tiles need fewer than 1.6 times as many rounds of 256
        // blocks (each of those tiles is half the work): a partial last
        // round of large tiles leaves compute units idle for a whole tile.
        const int64_t t256 = x32_tiles<256, 256, EP>(a);
        const int64_t r256 = (t256 + 255) / 256, r128 = (x32_tiles<128, 256, EP>(a) + 255) / 256;
        if (t256 > 128 && 10 * r128 >= 16 * r256) return launch_x32<256, 4, 2, EP>(a, stream);
    }
    if (x32_tiles<128, 256, EP>(a) > 128) return launch_x32<128, 2, 4, EP>(a, stream);
    return launch_x32<128, 2, 2, EP, 128>(a, stream);
}

template <int BM, int BN, int WM, int WN, Epilogue EP, int BK>
hipError_t launch_dma_tile(const ProductArgs& a, hipStream_t stream) {
    using T = Tile<BM, BN, WM, WN, EP>;
    const int64_t tiles = (int64_t)((a.N + T::kCols - 1) / T::kCols) * ((a.M + BM - 1) / BM);
    if (tiles * a.batch > 0x7fffffff) return hipErrorInvalidValue;  // one grid dimension
    const dim3 grid((unsigned)(tiles * a.batch));
    gemm_dma_kernel<BM, BN, WM, WN, EP, BK><<<grid, T::kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, Epilogue EP>
hipError_t launch_tile(const ProductArgs& a, hipStream_t stream) {
    using T = Tile<BM, BN, WM, WN, EP>;
    const int64_t tiles = (int64_t)((a.N + T::kCols - 1) / T::kCols) * ((a.M + BM - 1) / BM);
    if (tiles * a.batch > 0x7fffffff) return hipErrorInvalidValue;  // one grid dimension
    const dim3 grid((unsigned)(tiles * a.batch));
    gemm_kernel<BM, BN, WM, WN, EP><<<grid, T::kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

template <Epilogue EP>
hipError_t launch_ep(const ProductArgs& a, hipStream_t stream) {
    // Large problems: 256 x 256 tiles.  Small token counts: 64-token tiles so
    // that fewer padded rows are computed.
    const bool whole_stages = a.K % kBK == 0;
    if (a.M > 128) {
        // gemm_x32_kernel addresses a tile's weight rows as 32-bit byte
        // offsets from its first row; for the GLU the up rows sit N rows
        // further on.  Matrices too large for that take the 64-bit path.
        const int64_t span = (EP == Epilogue::kGluBf16 ? (int64_t)a.N : 0) + 256;
        const bool offs32 = span * (a.K / 4) < ((int64_t)1 << 32);
        if (!whole_stages || !offs32) return launch_tile<256, 256, 4, 2, EP>(a, stream);
        return launch_x32_sized<EP>(a, stream);
    }
    if (a.K % 256 == 0) return launch_dma_tile<64, 256, 1, 8, EP, 256>(a, stream);
    return whole_stages ? launch_dma_tile<64, 256, 1, 8, EP, 128>(a, stream)
                        : launch_tile<64, 256, 1, 8, EP>(a, stream);
}

}  // namespace

bool product_takes_residual(int M, int N, int K) {
    return M > 128 && K % kBK == 0 && (int64_t)256 * (K / 4) < ((int64_t)1 << 32) && N >= 1;
}

hipError_t launch_gemm_mfma(const ProductArgs& a, Epilogue ep, hipStream_t stream) {
    if (ep == Epilogue::kResBf16) {
        // The large-tile kernel with 64 x 64 wave tiles: each lane holds the
        // 64 residual values of its fragments before the stores.
        if (!product_takes_residual(a.M, a.N, a.K) || a.res == nullptr) return hipErrorInvalidValue;
        return launch_x32_sized<Epilogue::kResBf16>(a, stream);
    }
    if (skinny_supported(a.M, a.K, ep)) return launch_skinny(a, ep, stream);
    switch (ep) {
        case Epilogue::kF32: return launch_ep<Epilogue::kF32>(a, stream);
        case Epilogue::kI32: return launch_ep<Epilogue::kI32>(a, stream);
        case Epilogue::kGluBf16: return launch_ep<Epilogue::kGluBf16>(a, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace bl
