// skinny.hip -- the ternary product for a few tokens (5..16) on the int8
// matrix cores, streaming the packed weights from HBM into registers.
//
// With M <= 16 tokens the product is bound by reading the packed weights
// (N*K/4 bytes against 2*M*N*K operations), and a 16 x 16 x 64 MFMA covers
// all tokens of 16 weight rows at once ([jiqizhixin, "具有三值权重的 MatMul-free
// 密集层"]: the ternary product is an add/subtract accumulation; on the
// matrix cores it is the same integer sum, exactly):
//   * the block stages the int8 codes q of its M tokens in LDS once, rows
//     padded by 16 bytes so that the rows a read phase touches fall in
//     distinct banks; MFMA rows past M take zeros;
//   * each wave owns 16 * U weight rows and walks K in 256-wide chunks:
//     lane l loads 16 bytes (64 weights) of row l % 16, the quarter l / 16 of
//     the chunk, with plain vector loads double-buffered a few chunks ahead
//     (each load instruction thus reads 64 contiguous bytes of 16 rows, which
//     streams at about 5.3 TB/s, below the 512-byte runs of the one-token
//     kernel: the main limit of this kernel);
//   * step t (0..3) of a chunk multiplies word t of that quarter, i.e. the
//     chunk's k in 16 * (4 * (l / 16) + t) + 0..15, against the codes of the
//     same k read from LDS: MFMA lane l of A is token l % 16, of B weight row
//     l % 16, and both take k-slice l / 16, so each step sums 64 distinct k
//     and the four steps cover the chunk once (the order of k does not
//     change the integer sum);
//   * the accumulator of lane l holds tokens 4 * (l / 16) + v of weight row
//     l % 16 over the whole K, so no cross-lane reduction is needed; the
//     epilogue subtracts sum_k q (the weights are stored as w + 1) and
//     rescales ([datacamp, "Các thành phần lõi: MLGRU và GLU"]: scaled
//     ternary accumulation).
#include <algorithm>

#include "epilogue.h"
#include "quant_row.h"

namespace bl {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSkinnyThreads = 256;
constexpr int kSkinnyWaves = kSkinnyThreads / kWave;
constexpr int kSkinnyU = 2;      // 16-row weight groups per wave
constexpr int kChunkK = 256;     // k per chunk (64 packed bytes of a row)
constexpr int kGroup = 4;        // chunks per load group (double-buffered)

template <Epilogue EP>
__global__ __launch_bounds__(kSkinnyThreads) void skinny_kernel(ProductArgs a) {
    extern __shared__ int8_t qs[];  // [M][K + 16] int8 codes
    const int M = a.M, N = a.N, K = a.K;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane & 15, g = lane >> 4;
    const int pitch = K + 16;
    const int nchunks = K / kChunkK;
    const int ngroups = (nchunks + kGroup - 1) / kGroup;
    const int64_t row_bytes = K / 4;
    const int n0 = (blockIdx.x * kSkinnyWaves + wave) * 16 * kSkinnyU;

    // This lane's 16-byte quarter of each chunk of its weight rows (clamped
    // rows past N are read but never stored).
    const uint8_t* wrow[kSkinnyU];
#pragma unroll
    for (int u = 0; u < kSkinnyU; ++u)
        wrow[u] = a.packed + ((int64_t)b * N + min(n0 + 16 * u + r, N - 1)) * row_bytes + 16 * g;

    uint4 wv[2][kGroup][kSkinnyU];
    auto load_group = [&](int grp, uint4 (&dst)[kGroup][kSkinnyU]) {
#pragma unroll
        for (int c = 0; c < kGroup; ++c) {
            const int chunk = grp * kGroup + c;
#pragma unroll
            for (int u = 0; u < kSkinnyU; ++u) {
                dst[c][u] = make_uint4(0u, 0u, 0u, 0u);
                if (chunk < nchunks)
                    dst[c][u] = load_stream16(reinterpret_cast<const uint32_t*>(wrow[u] + 64 * chunk));
            }
        }
    };
    // The first weights are requested before the codes are staged, so HBM
    // is busy from the start.
    load_group(0, wv[0]);

    const int8_t* Q = a.q + (int64_t)b * M * K;
    const int kq = K / 16;  // 16-byte pieces per row
    for (int i = threadIdx.x; i < M * kq; i += kSkinnyThreads) {
        const int row = i / kq, piece = i - row * kq;
        *reinterpret_cast<int4*>(qs + row * pitch + 16 * piece) =
            *reinterpret_cast<const int4*>(Q + (int64_t)row * K + 16 * piece);
    }
    __syncthreads();

    i32x4 acc[kSkinnyU];
#pragma unroll
    for (int u = 0; u < kSkinnyU; ++u) acc[u] = i32x4{0, 0, 0, 0};
    const bool token = r < M;  // MFMA row r is a real token
    const int8_t* qrow = qs + min(r, M - 1) * pitch + 64 * g;

    auto compute_group = [&](int grp, const uint4 (&src)[kGroup][kSkinnyU]) {
#pragma unroll
        for (int c = 0; c < kGroup; ++c) {
            const int chunk = grp * kGroup + c;
            if (chunk >= nchunks) break;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                i32x4 av = *reinterpret_cast<const i32x4*>(qrow + kChunkK * chunk + 16 * t);
                if (!token) av = i32x4{0, 0, 0, 0};
#pragma unroll
                for (int u = 0; u < kSkinnyU; ++u) {
                    const uint32_t w = t == 0 ? src[c][u].x : (t == 1 ? src[c][u].y : (t == 2 ? src[c][u].z : src[c][u].w));
                    int32_t c0, c1, c2, c3;
                    decode_codes(w, c0, c1, c2, c3);
                    acc[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, i32x4{c0, c1, c2, c3}, acc[u], 0, 0, 0);
                }
            }
        }
    };
    for (int grp = 0; grp < ngroups; grp += 2) {
        if (grp + 1 < ngroups) load_group(grp + 1, wv[1]);
        compute_group(grp, wv[0]);
        if (grp + 1 < ngroups) {
            if (grp + 2 < ngroups) load_group(grp + 2, wv[0]);
            compute_group(grp + 1, wv[1]);
        }
    }

    // Epilogue: lane l holds tokens 4g + v of weight row n0 + 16u + r.
    const float gamma = EP == Epilogue::kI32 ? 0.0f : a.gamma[b];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m >= M) continue;
        const int64_t tk = (int64_t)b * M + m;
        const int32_t sq = a.sumq[tk];
        const float cs = EP == Epilogue::kI32 ? 0.0f : gamma / a.s[tk];
#pragma unroll
        for (int u = 0; u < kSkinnyU; ++u) {
            const int n = n0 + 16 * u + r;
            if (n >= N) continue;
            const int32_t val = acc[u][v] - sq;
            if (EP == Epilogue::kI32)
                static_cast<int32_t*>(a.out)[tk * N + n] = val;
            else
                static_cast<float*>(a.out)[tk * N + n] = rescale(val, cs);
        }
    }
}

// Same product for K <= 2048 (K % 512 == 0) with the weights read in runs of
// 128 contiguous bytes: a load instruction covers 8 rows x 128 bytes (lane l:
// row l / 8, bytes 16 * (l % 8) of a 512-wide k pair), which streams like
// the one-token kernel's long runs.  The wave writes each 16-row group into
// its own LDS buffer (row pitch K/4 + 16, so that writes and the quarter
// reads below are bank-conflict free) and reads it back in the MFMA layout;
// the buffer is private to the wave, so no barrier is needed.  The codes of
// the tokens for all of K stay in registers (NCH 256-wide chunks, at most
// 128 VGPRs), read once per block.  Blocks take runs of rows as in the
// kernel above, and each wave keeps the next group's loads in flight while
// it multiplies the current one.
template <int NCH, Epilogue EP>
__global__ __launch_bounds__(kSkinnyThreads) void skinny_runs_kernel(ProductArgs a, int rows_per_block) {
    extern __shared__ int8_t wbuf[];  // per wave: [16][K/4 + 16] packed bytes
    constexpr int kRowBytes = NCH * 64;
    constexpr int kPitch = kRowBytes + 16;
    constexpr int kPairs = NCH / 2;       // 128-byte runs per row
    constexpr int kLoads = 2 * kPairs;    // 16-byte loads per lane per group
    const int M = a.M, N = a.N;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane & 15, g = lane >> 4;
    int8_t* buf = wbuf + wave * 16 * kPitch;
    const int row0 = blockIdx.x * rows_per_block;
    const int rows = min(rows_per_block, N - row0);
    const int ngroups = (rows + 15) / 16;
    const uint8_t* P = a.packed + (int64_t)b * N * kRowBytes;

    // load k of a group: half h = k / kPairs (rows 8h..8h+7), pair p = k % kPairs
    auto load_group = [&](int grp, uint4 (&dst)[kLoads]) {
        const int rbase = row0 + 16 * (wave + kSkinnyWaves * grp);
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const int h = k / kPairs, p = k % kPairs;
            const int row = min(rbase + 8 * h + (lane >> 3), N - 1);
            dst[k] = load_stream16(reinterpret_cast<const uint32_t*>(P + (int64_t)row * kRowBytes + 128 * p +
                                                                     16 * (lane & 7)));
        }
    };
    const int my_groups = ngroups > wave ? (ngroups - wave + kSkinnyWaves - 1) / kSkinnyWaves : 0;
    uint4 wv[kLoads];
    if (my_groups > 0) load_group(0, wv);

    // Codes of token r for this lane's k-slices: chunk c, step t -> bytes
    // 256c + 64g + 16t (zeros for rows past M).
    i32x4 aq[NCH][4];
    const int8_t* Q = a.q + ((int64_t)b * M + min(r, M - 1)) * (NCH * 256) + 64 * g;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            aq[c][t] = i32x4{0, 0, 0, 0};
            if (r < M) aq[c][t] = *reinterpret_cast<const i32x4*>(Q + 256 * c + 16 * t);
        }
    const float gamma = EP == Epilogue::kI32 ? 0.0f : a.gamma[b];
    int32_t sq[4];
    float cs[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t tk = (int64_t)b * M + min(4 * g + v, M - 1);
        sq[v] = a.sumq[tk];
        cs[v] = EP == Epilogue::kI32 ? 0.0f : gamma / a.s[tk];
    }

    for (int grp = 0; grp < my_groups; ++grp) {
        // stage this group in the wave's buffer, then request the next one
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const int h = k / kPairs, p = k % kPairs;
            *reinterpret_cast<uint4*>(buf + (8 * h + (lane >> 3)) * kPitch + 128 * p + 16 * (lane & 7)) = wv[k];
        }
        if (grp + 1 < my_groups) load_group(grp + 1, wv);
        i32x4 acc = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint4 wq = *reinterpret_cast<const uint4*>(buf + r * kPitch + 64 * c + 16 * g);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t w = t == 0 ? wq.x : (t == 1 ? wq.y : (t == 2 ? wq.z : wq.w));
                int32_t c0, c1, c2, c3;
                decode_codes(w, c0, c1, c2, c3);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[c][t], i32x4{c0, c1, c2, c3}, acc, 0, 0, 0);
            }
        }
        const int n = row0 + 16 * (wave + kSkinnyWaves * grp) + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * g + v;
            if (m < M && n < N) {
                const int64_t tk = (int64_t)b * M + m;
                const int32_t val = acc[v] - sq[v];
                if (EP == Epilogue::kI32)
                    static_cast<int32_t*>(a.out)[tk * N + n] = val;
                else
                    static_cast<float*>(a.out)[tk * N + n] = rescale(val, cs[v]);
            }
        }
    }
}

// Same product for K = 1024 * NCHW (K = 2048 or 4096): the four waves of a
// block split K into quarters and walk the same 16-row groups together, so
// a wave holds the codes of a quarter of K only (NCHW 256-wide chunks) and
// keeps D groups of weights in flight instead of one. Each load instruction
// still covers 8 rows x 128 contiguous bytes (lane l: row l / 8, bytes
// 16 * (l % 8) of a 128-byte run of the wave's quarter); the group is
// reshaped through the wave's own LDS buffer as above. Each wave leaves its
// partial sums of a group in LDS; after every batch of four groups one
// barrier, then wave w adds the four quarters of group w of the batch
// (integer sums, exact in any order) and stores them. Partial sums are
// double-buffered by batch, so the barrier of batch i + 1 also orders the
// reads of batch i before their overwrite. The output writes, though only
// M * 4 bytes per 512-byte weight row, cost the stream more than their size:
// reads mixed with writes run slower on HBM than reads alone, whatever the
// store width or order.
constexpr int kSplitBatch = 4;  // 16-row groups per reduction: one per wave
constexpr int kSplitPartBytes = 2 * kSplitBatch * kSkinnyWaves * kWave * 16;  // partial-sum region

// FUSED: one launch for the whole layer, as the one-token decode kernel.
// Each block first quantises its problem's M token rows itself (wave w takes
// rows w, w + 4, ..., with the wave-per-row arithmetic of the streaming
// quantiser) into the partial-sum region of LDS, which is free until the
// first batch is added (M * K <= 32 KiB). The weight loads of the first
// groups are issued before, so HBM is busy from the start, and no codes are
// written to or read from HBM. Otherwise the codes, scales and sums come
// from an activation stage.
template <int NCHW, int D, Epilogue EP, bool FUSED>
__global__ __launch_bounds__(kSkinnyThreads) void skinny_split_kernel(ProductArgs a, DecodeArgs d,
                                                                      int rows_per_block) {
    static_assert(kSkinnyWaves == 4 && kSplitBatch == kSkinnyWaves, "four K quarters, one group per wave to add");
    static_assert((D > kSplitBatch ? D : kSplitBatch) % D == 0 && (D > kSplitBatch ? D : kSplitBatch) % kSplitBatch == 0,
                  "whole rings and batches per loop trip");
    constexpr int kSliceBytes = NCHW * 64;  // packed bytes of a row in one quarter of K
    constexpr int kPitch = kSliceBytes + 16;
    constexpr int kRuns = kSliceBytes / 128;
    constexpr int kLoads = 2 * kRuns;       // 16-byte loads per lane per group
    constexpr int K = 4 * NCHW * 256;
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    __shared__ float s_scale[kSkinnyMaxM];
    __shared__ int32_t s_sumq[kSkinnyMaxM];
    const int M = FUSED ? d.M : a.M, N = FUSED ? d.N : a.N;
    const uint8_t* const packed = FUSED ? d.packed : a.packed;
    const int64_t row_bytes = 4 * kSliceBytes;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane & 15, g = lane >> 4;
    int8_t* buf = smem + wave * 16 * kPitch;
    // partial sums: [2 batches][kSplitBatch groups][4 quarters][64 lanes] x int4
    i32x4* part = reinterpret_cast<i32x4*>(smem + kSkinnyWaves * 16 * kPitch);
    const int row0 = blockIdx.x * rows_per_block;
    const int rows = min(rows_per_block, N - row0);
    const int last_row = row0 + rows - 1;
    const int ngroups = (rows + 15) / 16;
    constexpr int kRing = D > kSplitBatch ? D : kSplitBatch;  // groups per loop trip (static ring slots)
    const int niters = (ngroups + kRing - 1) / kRing;
    const uint8_t* P = packed + (int64_t)b * N * row_bytes + wave * kSliceBytes;

    // Loads of group grp; rows past the block's last are clamped to it (read
    // again from cache, never stored).
    auto load_group = [&](int grp, uint4 (&dst)[kLoads]) {
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const int h = k / kRuns, p = k % kRuns;
            const int row = min(row0 + 16 * grp + 8 * h + (lane >> 3), last_row);
            dst[k] = load_stream16(reinterpret_cast<const uint32_t*>(P + (int64_t)row * row_bytes + 128 * p +
                                                                     16 * (lane & 7)));
        }
    };
    uint4 wv[D][kLoads];
#pragma unroll
    for (int s = 0; s < D; ++s) load_group(s, wv[s]);

    // The problem's codes [M][K], scales and code sums.
    const int8_t* qsrc;
    const float* ssrc;
    const int32_t* sqsrc;
    if constexpr (FUSED) {
        constexpr int CPL = K / 8 / kWave;  // 8-element chunks per lane
        int8_t* qlds = reinterpret_cast<int8_t*>(part);
        const uint16_t* X = d.x + (int64_t)b * M * K;
        const float* G = d.g + (int64_t)b * d.g_stride;
        auto g_chunk = [&](int c, float4& lo, float4& hi) {
            const int idx = lane + c * kWave;
            lo = *reinterpret_cast<const float4*>(G + 8 * idx);
            hi = *reinterpret_cast<const float4*>(G + 8 * idx + 4);
        };
        for (int m = wave; m < M; m += kSkinnyWaves) {
            uint4 xc[CPL];
            load_x_row<CPL, true>(X + (int64_t)m * K, lane, K / 8, xc);
            quant_row_regs<CPL, true>(xc, g_chunk, m, lane, K, d.eps, qlds, s_scale, s_sumq);
        }
        __syncthreads();
        qsrc = qlds;
        ssrc = s_scale;
        sqsrc = s_sumq;
    } else {
        qsrc = a.q + (int64_t)b * M * K;
        ssrc = a.s + (int64_t)b * M;
        sqsrc = a.sumq + (int64_t)b * M;
    }
    // Codes of token r for this lane's k-slices of the wave's quarter:
    // chunk c, step t -> k = K/4 * wave + 256c + 64g + 16t (zeros past M).
    i32x4 aq[NCHW][4];
    const int8_t* Q = qsrc + (int64_t)min(r, M - 1) * K + wave * (NCHW * 256) + 64 * g;
#pragma unroll
    for (int c = 0; c < NCHW; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            aq[c][t] = i32x4{0, 0, 0, 0};
            if (r < M) aq[c][t] = *reinterpret_cast<const i32x4*>(Q + 256 * c + 16 * t);
        }
    const float gamma = EP == Epilogue::kI32 ? 0.0f : (FUSED ? d.gamma : a.gamma)[b];
    int32_t sq[4];
    float cs[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int mm = min(4 * g + v, M - 1);
        sq[v] = sqsrc[mm];
        cs[v] = EP == Epilogue::kI32 ? 0.0f : gamma / ssrc[mm];
    }
    // the codes in LDS are read before the partial sums overwrite them
    if constexpr (FUSED) __syncthreads();

    for (int it = 0; it < niters; ++it) {
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            const int s = j % D;
            const int grp = it * kRing + j;
            i32x4* pb = part + ((grp / kSplitBatch) & 1) * (kSplitBatch * kSkinnyWaves * kWave);
#pragma unroll
            for (int k = 0; k < kLoads; ++k) {
                const int h = k / kRuns, p = k % kRuns;
                *reinterpret_cast<uint4*>(buf + (8 * h + (lane >> 3)) * kPitch + 128 * p + 16 * (lane & 7)) = wv[s][k];
            }
            load_group(grp + D, wv[s]);
            i32x4 acc = i32x4{0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < NCHW; ++c) {
                const uint4 wq = *reinterpret_cast<const uint4*>(buf + r * kPitch + 64 * c + 16 * g);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t w = t == 0 ? wq.x : (t == 1 ? wq.y : (t == 2 ? wq.z : wq.w));
                    int32_t c0, c1, c2, c3;
                    decode_codes(w, c0, c1, c2, c3);
                    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[c][t], i32x4{c0, c1, c2, c3}, acc, 0, 0, 0);
                }
            }
            pb[((j % kSplitBatch) * kSkinnyWaves + wave) * kWave + lane] = acc;
            if ((j + 1) % kSplitBatch != 0) continue;
            // the batch is complete: wave w adds the quarters of its group w
            __syncthreads();
            const int rgrp = grp + 1 - kSplitBatch + wave;
            if (rgrp < ngroups) {
                const i32x4* src = pb + wave * kSkinnyWaves * kWave + lane;
                const i32x4 sum = src[0] + src[kWave] + src[2 * kWave] + src[3 * kWave];
                const int n = row0 + 16 * rgrp + r;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 4 * g + v;
                    if (m < M && n <= last_row) {
                        const int64_t tk = (int64_t)b * M + m;
                        const int32_t val = sum[v] - sq[v];
                        void* out = FUSED ? d.out : a.out;
                        if (EP == Epilogue::kI32)
                            static_cast<int32_t*>(out)[tk * N + n] = val;
                        else
                            static_cast<float*>(out)[tk * N + n] = rescale(val, cs[v]);
                    }
                }
            }
        }
    }
}

template <int NCHW, int D, Epilogue EP, bool FUSED>
hipError_t launch_split(const ProductArgs& a, const DecodeArgs& d, hipStream_t stream) {
    const int64_t N = FUSED ? d.N : a.N, batch = FUSED ? d.batch : a.batch;
    const int64_t rpb = balanced_rows_per_block(N, batch, (int64_t)16 * kSplitBatch);
    const dim3 grid((unsigned)((N + rpb - 1) / rpb), (unsigned)batch);
    const size_t lds = (size_t)kSkinnyWaves * 16 * (NCHW * 64 + 16) + kSplitPartBytes;
    skinny_split_kernel<NCHW, D, EP, FUSED><<<grid, kSkinnyThreads, lds, stream>>>(a, d, (int)rpb);
    return hipGetLastError();
}

template <Epilogue EP>
hipError_t launch_split_ep(const ProductArgs& a, hipStream_t stream) {
    switch (a.K) {
        // weight groups in flight per wave: 8 at K = 2048 (3 waves per SIMD
        // fit), 4 at K = 4096 (the codes of a quarter take twice the registers)
        case 2048: return launch_split<2, 8, EP, false>(a, DecodeArgs{}, stream);
        case 4096: return launch_split<4, 4, EP, false>(a, DecodeArgs{}, stream);
    }
    return hipErrorInvalidValue;
}

template <int NCH, Epilogue EP>
hipError_t launch_runs(const ProductArgs& a, hipStream_t stream) {
    const int64_t rpb = balanced_rows_per_block(a.N, a.batch, (int64_t)kSkinnyWaves * 16);
    const dim3 grid((unsigned)((a.N + rpb - 1) / rpb), (unsigned)a.batch);
    const size_t lds = (size_t)kSkinnyWaves * 16 * (NCH * 64 + 16);
    skinny_runs_kernel<NCH, EP><<<grid, kSkinnyThreads, lds, stream>>>(a, (int)rpb);
    return hipGetLastError();
}

template <Epilogue EP>
hipError_t launch_runs_ep(const ProductArgs& a, hipStream_t stream) {
    switch (a.K / kChunkK) {
        case 2: return launch_runs<2, EP>(a, stream);
        case 4: return launch_runs<4, EP>(a, stream);
        case 6: return launch_runs<6, EP>(a, stream);
        case 8: return launch_runs<8, EP>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_few_supported(int M, int K) {
    return M >= 1 && M <= kSkinnyMaxM && (K == 2048 || K == 4096) && M * K <= kSplitPartBytes;
}

hipError_t launch_decode_few(const DecodeArgs& d, hipStream_t stream) {
    if (!decode_few_supported(d.M, d.K)) return hipErrorInvalidValue;
    return d.K == 2048 ? launch_split<2, 8, Epilogue::kF32, true>(ProductArgs{}, d, stream)
                       : launch_split<4, 4, Epilogue::kF32, true>(ProductArgs{}, d, stream);
}

bool skinny_supported(int M, int K, Epilogue ep) {
    return M >= 1 && M <= kSkinnyMaxM && K % kChunkK == 0 && ep != Epilogue::kGluBf16 &&
           (size_t)M * (K + 16) <= 64 * 1024;
}

hipError_t launch_skinny(const ProductArgs& a, Epilogue ep, hipStream_t stream) {
    if (!skinny_supported(a.M, a.K, ep)) return hipErrorInvalidValue;
    if (a.K == 2048 || a.K == 4096)
        return ep == Epilogue::kI32 ? launch_split_ep<Epilogue::kI32>(a, stream)
                                    : launch_split_ep<Epilogue::kF32>(a, stream);
    if (a.K % 512 == 0 && a.K <= 2048)
        return ep == Epilogue::kI32 ? launch_runs_ep<Epilogue::kI32>(a, stream)
                                    : launch_runs_ep<Epilogue::kF32>(a, stream);
    constexpr int kRowsPerBlock = kSkinnyWaves * 16 * kSkinnyU;
    const dim3 grid((unsigned)((a.N + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)a.batch);
    const size_t lds = (size_t)a.M * (a.K + 16);
    if (ep == Epilogue::kI32)
        skinny_kernel<Epilogue::kI32><<<grid, kSkinnyThreads, lds, stream>>>(a);
    else
        skinny_kernel<Epilogue::kF32><<<grid, kSkinnyThreads, lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace bl
