// mlgru.hip -- the MLGRU token mixer's recurrence and the layer's residual
// stream (gfx950).
//
// [datacamp, "Các thành phần lõi: MLGRU và GLU"]: the MLGRU takes a
// sequence token by token, mixing the current token into a hidden state
// through element-wise operations and gates with values in (0, 1);
// [jiqizhixin, "MatMul-free 语言模型架构"]: a ternary RNN of element-wise
// products and accumulation built on the GRU; [ld246, "线性操作的引入"]:
// element-wise operations in place of the GRU's matrix products.  With the
// gates taken from the token alone (one BitLinear gives z = z_f | z_c | z_g
// per token), the recurrence per channel is linear in the state:
//   f = sigmoid(z_f), c = SiLU(z_c), g = sigmoid(z_g),
//   h_t = f h_{t-1} + (1 - f) c,       p_t = bf16(g h_t).
// It is bound by HBM (12 bytes of z read and 2 bytes of p written per token
// and channel), and sequential in t only.  So that a single sequence still
// fills the GPU, the tokens are cut into chunks that run in parallel:
//   A. each chunk j < last computes its summary over its tokens, the
//      product of its forget gates A_j and its end state H_j from h = 0;
//   M. the states entering the chunks, S_0 = h_0 and S_{j+1} = A_j S_j +
//      H_j, from a parallel prefix over the chunks (one wave per channel
//      pair; the maps h -> A h + H compose associatively);
//   B. each chunk reruns its tokens from S_j, writing p_t; the last chunk
//      writes the final state.
// The linear map h -> f h + (1 - f) c composes exactly as A and H do, so the
// chunked order gives the same states up to fp32 rounding.  One chunk (many
// channels, or one token) runs B alone.
//
// Layouts: z fp32 [B][T][3d] (rows of a token: z_f | z_c | z_g), state fp32
// [B][d] (h_0 in, h_T out), p bf16 [B][T][d]; a thread owns channels
// 2 c2 and 2 c2 + 1 (c2 = (b * d + n) / 2, d even).
#include <algorithm>

#include "epilogue.h"

namespace bl {
namespace {

constexpr int kScanThreads = 256;
constexpr int kMaxChunks = 2 * kWave;      // two per lane of the chunk-start scan
constexpr int64_t kTargetThreads = 131072;  // pairs of channels: about 8 waves per CU over 256 CUs
constexpr int64_t kSinglePassThreads = 32768;

// One thread owns two adjacent channels (d is even), so each wave moves
// 512 contiguous bytes per token and per stream.
struct ScanArgs {
    const float* z;
    float* state;
    uint16_t* p;
    float2* A;  // [nc - 1][C/2]
    float2* H;  // [nc - 1][C/2]
    float2* S;  // [nc][C/2]
    int B, T, d, L, nc;
};

// Token range of chunk j.
__device__ __forceinline__ void chunk_range(const ScanArgs& a, int j, int& t0, int& t1) {
    t0 = j * a.L;
    t1 = min(a.T, t0 + a.L);
}

// The loads of kU tokens are issued before their state updates: only the
// updates form a chain.
constexpr int kU = 16;

__device__ __forceinline__ void step(float zf, float zc, float& h, float& prod) {
    float f, omf;
    sigmoid_pair(zf, f, omf);
    h = fmaf(f, h, omf * silu_f32(zc));
    prod *= f;
}

// Pass A: summaries of chunks 0 .. nc-2.
__global__ __launch_bounds__(kScanThreads) void mlgru_summary_kernel(ScanArgs a) {
    const int64_t C2 = (int64_t)a.B * a.d / 2;
    const int64_t c2 = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;
    const int j = blockIdx.y;
    if (c2 >= C2) return;
    const int b = (int)(2 * c2 / a.d), n = (int)(2 * c2 % a.d);
    const int64_t d3 = 3 * (int64_t)a.d;
    int t0, t1;
    chunk_range(a, j, t0, t1);
    const float* zb = a.z + ((int64_t)b * a.T) * d3 + n;
    float2 prod = make_float2(1.0f, 1.0f), h = make_float2(0.0f, 0.0f);
    for (int t = t0; t < t1; t += kU) {
        float2 zf[kU], zc[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int tt = min(t + u, t1 - 1);
            zf[u] = *reinterpret_cast<const float2*>(zb + (int64_t)tt * d3);
            zc[u] = *reinterpret_cast<const float2*>(zb + (int64_t)tt * d3 + a.d);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (t + u < t1) {
                step(zf[u].x, zc[u].x, h.x, prod.x);
                step(zf[u].y, zc[u].y, h.y, prod.y);
            }
        }
    }
    a.A[(int64_t)j * C2 + c2] = prod;
    a.H[(int64_t)j * C2 + c2] = h;
}

// Pass M: the state entering each chunk, S_0 = h_0 and S_{j+1} = A_j S_j +
// H_j.  Chunk j's summary is the affine map h -> A_j h + H_j, and maps
// compose associatively ((A', H') after (A, H) is (A' A, A' H + H')), so one
// wave per channel pair scans them in parallel: lane l composes chunks 2l
// and 2l + 1, an inclusive scan over the lanes gives the map of chunks
// 0 .. 2l + 1, and lane l applies the map of the chunks before its own to h_0.
__global__ __launch_bounds__(kScanThreads) void mlgru_chunk_start_kernel(ScanArgs a) {
    const int64_t C2 = (int64_t)a.B * a.d / 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t c2 = (int64_t)blockIdx.x * (kScanThreads / kWave) + threadIdx.x / kWave;
    if (c2 >= C2) return;  // whole waves leave together
    const int j0 = 2 * lane, j1 = 2 * lane + 1, last = a.nc - 1;  // summaries exist for j < last
    float2 A0 = make_float2(1.0f, 1.0f), H0 = make_float2(0.0f, 0.0f), A1 = A0, H1 = H0;
    if (j0 < last) {
        A0 = a.A[(int64_t)j0 * C2 + c2];
        H0 = a.H[(int64_t)j0 * C2 + c2];
    }
    if (j1 < last) {
        A1 = a.A[(int64_t)j1 * C2 + c2];
        H1 = a.H[(int64_t)j1 * C2 + c2];
    }
    // this lane's pair: chunk j1 after chunk j0
    float2 Ap = make_float2(A1.x * A0.x, A1.y * A0.y);
    float2 Hp = make_float2(fmaf(A1.x, H0.x, H1.x), fmaf(A1.y, H0.y, H1.y));
    // inclusive scan over lanes: lane l ends with the map of chunks 0 .. j1
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float ax = __shfl_up(Ap.x, off, kWave), ay = __shfl_up(Ap.y, off, kWave);
        const float hx = __shfl_up(Hp.x, off, kWave), hy = __shfl_up(Hp.y, off, kWave);
        if (lane >= off) {
            Hp = make_float2(fmaf(Ap.x, hx, Hp.x), fmaf(Ap.y, hy, Hp.y));
            Ap = make_float2(Ap.x * ax, Ap.y * ay);
        }
    }
    // map of the chunks before j0 (identity for lane 0), applied to h_0
    float ex_ax = __shfl_up(Ap.x, 1, kWave), ex_ay = __shfl_up(Ap.y, 1, kWave);
    float ex_hx = __shfl_up(Hp.x, 1, kWave), ex_hy = __shfl_up(Hp.y, 1, kWave);
    if (lane == 0) {
        ex_ax = ex_ay = 1.0f;
        ex_hx = ex_hy = 0.0f;
    }
    const float2 h0 = reinterpret_cast<const float2*>(a.state)[c2];
    const float2 s0 = make_float2(fmaf(ex_ax, h0.x, ex_hx), fmaf(ex_ay, h0.y, ex_hy));
    if (j0 < a.nc) a.S[(int64_t)j0 * C2 + c2] = s0;
    if (j1 < a.nc) a.S[(int64_t)j1 * C2 + c2] = make_float2(fmaf(A0.x, s0.x, H0.x), fmaf(A0.y, s0.y, H0.y));
}

// Pass B: the recurrence over each chunk from its start state, writing p.
// With a single chunk the start state is h_0 itself (S unused).
__global__ __launch_bounds__(kScanThreads) void mlgru_scan_kernel(ScanArgs a) {
    const int64_t C2 = (int64_t)a.B * a.d / 2;
    const int64_t c2 = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;
    const int j = blockIdx.y;
    if (c2 >= C2) return;
    const int b = (int)(2 * c2 / a.d), n = (int)(2 * c2 % a.d);
    const int64_t d3 = 3 * (int64_t)a.d;
    int t0, t1;
    chunk_range(a, j, t0, t1);
    const float* zb = a.z + ((int64_t)b * a.T) * d3 + n;
    uint32_t* pb = reinterpret_cast<uint32_t*>(a.p + ((int64_t)b * a.T) * a.d + n);
    float2 h = a.nc == 1 ? reinterpret_cast<const float2*>(a.state)[c2] : a.S[(int64_t)j * C2 + c2];
    for (int t = t0; t < t1; t += kU) {
        float2 zf[kU], zc[kU], zg[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int tt = min(t + u, t1 - 1);
            zf[u] = *reinterpret_cast<const float2*>(zb + (int64_t)tt * d3);
            zc[u] = *reinterpret_cast<const float2*>(zb + (int64_t)tt * d3 + a.d);
            zg[u] = *reinterpret_cast<const float2*>(zb + (int64_t)tt * d3 + 2 * a.d);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (t + u < t1) {
                const uint32_t p0 = mlgru_token(zf[u].x, zc[u].x, zg[u].x, h.x);
                const uint32_t p1 = mlgru_token(zf[u].y, zc[u].y, zg[u].y, h.y);
                pb[(int64_t)(t + u) * (a.d / 2)] = p0 | (p1 << 16);
            }
        }
    }
    if (j == a.nc - 1) reinterpret_cast<float2*>(a.state)[c2] = h;
}

// Residual stream: out = bf16(float(x) + y), 8 elements per thread.
__global__ __launch_bounds__(256) void residual_bf16_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ y,
                                                             uint16_t* __restrict__ out, int64_t n8) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const uint4 xv = reinterpret_cast<const uint4*>(x)[i];
    const float4 y0 = reinterpret_cast<const float4*>(y)[2 * i];
    const float4 y1 = reinterpret_cast<const float4*>(y)[2 * i + 1];
    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
    const float ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = f32_to_bf16_bits(bf16_lo(xs[k]) + ys[2 * k]);
        const uint32_t hi = f32_to_bf16_bits(bf16_hi(xs[k]) + ys[2 * k + 1]);
        o[k] = lo | (hi << 16);
    }
    reinterpret_cast<uint4*>(out)[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

struct ScanPlan {
    int L, nc;
};

// Chunks: one when the channel pairs alone fill the GPU; otherwise enough
// for about kTargetThreads threads (at most kMaxChunks, two per lane of pass
// M's scan), never shorter than one token.
ScanPlan scan_plan(int64_t B, int64_t T, int64_t d) {
    const int64_t C2 = B * d / 2;
    // With 2 waves per CU or more a single pass streams well (it reads z
    // once, where chunking reads z_f and z_c twice).
    if (C2 >= kSinglePassThreads) return ScanPlan{(int)T, 1};
    int64_t nc = (kTargetThreads + C2 - 1) / C2;
    nc = std::max<int64_t>(1, std::min<int64_t>({nc, (int64_t)kMaxChunks, T}));
    const int64_t L = (T + nc - 1) / nc;
    nc = (T + L - 1) / L;
    return ScanPlan{(int)L, (int)nc};
}

}  // namespace

size_t mlgru_scan_workspace_bytes(int64_t B, int64_t T, int64_t d) {
    const ScanPlan pl = scan_plan(B, T, d);
    if (pl.nc == 1) return 0;
    const int64_t C = B * d;
    return (size_t)(2 * round_up((int64_t)(pl.nc - 1) * C * 4, 256) + round_up((int64_t)pl.nc * C * 4, 256));
}

hipError_t launch_mlgru_scan(const float* z, int64_t B, int64_t T, int64_t d, float* state,
                             uint16_t* p, void* ws, hipStream_t stream) {
    const ScanPlan pl = scan_plan(B, T, d);
    const int64_t C = B * d;
    ScanArgs a;
    a.z = z;
    a.state = state;
    a.p = p;
    a.B = (int)B;
    a.T = (int)T;
    a.d = (int)d;
    a.L = pl.L;
    a.nc = pl.nc;
    a.A = a.H = a.S = nullptr;
    const unsigned cblocks = (unsigned)((C / 2 + kScanThreads - 1) / kScanThreads);
    if (pl.nc > 1) {
        char* w = static_cast<char*>(ws);
        a.A = reinterpret_cast<float2*>(w);
        w += round_up((int64_t)(pl.nc - 1) * C * 4, 256);
        a.H = reinterpret_cast<float2*>(w);
        w += round_up((int64_t)(pl.nc - 1) * C * 4, 256);
        a.S = reinterpret_cast<float2*>(w);
        mlgru_summary_kernel<<<dim3(cblocks, (unsigned)(pl.nc - 1)), kScanThreads, 0, stream>>>(a);
        const unsigned mblocks = (unsigned)((C / 2 + kScanThreads / kWave - 1) / (kScanThreads / kWave));
        mlgru_chunk_start_kernel<<<dim3(mblocks), kScanThreads, 0, stream>>>(a);
    }
    mlgru_scan_kernel<<<dim3(cblocks, (unsigned)pl.nc), kScanThreads, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_residual_bf16(const uint16_t* x, const float* y, uint16_t* out, int64_t n,
                                hipStream_t stream) {
    const int64_t n8 = n / 8;  // n % 16 == 0 (rows of d elements, d % 16 == 0)
    if (n8 == 0) return hipSuccess;
    residual_bf16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, stream>>>(x, y, out, n8);
    return hipGetLastError();
}

}  // namespace bl
