// pack.hip -- absmean ternarisation of fp32 weights into the 2-bit format.
//
// [datacamp, "Thay MatMul bằng các phép toán tam phân"]: the weight matrix is
// scaled by its mean absolute value (gamma) and every element rounded to the
// nearest of -1, 0, +1.  Readings: one gamma per matrix, sum of |W| in fp64,
// w = clip(rint(W / (gamma + 1e-5)), -1, 1) with an IEEE fp32 division.
//
// Kernels (all HBM-bound; W is read twice, packed written once), each over a
// batch of matrices of one shape along grid y (one gamma per matrix):
//   gamma_partial  -- fixed-range fp64 partial sums of |W| (one per block)
//   gamma_final    -- one block per matrix sums its partials in a fixed order
//   ternarize_pack -- one thread per 16-weight group -> one packed word
#include "device_common.h"
#include "launch.h"

namespace bl {
namespace {

constexpr int kPackThreads = 256;
constexpr int kMaxPartials = 1024;

__global__ __launch_bounds__(kPackThreads) void gamma_partial_kernel(const float* __restrict__ W,
                                                                     int64_t total, int64_t chunk,
                                                                     double* __restrict__ partial) {
    __shared__ double scratch[kPackThreads / kWave];
    W += (int64_t)blockIdx.y * total;  // matrix blockIdx.y of the batch
    const int64_t begin = (int64_t)blockIdx.x * chunk;
    const int64_t end = begin + chunk < total ? begin + chunk : total;
    constexpr int64_t kStep = 4 * kPackThreads;
    double acc = 0.0;
    // chunk and total are multiples of 4, so float4 loads stay aligned.  Four
    // loads are issued before their sums; the order of the sums is that of
    // the one-load loop.
    auto add = [&](const float4 v) {
        acc += (double)fabsf(v.x);
        acc += (double)fabsf(v.y);
        acc += (double)fabsf(v.z);
        acc += (double)fabsf(v.w);
    };
    int64_t i = begin + 4 * (int64_t)threadIdx.x;
    for (; i + 3 * kStep < end; i += 4 * kStep) {
        const float4 v0 = *reinterpret_cast<const float4*>(W + i);
        const float4 v1 = *reinterpret_cast<const float4*>(W + i + kStep);
        const float4 v2 = *reinterpret_cast<const float4*>(W + i + 2 * kStep);
        const float4 v3 = *reinterpret_cast<const float4*>(W + i + 3 * kStep);
        add(v0);
        add(v1);
        add(v2);
        add(v3);
    }
    for (; i < end; i += kStep) add(*reinterpret_cast<const float4*>(W + i));
    acc = block_sum(acc, scratch);
    if (threadIdx.x == 0) partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = acc;
}

// One block per matrix of the batch.
__global__ __launch_bounds__(kPackThreads) void gamma_final_kernel(const double* __restrict__ partial,
                                                                   int nparts, int64_t total,
                                                                   float* __restrict__ gamma) {
    __shared__ double scratch[kPackThreads / kWave];
    partial += (int64_t)blockIdx.x * nparts;
    double acc = 0.0;
    for (int i = threadIdx.x; i < nparts; i += kPackThreads) acc += partial[i];
    acc = block_sum(acc, scratch);
    if (threadIdx.x == 0) gamma[blockIdx.x] = (float)(acc / (double)total);
}

__global__ __launch_bounds__(kPackThreads) void ternarize_pack_kernel(const float* __restrict__ W,
                                                                      int64_t nwords,
                                                                      const float* __restrict__ gamma,
                                                                      uint32_t* __restrict__ packed) {
    const int64_t i = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (i >= nwords) return;
    const int64_t b = blockIdx.y;  // matrix of the batch
    const float d = gamma[b] + 1e-5f;
    const float4* src = reinterpret_cast<const float4*>(W + 16 * (b * nwords + i));
    float v[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float4 f = src[c];
        v[4 * c + 0] = f.x;
        v[4 * c + 1] = f.y;
        v[4 * c + 2] = f.z;
        v[4 * c + 3] = f.w;
    }
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float t = rintf(v[j] / d);  // IEEE division (no fast-math), ties to even
        t = fminf(fmaxf(t, -1.0f), 1.0f);
        const uint32_t code = (uint32_t)((int)t + 1);
        word |= code << (8 * (j & 3) + 2 * (j >> 2));
    }
    packed[b * nwords + i] = word;
}

__global__ __launch_bounds__(kPackThreads) void unpack_kernel(const uint32_t* __restrict__ packed,
                                                              int64_t nwords, int8_t* __restrict__ w) {
    const int64_t i = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (i >= nwords) return;
    int32_t c[4];
    decode_codes(packed[i], c[0], c[1], c[2], c[3]);
    uint4 out;
    // code - 1 in every byte without borrows: set bit 7, subtract, flip bit 7.
    out.x = (((uint32_t)c[0] | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
    out.y = (((uint32_t)c[1] | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
    out.z = (((uint32_t)c[2] | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
    out.w = (((uint32_t)c[3] | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
    *reinterpret_cast<uint4*>(w + 16 * i) = out;
}

inline unsigned grid_for(int64_t n, int per_block) { return (unsigned)((n + per_block - 1) / per_block); }

}  // namespace

int gamma_partials(int64_t total) {
    int64_t n = (total + 16 * kPackThreads - 1) / (16 * kPackThreads);
    if (n < 1) n = 1;
    return n > kMaxPartials ? kMaxPartials : (int)n;
}

hipError_t launch_gamma(const float* W, int64_t total, int64_t batch, double* partial, float* gamma,
                        hipStream_t stream) {
    const int nparts = gamma_partials(total);
    const int64_t chunk = round_up((total + nparts - 1) / nparts, 4);
    gamma_partial_kernel<<<dim3((unsigned)nparts, (unsigned)batch), kPackThreads, 0, stream>>>(W, total, chunk,
                                                                                              partial);
    gamma_final_kernel<<<(unsigned)batch, kPackThreads, 0, stream>>>(partial, nparts, total, gamma);
    return hipGetLastError();
}

hipError_t launch_ternarize_pack(const float* W, int64_t total, int64_t batch, const float* gamma,
                                 uint32_t* packed, hipStream_t stream) {
    const int64_t nwords = total / 16;
    ternarize_pack_kernel<<<dim3(grid_for(nwords, kPackThreads), (unsigned)batch), kPackThreads, 0, stream>>>(
        W, nwords, gamma, packed);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* packed, int64_t nwords, int8_t* w, hipStream_t stream) {
    unpack_kernel<<<grid_for(nwords, kPackThreads), kPackThreads, 0, stream>>>(packed, nwords, w);
    return hipGetLastError();
}

}  // namespace bl
