// launch.h -- host-side launchers of the BitLinear kernels (library internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Compute units of the current device, queried once per device.
int device_cu_count();
// Rows per block, a multiple of `gran`, for `batch` problems of N rows each,
// when a block stays inside one problem: equal blocks, split so that the
// busiest compute unit has the fewest rows.
int64_t balanced_rows_per_block(int64_t N, int64_t batch, int64_t gran);

// Per-token activation stage produced by the quantisation kernel:
// q int8 [rows][K] (row stride K), s fp32 [rows], sumq int32 [rows] = sum_k q.
struct ActStage {
    int8_t* q;
    float* s;
    int32_t* sumq;
};

// Workspace layout of one activation stage (each part 256-byte aligned).
size_t act_stage_bytes(int64_t rows, int64_t K);
ActStage act_stage_carve(void* base, int64_t rows, int64_t K);

// --- weights ---------------------------------------------------------------
// Number of fp64 partial sums the gamma reduction uses for `total` weights.
int gamma_partials(int64_t total);
// `batch` matrices of `total` elements each, back to back; partial holds
// gamma_partials(total) sums per matrix and gamma one value per matrix.
hipError_t launch_gamma(const float* W, int64_t total, int64_t batch, double* partial, float* gamma,
                        hipStream_t stream);
hipError_t launch_ternarize_pack(const float* W, int64_t total, int64_t batch, const float* gamma,
                                 uint32_t* packed, hipStream_t stream);
hipError_t launch_unpack(const uint32_t* packed, int64_t nwords, int8_t* w, hipStream_t stream);

// --- activations -------------------------------------------------------------
// RMSNorm + absmax int8 over `rows` rows of length K.  Row r uses the RMSNorm
// weight vector g + (r / rows_per_g) * K (rows_per_g = rows for one shared
// vector).
hipError_t launch_quant(const uint16_t* x, const float* g, int64_t rows, int64_t rows_per_g,
                        int K, float eps, ActStage out, hipStream_t stream);
// sumq[r] = sum_k q[r][k] for caller-provided codes.
hipError_t launch_row_sums(const int8_t* q, int64_t rows, int K, int32_t* sumq,
                           hipStream_t stream);

// --- ternary product -----------------------------------------------------------
enum class Epilogue {
    kF32,        // y[m][n] = float(acc) * (gamma / s[m])
    kI32,        // acc[m][n]
    kGluBf16,    // h[m][f] = bf16(silu(z[m][f]) * z[m][F + f]), z = float(acc) * gamma / s
    kResBf16,    // u[m][n] = bf16(res[m][n] + y[m][n]): a residual added (fused decode kernel, and
                 // the large-tile product where product_takes_residual() holds)
    kMlgruStep,  // one MLGRU token per row m (its own sequence): z = y over rows n, d + n, 2d + n,
                 // state[m][n] updated, p[m][n] = bf16(g h) (fused decode kernel only)
};

// One problem, or `batch` problems of the same shape laid out back to back:
// problem b uses q rows [b*M, (b+1)*M), packed + b*Nrows*K/4, gamma + b and
// out + b*M*Ncols, where Nrows = N (or 2F for the GLU) and Ncols = N (or F).
struct ProductArgs {
    const int8_t* q;
    const float* s;
    const int32_t* sumq;
    const uint8_t* packed;
    const float* gamma;
    int M;      // tokens per problem
    int N;      // output columns per problem (F for the GLU epilogue)
    int K;
    int batch;
    void* out;  // float*, int32_t* or uint16_t* by epilogue
    const uint16_t* res = nullptr;  // kResBf16: bf16 [batch][M][N], the same layout as out
};

// Whether launch_gemm_mfma takes Epilogue::kResBf16 for this shape (the
// large-tile kernel: more than 128 tokens, K a multiple of 128).
bool product_takes_residual(int M, int N, int K);

hipError_t launch_gemv(const ProductArgs& a, Epilogue ep, hipStream_t stream);
hipError_t launch_gemm_mfma(const ProductArgs& a, Epilogue ep, hipStream_t stream);

// Few-token product on the matrix cores (weights streamed into registers):
// M <= kSkinnyMaxM, K % 256 == 0, F32 or I32 epilogue.
constexpr int kSkinnyMaxM = 16;
bool skinny_supported(int M, int K, Epilogue ep);
hipError_t launch_skinny(const ProductArgs& a, Epilogue ep, hipStream_t stream);

// Largest M the GEMV kernel takes.
constexpr int kGemvMaxM = 8;

// Fused decode (quantisation + product in one kernel) for M <= kDecodeMaxM:
// x bf16 [batch][M][K], g fp32 at g + b * g_stride (g_stride 0 = shared),
// packed [batch][Nrows][K/4], gamma [batch], out [batch][M][N].
constexpr int kDecodeMaxM = 4;
struct DecodeArgs {
    const uint16_t* x;
    const float* g;
    int64_t g_stride;
    const uint8_t* packed;
    const float* gamma;
    int M, N, K;
    int batch;
    float eps;
    void* out;
    const uint16_t* res = nullptr;  // kResBf16: bf16 [batch][M][N]
    float* state = nullptr;         // kMlgruStep: fp32 [batch][M][N], read and written
};
bool decode_supported(int M, int K);
hipError_t launch_decode(const DecodeArgs& a, Epilogue ep, hipStream_t stream);
// The same for 5..16 tokens (fp32 epilogue): quantisation fused into the
// K-split few-token product; K = 2048 or 4096 with M * K <= 32 KiB.
bool decode_few_supported(int M, int K);
hipError_t launch_decode_few(const DecodeArgs& a, hipStream_t stream);

// --- MLGRU token mixer and the layer's residual stream ---------------------------
// Recurrence of the token mixer from its pre-activations z fp32 [B][T][3d]
// (z_f | z_c | z_g per token): p bf16 [B][T][d]; state fp32 [B][d] holds h_0
// on entry and h_T on return.  ws: mlgru_scan_workspace_bytes(B, T, d)
// bytes, 256-byte aligned (0 when one chunk suffices).
size_t mlgru_scan_workspace_bytes(int64_t B, int64_t T, int64_t d);
hipError_t launch_mlgru_scan(const float* z, int64_t B, int64_t T, int64_t d, float* state,
                             uint16_t* p, void* ws, hipStream_t stream);
// out = bf16(float(x) + y) over n elements (n % 16 == 0).
hipError_t launch_residual_bf16(const uint16_t* x, const float* y, uint16_t* out, int64_t n,
                                hipStream_t stream);

// --- backward (straight-through estimator) -------------------------------------
// x bf16 [M][K], g fp32 [K], packed [N][K/4], gamma (device scalar), dy fp32
// [M][N] -> dx fp32 [M][K], dg fp32 [K], dW fp32 [N][K]; ws of
// backward_workspace_bytes(M, N, K) bytes, 256-byte aligned.
struct BackwardArgs {
    const uint16_t* x;
    const float* g;
    const uint8_t* packed;
    const float* gamma;
    const float* dy;
    int64_t M, N, K;
    float eps;
    float* dx;
    float* dg;
    float* dW;
    void* ws;
};
size_t backward_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);

}  // namespace bl
