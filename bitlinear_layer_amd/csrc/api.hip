// api.hip -- the C ABI declared in include/bitlinear.h: argument checks,
// workspace carving and kernel dispatch.  No allocation, no host sync.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "bitlinear.h"
#include "launch.h"

// Scratch of bitlinear_forward_noalloc (the activation stage: int8 codes,
// per-token scales and code sums), resident on every GPU the library runs
// on from module load until the process ends.  In host code this name is a
// host-side stand-in, not a device address: the address of each device's
// copy comes from hipGetSymbolAddress (noalloc_scratch below), and only that
// address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[BITLINEAR_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return BITLINEAR_OK;
    return fail(BITLINEAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // any one matrix, in elements
constexpr int64_t kMaxBatch = 65535;             // grid y limit

#define CHECK(cond, status, ...)                   \
    do {                                           \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

#define CHECK_SCALAR(p)                                                                    \
    do {                                                                                   \
        CHECK((p) != nullptr && aligned((p), 4), BITLINEAR_ERR_INVALID_ARG,                \
              "%s must be a non-NULL 4-byte aligned device pointer", #p);                  \
    } while (0)

#define CHECK_PTR(p)                                                                      \
    do {                                                                                  \
        CHECK((p) != nullptr, BITLINEAR_ERR_INVALID_ARG, "%s must not be NULL", #p);      \
        CHECK(aligned((p), 16), BITLINEAR_ERR_INVALID_ARG, "%s must be 16-byte aligned", #p); \
    } while (0)

int check_k(int64_t K, const char* name) {
    CHECK(K > 0, BITLINEAR_ERR_INVALID_ARG, "%s must be > 0 (got %lld)", name, (long long)K);
    CHECK(K % 16 == 0, BITLINEAR_ERR_INVALID_ARG, "%s must be a multiple of 16 (got %lld)", name,
          (long long)K);
    CHECK(K <= BITLINEAR_MAX_K, BITLINEAR_ERR_INVALID_ARG, "%s exceeds BITLINEAR_MAX_K", name);
    return BITLINEAR_OK;
}

int check_rows(int64_t R, const char* name) {
    CHECK(R >= 0, BITLINEAR_ERR_INVALID_ARG, "%s must be >= 0 (got %lld)", name, (long long)R);
    CHECK(R <= BITLINEAR_MAX_DIM, BITLINEAR_ERR_INVALID_ARG, "%s exceeds BITLINEAR_MAX_DIM", name);
    return BITLINEAR_OK;
}

int check_eps(float eps) {
    CHECK(isfinite(eps) && eps > 0.0f, BITLINEAR_ERR_INVALID_ARG, "eps must be finite and > 0");
    return BITLINEAR_OK;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return BITLINEAR_OK;
    CHECK(ws != nullptr, BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    CHECK(aligned(ws, 256), BITLINEAR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    CHECK(ws_bytes >= need, BITLINEAR_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes,
          need);
    return BITLINEAR_OK;
}

#define TRY(expr)                        \
    do {                                 \
        int _st = (expr);                \
        if (_st != BITLINEAR_OK) return _st; \
    } while (0)

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Kernel for the product from a quantised stage: the GEMV up to 4 tokens,
// the MFMA tiles above (or whatever the caller forces).
bool use_gemv(int64_t M, int kernel) {
    if (kernel == BITLINEAR_KERNEL_GEMV) return true;
    if (kernel == BITLINEAR_KERNEL_MFMA) return false;
    return M <= 4;
}

// Whether a whole layer can run as one fused kernel (quantisation inside):
// the one-token decode kernel for M <= 4 (either epilogue), the K-split
// few-token kernel for 5..16 tokens (fp32 epilogue only).
bool fused_supported(int64_t M, int64_t K, bool glu) {
    return bl::decode_supported((int)M, (int)K) || (!glu && bl::decode_few_supported((int)M, (int)K));
}

// Whether a full forward runs as a single fused kernel.
bool use_decode(int64_t M, int64_t K, int kernel, bool glu) {
    if (kernel == BITLINEAR_KERNEL_DECODE) return true;
    return kernel == BITLINEAR_KERNEL_AUTO && fused_supported(M, K, glu);
}

int check_kernel(int kernel, int64_t M, int64_t K, bool fused_allowed, bool glu = false) {
    CHECK(kernel == BITLINEAR_KERNEL_AUTO || kernel == BITLINEAR_KERNEL_GEMV ||
              kernel == BITLINEAR_KERNEL_MFMA || (fused_allowed && kernel == BITLINEAR_KERNEL_DECODE),
          BITLINEAR_ERR_INVALID_ARG, "kernel choice %d not available here", kernel);
    CHECK(kernel != BITLINEAR_KERNEL_GEMV || M <= bl::kGemvMaxM, BITLINEAR_ERR_INVALID_ARG,
          "the GEMV kernel takes M <= %d (got %lld)", bl::kGemvMaxM, (long long)M);
    CHECK(kernel != BITLINEAR_KERNEL_DECODE || M == 0 || fused_supported(M, K, glu),
          BITLINEAR_ERR_INVALID_ARG, "the fused decode kernel does not take M=%lld, K=%lld",
          (long long)M, (long long)K);
    return BITLINEAR_OK;
}

int run_decode(const uint16_t* x, const float* g, int64_t g_stride, const uint8_t* packed,
               const float* gamma, int64_t B, int64_t M, int64_t N, int64_t K, float eps, void* out,
               bl::Epilogue ep, hipStream_t stream, const uint16_t* res = nullptr, float* state = nullptr) {
    bl::DecodeArgs d;
    d.res = res;
    d.state = state;
    d.x = x;
    d.g = g;
    d.g_stride = g_stride;
    d.packed = packed;
    d.gamma = gamma;
    d.M = (int)M;
    d.N = (int)N;
    d.K = (int)K;
    d.batch = (int)B;
    d.eps = eps;
    d.out = out;
    // fused_supported() has admitted (M, K, ep) for one of the two kernels
    if (bl::decode_supported(d.M, d.K)) return hip_status(bl::launch_decode(d, ep, stream), "fused decode launch");
    return hip_status(bl::launch_decode_few(d, stream), "fused few-token launch");
}

// Ternary product + epilogue for `batch` problems whose activation stage is
// already in `act`.
int run_product(const bl::ActStage& act, const uint8_t* packed, const float* gamma, int64_t M,
                int64_t N, int64_t K, int64_t batch, void* out, bl::Epilogue ep, int kernel,
                hipStream_t stream, const uint16_t* res = nullptr) {
    bl::ProductArgs a;
    a.res = res;
    a.q = act.q;
    a.s = act.s;
    a.sumq = act.sumq;
    a.packed = packed;
    a.gamma = gamma;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.batch = (int)batch;
    a.out = out;
    hipError_t e = use_gemv(M, kernel) ? bl::launch_gemv(a, ep, stream)
                                       : bl::launch_gemm_mfma(a, ep, stream);
    return hip_status(e, "ternary product launch");
}

int forward_impl(const uint16_t* x, const float* rms_weight, const uint8_t* packed,
                 const float* gamma, int64_t B, int64_t M, int64_t N, int64_t K, float eps,
                 float* y, void* ws, size_t ws_bytes, void* stream, int kernel) {
    TRY(check_rows(M, "M"));
    TRY(check_rows(N, "N"));
    TRY(check_k(K, "K"));
    TRY(check_eps(eps));
    CHECK(B >= 1 && B <= kMaxBatch, BITLINEAR_ERR_INVALID_ARG, "batch must be in [1, %lld]",
          (long long)kMaxBatch);
    CHECK(B * M <= BITLINEAR_MAX_DIM, BITLINEAR_ERR_INVALID_ARG, "B*M exceeds BITLINEAR_MAX_DIM");
    CHECK(M * K <= kMaxElems && N * K <= kMaxElems && M * N <= kMaxElems,
          BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    TRY(check_kernel(kernel, M, K, true, false));
    if (M == 0 || N == 0) return BITLINEAR_OK;
    CHECK_PTR(x);
    CHECK_PTR(rms_weight);
    CHECK_PTR(packed);
    CHECK_SCALAR(gamma);
    CHECK_PTR(y);
    const size_t need = bl::act_stage_bytes(B * M, K);
    TRY(check_ws(ws, ws_bytes, need));
    hipStream_t st = as_stream(stream);
    if (use_decode(M, K, kernel, false))
        return run_decode(x, rms_weight, B > 1 ? K : 0, packed, gamma, B, M, N, K, eps, y,
                          bl::Epilogue::kF32, st);
    bl::ActStage act = bl::act_stage_carve(ws, B * M, K);
    TRY(hip_status(bl::launch_quant(x, rms_weight, B * M, M, (int)K, eps, act, st), "quantise launch"));
    return run_product(act, packed, gamma, M, N, K, B, y, bl::Epilogue::kF32, kernel, st);
}

// B independent GLU mixers of one shape (B = 1 for bitlinear_glu_forward).
// With res (bf16 [B][M][D]) the mixer adds its output to res and writes the
// bf16 sum to out_res instead of y (fused into the down projection when
// that runs on the one-token decode kernel or on the large-tile product;
// y is then scratch).
int glu_impl(const uint16_t* x, const float* rms_w_gu, const uint8_t* packed_gu,
             const float* gamma_gu, const float* rms_w_down, const uint8_t* packed_down,
             const float* gamma_down, int64_t B, int64_t M, int64_t D, int64_t F, float eps,
             float* y, void* ws, size_t ws_bytes, void* stream, const uint16_t* res = nullptr,
             uint16_t* out_res = nullptr) {
    TRY(check_rows(M, "M"));
    TRY(check_k(D, "D"));
    TRY(check_k(F, "F"));
    TRY(check_eps(eps));
    CHECK(B >= 1 && B <= kMaxBatch, BITLINEAR_ERR_INVALID_ARG, "batch must be in [1, %lld]",
          (long long)kMaxBatch);
    CHECK(B * M <= BITLINEAR_MAX_DIM, BITLINEAR_ERR_INVALID_ARG, "B*M exceeds BITLINEAR_MAX_DIM");
    CHECK(B * M * D <= kMaxElems && 2 * F * D <= kMaxElems && B * M * F <= kMaxElems,
          BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    if (M == 0) return BITLINEAR_OK;
    CHECK_PTR(x);
    CHECK_PTR(rms_w_gu);
    CHECK_PTR(packed_gu);
    CHECK_SCALAR(gamma_gu);
    CHECK_PTR(rms_w_down);
    CHECK_PTR(packed_down);
    CHECK_SCALAR(gamma_down);
    CHECK_PTR(y);
    const int64_t rows = B * M;
    TRY(check_ws(ws, ws_bytes, bitlinear_glu_workspace_bytes(rows, D, F)));
    hipStream_t st = as_stream(stream);
    char* base = static_cast<char*>(ws);
    bl::ActStage act_x = bl::act_stage_carve(base, rows, D);
    base += bl::act_stage_bytes(rows, D);
    uint16_t* h = reinterpret_cast<uint16_t*>(base);
    base += bl::round_up(rows * F * 2, 256);
    bl::ActStage act_h = bl::act_stage_carve(base, rows, F);
    if (use_decode(M, D, BITLINEAR_KERNEL_AUTO, true)) {
        TRY(run_decode(x, rms_w_gu, B > 1 ? D : 0, packed_gu, gamma_gu, B, M, F, D, eps, h,
                       bl::Epilogue::kGluBf16, st));
    } else {
        TRY(hip_status(bl::launch_quant(x, rms_w_gu, rows, M, (int)D, eps, act_x, st), "quantise launch"));
        TRY(run_product(act_x, packed_gu, gamma_gu, M, F, D, B, h, bl::Epilogue::kGluBf16,
                        BITLINEAR_KERNEL_AUTO, st));
    }
    if (res != nullptr && bl::decode_supported((int)M, (int)F))
        return run_decode(h, rms_w_down, B > 1 ? F : 0, packed_down, gamma_down, B, M, D, F, eps, out_res,
                          bl::Epilogue::kResBf16, st, res);
    if (res != nullptr && B == 1 && bl::product_takes_residual((int)M, (int)D, (int)F)) {
        // the residual added in the down projection's epilogue: u is read and
        // out written in bf16, and no fp32 output passes through HBM
        TRY(hip_status(bl::launch_quant(h, rms_w_down, rows, M, (int)F, eps, act_h, st), "quantise launch"));
        return run_product(act_h, packed_down, gamma_down, M, D, F, 1, out_res, bl::Epilogue::kResBf16,
                           BITLINEAR_KERNEL_AUTO, st, res);
    }
    if (use_decode(M, F, BITLINEAR_KERNEL_AUTO, false)) {
        TRY(run_decode(h, rms_w_down, B > 1 ? F : 0, packed_down, gamma_down, B, M, D, F, eps, y,
                       bl::Epilogue::kF32, st));
    } else {
        TRY(hip_status(bl::launch_quant(h, rms_w_down, rows, M, (int)F, eps, act_h, st), "quantise launch"));
        TRY(run_product(act_h, packed_down, gamma_down, M, D, F, B, y, bl::Epilogue::kF32,
                        BITLINEAR_KERNEL_AUTO, st));
    }
    if (res != nullptr)
        return hip_status(bl::launch_residual_bf16(res, y, out_res, rows * D, st), "residual launch");
    return BITLINEAR_OK;
}

// B matrices of one shape, back to back (B = 1 for bitlinear_pack_weights).
int pack_impl(const float* W, int64_t B, int64_t N, int64_t K, uint8_t* packed, float* gamma,
              void* ws, size_t ws_bytes, void* stream) {
    TRY(check_k(K, "K"));
    CHECK(N >= 1 && N <= BITLINEAR_MAX_DIM, BITLINEAR_ERR_INVALID_ARG, "N must be in [1, MAX_DIM]");
    CHECK(B >= 1 && B <= kMaxBatch, BITLINEAR_ERR_INVALID_ARG, "batch must be in [1, %lld]",
          (long long)kMaxBatch);
    CHECK(N * K <= kMaxElems && B * N * K / 16 <= kMaxElems, BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    CHECK_PTR(W);
    CHECK_PTR(packed);
    CHECK_SCALAR(gamma);
    TRY(check_ws(ws, ws_bytes, bitlinear_pack_batched_workspace_bytes(B, N, K)));
    hipStream_t st = as_stream(stream);
    const int64_t total = N * K;
    TRY(hip_status(bl::launch_gamma(W, total, B, static_cast<double*>(ws), gamma, st), "gamma launch"));
    return hip_status(bl::launch_ternarize_pack(W, total, B, gamma, reinterpret_cast<uint32_t*>(packed), st),
                      "pack launch");
}

// Workspace of the MLGRU token mixer over M = B * T tokens: one activation
// stage (reused by the input and the output projection), the
// pre-activations z fp32 [M][3d], the gated state p bf16 [M][d] and the
// scan's chunk summaries; each part 256-byte aligned.
struct MlgruWs {
    char* act;
    float* z;
    uint16_t* p;
    void* scan;
    size_t act_bytes;
};

size_t mlgru_ws_bytes(int64_t B, int64_t T, int64_t d) {
    const int64_t M = B * T;
    return bl::act_stage_bytes(M, d) + (size_t)bl::round_up(M * 3 * d * 4, 256) +
           (size_t)bl::round_up(M * d * 2, 256) + bl::mlgru_scan_workspace_bytes(B, T, d);
}

MlgruWs mlgru_ws_carve(void* base, int64_t B, int64_t T, int64_t d) {
    const int64_t M = B * T;
    char* w = static_cast<char*>(base);
    MlgruWs m;
    m.act = w;
    m.act_bytes = bl::act_stage_bytes(M, d);
    w += m.act_bytes;
    m.z = reinterpret_cast<float*>(w);
    w += bl::round_up(M * 3 * d * 4, 256);
    m.p = reinterpret_cast<uint16_t*>(w);
    w += bl::round_up(M * d * 2, 256);
    m.scan = w;
    return m;
}

int check_mlgru_shape(int64_t B, int64_t T, int64_t d) {
    TRY(check_rows(B, "B"));
    TRY(check_rows(T, "T"));
    TRY(check_k(d, "d"));
    CHECK(B * T <= BITLINEAR_MAX_DIM, BITLINEAR_ERR_INVALID_ARG, "B*T exceeds BITLINEAR_MAX_DIM");
    CHECK(B * T * 3 * d <= kMaxElems && 3 * d * d <= kMaxElems, BITLINEAR_ERR_INVALID_ARG,
          "matrix too large");
    return BITLINEAR_OK;
}

// The token mixer: z = BitLinear_in(x) over all B*T tokens, the recurrence,
// y = BitLinear_out(p).  The projections go through the forward's own
// dispatch (fused decode kernel for a few tokens, MFMA tiles for many).
// With res (bf16 [B][T][d]) the mixer adds its output to res and writes the
// bf16 sum to out_res instead of y (y is then scratch).  One token per
// sequence (T = 1, B <= 4) runs as two launches: the input projection's
// decode kernel gathers the f, c and g rows of each channel and applies the
// recurrence step in its epilogue, and the output projection's adds the
// residual in its epilogue (same fp32 arithmetic as the separate kernels,
// so the same bits).  Above 128 tokens the output projection's large-tile
// product adds the residual in its epilogue likewise.
int mlgru_impl(const uint16_t* x, const float* rms_w_in, const uint8_t* packed_in,
               const float* gamma_in, const float* rms_w_out, const uint8_t* packed_out,
               const float* gamma_out, int64_t B, int64_t T, int64_t d, float eps, float* state,
               float* y, void* ws, size_t ws_bytes, hipStream_t st, const uint16_t* res = nullptr,
               uint16_t* out_res = nullptr) {
    TRY(check_mlgru_shape(B, T, d));
    TRY(check_eps(eps));
    if (B == 0 || T == 0) return BITLINEAR_OK;
    CHECK_PTR(x);
    CHECK_PTR(rms_w_in);
    CHECK_PTR(packed_in);
    CHECK_SCALAR(gamma_in);
    CHECK_PTR(rms_w_out);
    CHECK_PTR(packed_out);
    CHECK_SCALAR(gamma_out);
    CHECK_PTR(state);
    CHECK_PTR(y);
    TRY(check_ws(ws, ws_bytes, mlgru_ws_bytes(B, T, d)));
    const MlgruWs w = mlgru_ws_carve(ws, B, T, d);
    const int64_t M = B * T;
    if (T == 1 && bl::decode_supported((int)B, (int)d)) {
        TRY(run_decode(x, rms_w_in, 0, packed_in, gamma_in, 1, B, d, d, eps, w.p, bl::Epilogue::kMlgruStep, st,
                       nullptr, state));
    } else {
        TRY(forward_impl(x, rms_w_in, packed_in, gamma_in, 1, M, 3 * d, d, eps, w.z, w.act, w.act_bytes,
                         st, BITLINEAR_KERNEL_AUTO));
        TRY(hip_status(bl::launch_mlgru_scan(w.z, B, T, d, state, w.p, w.scan, st), "mlgru scan launch"));
    }
    if (res != nullptr && bl::decode_supported((int)M, (int)d))
        return run_decode(w.p, rms_w_out, 0, packed_out, gamma_out, 1, M, d, d, eps, out_res,
                          bl::Epilogue::kResBf16, st, res);
    if (res != nullptr && bl::product_takes_residual((int)M, (int)d, (int)d)) {
        // the residual added in the output projection's epilogue
        bl::ActStage act = bl::act_stage_carve(w.act, M, d);
        TRY(hip_status(bl::launch_quant(w.p, rms_w_out, M, M, (int)d, eps, act, st), "quantise launch"));
        return run_product(act, packed_out, gamma_out, M, d, d, 1, out_res, bl::Epilogue::kResBf16,
                           BITLINEAR_KERNEL_AUTO, st, res);
    }
    TRY(forward_impl(w.p, rms_w_out, packed_out, gamma_out, 1, M, d, d, eps, y, w.act, w.act_bytes, st,
                     BITLINEAR_KERNEL_AUTO));
    if (res != nullptr)
        return hip_status(bl::launch_residual_bf16(res, y, out_res, M * d, st), "residual launch");
    return BITLINEAR_OK;
}

// Workspace of one layer: a region shared by the two mixers (each needs it
// only while it runs), the mixers' fp32 outputs [M][d] and the bf16 residual
// stream u [M][d] between them.
size_t layer_shared_bytes(int64_t B, int64_t T, int64_t d, int64_t F) {
    return std::max(mlgru_ws_bytes(B, T, d), bitlinear_glu_workspace_bytes(B * T, d, F));
}

size_t layer_ws_bytes(int64_t B, int64_t T, int64_t d, int64_t F) {
    const int64_t M = B * T;
    return bl::round_up((int64_t)layer_shared_bytes(B, T, d, F), 256) + (size_t)bl::round_up(M * d * 4, 256) +
           (size_t)bl::round_up(M * d * 2, 256);
}

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) on the first no-allocation call there.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];

int noalloc_scratch(void** out) {
    int dev = -1;
    TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
    CHECK(dev >= 0 && dev < kMaxScratchDevices, BITLINEAR_ERR_UNSUPPORTED,
          "device %d is beyond the %d devices the no-allocation scratch is tracked for", dev,
          kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
        CHECK(p != nullptr && aligned(p, 256), BITLINEAR_ERR_HIP,
              "the scratch array has no usable device address on device %d", dev);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BITLINEAR_OK;
}

int layer_impl(const uint16_t* x, const float* rms_w_in, const uint8_t* packed_in,
               const float* gamma_in, const float* rms_w_out, const uint8_t* packed_out,
               const float* gamma_out, const float* rms_w_gu, const uint8_t* packed_gu,
               const float* gamma_gu, const float* rms_w_down, const uint8_t* packed_down,
               const float* gamma_down, int64_t B, int64_t T, int64_t d, int64_t F, float eps,
               float* state, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t st) {
    TRY(check_mlgru_shape(B, T, d));
    TRY(check_k(F, "F"));
    TRY(check_eps(eps));
    CHECK(B * T * F <= kMaxElems && 2 * F * d <= kMaxElems, BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    if (B == 0 || T == 0) return BITLINEAR_OK;
    CHECK_PTR(out);
    CHECK_PTR(rms_w_gu);
    CHECK_PTR(packed_gu);
    CHECK_SCALAR(gamma_gu);
    CHECK_PTR(rms_w_down);
    CHECK_PTR(packed_down);
    CHECK_SCALAR(gamma_down);
    TRY(check_ws(ws, ws_bytes, layer_ws_bytes(B, T, d, F)));
    const int64_t M = B * T;
    char* base = static_cast<char*>(ws);
    const size_t shared = (size_t)bl::round_up((int64_t)layer_shared_bytes(B, T, d, F), 256);
    float* ymix = reinterpret_cast<float*>(base + shared);
    uint16_t* u = reinterpret_cast<uint16_t*>(base + shared + bl::round_up(M * d * 4, 256));
    TRY(mlgru_impl(x, rms_w_in, packed_in, gamma_in, rms_w_out, packed_out, gamma_out, B, T, d, eps, state,
                   ymix, base, mlgru_ws_bytes(B, T, d), st, x, u));
    return glu_impl(u, rms_w_gu, packed_gu, gamma_gu, rms_w_down, packed_down, gamma_down, 1, M, d, F, eps,
                    ymix, base, bitlinear_glu_workspace_bytes(M, d, F), st, u, out);
}

}  // namespace

extern "C" {

int bitlinear_abi_version(void) { return 1; }

int bitlinear_decode_supported(int64_t M, int64_t K) {
    if (M < 1 || K < 1 || M > BITLINEAR_MAX_DIM || K > BITLINEAR_MAX_K) return 0;
    return fused_supported(M, K, false) ? 1 : 0;
}

const char* bitlinear_last_error(void) { return g_last_error.c_str(); }

size_t bitlinear_packed_bytes(int64_t N, int64_t K) {
    if (N < 0 || K < 0 || K % 16 != 0) return 0;
    return (size_t)(N * (K / 4));
}

size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K) {
    return bitlinear_pack_batched_workspace_bytes(1, N, K);
}

size_t bitlinear_pack_batched_workspace_bytes(int64_t B, int64_t N, int64_t K) {
    if (B <= 0 || N <= 0 || K <= 0 || B > kMaxBatch || N > kMaxElems / K) return 0;
    return (size_t)bl::round_up(B * (int64_t)bl::gamma_partials(N * K) * 8, 256);
}

int bitlinear_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                           void* ws, size_t ws_bytes, void* stream) {
    return pack_impl(W, 1, N, K, packed, gamma, ws, ws_bytes, stream);
}

int bitlinear_pack_weights_batched(const float* W, int64_t B, int64_t N, int64_t K, uint8_t* packed,
                                   float* gamma, void* ws, size_t ws_bytes, void* stream) {
    return pack_impl(W, B, N, K, packed, gamma, ws, ws_bytes, stream);
}

int bitlinear_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* w, void* stream) {
    TRY(check_k(K, "K"));
    TRY(check_rows(N, "N"));
    CHECK(N * K <= kMaxElems, BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    if (N == 0) return BITLINEAR_OK;
    CHECK_PTR(packed);
    CHECK_PTR(w);
    return hip_status(bl::launch_unpack(reinterpret_cast<const uint32_t*>(packed), N * K / 16, w,
                                        as_stream(stream)),
                      "unpack launch");
}

size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    (void)N;
    if (M <= 0 || K <= 0) return 0;
    return bl::act_stage_bytes(M, K);
}

size_t bitlinear_forward_batched_workspace_bytes(int64_t B, int64_t M, int64_t N, int64_t K) {
    (void)N;
    if (B <= 0 || M <= 0 || K <= 0) return 0;
    return bl::act_stage_bytes(B * M, K);
}

int bitlinear_forward(const uint16_t* x, const float* rms_weight, const uint8_t* packed,
                      const float* gamma, int64_t M, int64_t N, int64_t K, float eps, float* y,
                      void* ws, size_t ws_bytes, void* stream) {
    return forward_impl(x, rms_weight, packed, gamma, 1, M, N, K, eps, y, ws, ws_bytes, stream,
                        BITLINEAR_KERNEL_AUTO);
}

int bitlinear_forward_noalloc(const uint16_t* x, const float* rms_weight, const uint8_t* packed,
                              const float* gamma, int64_t M, int64_t N, int64_t K, float eps,
                              float* y, void* stream) {
    // Sizes first: a call beyond the scratch is refused before any HIP call.
    TRY(check_rows(M, "M"));
    TRY(check_rows(N, "N"));
    TRY(check_k(K, "K"));
    if (M == 0 || N == 0) return BITLINEAR_OK;
    CHECK(M * K <= kMaxElems, BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    const size_t need = bl::act_stage_bytes(M, K);
    CHECK(need <= (size_t)BITLINEAR_NOALLOC_SCRATCH_BYTES, BITLINEAR_ERR_INVALID_ARG,
          "bitlinear_forward_noalloc: M=%lld, K=%lld need %zu bytes of scratch, more than the %zu it "
          "holds (use bitlinear_forward with a workspace)",
          (long long)M, (long long)K, need, (size_t)BITLINEAR_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    TRY(noalloc_scratch(&ws));
    return forward_impl(x, rms_weight, packed, gamma, 1, M, N, K, eps, y, ws, need, stream,
                        BITLINEAR_KERNEL_AUTO);
}

int bitlinear_forward_ex(const uint16_t* x, const float* rms_weight, const uint8_t* packed,
                         const float* gamma, int64_t M, int64_t N, int64_t K, float eps, float* y,
                         void* ws, size_t ws_bytes, void* stream, int kernel) {
    return forward_impl(x, rms_weight, packed, gamma, 1, M, N, K, eps, y, ws, ws_bytes, stream,
                        kernel);
}

int bitlinear_prepare_activations(const uint16_t* x, const float* rms_weight, int64_t M, int64_t K,
                                  float eps, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_rows(M, "M"));
    TRY(check_k(K, "K"));
    TRY(check_eps(eps));
    CHECK(M * K <= kMaxElems, BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    if (M == 0) return BITLINEAR_OK;
    CHECK_PTR(x);
    CHECK_PTR(rms_weight);
    TRY(check_ws(ws, ws_bytes, bl::act_stage_bytes(M, K)));
    bl::ActStage act = bl::act_stage_carve(ws, M, K);
    return hip_status(bl::launch_quant(x, rms_weight, M, M, (int)K, eps, act, as_stream(stream)),
                      "quantise launch");
}

int bitlinear_forward_prepared(const uint8_t* packed, const float* gamma, int64_t M, int64_t N,
                               int64_t K, float* y, void* ws, size_t ws_bytes, void* stream,
                               int kernel) {
    TRY(check_rows(M, "M"));
    TRY(check_rows(N, "N"));
    TRY(check_k(K, "K"));
    CHECK(M * K <= kMaxElems && N * K <= kMaxElems && M * N <= kMaxElems,
          BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    TRY(check_kernel(kernel, M, K, false));
    if (M == 0 || N == 0) return BITLINEAR_OK;
    CHECK_PTR(packed);
    CHECK_SCALAR(gamma);
    CHECK_PTR(y);
    TRY(check_ws(ws, ws_bytes, bl::act_stage_bytes(M, K)));
    bl::ActStage act = bl::act_stage_carve(ws, M, K);
    return run_product(act, packed, gamma, M, N, K, 1, y, bl::Epilogue::kF32, kernel,
                       as_stream(stream));
}

int bitlinear_forward_batched(const uint16_t* x, const float* rms_weight, const uint8_t* packed,
                              const float* gamma, int64_t B, int64_t M, int64_t N, int64_t K,
                              float eps, float* y, void* ws, size_t ws_bytes, void* stream) {
    CHECK(B >= 1, BITLINEAR_ERR_INVALID_ARG, "B must be >= 1");
    return forward_impl(x, rms_weight, packed, gamma, B, M, N, K, eps, y, ws, ws_bytes, stream,
                        BITLINEAR_KERNEL_AUTO);
}

size_t bitlinear_glu_workspace_bytes(int64_t M, int64_t D, int64_t F) {
    if (M <= 0 || D <= 0 || F <= 0) return 0;
    return bl::act_stage_bytes(M, D) + (size_t)bl::round_up(M * F * 2, 256) +
           bl::act_stage_bytes(M, F);
}

int bitlinear_glu_hidden(const uint16_t* x, const float* rms_w_gu, const uint8_t* packed_gu,
                         const float* gamma_gu, int64_t M, int64_t D, int64_t F, float eps,
                         uint16_t* h, void* ws, size_t ws_bytes, void* stream, int kernel) {
    TRY(check_rows(M, "M"));
    TRY(check_k(D, "D"));
    TRY(check_k(F, "F"));
    TRY(check_eps(eps));
    CHECK(M * D <= kMaxElems && 2 * F * D <= kMaxElems && M * F <= kMaxElems,
          BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    TRY(check_kernel(kernel, M, D, true, true));
    if (M == 0) return BITLINEAR_OK;
    CHECK_PTR(x);
    CHECK_PTR(rms_w_gu);
    CHECK_PTR(packed_gu);
    CHECK_SCALAR(gamma_gu);
    CHECK_PTR(h);
    TRY(check_ws(ws, ws_bytes, bl::act_stage_bytes(M, D)));
    hipStream_t st = as_stream(stream);
    if (use_decode(M, D, kernel, true))
        return run_decode(x, rms_w_gu, 0, packed_gu, gamma_gu, 1, M, F, D, eps, h,
                          bl::Epilogue::kGluBf16, st);
    bl::ActStage act = bl::act_stage_carve(ws, M, D);
    TRY(hip_status(bl::launch_quant(x, rms_w_gu, M, M, (int)D, eps, act, st), "quantise launch"));
    return run_product(act, packed_gu, gamma_gu, M, F, D, 1, h, bl::Epilogue::kGluBf16, kernel, st);
}

int bitlinear_glu_forward(const uint16_t* x, const float* rms_w_gu, const uint8_t* packed_gu,
                          const float* gamma_gu, const float* rms_w_down,
                          const uint8_t* packed_down, const float* gamma_down, int64_t M, int64_t D,
                          int64_t F, float eps, float* y, void* ws, size_t ws_bytes, void* stream) {
    return glu_impl(x, rms_w_gu, packed_gu, gamma_gu, rms_w_down, packed_down, gamma_down, 1, M, D,
                    F, eps, y, ws, ws_bytes, stream);
}

size_t bitlinear_glu_batched_workspace_bytes(int64_t B, int64_t M, int64_t D, int64_t F) {
    if (B <= 0) return 0;
    return bitlinear_glu_workspace_bytes(B * M, D, F);
}

int bitlinear_glu_forward_batched(const uint16_t* x, const float* rms_w_gu,
                                  const uint8_t* packed_gu, const float* gamma_gu,
                                  const float* rms_w_down, const uint8_t* packed_down,
                                  const float* gamma_down, int64_t B, int64_t M, int64_t D,
                                  int64_t F, float eps, float* y, void* ws, size_t ws_bytes,
                                  void* stream) {
    return glu_impl(x, rms_w_gu, packed_gu, gamma_gu, rms_w_down, packed_down, gamma_down, B, M, D,
                    F, eps, y, ws, ws_bytes, stream);
}

int bitlinear_quantize(const uint16_t* x, const float* rms_weight, int64_t M, int64_t K, float eps,
                       int8_t* q, float* s, void* stream) {
    TRY(check_rows(M, "M"));
    TRY(check_k(K, "K"));
    TRY(check_eps(eps));
    CHECK(M * K <= kMaxElems, BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    if (M == 0) return BITLINEAR_OK;
    CHECK_PTR(x);
    CHECK_PTR(rms_weight);
    CHECK_PTR(q);
    CHECK_PTR(s);
    // The stage call returns q and s only; a NULL code-sum pointer tells the
    // kernel to skip that output.
    bl::ActStage act;
    act.q = q;
    act.s = s;
    act.sumq = nullptr;
    return hip_status(bl::launch_quant(x, rms_weight, M, M, (int)K, eps, act, as_stream(stream)),
                      "quantise launch");
}

int bitlinear_ternary_matmul_i32(const int8_t* q, const uint8_t* packed, int64_t M, int64_t N,
                                 int64_t K, int32_t* acc, void* ws, size_t ws_bytes, void* stream,
                                 int kernel) {
    TRY(check_rows(M, "M"));
    TRY(check_rows(N, "N"));
    TRY(check_k(K, "K"));
    CHECK(M * K <= kMaxElems && N * K <= kMaxElems && M * N <= kMaxElems,
          BITLINEAR_ERR_INVALID_ARG, "matrix too large");
    TRY(check_kernel(kernel, M, K, false));
    if (M == 0 || N == 0) return BITLINEAR_OK;
    CHECK_PTR(q);
    CHECK_PTR(packed);
    CHECK_PTR(acc);
    TRY(check_ws(ws, ws_bytes, bitlinear_forward_workspace_bytes(M, N, K)));
    hipStream_t st = as_stream(stream);
    bl::ActStage act = bl::act_stage_carve(ws, M, K);
    act.q = const_cast<int8_t*>(q);
    TRY(hip_status(bl::launch_row_sums(q, M, (int)K, act.sumq, st), "row sums launch"));
    return run_product(act, packed, nullptr, M, N, K, 1, acc, bl::Epilogue::kI32, kernel, st);
}


size_t bitlinear_backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K <= 0 || K % 16 != 0 || K > BITLINEAR_MAX_K || M > BITLINEAR_MAX_DIM ||
        N > BITLINEAR_MAX_DIM)
        return 0;
    return bl::backward_workspace_bytes(M, N, K);
}

int bitlinear_backward(const uint16_t* x, const float* rms_weight, const uint8_t* packed,
                       const float* gamma, const float* dy, int64_t M, int64_t N, int64_t K, float eps,
                       float* dx, float* dg, float* dW, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_rows(M, "M"));
    TRY(check_rows(N, "N"));
    TRY(check_k(K, "K"));
    TRY(check_eps(eps));
    CHECK(M * K <= kMaxElems && N * K <= kMaxElems && M * N <= kMaxElems, BITLINEAR_ERR_INVALID_ARG,
          "matrix too large");
    CHECK_PTR(rms_weight);
    CHECK_SCALAR(gamma);
    CHECK_PTR(dg);
    if (M > 0) {
        CHECK_PTR(x);
        CHECK_PTR(dx);
    }
    if (N > 0) {
        CHECK_PTR(packed);
        CHECK_PTR(dW);
    }
    if (M > 0 && N > 0) CHECK_PTR(dy);
    TRY(check_ws(ws, ws_bytes, bl::backward_workspace_bytes(M, N, K)));
    bl::BackwardArgs a{x, rms_weight, packed, gamma, dy, M, N, K, eps, dx, dg, dW, ws};
    return hip_status(bl::launch_backward(a, as_stream(stream)), "backward launch");
}

size_t bitlinear_mlgru_scan_workspace_bytes(int64_t B, int64_t T, int64_t d) {
    if (B <= 0 || T <= 0 || d <= 0 || d % 16 != 0 || d > BITLINEAR_MAX_K || B * T > BITLINEAR_MAX_DIM) return 0;
    return bl::mlgru_scan_workspace_bytes(B, T, d);
}

int bitlinear_mlgru_scan(const float* z, int64_t B, int64_t T, int64_t d, float* state, uint16_t* p,
                         void* ws, size_t ws_bytes, void* stream) {
    TRY(check_mlgru_shape(B, T, d));
    if (B == 0 || T == 0) return BITLINEAR_OK;
    CHECK_PTR(z);
    CHECK_PTR(state);
    CHECK_PTR(p);
    TRY(check_ws(ws, ws_bytes, bl::mlgru_scan_workspace_bytes(B, T, d)));
    return hip_status(bl::launch_mlgru_scan(z, B, T, d, state, p, ws, as_stream(stream)), "mlgru scan launch");
}

size_t bitlinear_mlgru_workspace_bytes(int64_t B, int64_t T, int64_t d) {
    if (B <= 0 || T <= 0 || d <= 0 || d % 16 != 0 || d > BITLINEAR_MAX_K || B * T > BITLINEAR_MAX_DIM) return 0;
    return mlgru_ws_bytes(B, T, d);
}

int bitlinear_mlgru_forward(const uint16_t* x, const float* rms_w_in, const uint8_t* packed_in,
                            const float* gamma_in, const float* rms_w_out, const uint8_t* packed_out,
                            const float* gamma_out, int64_t B, int64_t T, int64_t d, float eps,
                            float* state, float* y, void* ws, size_t ws_bytes, void* stream) {
    return mlgru_impl(x, rms_w_in, packed_in, gamma_in, rms_w_out, packed_out, gamma_out, B, T, d, eps,
                      state, y, ws, ws_bytes, as_stream(stream));
}

size_t bitlinear_layer_workspace_bytes(int64_t B, int64_t T, int64_t d, int64_t F) {
    if (B <= 0 || T <= 0 || d <= 0 || F <= 0 || d % 16 != 0 || F % 16 != 0 || d > BITLINEAR_MAX_K ||
        F > BITLINEAR_MAX_K || B * T > BITLINEAR_MAX_DIM)
        return 0;
    return layer_ws_bytes(B, T, d, F);
}

int bitlinear_layer_forward(const uint16_t* x, const float* rms_w_in, const uint8_t* packed_in,
                            const float* gamma_in, const float* rms_w_out, const uint8_t* packed_out,
                            const float* gamma_out, const float* rms_w_gu, const uint8_t* packed_gu,
                            const float* gamma_gu, const float* rms_w_down, const uint8_t* packed_down,
                            const float* gamma_down, int64_t B, int64_t T, int64_t d, int64_t F,
                            float eps, float* state, uint16_t* out, void* ws, size_t ws_bytes,
                            void* stream) {
    return layer_impl(x, rms_w_in, packed_in, gamma_in, rms_w_out, packed_out, gamma_out, rms_w_gu, packed_gu,
                      gamma_gu, rms_w_down, packed_down, gamma_down, B, T, d, F, eps, state, out, ws, ws_bytes,
                      as_stream(stream));
}

}  // extern "C"
