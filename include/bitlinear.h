/*
 * bitlinear.h -- C ABI of the fused BitLinear layer for AMD Instinct MI355X
 * (gfx950 / CDNA4).
 *
 * BitLinear is the dense layer of "Scalable MatMul-free Language Modeling".
 * Sources, as the pages that describe it:
 *   [ld246]      ld246.com article 1724132886152: section "三值权重的应用"
 *                (weights are -1, 0 or +1, so +1 adds the input, -1
 *                subtracts it and 0 skips it) and section "融合 BitLinear 层的
 *                创新" (RMSNorm and quantisation fused in front of the product,
 *                activations read from HBM once).
 *   [jiqizhixin] jiqizhixin.com article 2024-06-11-4: section "具有三值权重的
 *                MatMul-free 密集层" (ternary dense layer; Algorithm 1: RMSNorm
 *                fused with quantisation and BitLinear), section "MatMul-free
 *                语言模型架构" (GLU channel mixer built from BitLinear) and
 *                section "MatMul-free 语言模型的扩展规律" (BitLinear activations
 *                are BF16).
 *   [datacamp]   datacamp.com/vi/blog/matmul-free-language-models: section
 *                "Thay MatMul bằng các phép toán tam phân" (absmean
 *                ternarisation of the weight matrix) and section "Các thành
 *                phần lõi: MLGRU và GLU" (RMSNorm before quantisation, scaled
 *                ternary accumulation, GLU = two BitLinear, SiLU on one,
 *                element-wise product, third BitLinear).
 *
 * What the layer computes (per token row m of x, output feature n):
 *   gamma   = mean_{n,k} |W[n][k]|                        (sum in fp64)
 *   w[n][k] = clip(round(W[n][k] / (gamma + 1e-5)), -1, 1)   (fp32, ties even)
 *   r_m     = 1 / sqrt(fp32(sum_k x^2 / K) + eps)         (sum in fp64)
 *   xn      = (x * r_m) * rms_weight                      (fp32)
 *   s_m     = 127 / max(max_k |xn|, 1e-5)                 (fp32)
 *   q       = clip(round(xn * s_m), -128, 127)            (int8, ties even)
 *   acc     = sum_k (w=+1: +q, w=-1: -q, w=0: skip)       (int32, exact)
 *   y[m][n] = float(acc) * (gamma / s_m)                  (fp32)
 * The pages print none of these formulas; the readings (divide rather than
 * multiply by the mean, symmetric 127 scale, the 1e-5 guards, fp64 sums) are
 * the library's, chosen as the plainest ones consistent with the pages.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to caller-owned memory; the library
 *     allocates nothing and keeps no device state, apart from the fixed
 *     scratch array of bitlinear_forward_noalloc (part of the loaded code,
 *     one per GPU).  All matrices are row-major and densely packed (row
 *     stride = row length).
 *   - x and h are bf16 stored as uint16 bit patterns.  W and rms weights are
 *     fp32.  gamma is a device fp32 scalar (no host round trip).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work and return; nothing synchronises the host.
 *     No entry point allocates, copies or clears memory: each only launches
 *     kernels on `stream`, so a sequence of calls can be captured into a HIP
 *     graph and replayed (with the same pointers and sizes).
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Return value: BITLINEAR_OK (0) or a bitlinear_status; on error nothing
 *     was launched (argument and workspace checks run before any launch)
 *     unless the status is BITLINEAR_ERR_HIP, and bitlinear_last_error()
 *     returns a message (per calling thread).
 *   - Checked before launch: non-NULL pointers for non-empty tensors; sizes
 *     >= 0 with K > 0; K (and D, F for the GLU) multiples of 16 and at most
 *     BITLINEAR_MAX_K; row counts at most BITLINEAR_MAX_DIM; 16-byte
 *     alignment of every pointer and 256-byte alignment of the workspace;
 *     workspace size; eps > 0 and finite.  M = 0 or N = 0 is a valid empty call that does nothing.
 *   - Inputs are read-only; outputs are fully overwritten; outputs, inputs
 *     and workspace must not overlap.  NaN/Inf inputs are outside the
 *     contract.
 *   - Workspace: caller-provided device scratch of at least the size the
 *     matching *_workspace_bytes() query returns for the same sizes.  Its
 *     contents are undefined after a call; calls that share a workspace must
 *     be ordered on one stream.
 *   - Entry points are reentrant and thread-safe.
 *
 * Packed ternary format (the pages print none; this is the library's own):
 *   - row n of the [N][K] ternary matrix occupies K/4 bytes, rows back to
 *     back, so the packed matrix is [N][K/4] bytes; K % 16 == 0;
 *   - along a row, weights go in groups of 16, one little-endian 32-bit word
 *     per group (k = 16*grp + j -> word grp of the row);
 *   - weight j = 4*i + t of a group sits in byte t of the word, bits
 *     2i+1..2i (so (word >> 2i) & 0x03030303 yields weights 4i..4i+3 of the
 *     group, one per byte, in order);
 *   - the 2-bit code is w + 1: 0 -> -1, 1 -> 0, 2 -> +1; code 3 is never
 *     written (bitlinear_unpack_weights decodes it to 2).
 *   The offset code lets the kernels feed masked codes c = w + 1 straight
 *   into int8 dot products and MFMA, since sum_k q w = sum_k q c - sum_k q,
 *   with sum_k q computed once per token.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BITLINEAR_OK = 0,
    BITLINEAR_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment or eps   */
    BITLINEAR_ERR_WORKSPACE = 2,   /* workspace missing or too small        */
    BITLINEAR_ERR_UNSUPPORTED = 3, /* no GPU of the supported kind          */
    BITLINEAR_ERR_HIP = 4          /* a HIP call or launch failed           */
} bitlinear_status;

/* Largest M, N, K, B*M, D or F accepted (keeps every in-kernel row index and
 * every row length in 32 bits). */
#define BITLINEAR_MAX_DIM ((int64_t)1 << 30)

/* Largest reduction length accepted: K, and D and F for the GLU.  Codes lie
 * in [-127, 127], so every accumulation and every code sum stays below
 * 127 * 2^24 < 2^31 in magnitude and the int32 results are exact. */
#define BITLINEAR_MAX_K ((int64_t)1 << 24)

/* Kernel choice for bitlinear_forward_ex. */
typedef enum {
    BITLINEAR_KERNEL_AUTO = 0,   /* by token count M (what bitlinear_forward does)  */
    BITLINEAR_KERNEL_GEMV = 1,   /* quantise, then weight-streaming GEMV (M <= 8)   */
    BITLINEAR_KERNEL_MFMA = 2,   /* quantise, then int8 MFMA tiles                  */
    BITLINEAR_KERNEL_DECODE = 3  /* one fused kernel, quantisation inside; takes
                                    M <= 4 with K % 64 == 0 and K <= 16384
                                    (M = 1), 8192 (M = 2) or 4096 (M = 3, 4);
                                    and M <= 16 with K = 2048 or 4096 and
                                    M * K <= 32768 (the fp32 forward only)   */
} bitlinear_kernel;

/* 1 when a fused kernel (BITLINEAR_KERNEL_DECODE) takes M tokens of length K
 * in bitlinear_forward, else 0. */
int bitlinear_decode_supported(int64_t M, int64_t K);

/* Version of this ABI (bumped on any incompatible change). */
int bitlinear_abi_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char* bitlinear_last_error(void);

/* ---------------------------------------------------------------------------
 * Weights.  [datacamp, "Thay MatMul bằng các phép toán tam phân"]: absmean
 * ternarisation -- the matrix is scaled by its mean absolute value and each
 * element rounded to the nearest of -1, 0, +1 ([ld246, "三值权重的应用"]).
 * ------------------------------------------------------------------------- */

/* Bytes of the packed [N][K/4] matrix (0 when K % 16 != 0 or a size is
 * negative). */
size_t bitlinear_packed_bytes(int64_t N, int64_t K);

/* Workspace bytes for bitlinear_pack_weights (fp64 partial sums of |W|). */
size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K);

/* W: device fp32 [N][K].  Writes packed (device, [N][K/4] bytes) and *gamma
 * (device fp32 scalar, the mean |W|).  The fp64 sum of |W| is reduced in a
 * fixed order, so the result is deterministic.  N >= 1. */
int bitlinear_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* packed,
                           float* gamma, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for bitlinear_pack_weights_batched (0 for an invalid
 * shape). */
size_t bitlinear_pack_batched_workspace_bytes(int64_t B, int64_t N, int64_t K);

/* B matrices of one shape ternarised in one call -- the re-ternarisation of
 * a stack of layers from their fp32 master weights, e.g. once per training
 * step ([ld246, "训练与优化：新的策略"]: training passes gradients straight
 * through the ternarisation, so the full-precision weights are kept, updated
 * and ternarised again).
 * W: device fp32 [B][N][K]; packed: device [B][N][K/4]; gamma: device fp32
 * [B], one mean |W| per matrix.  Each matrix gets exactly the bytes and gamma
 * that bitlinear_pack_weights gives it.  1 <= B <= 65535. */
int bitlinear_pack_weights_batched(const float* W, int64_t B, int64_t N, int64_t K,
                                   uint8_t* packed, float* gamma, void* ws, size_t ws_bytes,
                                   void* stream);

/* Test/inspection: decode packed [N][K/4] into int8 [N][K] as code - 1.
 * Valid codes give -1, 0, +1; the unused code 3 decodes to 2, outside the
 * ternary set, so that a corrupted matrix is visible to a check of w. */
int bitlinear_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* w,
                             void* stream);

/* ---------------------------------------------------------------------------
 * Forward.  [jiqizhixin, "具有三值权重的 MatMul-free 密集层", Algorithm 1] and
 * [ld246, "融合 BitLinear 层的创新"]: RMSNorm and activation quantisation
 * fused in front of the ternary product; [datacamp, "Các thành phần lõi:
 * MLGRU và GLU", panels "RMS norm" and "MatMul vs scaled ternary
 * accumulation"]: normalise, quantise, accumulate with +/-, rescale.
 * ------------------------------------------------------------------------- */

/* Workspace bytes for bitlinear_forward / bitlinear_forward_ex (int8 codes
 * [M][K], per-token scale and code sum, each part 256-byte aligned). */
size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* x: bf16 [M][K]; rms_weight: fp32 [K]; packed: [N][K/4] (from
 * bitlinear_pack_weights); gamma: device fp32 scalar; y: fp32 [M][N].
 * Dispatches on M: one fused kernel (quantisation and product) for M <= 4
 * and K % 64 == 0; otherwise the quantisation pass, then the ternary product
 * on the int8 matrix cores (or the GEMV for M <= 4). */
int bitlinear_forward(const uint16_t* x, const float* rms_weight, const uint8_t* packed,
                      const float* gamma, int64_t M, int64_t N, int64_t K, float eps,
                      float* y, void* ws, size_t ws_bytes, void* stream);

/* bitlinear_forward with an explicit kernel choice (results are identical
 * for every choice; used to test and time each kernel on the same shape). */
int bitlinear_forward_ex(const uint16_t* x, const float* rms_weight,
                         const uint8_t* packed, const float* gamma, int64_t M, int64_t N,
                         int64_t K, float eps, float* y, void* ws, size_t ws_bytes,
                         void* stream, int kernel);

/* Bytes of device scratch that bitlinear_forward_noalloc holds per GPU. */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)

/* bitlinear_forward for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without a workspace, the same kernels and bit-identical y.  The
 * activation stage lives in a static device array of
 * BITLINEAR_NOALLOC_SCRATCH_BYTES (48 MiB), one per GPU, held from the
 * library's load until the process ends; the call allocates nothing and
 * calls no allocating routine.  Limit: bitlinear_forward_workspace_bytes(M,
 * N, K) <= BITLINEAR_NOALLOC_SCRATCH_BYTES (M * K up to about 50 M codes,
 * e.g. 16384 x 2560); larger calls return BITLINEAR_ERR_INVALID_ARG before
 * touching the GPU.  The first call on each device looks up that device's
 * array (hipGetSymbolAddress) with the device current: make it before any
 * graph capture, on the stream's device.  Every call on one GPU shares its
 * array, and nothing in it needs clearing (each call writes every byte it
 * reads); calls that overlap in time on one GPU (other streams, other
 * threads) race on it, so order them. */
int bitlinear_forward_noalloc(const uint16_t* x, const float* rms_weight, const uint8_t* packed,
                              const float* gamma, int64_t M, int64_t N, int64_t K, float eps,
                              float* y, void* stream);

/* The two halves of bitlinear_forward, for callers that feed one input to
 * several weight matrices (quantise once, multiply many times) or that time
 * the halves apart.  bitlinear_prepare_activations runs RMSNorm + absmax
 * quantisation of x [M][K] into the workspace (a private layout, sized by
 * bitlinear_forward_workspace_bytes(M, N, K)); bitlinear_forward_prepared
 * then runs the ternary product and rescale from that workspace into y
 * [M][N].  The workspace must not be modified in between; the pair computes
 * exactly what bitlinear_forward computes. */
int bitlinear_prepare_activations(const uint16_t* x, const float* rms_weight, int64_t M,
                                  int64_t K, float eps, void* ws, size_t ws_bytes,
                                  void* stream);
int bitlinear_forward_prepared(const uint8_t* packed, const float* gamma, int64_t M,
                               int64_t N, int64_t K, float* y, void* ws, size_t ws_bytes,
                               void* stream, int kernel);

/* B independent layers of the same shape in one launch sequence, e.g. one
 * decode step through a stack of layers that do not depend on each other:
 * x bf16 [B][M][K], rms_weight fp32 [B][K], packed [B][N][K/4], gamma fp32
 * [B] (device), y fp32 [B][M][N].  Layer b computes exactly what
 * bitlinear_forward computes on its slices.  B*M <= BITLINEAR_MAX_DIM. */
size_t bitlinear_forward_batched_workspace_bytes(int64_t B, int64_t M, int64_t N, int64_t K);
int bitlinear_forward_batched(const uint16_t* x, const float* rms_weight,
                              const uint8_t* packed, const float* gamma, int64_t B,
                              int64_t M, int64_t N, int64_t K, float eps, float* y,
                              void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * GLU channel mixer.  [datacamp, "Các thành phần lõi: MLGRU và GLU"]: two
 * BitLinear projections of the input, SiLU on one, element-wise product with
 * the other, then a third BitLinear; [jiqizhixin, "MatMul-free 语言模型架构"].
 * Readings: gate and up are one fused [2F][D] packed matrix with one gamma
 * (rows 0..F-1 gate, F..2F-1 up); SiLU(v) = v / (1 + exp(-v)) in fp32; the
 * product h is rounded to bf16 (the layer-boundary activation type) before
 * the down projection, which applies its own RMSNorm and quantisation.
 * ------------------------------------------------------------------------- */

size_t bitlinear_glu_workspace_bytes(int64_t M, int64_t D, int64_t F);

/* x: bf16 [M][D]; rms_w_gu: fp32 [D]; packed_gu: [2F][D/4]; gamma_gu:
 * device scalar; rms_w_down: fp32 [F]; packed_down: [D][F/4]; gamma_down:
 * device scalar; y: fp32 [M][D]. */
int bitlinear_glu_forward(const uint16_t* x, const float* rms_w_gu,
                          const uint8_t* packed_gu, const float* gamma_gu,
                          const float* rms_w_down, const uint8_t* packed_down,
                          const float* gamma_down, int64_t M, int64_t D, int64_t F,
                          float eps, float* y, void* ws, size_t ws_bytes, void* stream);

/* B independent mixers of the same shape, e.g. one decode step through a
 * stack of layers: x bf16 [B][M][D], rms_w_gu fp32 [B][D], packed_gu
 * [B][2F][D/4], gamma_gu fp32 [B], rms_w_down fp32 [B][F], packed_down
 * [B][D][F/4], gamma_down fp32 [B] (device), y fp32 [B][M][D].  Mixer b
 * computes exactly what bitlinear_glu_forward computes on its slices.
 * B*M <= BITLINEAR_MAX_DIM. */
size_t bitlinear_glu_batched_workspace_bytes(int64_t B, int64_t M, int64_t D, int64_t F);
int bitlinear_glu_forward_batched(const uint16_t* x, const float* rms_w_gu,
                                  const uint8_t* packed_gu, const float* gamma_gu,
                                  const float* rms_w_down, const uint8_t* packed_down,
                                  const float* gamma_down, int64_t B, int64_t M, int64_t D,
                                  int64_t F, float eps, float* y, void* ws, size_t ws_bytes,
                                  void* stream);

/* First half of the mixer alone: h = bf16(SiLU(gate) * up), h bf16 [M][F].
 * Workspace: bitlinear_forward_workspace_bytes(M, 2F, D). */
int bitlinear_glu_hidden(const uint16_t* x, const float* rms_w_gu,
                         const uint8_t* packed_gu, const float* gamma_gu, int64_t M,
                         int64_t D, int64_t F, float eps, uint16_t* h, void* ws,
                         size_t ws_bytes, void* stream, int kernel);

/* ---------------------------------------------------------------------------
 * MLGRU token mixer.  [datacamp, "Các thành phần lõi: MLGRU và GLU"]: the
 * MLGRU takes a sequence token by token, updating a hidden state, the
 * memory of earlier tokens, through element-wise operations and gates with
 * values between 0 and 1; [jiqizhixin, "MatMul-free 语言模型架构"]: a ternary
 * RNN of element-wise products and accumulation built on the GRU; [ld246,
 * "线性操作的引入"]: element-wise operations in place of the GRU's matrix
 * products.  Readings (the pages print no equations): the gates depend on
 * the token only, through one BitLinear whose fused [3d][d] matrix (one
 * gamma, one RMSNorm weight) gives z = z_f | z_c | z_g (rows 0..d-1, d..2d-1,
 * 2d..3d-1); per channel
 *   f = sigmoid(z_f), c = SiLU(z_c), g = sigmoid(z_g),
 *   h_t = f h_{t-1} + (1 - f) c,  p_t = bf16(g h_t),  y_t = BitLinear_out(p_t)
 * with a second BitLinear [d][d].  Sigmoid and SiLU are evaluated in fp32
 * from 2^x and a reciprocal (about one ulp each); the state is fp32.
 * ------------------------------------------------------------------------- */

/* Workspace bytes for bitlinear_mlgru_scan (0 when the sequence needs no
 * chunk summaries, or for an invalid shape). */
size_t bitlinear_mlgru_scan_workspace_bytes(int64_t B, int64_t T, int64_t d);

/* The recurrence alone, from the pre-activations: z fp32 [B][T][3d] (device),
 * state fp32 [B][d] (device; h_0 on entry, h_T on return), p bf16 [B][T][d]
 * (device, written).  The tokens of a sequence are cut into chunks that run
 * in parallel (summaries, then chunk start states, then each chunk again),
 * which equals the token-by-token recurrence up to fp32 rounding.  d % 16 ==
 * 0; B = 0 or T = 0 leaves the state as it is. */
int bitlinear_mlgru_scan(const float* z, int64_t B, int64_t T, int64_t d, float* state,
                         uint16_t* p, void* ws, size_t ws_bytes, void* stream);

size_t bitlinear_mlgru_workspace_bytes(int64_t B, int64_t T, int64_t d);

/* The token mixer: x bf16 [B][T][d]; rms_w_in fp32 [d], packed_in [3d][d/4]
 * (rows f | c | g) and gamma_in; rms_w_out fp32 [d], packed_out [d][d/4] and
 * gamma_out; state fp32 [B][d] (h_0 in, h_T out; zero it for new
 * sequences); y fp32 [B][T][d].  The two projections run through the
 * forward's dispatch over all B*T tokens (one fused kernel each for a
 * single token).  Decoding token by token is this call with T = 1, carrying
 * the state. */
int bitlinear_mlgru_forward(const uint16_t* x, const float* rms_w_in, const uint8_t* packed_in,
                            const float* gamma_in, const float* rms_w_out,
                            const uint8_t* packed_out, const float* gamma_out, int64_t B,
                            int64_t T, int64_t d, float eps, float* state, float* y, void* ws,
                            size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * One layer: the MLGRU token mixer, then the GLU channel mixer
 * ([jiqizhixin, "MatMul-free 语言模型架构"]: a layer is a token mixer and a
 * channel mixer, in the Metaformer view).  Reading: each mixer adds its
 * output to its input, and the residual stream is bf16:
 *   u = bf16(x + MLGRU(x)),   out = bf16(u + GLU(u)).
 * ------------------------------------------------------------------------- */

size_t bitlinear_layer_workspace_bytes(int64_t B, int64_t T, int64_t d, int64_t F);

/* x bf16 [B][T][d]; the MLGRU's weights as for bitlinear_mlgru_forward; the
 * GLU's as for bitlinear_glu_forward (inner size F); state fp32 [B][d] (in
 * and out); out bf16 [B][T][d]. */
int bitlinear_layer_forward(const uint16_t* x, const float* rms_w_in, const uint8_t* packed_in,
                            const float* gamma_in, const float* rms_w_out,
                            const uint8_t* packed_out, const float* gamma_out,
                            const float* rms_w_gu, const uint8_t* packed_gu, const float* gamma_gu,
                            const float* rms_w_down, const uint8_t* packed_down,
                            const float* gamma_down, int64_t B, int64_t T, int64_t d, int64_t F,
                            float eps, float* state, uint16_t* out, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------------------
 * Stages (exposed so that each step can be compared on its own).
 * ------------------------------------------------------------------------- */

/* RMSNorm + per-token absmax quantisation ([jiqizhixin, "具有三值权重的
 * MatMul-free 密集层", Algorithm 1: the activation quantiser fused with
 * RMSNorm]; [datacamp, "Các thành phần lõi: MLGRU và GLU", panel "RMS norm":
 * normalise before quantising]): q int8 [M][K] and s fp32 [M]
 * (q ~= s * RMSNorm(x)).  Same arithmetic as the first half of
 * bitlinear_forward. */
int bitlinear_quantize(const uint16_t* x, const float* rms_weight, int64_t M, int64_t K,
                       float eps, int8_t* q, float* s, void* stream);

/* Ternary accumulation alone ([ld246, "三值权重的应用"]: +1 adds the input,
 * -1 subtracts it, 0 skips it; [jiqizhixin, "具有三值权重的 MatMul-free
 * 密集层"]: the ternary product as additions and subtractions):
 * acc int32 [M][N] = sum_k q[m][k] * w[n][k] from int8 q [M][K] and packed
 * [N][K/4], exact.  Workspace:
 * bitlinear_forward_workspace_bytes(M, N, K). */
int bitlinear_ternary_matmul_i32(const int8_t* q, const uint8_t* packed, int64_t M,
                                 int64_t N, int64_t K, int32_t* acc, void* ws,
                                 size_t ws_bytes, void* stream, int kernel);

/* ---------------------------------------------------------------------------
 * Backward pass (training)
 * ------------------------------------------------------------------------- */

/* Workspace bytes for bitlinear_backward (0 for an invalid shape). */
size_t bitlinear_backward_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Gradients of the layer with the straight-through estimator ([ld246,
 * "训练与优化：新的策略"]: gradients pass straight through the ternary weights
 * and the activation quantiser; [ld246, "融合 BitLinear 层的创新"]: RMSNorm and
 * quantisation fused, activations read once).  Reading: both quantisers are
 * the identity in the backward, gamma and s held constant, so for
 * y = (q / s) (gamma w)^T:
 *   dxn = gamma dy w,  dW = dy^T (q / s),
 *   dg[k] = sum_m dxn[m][k] x[m][k] r[m],
 *   dx[m][k] = r g[k] dxn[m][k] - x[m][k] r^3 / K sum_j dxn[m][j] g[j] x[m][j],
 *   r = (mean_k x[m][k]^2 + eps)^-1/2.
 * Inputs (device): x bf16 [M][K], rms_weight fp32 [K], packed [N][K/4] and
 * gamma (fp32 scalar) of the forward, dy fp32 [M][N].  Outputs (device):
 * dx fp32 [M][K], dg fp32 [K], dW fp32 [N][K] (the gradient with respect to
 * the fp32 master weights).  q and s are recomputed from x with the
 * forward's own quantisation arithmetic, so they are the forward's bits.  The two products
 * run in bf16 with fp32 accumulation: dy and dy * (1 / s) (one fp32
 * reciprocal per token) are rounded to bf16 (nearest even); w and q are
 * exact.  M = 0 gives dg = 0 and dW = 0; N = 0
 * gives dx = 0 and dg = 0.  Deterministic (fixed reduction orders). */
int bitlinear_backward(const uint16_t* x, const float* rms_weight, const uint8_t* packed,
                       const float* gamma, const float* dy, int64_t M, int64_t N, int64_t K, float eps,
                       float* dx, float* dg, float* dW, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
