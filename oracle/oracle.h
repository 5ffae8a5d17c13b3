/*
 * oracle.h -- plain, slow CPU definition of the BitLinear forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the checker that the HIP
 * implementation is compared against.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, table or constant with the HIP path.
 *
 * Sources (pages about "Scalable MatMul-free Language Modeling"):
 *   [ld246]      ld246.com article 1724132886152, sections "三值权重的应用"
 *                (ternary weights: +1 adds, -1 subtracts, 0 skips) and
 *                "融合 BitLinear 层的创新" (RMSNorm and quantisation fused in
 *                front of the ternary product) and "训练与优化：新的策略"
 *                (straight-through gradients in training).
 *   [jiqizhixin] jiqizhixin.com 2024-06-11-4, section "具有三值权重的
 *                MatMul-free 密集层" (ternary dense layer, Algorithm 1:
 *                quantisation fused with RMSNorm and BitLinear) and section
 *                "MatMul-free 语言模型架构" (GLU channel mixer built from
 *                BitLinear), section "MatMul-free 语言模型的扩展规律"
 *                (BitLinear activations are BF16).
 *   [datacamp]   datacamp.com/vi/blog/matmul-free-language-models, section
 *                "Thay MatMul bằng các phép toán tam phân" (absmean
 *                quantisation of the weight matrix) and section "Các thành
 *                phần lõi: MLGRU và GLU" (RMSNorm before quantisation; GLU
 *                = two BitLinear, SiLU on one, Hadamard product, third
 *                BitLinear).
 *
 * Where the pages are silent the readings are listed beside each function.
 * Floating point that decides an integer (the ternary code, the int8 code)
 * is taken in fp32, the precision the GPU kernels decide it in; everything
 * else (the weight mean, the sum of squares, the rescale, SiLU) is fp64.
 *
 * Layouts: row-major.  x is bf16 stored as uint16 bit patterns [M][K];
 * W is fp32 [N][K] (out x in, y = x W^T); q int8 [M][K]; w int8 [N][K];
 * acc int32 [M][N]; y fp64 [M][N].
 */
#ifndef BITLINEAR_ORACLE_H
#define BITLINEAR_ORACLE_H

#include <stdint.h>

/* absmean weight scale: gamma = mean over the whole matrix of |W|. */
float orc_absmean_gamma(const float* W, int64_t N, int64_t K);

/* ternary code of every weight: clip(round(W / (gamma + 1e-5)), -1, 1). */
void orc_ternarize(const float* W, int64_t N, int64_t K, float gamma, int8_t* w);

/* 2-bit packed storage of a ternary matrix (format defined in oracle.c).
 * Return 0, or -1 when K % 16 != 0 (pack) or a byte holds the unused code
 * (unpack). */
int orc_pack(const int8_t* w, int64_t N, int64_t K, uint8_t* packed);
int orc_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* w);

/* bf16 bit pattern -> float (exact) and double -> nearest bf16 (ties even). */
float orc_bf16_to_float(uint16_t h);
uint16_t orc_double_to_bf16(double v);

/* RMSNorm then per-token absmax int8 quantisation.  Writes q [M][K] and the
 * per-token scale s [M] (q ~= s * normalised x). */
void orc_rmsnorm_quant(const uint16_t* x, const float* g, int64_t M, int64_t K,
                       float eps, int8_t* q, float* s);

/* Ternary accumulation: explicit add / subtract / skip loop, int32. */
void orc_ternary_accumulate(const int8_t* q, const int8_t* w, int64_t M, int64_t N,
                            int64_t K, int32_t* acc);

/* Rescale: y = acc * gamma / s (fp64). */
void orc_rescale(const int32_t* acc, float gamma, const float* s, int64_t M,
                 int64_t N, double* y);

/* Whole BitLinear forward from the fp32 master weights.  Any of the
 * intermediate outputs may be NULL. */
void orc_bitlinear(const uint16_t* x, const float* g, const float* W, int64_t M,
                   int64_t N, int64_t K, float eps, double* y, float* gamma_out,
                   int8_t* w_out, int8_t* q_out, float* s_out, int32_t* acc_out);

/* The same forward from an already ternarised matrix w and its gamma. */
void orc_bitlinear_ternary(const uint16_t* x, const float* g, const int8_t* w,
                           float gamma, int64_t M, int64_t N, int64_t K, float eps,
                           double* y, int8_t* q_out, float* s_out, int32_t* acc_out);

/* BitLinear GLU channel mixer.  W_gu is the fused [2F][D] matrix (rows 0..F-1
 * gate, F..2F-1 up, one gamma); W_down is [D][F].  h_out (bf16 [M][F]) may
 * be NULL. */
void orc_glu(const uint16_t* x, const float* g_gu, const float* W_gu,
             const float* g_down, const float* W_down, int64_t M, int64_t D,
             int64_t F, float eps, double* y, uint16_t* h_out);

/* The same mixer from ternarised matrices. */
void orc_glu_ternary(const uint16_t* x, const float* g_gu, const int8_t* w_gu,
                     float gamma_gu, const float* g_down, const int8_t* w_down,
                     float gamma_down, int64_t M, int64_t D, int64_t F, float eps,
                     double* y, uint16_t* h_out);

/* MLGRU recurrence from the pre-activations z [B][T][3d] (rows of each
 * token: z_f | z_c | z_g): f = sigmoid(z_f), c = SiLU(z_c),
 * g = sigmoid(z_g), h_t = f h_{t-1} + (1 - f) c, p_t = bf16(g h_t).
 * state [B][d] holds h_0 on entry and h_T on return; p is bf16 [B][T][d].
 * Readings in oracle.c. */
void orc_mlgru_scan(const double* z, int64_t B, int64_t T, int64_t d, double* state,
                    uint16_t* p);

/* MLGRU token mixer: z = BitLinear(x; g_in, w_in [3d][d], gamma_in), the
 * recurrence above, y = BitLinear(p; g_out, w_out [d][d], gamma_out).
 * x bf16 [B][T][d], y fp64 [B][T][d], state as above, p_out (bf16
 * [B][T][d]) may be NULL. */
void orc_mlgru_ternary(const uint16_t* x, const float* g_in, const int8_t* w_in,
                       float gamma_in, const float* g_out, const int8_t* w_out,
                       float gamma_out, int64_t B, int64_t T, int64_t d, float eps,
                       double* state, double* y, uint16_t* p_out);

/* The same from the fp32 master weights W_in [3d][d] and W_out [d][d]. */
void orc_mlgru(const uint16_t* x, const float* g_in, const float* W_in, const float* g_out,
               const float* W_out, int64_t B, int64_t T, int64_t d, float eps, double* state,
               double* y, uint16_t* p_out);

/* One layer: u = bf16(x + MLGRU(x)), out = bf16(u + GLU(u)) (bf16 [B][T][d]);
 * the GLU as orc_glu_ternary with inner size F. */
void orc_lm_layer_ternary(const uint16_t* x, const float* g_in, const int8_t* w_in,
                          float gamma_in, const float* g_out, const int8_t* w_out,
                          float gamma_out, const float* g_gu, const int8_t* w_gu,
                          float gamma_gu, const float* g_down, const int8_t* w_down,
                          float gamma_down, int64_t B, int64_t T, int64_t d, int64_t F,
                          float eps, double* state, uint16_t* out, uint16_t* u_out);

/* Backward pass of BitLinear with the straight-through estimator, from a
 * ternarised w and its gamma: given dy [M][N] (fp32), writes dx [M][K],
 * dg [K] and dW [N][K] (fp64).  Readings in oracle.c. */
void orc_bitlinear_backward(const uint16_t* x, const float* g, const int8_t* w,
                            float gamma, const float* dy, int64_t M, int64_t N,
                            int64_t K, float eps, double* dx, double* dg, double* dW);

#endif
