/*
 * oracle.c -- plain, slow CPU definition of the BitLinear forward pass (and
 * of its straight-through backward, at the end of the file).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the library.  It is written
 * from the method's definition, one step per function, in the order the
 * pages give (RMSNorm -> quantise -> ternary add/subtract -> rescale), with
 * no blocking, fusion or reordering.  Source tags ([ld246], [jiqizhixin],
 * [datacamp]) are expanded in oracle.h.
 *
 * Build: gcc -std=c11 -O2 (ISO mode: no FMA contraction, no fast-math), so
 * every fp32 expression below rounds once per operation, round-half-even.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 <-> float                                                            */
/* ------------------------------------------------------------------------ */

/* A bf16 value is the top 16 bits of the fp32 value with the same sign,
 * exponent and leading 7 fraction bits, so widening is exact. */
float orc_bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Nearest bf16 to v, ties to even, from the definition: bf16 carries 8
 * significant bits, so the spacing of representable values at |v| in
 * [2^(e-1), 2^e) is 2^(e-8), and never below the subnormal spacing 2^-133.
 * Round |v| to a whole number of spacings, then read the bit pattern off the
 * (exactly representable) fp32 value.  Inf/NaN are outside the contract. */
uint16_t orc_double_to_bf16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);              /* a = f * 2^e, 0.5 <= f < 1 */
    int qe = e - 8;
    if (qe < -133) qe = -133;
    double n = rint(ldexp(a, -qe));  /* default rounding mode: ties to even */
    float f = (float)ldexp(n, qe);   /* exact: at most 9 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------------------------------ */
/* Weights: absmean ternarisation and 2-bit storage                          */
/* ------------------------------------------------------------------------ */

/* [datacamp, "Thay MatMul bằng các phép toán tam phân"]: the weight scale is
 * the mean absolute value of the matrix ("its" mean, one scalar per
 * matrix).  Reading: the sum is taken in fp64 in row-major order, divided in
 * fp64 and rounded once to fp32. */
float orc_absmean_gamma(const float* W, int64_t N, int64_t K) {
    double sum = 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            sum += fabs((double)W[n * K + k]);
    return (float)(sum / (double)(N * K));
}

/* [datacamp, same section]: each weight is scaled by the matrix's mean
 * absolute value and rounded to the nearest of -1, 0, +1; [ld246,
 * "三值权重的应用"] restricts weights to {-1, 0, +1}.  Readings: the scaling
 * divides by gamma + 1e-5 (the page's "multiply" would send almost every
 * weight to 0), the division and the rounding are fp32, ties go to even. */
void orc_ternarize(const float* W, int64_t N, int64_t K, float gamma, int8_t* w) {
    float d = gamma + 1e-5f;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            float t = rintf(W[n * K + k] / d);
            if (t > 1.0f) t = 1.0f;
            if (t < -1.0f) t = -1.0f;
            w[n * K + k] = (int8_t)t;
        }
    }
}

/* Storage format (the pages give none; this is the library's own):
 *   - row n of w occupies K/4 bytes, rows back to back; K % 16 == 0;
 *   - along a row, weights go in groups of 16 (k = 16*grp + j, j = 0..15);
 *     group grp lives in bytes 4*grp .. 4*grp+3 of the row;
 *   - weight j = 4*i + t of a group sits in byte 4*grp + t, bits 2i+1..2i;
 *   - the 2-bit code is w + 1: 0 -> -1, 1 -> 0, 2 -> +1; code 3 is unused.
 * The function reads the format straight off this description. */
static int64_t orc_code_byte(int64_t K, int64_t n, int64_t k) {
    int64_t grp = k / 16, j = k % 16, t = j % 4;
    return n * (K / 4) + 4 * grp + t;
}
static int orc_code_shift(int64_t k) {
    int64_t j = k % 16, i = j / 4;
    return (int)(2 * i);
}

int orc_pack(const int8_t* w, int64_t N, int64_t K, uint8_t* packed) {
    if (K % 16 != 0) return -1;
    memset(packed, 0, (size_t)(N * (K / 4)));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int v = w[n * K + k];
            if (v < -1 || v > 1) return -1;
            uint8_t code = (uint8_t)(v + 1);
            packed[orc_code_byte(K, n, k)] |= (uint8_t)(code << orc_code_shift(k));
        }
    }
    return 0;
}

int orc_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* w) {
    if (K % 16 != 0) return -1;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int code = (packed[orc_code_byte(K, n, k)] >> orc_code_shift(k)) & 3;
            if (code == 3) return -1;
            w[n * K + k] = (int8_t)(code - 1);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Activations: RMSNorm then per-token absmax int8                            */
/* ------------------------------------------------------------------------ */

/* [datacamp, "Các thành phần lõi: MLGRU và GLU", figure panel "RMS norm"]:
 * activations are RMS-normalised before quantisation; [ld246, "融合
 * BitLinear 层的创新"] and [jiqizhixin, Algorithm 1 title]: the quantisation
 * follows RMSNorm inside BitLinear.  Readings (pages silent):
 *   RMSNorm:  r = 1 / sqrt(mean(x^2) + eps), xn = (x * r) * g;
 *             sum of squares in fp64 (k ascending), mean rounded to fp32,
 *             then fp32 add, sqrt and divide (each correctly rounded);
 *   quantise: per token (row), symmetric absmax to 127:
 *             s = 127 / max(max|xn|, 1e-5), q = clip(round(xn * s), -128, 127),
 *             fp32, round half to even. */
void orc_rmsnorm_quant(const uint16_t* x, const float* g, int64_t M, int64_t K,
                       float eps, int8_t* q, float* s) {
    float* xn = (float*)malloc((size_t)K * sizeof(float));
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)orc_bf16_to_float(row[k]);
            ss += v * v;
        }
        float ms = (float)(ss / (double)K);
        float r = 1.0f / sqrtf(ms + eps);
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            xn[k] = (orc_bf16_to_float(row[k]) * r) * g[k];
            float a = fabsf(xn[k]);
            if (a > amax) amax = a;
        }
        float scale = 127.0f / (amax > 1e-5f ? amax : 1e-5f);
        for (int64_t k = 0; k < K; ++k) {
            float v = rintf(xn[k] * scale);
            if (v > 127.0f) v = 127.0f;
            if (v < -128.0f) v = -128.0f;
            q[m * K + k] = (int8_t)v;
        }
        s[m] = scale;
    }
    free(xn);
}

/* ------------------------------------------------------------------------ */
/* Ternary accumulation and rescale                                          */
/* ------------------------------------------------------------------------ */

/* [ld246, "三值权重的应用"]: weight +1 adds the input, -1 subtracts it, 0
 * does nothing; [jiqizhixin, "具有三值权重的 MatMul-free 密集层"]: the
 * ternary product is written with additions and subtractions only. */
void orc_ternary_accumulate(const int8_t* q, const int8_t* w, int64_t M, int64_t N,
                            int64_t K, int32_t* acc) {
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t a = 0;
            for (int64_t k = 0; k < K; ++k) {
                if (w[n * K + k] == 1)
                    a += q[m * K + k];
                else if (w[n * K + k] == -1)
                    a -= q[m * K + k];
            }
            acc[m * N + n] = a;
        }
    }
}

/* [datacamp, figure panel "MatMul vs scaled ternary accumulation"]: the
 * integer accumulation is scaled back.  Reading: q ~= s * xn and W ~= gamma
 * * w, so y = acc * gamma / s; no bias. */
void orc_rescale(const int32_t* acc, float gamma, const float* s, int64_t M,
                 int64_t N, double* y) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (double)acc[m * N + n] * (double)gamma / (double)s[m];
}

/* ------------------------------------------------------------------------ */
/* Compositions                                                              */
/* ------------------------------------------------------------------------ */

void orc_bitlinear_ternary(const uint16_t* x, const float* g, const int8_t* w,
                           float gamma, int64_t M, int64_t N, int64_t K, float eps,
                           double* y, int8_t* q_out, float* s_out, int32_t* acc_out) {
    int8_t* q = q_out ? q_out : (int8_t*)malloc((size_t)(M * K));
    float* s = s_out ? s_out : (float*)malloc((size_t)M * sizeof(float));
    int32_t* acc = acc_out ? acc_out : (int32_t*)malloc((size_t)(M * N) * sizeof(int32_t));
    orc_rmsnorm_quant(x, g, M, K, eps, q, s);
    orc_ternary_accumulate(q, w, M, N, K, acc);
    orc_rescale(acc, gamma, s, M, N, y);
    if (!q_out) free(q);
    if (!s_out) free(s);
    if (!acc_out) free(acc);
}

void orc_bitlinear(const uint16_t* x, const float* g, const float* W, int64_t M,
                   int64_t N, int64_t K, float eps, double* y, float* gamma_out,
                   int8_t* w_out, int8_t* q_out, float* s_out, int32_t* acc_out) {
    int8_t* w = w_out ? w_out : (int8_t*)malloc((size_t)(N * K));
    float gamma = orc_absmean_gamma(W, N, K);
    orc_ternarize(W, N, K, gamma, w);
    orc_bitlinear_ternary(x, g, w, gamma, M, N, K, eps, y, q_out, s_out, acc_out);
    if (gamma_out) *gamma_out = gamma;
    if (!w_out) free(w);
}

/* [datacamp, "Các thành phần lõi: MLGRU và GLU"]: the input goes through two
 * BitLinear layers, one output passes SiLU and is multiplied element-wise by
 * the other, and a third BitLinear maps the result to the output;
 * [jiqizhixin, "MatMul-free 语言模型架构"]: the GLU channel mixer is built from
 * BitLinear only.  Readings: gate and up are one fused [2F][D] matrix with
 * one gamma (gate = rows 0..F-1), SiLU(v) = v / (1 + exp(-v)) in fp64, and
 * the product is stored as bf16 (activations between layers are BF16,
 * [jiqizhixin, "MatMul-free 语言模型的扩展规律"]) before the down layer, which
 * applies its own RMSNorm and quantisation.  The other reading of "two
 * BitLinear layers" -- a gamma and an RMSNorm weight for each of gate and up
 * -- ternarises differently wherever the two gammas differ; it is not the
 * one implemented here. */
void orc_glu_ternary(const uint16_t* x, const float* g_gu, const int8_t* w_gu,
                     float gamma_gu, const float* g_down, const int8_t* w_down,
                     float gamma_down, int64_t M, int64_t D, int64_t F, float eps,
                     double* y, uint16_t* h_out) {
    double* z = (double*)malloc((size_t)(M * 2 * F) * sizeof(double));
    uint16_t* h = h_out ? h_out : (uint16_t*)malloc((size_t)(M * F) * sizeof(uint16_t));
    orc_bitlinear_ternary(x, g_gu, w_gu, gamma_gu, M, 2 * F, D, eps, z, NULL, NULL, NULL);
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t f = 0; f < F; ++f) {
            double gate = z[m * 2 * F + f];
            double up = z[m * 2 * F + F + f];
            double silu = gate / (1.0 + exp(-gate));
            h[m * F + f] = orc_double_to_bf16(silu * up);
        }
    }
    orc_bitlinear_ternary(h, g_down, w_down, gamma_down, M, D, F, eps, y, NULL, NULL, NULL);
    free(z);
    if (!h_out) free(h);
}

void orc_glu(const uint16_t* x, const float* g_gu, const float* W_gu,
             const float* g_down, const float* W_down, int64_t M, int64_t D,
             int64_t F, float eps, double* y, uint16_t* h_out) {
    int8_t* w_gu = (int8_t*)malloc((size_t)(2 * F * D));
    int8_t* w_down = (int8_t*)malloc((size_t)(D * F));
    float gamma_gu = orc_absmean_gamma(W_gu, 2 * F, D);
    float gamma_down = orc_absmean_gamma(W_down, D, F);
    orc_ternarize(W_gu, 2 * F, D, gamma_gu, w_gu);
    orc_ternarize(W_down, D, F, gamma_down, w_down);
    orc_glu_ternary(x, g_gu, w_gu, gamma_gu, g_down, w_down, gamma_down, M, D, F, eps,
                    y, h_out);
    free(w_gu);
    free(w_down);
}

/* ------------------------------------------------------------------------ */
/* MLGRU token mixer                                                         */
/* ------------------------------------------------------------------------ */

/* [datacamp, "Các thành phần lõi: MLGRU và GLU"]: the MLGRU takes the tokens
 * of a sequence one at a time; each step combines the current token's
 * embedding with the previous hidden state, the memory of earlier tokens,
 * through element-wise operations and gates -- vectors of values between 0
 * and 1 -- that decide how much of the previous state and of the current
 * token carry on; [jiqizhixin, "MatMul-free 语言模型架构"]: a ternary RNN of
 * element-wise products and accumulation, with the GRU as its base;
 * [ld246, "线性操作的引入"]: the GRU's matrix products become element-wise
 * operations (a linear GRU).  Readings (the pages print no equations):
 *   - the state enters element-wise only (no state-to-state product), so
 *     the gates are functions of the token alone, through BitLinear;
 *   - one BitLinear of the token gives z = [z_f | z_c | z_g]: rows 0..d-1,
 *     d..2d-1 and 2d..3d-1 of one [3d][d] ternary matrix with one gamma and
 *     one RMSNorm weight, as for the GLU's fused gate|up;
 *   - forget gate f = sigmoid(z_f), in (0, 1); candidate c = SiLU(z_c) (the
 *     activation the pages name for the model); output gate
 *     g = sigmoid(z_g);
 *   - h_t = f * h_{t-1} + (1 - f) * c, element-wise, from a given h_0 (zero
 *     for a new sequence);
 *   - p_t = g * h_t is stored as bf16 (the activation type between BitLinear
 *     layers) and mapped by a second BitLinear, [d][d], to the output.
 * Everything here is fp64. */
static double orc_sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }
static double orc_silu(double v) { return v / (1.0 + exp(-v)); }

void orc_mlgru_scan(const double* z, int64_t B, int64_t T, int64_t d, double* state,
                    uint16_t* p) {
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t n = 0; n < d; ++n) {
            double h = state[b * d + n];
            for (int64_t t = 0; t < T; ++t) {
                const double* zt = z + (b * T + t) * 3 * d;
                double f = orc_sigmoid(zt[n]);
                double c = orc_silu(zt[d + n]);
                double g = orc_sigmoid(zt[2 * d + n]);
                h = f * h + (1.0 - f) * c;
                p[(b * T + t) * d + n] = orc_double_to_bf16(g * h);
            }
            state[b * d + n] = h;
        }
    }
}

void orc_mlgru_ternary(const uint16_t* x, const float* g_in, const int8_t* w_in,
                       float gamma_in, const float* g_out, const int8_t* w_out,
                       float gamma_out, int64_t B, int64_t T, int64_t d, float eps,
                       double* state, double* y, uint16_t* p_out) {
    int64_t M = B * T;
    double* z = (double*)malloc((size_t)(M * 3 * d) * sizeof(double));
    uint16_t* p = p_out ? p_out : (uint16_t*)malloc((size_t)(M * d) * sizeof(uint16_t));
    orc_bitlinear_ternary(x, g_in, w_in, gamma_in, M, 3 * d, d, eps, z, NULL, NULL, NULL);
    orc_mlgru_scan(z, B, T, d, state, p);
    orc_bitlinear_ternary(p, g_out, w_out, gamma_out, M, d, d, eps, y, NULL, NULL, NULL);
    free(z);
    if (!p_out) free(p);
}

void orc_mlgru(const uint16_t* x, const float* g_in, const float* W_in, const float* g_out,
               const float* W_out, int64_t B, int64_t T, int64_t d, float eps, double* state,
               double* y, uint16_t* p_out) {
    int8_t* w_in = (int8_t*)malloc((size_t)(3 * d * d));
    int8_t* w_out = (int8_t*)malloc((size_t)(d * d));
    float gamma_in = orc_absmean_gamma(W_in, 3 * d, d);
    float gamma_out = orc_absmean_gamma(W_out, d, d);
    orc_ternarize(W_in, 3 * d, d, gamma_in, w_in);
    orc_ternarize(W_out, d, d, gamma_out, w_out);
    orc_mlgru_ternary(x, g_in, w_in, gamma_in, g_out, w_out, gamma_out, B, T, d, eps, state,
                      y, p_out);
    free(w_in);
    free(w_out);
}

/* ------------------------------------------------------------------------ */
/* One layer: token mixer, then channel mixer                                */
/* ------------------------------------------------------------------------ */

/* [jiqizhixin, "MatMul-free 语言模型架构"]: in the Metaformer view a layer is
 * a token mixer followed by a channel mixer; here the MLGRU and the GLU.
 * Readings: each mixer's output is added to its input (the residual
 * connections of a Metaformer block; the normalisation is the RMSNorm inside
 * each BitLinear), and the residual stream is bf16 between the mixers and
 * at the layer output:
 *   u = bf16(x + MLGRU(x)),   out = bf16(u + GLU(u)).
 * u_out (bf16 [B*T][d]) may be NULL. */
void orc_lm_layer_ternary(const uint16_t* x, const float* g_in, const int8_t* w_in,
                          float gamma_in, const float* g_out, const int8_t* w_out,
                          float gamma_out, const float* g_gu, const int8_t* w_gu,
                          float gamma_gu, const float* g_down, const int8_t* w_down,
                          float gamma_down, int64_t B, int64_t T, int64_t d, int64_t F,
                          float eps, double* state, uint16_t* out, uint16_t* u_out) {
    int64_t M = B * T;
    double* y = (double*)malloc((size_t)(M * d) * sizeof(double));
    uint16_t* u = u_out ? u_out : (uint16_t*)malloc((size_t)(M * d) * sizeof(uint16_t));
    orc_mlgru_ternary(x, g_in, w_in, gamma_in, g_out, w_out, gamma_out, B, T, d, eps, state,
                      y, NULL);
    for (int64_t i = 0; i < M * d; ++i)
        u[i] = orc_double_to_bf16((double)orc_bf16_to_float(x[i]) + y[i]);
    orc_glu_ternary(u, g_gu, w_gu, gamma_gu, g_down, w_down, gamma_down, M, d, F, eps, y,
                    NULL);
    for (int64_t i = 0; i < M * d; ++i)
        out[i] = orc_double_to_bf16((double)orc_bf16_to_float(u[i]) + y[i]);
    free(y);
    if (!u_out) free(u);
}

/* ------------------------------------------------------------------------ */
/* Backward pass through BitLinear (straight-through estimator)              */
/* ------------------------------------------------------------------------ */

/* [ld246, "训练与优化：新的策略"]: the ternary weights and the activation
 * quantisation are not differentiable, and training passes gradients
 * through them with the straight-through estimator; [ld246, "融合 BitLinear
 * 层的创新"]: the training-time layer fuses RMSNorm with the quantisation.
 * Readings (pages silent on the details):
 *   - both quantisers are the identity in the backward pass: the forward
 *     value is y = xq W~^T with xq = q / s (the dequantised activations) and
 *     W~ = gamma * w, and d xq / d xn = I, d W~ / d W = I (no clipping mask,
 *     gamma and s held constant);
 *   - hence, with dy the gradient of the loss with respect to y:
 *       dxn = dy W~ = gamma * dy w            (ternary add/subtract per n),
 *       dW  = dy^T xq,
 *     and the RMSNorm xn = x * r * g, r = (mean(x^2) + eps)^(-1/2), gives
 *       dg[k]   = sum_m dxn[m][k] * x[m][k] * r[m],
 *       dx[m][k] = r g[k] dxn[m][k] - x[m][k] r^3 / K * sum_j dxn[m][j] g[j] x[m][j];
 *   - q and s are the forward's own codes and scales (orc_rmsnorm_quant);
 *     everything else is fp64. */
void orc_bitlinear_backward(const uint16_t* x, const float* g, const int8_t* w,
                            float gamma, const float* dy, int64_t M, int64_t N,
                            int64_t K, float eps, double* dx, double* dg, double* dW) {
    int8_t* q = (int8_t*)malloc((size_t)(M * K) + 1);
    float* s = (float*)malloc((size_t)M * sizeof(float) + 1);
    double* dxn = (double*)malloc((size_t)(M * K) * sizeof(double) + 1);
    orc_rmsnorm_quant(x, g, M, K, eps, q, s);

    /* dxn = gamma * dy w: weight +1 adds dy, -1 subtracts it, 0 skips. */
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            double a = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const int wnk = w[n * K + k];
                if (wnk == 1)
                    a += (double)dy[m * N + n];
                else if (wnk == -1)
                    a -= (double)dy[m * N + n];
            }
            dxn[m * K + k] = (double)gamma * a;
        }
    }

    /* RMSNorm backward. */
    for (int64_t k = 0; k < K; ++k) dg[k] = 0.0;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double v = (double)orc_bf16_to_float(row[k]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)K + (double)eps);
        double S = 0.0;
        for (int64_t k = 0; k < K; ++k)
            S += dxn[m * K + k] * (double)g[k] * (double)orc_bf16_to_float(row[k]);
        for (int64_t k = 0; k < K; ++k) {
            double xv = (double)orc_bf16_to_float(row[k]);
            dg[k] += dxn[m * K + k] * xv * r;
            dx[m * K + k] = r * (double)g[k] * dxn[m * K + k] - xv * r * r * r * S / (double)K;
        }
    }

    /* dW = dy^T xq, xq = q / s. */
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            double a = 0.0;
            for (int64_t m = 0; m < M; ++m)
                a += (double)dy[m * N + n] * ((double)q[m * K + k] / (double)s[m]);
            dW[n * K + k] = a;
        }
    }
    free(q);
    free(s);
    free(dxn);
}
