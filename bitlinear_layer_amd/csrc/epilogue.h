// epilogue.h -- the rescale / GLU epilogue shared by the GEMV and MFMA kernels.
//
// The kernels accumulate sum_k q * c with c = w + 1 (the packed code), so the
// ternary accumulation is acc = sum_k q c - sum_k q ([ld246, "三值权重的应用"]:
// +1 adds, -1 subtracts, 0 skips -- the same integer, exactly).  Then
// [datacamp, "Các thành phần lõi: MLGRU và GLU", panel "MatMul vs scaled
// ternary accumulation"]: y = float(acc) * (gamma / s).  The GLU epilogue
// ([datacamp, same section]; [jiqizhixin, "MatMul-free 语言模型架构"]) forms
// h = bf16(SiLU(gate) * up) from the two accumulations of one (m, f).
#pragma once

#include "device_common.h"
#include "launch.h"

namespace bl {

__device__ __forceinline__ float rescale(int32_t acc, float c) { return (float)acc * c; }

// SiLU(v) = v * sigmoid(v), with e = e^-|v| = 2^(-|v| log2 e) in (0, 1] from
// v_exp_f32 and the reciprocal of 1 + e (in (1, 2]) from v_rcp_f32:
// sigmoid(|v|) = 1 / (1 + e) and sigmoid(-|v|) = e / (1 + e). Nothing can
// overflow; for large negative v the result tends to -0 as e underflows.
// Each step is within about 1 fp32 ulp, apart from the rounding of
// -|v| log2 e, whose effect on the result is near a * 2^-24 relative for
// v = -a < 0 — far below the half-ulp of the bf16 the product is stored in.
__device__ __forceinline__ float silu_f32(float v) {
    constexpr float kNegLog2e = -1.44269502e+00f;   // -log2(e) rounded to fp32
    const float e = __builtin_amdgcn_exp2f(fabsf(v) * kNegLog2e);
    const float q = __builtin_amdgcn_rcpf(1.0f + e);
    return v * (v < 0.0f ? e * q : q);
}

__device__ __forceinline__ uint16_t glu_bf16(float zg, float zu) {
    return (uint16_t)f32_to_bf16_bits(silu_f32(zg) * zu);
}

// sigmoid(v) and 1 - sigmoid(v) = sigmoid(-v), each from e = 2^(-|v| log2 e)
// in (0, 1] and the reciprocal of 1 + e (as silu_f32 does): for v >= 0,
// sigmoid(v) = 1 / (1 + e) and sigmoid(-v) = e / (1 + e); mirrored for
// v < 0.  Neither value is formed as 1 - x, so both keep their relative
// precision when the other is close to 1.
__device__ __forceinline__ void sigmoid_pair(float v, float& s, float& oms) {
    constexpr float kNegLog2e = -1.44269502e+00f;
    const float e = __builtin_amdgcn_exp2f(fabsf(v) * kNegLog2e);
    const float q = __builtin_amdgcn_rcpf(1.0f + e);
    const float eq = e * q;
    s = v < 0.0f ? eq : q;
    oms = v < 0.0f ? q : eq;
}

// One token of the MLGRU recurrence for one channel ([datacamp, "Các thành
// phần lõi: MLGRU và GLU"]: gates in (0, 1) mix the previous state and the
// current token): forget gate f = sigmoid(zf), candidate c = SiLU(zc),
// output gate g = sigmoid(zg); h = f h + (1 - f) c; returns bf16(g h).
__device__ __forceinline__ uint32_t mlgru_token(float zf, float zc, float zg, float& h) {
    float f, omf, g, omg;
    sigmoid_pair(zf, f, omf);
    sigmoid_pair(zg, g, omg);
    h = fmaf(f, h, omf * silu_f32(zc));
    return f32_to_bf16_bits(g * h);
}

}  // namespace bl
