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

__device__ __forceinline__ uint16_t glu_bf16(float zg, float zu) {
    const float silu = zg / (1.0f + expf(-zg));
    return (uint16_t)f32_to_bf16_bits(silu * zu);
}

}  // namespace bl
