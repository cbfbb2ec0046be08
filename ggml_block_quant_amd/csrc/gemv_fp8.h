// gemv_fp8.h -- the one-shot GEMV for FP8 E4M3 weights with per-row fp32
// scales (page "Quantization types", section "FP8": weight-only FP8 with
// 16-bit activations).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

// Y[m][n] = s[n] * sum_k e4m3(code[n][k]) * X[m][k] for one or two tokens.
// Returns false (nothing launched) where the shape needs the generic
// kernel: M > 2, K > 16384 (one token) or K > 8192 (two tokens); else
// launches and sets e to the launch status.
bool launch_gemv_fp8(const uint8_t *blocks, const uint16_t *X, float *Y, int M, int64_t N, int64_t K,
                     hipStream_t s, hipError_t &e);

}  // namespace ql
