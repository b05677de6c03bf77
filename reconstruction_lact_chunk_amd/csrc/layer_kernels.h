// Launchers of the elementwise kernels around the TTT layer (layer_kernels.hip).
#pragma once

#include "zm_internal.h"

namespace zm {

// eta[t][h] = scale * sigmoid(y[t][col0 + h]), y bf16 rows of stride ldy.
hipError_t launch_eta_from_logits(const uint16_t* y, int64_t ldy, int64_t col0, int heads,
                                  float scale, float* eta, int64_t n, hipStream_t st);

// o[t] = RMSNorm(op[t]) * SiLU(g[t]) with RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma.
hipError_t launch_rmsnorm_gate(const uint16_t* op, int64_t ldo, const uint16_t* g, int64_t ldg,
                               const float* gamma, float eps, uint16_t* o, int64_t ldout,
                               int width, int64_t n, hipStream_t st);

}  // namespace zm
