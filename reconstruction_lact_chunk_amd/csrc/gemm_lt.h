// Plain GEMMs through hipBLASLt (bf16 operands, fp32 accumulation), row-major
// helpers.  Failures return false and record the reason (zm_ttt_last_error).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "zm_internal.h"

namespace zm {

constexpr size_t kLtWorkspace = (size_t)64 << 20;  // GEMM library workspace per call

struct LtWs {
  void* p;
  size_t bytes;
};

// Row-major C (M x N, ldc) = A (M x K, lda) B (N x K, ldb)^T, plus beta C; C bf16
// or fp32; `count` products with element strides sa (A), sb (B), sc (C).
bool lt_rm_nt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb, void* C, int64_t ldc, bool out_f32, LtWs ws, hipStream_t st,
              int count = 1, int64_t sa = 0, int64_t sb = 0, int64_t sc = 0, float beta = 0.f);

// Row-major C (M x N, ldc) = A (K x M, lda)^T B (K x N, ldb), plus beta C;
// `count` products with element strides sa (A), sb (B), sc (C).
bool lt_rm_tn(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb, void* C, int64_t ldc, bool out_f32, LtWs ws, hipStream_t st,
              int count = 1, int64_t sa = 0, int64_t sb = 0, int64_t sc = 0, float beta = 0.f);

}  // namespace zm
