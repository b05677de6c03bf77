// Reduction kernel of the full-width fast weight (one head of d = 1024, hidden
// h = 2048: the 6 d^2 state of the ZipMap paper-reading notes' state-size
// paragraph): k_wide_reduce, the fixed-order sum of the block partials, the
// step, the row renorm and the bf16 operand copies, one workgroup per weight
// row (rows of 1024 or 2048 elements).  Formulas: review of ZipMap
// (kimjy99.github.io), Method 2, Eq. (1)-(4) and the renormalised update
// display after Eq. (3).
#include "wide_path.h"

namespace zm {

// Sum over the 256 threads of a workgroup, the same bits on every thread:
// butterflies within each wave, then the four wave sums in a fixed order.
__device__ __forceinline__ float block_sum256(float x, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();  // earlier readers of red are done
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// One workgroup of 256 threads per weight row: rows of W1 and W3 (length d)
// and of W2 (length h), heads x (2 h + d) rows.  Partials: [S][heads][3][h d]
// (W1, W3 as [h][d], W2 as [d][h]).  Adds the S slots in order to W, rescales
// the row to its pre-update norm when renorm is set (guard max(., 1e-12)),
// writes W_hat and, when emit is set, the bf16 operand copies.
template <int EPT>  // elements per thread: row length / 256
__device__ __forceinline__ void wide_row(const float* __restrict__ part, int splits,
                                         int64_t pstride, int64_t e0, const float* win,
                                         float* wout, int renorm, float* red, float (&nv)[EPT]) {
  const int tid = threadIdx.x;
  float so = 0.f, sn = 0.f;
#pragma unroll
  for (int q = 0; q < EPT; q += 4) {
    const int64_t off = 4 * tid + 1024 * (q / 4);
    const f32x4 wv = *(const f32x4*)(win + off);
    const f32x4 sum = sum_slots(part + e0 + off, pstride, splits);
    const f32x4 n4 = wv + sum;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      nv[q + r] = n4[r];
      so = fmaf(wv[r], wv[r], so);
      sn = fmaf(n4[r], n4[r], sn);
    }
  }
  if (renorm) {
    so = block_sum256(so, red);
    sn = block_sum256(sn, red);
    const float scale = sqrtf(so) / fmaxf(sqrtf(sn), 1e-12f);
#pragma unroll
    for (int q = 0; q < EPT; ++q) nv[q] *= scale;
  }
#pragma unroll
  for (int q = 0; q < EPT; q += 4) {
    const int64_t off = 4 * tid + 1024 * (q / 4);
    *(f32x4*)(wout + off) = f32x4{nv[q], nv[q + 1], nv[q + 2], nv[q + 3]};
  }
}

template <int D, int HID>
__global__ __launch_bounds__(256) void k_wide_reduce(const float* __restrict__ part, int splits,
                                                     int heads, const float* w1, const float* w2,
                                                     const float* w3, float* o1, float* o2,
                                                     float* o3, int renorm, WSet ob,
                                                     int emit_bf16) {
  __shared__ float red[4];
  constexpr int64_t HD = (int64_t)HID * D;
  const int rows_per_head = 2 * HID + D;
  const int head = blockIdx.x / rows_per_head;
  const int r = blockIdx.x - head * rows_per_head;
  const int64_t pstride = (int64_t)heads * 3 * HD;
  const int tid = threadIdx.x;
  if (r < 2 * HID) {  // a row of W1 (r < h) or W3, length d
    const int mat = r < HID ? 0 : 1;
    const int j = r - mat * HID;
    const int64_t off = (int64_t)head * HD + (int64_t)j * D;
    const int64_t e0 = (int64_t)head * 3 * HD + mat * HD + (int64_t)j * D;
    float nv[D / 256];
    wide_row<D / 256>(part, splits, pstride, e0, (mat == 0 ? w1 : w3) + off,
                      (mat == 0 ? o1 : o3) + off, renorm, red, nv);
    if (emit_bf16) {
      uint16_t* dst = (mat == 0 ? ob.w1b : ob.w3b) + off;
      const float f = mat == 0 ? kNegLog2e : 1.f;
#pragma unroll
      for (int q = 0; q < D / 256; q += 4) {
        const int c = 4 * tid + 1024 * (q / 4);
        *(u32x2*)(dst + c) =
            u32x2{pack_bf16x2(f * nv[q], f * nv[q + 1]), pack_bf16x2(f * nv[q + 2], f * nv[q + 3])};
      }
    }
  } else {  // a row c of W2, length h
    const int c = r - 2 * HID;
    const int64_t off = (int64_t)head * HD + (int64_t)c * HID;
    const int64_t e0 = (int64_t)head * 3 * HD + 2 * HD + (int64_t)c * HID;
    float nv[HID / 256];
    wide_row<HID / 256>(part, splits, pstride, e0, w2 + off, o2 + off, renorm, red, nv);
    if (emit_bf16) {
#pragma unroll
      for (int q = 0; q < HID / 256; q += 4) {
        const int j = 4 * tid + 1024 * (q / 4);
        *(u32x2*)(ob.w2b + off + j) =
            u32x2{pack_bf16x2(kNegInvLog2e * nv[q], kNegInvLog2e * nv[q + 1]),
                  pack_bf16x2(kNegInvLog2e * nv[q + 2], kNegInvLog2e * nv[q + 3])};
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          ob.w2tb[((int64_t)head * HID + j + r4) * D + c] = to_bf16(nv[q + r4]);
      }
    }
  }
}

hipError_t launch_wide_reduce(const float* part, int splits, int heads, int d, int h,
                              const float* w1, const float* w2, const float* w3, float* o1,
                              float* o2, float* o3, int renorm, const WSet* out_bf16,
                              hipStream_t st) {
  if (d != 1024 || h != 2048) return hipErrorInvalidValue;
  const WSet ob = out_bf16 ? *out_bf16 : WSet{nullptr, nullptr, nullptr, nullptr};
  hipLaunchKernelGGL((k_wide_reduce<1024, 2048>), dim3(heads * (2 * h + d)), dim3(256), 0, st,
                     part, splits, heads, w1, w2, w3, o1, o2, o3, renorm, ob,
                     out_bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace zm
