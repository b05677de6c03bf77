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

// The reduction products leave each partial slot transposed: per head, the
// slot holds [D1; D3]^T as a row-major d x 2h matrix, then D2^T as h x d (the
// library runs those orientations faster).  This kernel adds the S slots in
// slot order and writes the sum in the natural layouts, [D1; D3] (2h x d)
// and D2 (d x h), to sum[heads][3][h d]: one 64 x 64 tile per workgroup,
// transposed through LDS (row pitch 65: the tile's writes and its transposed
// reads are both free of bank conflicts).  Tiles 0 .. 2h d / 4096 - 1 of
// each head belong to the first matrix, the rest to the second.
template <int D, int HID>
__global__ __launch_bounds__(256) void k_wide_tsum(const float* __restrict__ part, int splits,
                                                   int heads, float* __restrict__ sum) {
  constexpr int64_t HD = (int64_t)HID * D;
  constexpr int T13 = (D / 64) * (2 * HID / 64);
  __shared__ float tile[64][65];
  const int head = blockIdx.y;
  int t = blockIdx.x;
  const bool m2 = t >= T13;
  if (m2) t -= T13;
  // input matrix R x C (row-major), output C x R
  const int R = m2 ? HID : D, C = m2 ? D : 2 * HID;
  const int64_t base = (int64_t)head * 3 * HD + (m2 ? 2 * HD : 0);
  const int r0 = 64 * (t / (C / 64)), c0 = 64 * (t % (C / 64));
  const int64_t pstride = (int64_t)heads * 3 * HD;
  const int tid = threadIdx.x, tr = tid >> 4, tc = 4 * (tid & 15);
  const float* src = part + base + (int64_t)(r0 + tr) * C + c0 + tc;
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // slots in groups of two, four rows each: eight loads in flight, added in
  // slot order
  for (int s0 = 0; s0 < splits; s0 += 2) {
    f32x4 v[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (s0 + k < splits) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[k][i] = *(const f32x4*)(src + (int64_t)(s0 + k) * pstride + (int64_t)16 * i * C);
      }
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (s0 + k < splits) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += v[k][i];
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) tile[tr + 16 * i][tc + k] = acc[i][k];
  __syncthreads();
  float* dst = sum + base + (int64_t)(c0 + tr) * R + r0 + tc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cc = tr + 16 * i;
    *(f32x4*)(dst + (int64_t)16 * i * R) =
        f32x4{tile[tc][cc], tile[tc + 1][cc], tile[tc + 2][cc], tile[tc + 3][cc]};
  }
}

hipError_t launch_wide_tsum(const float* part, int splits, int heads, int d, int h, float* sum,
                            hipStream_t st) {
  if (d != 1024 || h != 2048) return hipErrorInvalidValue;
  const unsigned tiles = (unsigned)((d / 64) * (2 * h / 64) + (h / 64) * (d / 64));
  hipLaunchKernelGGL((k_wide_tsum<1024, 2048>), dim3(tiles, (unsigned)heads), dim3(256), 0, st,
                     part, splits, heads, sum);
  return hipGetLastError();
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
