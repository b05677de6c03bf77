// The per-element reduce/step/renorm of the partial gradient sums, shared by
// the reduce kernel (weights.hip) and the reduce workgroups of the shared
// read-and-update launch (frame_bf16.hip): both run this code on the same
// elements, so their results are equal bit for bit.
//
// The step follows the review of ZipMap (kimjy99.github.io), Method 2:
// W' = W - g with g the chunk gradient of Eq. (3) (the partials hold -g), and
// the norm-preserving rescale shown after Eq. (3), read per row: row r of W'
// is scaled by ||W_r|| / max(||W'_r||, 1e-12).
#pragma once

#include "zm_internal.h"

namespace zm {

// Sum over the TPR lanes of an aligned lane group (TPR a power of two <= 64)
// by butterfly: every lane of the group ends with the same bits, since each
// step adds the same two operands on both partner lanes.
template <int TPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// One thread per 4 consecutive elements of the [H][3][h*d] weight space (the
// partials' layout): rows of W1, W3 (length d) and W2 (length h) are
// contiguous, so the LEN / 4 threads of a row form an aligned lane group of
// one wave.  Each thread adds the S partials of its 4 elements in split order
// (fixed order: bitwise reproducible), forms W' = W + sum, and for renorm
// scales its row by ||W_row|| / max(||W'_row||, 1e-12) with both norms summed
// over the row's lane group.
template <int LEN>
__device__ __forceinline__ void reduce_row4(const float* __restrict__ part, int splits,
                                            int64_t pstride, int64_t e, const float* win,
                                            float* wout, int renorm, f32x4& nv) {
  const f32x4 wv = *(const f32x4*)(win);
  const f32x4 sum = sum_slots(part + e, pstride, splits);
  nv = wv + sum;
  if (renorm) {
    float so = 0.f, sn = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      so = fmaf(wv[q], wv[q], so);
      sn = fmaf(nv[q], nv[q], sn);
    }
    so = group_sum<LEN / 4>(so);
    sn = group_sum<LEN / 4>(sn);
    // Same code on identical values: an unchanged row gets scale exactly 1.
    const float scale = sqrtf(so) / fmaxf(sqrtf(sn), 1e-12f);
    nv *= scale;
  }
  *(f32x4*)(wout) = nv;
}

// The 1024 consecutive elements [e0, e0 + 1024) of the weight space (e0 a
// multiple of 1024, so they lie in one matrix: h d is a multiple of 1024 for
// every supported shape), by a group of 256 threads (t = 0 .. 255 within the
// group) with `tr` 1024 floats of LDS of its own.  W2 groups synchronise the
// whole workgroup once, so every group of a workgroup must take the same
// matrix.  With bad, the outputs are NaN (a failed wait upstream).
template <int D, int HID>
__device__ __forceinline__ void reduce_1k(const float* __restrict__ part, int splits, int heads,
                                          int64_t e0, int t, const ReduceOut& r, float* tr,
                                          bool bad = false) {
  constexpr int64_t HD = (int64_t)HID * D;
  static_assert(HD % 1024 == 0 && (HID == 128 || HID == 256), "groups within one matrix");
  const int64_t e = e0 + 4 * t;  // element index
  const int64_t head = e / (3 * HD);
  const int64_t rem = e - head * 3 * HD;
  const int mat = (int)(rem / HD);
  const int64_t local = rem - mat * HD;
  const int64_t off = head * HD + local;  // offset in the weight and bf16 arrays
  const int64_t pstride = (int64_t)heads * 3 * HD;
  f32x4 nv;
  if (mat == 2) {  // W2 rows have length h
    reduce_row4<HID>(part, splits, pstride, e, r.w2 + off, r.o2 + off, r.renorm, nv);
  } else {         // W1 / W3 rows have length d
    reduce_row4<D>(part, splits, pstride, e, (mat == 0 ? r.w1 : r.w3) + off,
                   (mat == 0 ? r.o1 : r.o3) + off, r.renorm, nv);
  }
  if (bad) {
    const float qn = __builtin_nanf("");
    nv = f32x4{qn, qn, qn, qn};
    *(f32x4*)((mat == 0 ? r.o1 : mat == 1 ? r.o3 : r.o2) + off) = nv;
  }
  if (!r.emit) return;
  const WSet& ob = r.ob;
  if (mat == 0) {
    u32x2 pk = {pack_bf16x2(kNegLog2e * nv[0], kNegLog2e * nv[1]),
                pack_bf16x2(kNegLog2e * nv[2], kNegLog2e * nv[3])};
    *(u32x2*)(ob.w1b + off) = pk;
  } else if (mat == 1) {
    u32x2 pk = {pack_bf16x2(nv[0], nv[1]), pack_bf16x2(nv[2], nv[3])};
    *(u32x2*)(ob.w3b + off) = pk;
  } else {
    u32x2 pk = {pack_bf16x2(kNegInvLog2e * nv[0], kNegInvLog2e * nv[1]),
                pack_bf16x2(kNegInvLog2e * nv[2], kNegInvLog2e * nv[3])};
    *(u32x2*)(ob.w2b + off) = pk;
    // Transposed copy w2tb[head][j][c] = W2[head][c][j] through LDS: the
    // group's 1024 elements are RW whole rows c0 .. c0 + RW - 1 of W2 (a row
    // block starts on a multiple of 1024 elements), so thread j writes rows'
    // column j as one RW-element piece of w2tb row j.
    constexpr int RW = 1024 / HID;
    *(f32x4*)&tr[4 * t] = nv;
    __syncthreads();
    if (t < HID) {
      const int64_t c0 = (local - 4 * (int64_t)t) / HID;
      unsigned pk2[RW / 2];
#pragma unroll
      for (int q = 0; q < RW; q += 2)
        pk2[q / 2] = (unsigned)to_bf16(tr[q * HID + t]) |
                     ((unsigned)to_bf16(tr[(q + 1) * HID + t]) << 16);
      uint16_t* dst = ob.w2tb + (head * HID + t) * D + c0;
      if constexpr (RW == 4) {
        *(u32x2*)dst = u32x2{pk2[0], pk2[1]};
      } else {
        *(u32x4*)dst = u32x4{pk2[0], pk2[1], pk2[2], pk2[3]};
      }
    }
  }
}

}  // namespace zm
