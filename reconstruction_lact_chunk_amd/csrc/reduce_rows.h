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

// Global-memory access through a plain pointer: the weight pointers reach
// the kernels inside a struct, where the compiler cannot tell their address
// space and would emit flat accesses, which also hold up every later wait on
// LDS and scalar loads.
template <typename T>
__device__ __forceinline__ T gld(const void* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
template <typename T>
__device__ __forceinline__ void gst(void* p, T v) {
  *(__attribute__((address_space(1))) T*)p = v;
}

// Where thread t's 4 consecutive elements of the 1024-element group at e0
// lie (e0 a multiple of 1024, so the group lies in one matrix: h d is a
// multiple of 1024 for every supported shape).  e0 is uniform over the wave,
// so head and matrix are scalars.
struct RowPos {
  int64_t e;      // element index in the partials' layout [H][3][h d]
  int64_t head;
  int64_t local;  // index inside the matrix
  int64_t off;    // offset in the weight and bf16 arrays: head * h d + local
  int mat;        // 0: W1, 1: W3, 2: W2
};

template <int D, int HID>
__device__ __forceinline__ RowPos row_pos(int64_t e0, int t) {
  constexpr int64_t HD = (int64_t)HID * D;
  static_assert(HD % 1024 == 0 && (HID == 128 || HID == 256), "groups within one matrix");
  RowPos p;
  p.head = e0 / (3 * HD);
  const int64_t rem0 = e0 - p.head * 3 * HD;
  p.mat = (int)(rem0 / HD);
  p.local = rem0 - p.mat * HD + 4 * t;
  p.e = e0 + 4 * t;
  p.off = p.head * HD + p.local;
  return p;
}

// W's 4 elements at p (read before the partial sums, which may still be in
// flight elsewhere when the caller issues this load).
__device__ __forceinline__ f32x4 load_w(const RowPos& p, ReduceOut r) {
  return gld<f32x4>((p.mat == 0 ? r.w1 : p.mat == 1 ? r.w3 : r.w2) + p.off);
}

// The reduce of nu <= U groups of 1024 elements by one group of 256 threads
// (t = 0 .. 255 within the group), W's elements already in wv.  One thread
// per 4 consecutive elements of the [H][3][h*d] weight space (the partials'
// layout): rows of W1, W3 (length d) and W2 (length h) are contiguous, so the
// LEN / 4 threads of a row form an aligned lane group of one wave.  Each
// thread adds the S partials of its elements in split order (fixed order:
// bitwise reproducible; the loads of all nu groups are issued together),
// forms W' = W + sum, and for renorm scales its row by
// ||W_row|| / max(||W'_row||, 1e-12) with both norms summed over the row's
// lane group.  The emitted transposed W2 copy goes through LDS: `tr` holds
// 1024 floats per group, tr_stride apart, and the whole workgroup
// synchronises once when any group is in W2, so every group of 256 threads
// of a workgroup must take the same matrices.  With bad, the outputs are NaN
// (a failed wait upstream).
template <int D, int HID, int U>
__device__ __forceinline__ void reduce_groups(const float* __restrict__ part, int splits,
                                              int heads, const RowPos (&p)[U],
                                              const f32x4 (&wv)[U], int nu, int t,
                                              ReduceOut r, float* tr, int tr_stride,
                                              bool bad = false) {
  constexpr int64_t HD = (int64_t)HID * D;
  constexpr int G = 8;
  const int64_t pstride = (int64_t)heads * 3 * HD;
  f32x4 sum[U];
#pragma unroll
  for (int u = 0; u < U; ++u) sum[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += G) {
    f32x4 v[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < G; ++i)
        if (u < nu && s0 + i < splits)
          v[u][i] = *(const f32x4*)(part + p[u].e + (int64_t)(s0 + i) * pstride);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < G; ++i)
        if (u < nu && s0 + i < splits) sum[u] += v[u][i];
  }
  bool any_w2 = false;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= nu) continue;
    const int mat = p[u].mat;
    f32x4 nv = wv[u] + sum[u];
    if (r.renorm) {
      float so = 0.f, sn = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        so = fmaf(wv[u][q], wv[u][q], so);
        sn = fmaf(nv[q], nv[q], sn);
      }
      if (mat == 2) {  // W2 rows have length h
        so = group_sum<HID / 4>(so);
        sn = group_sum<HID / 4>(sn);
      } else {         // W1 / W3 rows have length d
        so = group_sum<D / 4>(so);
        sn = group_sum<D / 4>(sn);
      }
      // Same code on identical values: an unchanged row gets scale exactly 1.
      const float scale = sqrtf(so) / fmaxf(sqrtf(sn), 1e-12f);
      nv *= scale;
    }
    if (bad) {
      const float qn = __builtin_nanf("");
      nv = f32x4{qn, qn, qn, qn};
    }
    const int64_t off = p[u].off;
    gst<f32x4>((mat == 0 ? r.o1 : mat == 1 ? r.o3 : r.o2) + off, nv);
    if (!r.emit) continue;
    const WSet& ob = r.ob;
    if (mat == 0) {
      gst<u32x2>(ob.w1b + off, u32x2{pack_bf16x2(kNegLog2e * nv[0], kNegLog2e * nv[1]),
                                     pack_bf16x2(kNegLog2e * nv[2], kNegLog2e * nv[3])});
    } else if (mat == 1) {
      gst<u32x2>(ob.w3b + off, u32x2{pack_bf16x2(nv[0], nv[1]), pack_bf16x2(nv[2], nv[3])});
    } else {
      gst<u32x2>(ob.w2b + off, u32x2{pack_bf16x2(kNegInvLog2e * nv[0], kNegInvLog2e * nv[1]),
                                     pack_bf16x2(kNegInvLog2e * nv[2], kNegInvLog2e * nv[3])});
      *(f32x4*)&tr[u * tr_stride + 4 * t] = nv;
      any_w2 = true;
    }
  }
  if (!any_w2) return;
  // Transposed copy w2tb[head][j][c] = W2[head][c][j]: a group's 1024
  // elements are RW whole rows c0 .. c0 + RW - 1 of W2 (a row block starts on
  // a multiple of 1024 elements), so thread j writes rows' column j as one
  // RW-element piece of w2tb row j.
  constexpr int RW = 1024 / HID;
  __syncthreads();
  if (t >= HID) return;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= nu || p[u].mat != 2) continue;
    const float* tu = tr + u * tr_stride;
    const int64_t c0 = (p[u].local - 4 * (int64_t)t) / HID;
    unsigned pk2[RW / 2];
#pragma unroll
    for (int q = 0; q < RW; q += 2)
      pk2[q / 2] = (unsigned)to_bf16(tu[q * HID + t]) |
                   ((unsigned)to_bf16(tu[(q + 1) * HID + t]) << 16);
    uint16_t* dst = r.ob.w2tb + (p[u].head * HID + t) * D + c0;
    if constexpr (RW == 4) {
      gst<u32x2>(dst, u32x2{pk2[0], pk2[1]});
    } else {
      gst<u32x4>(dst, u32x4{pk2[0], pk2[1], pk2[2], pk2[3]});
    }
  }
}

}  // namespace zm
