// Weight-side kernels: the fp32 -> bf16 operand cast of a fast-weight set,
// and the deterministic reduction of the per-chunk partial gradients into
// the stepped, optionally row-renormalised weights.
//
// The step follows the review of ZipMap (kimjy99.github.io), Method 2:
// W' = W - g with g the chunk gradient of Eq. (3) (the partials hold -g), and
// the norm-preserving rescale shown after Eq. (3), read per row: row r of W'
// is scaled by ||W_r|| / max(||W'_r||, 1e-12).  The LaCT summary (mhpn.cn,
// part 二, 2、架构) likewise normalises after summing the chunk's gradients.
#include "zm_internal.h"

namespace zm {

// One thread per element of the [H][h][d] index space.
__global__ __launch_bounds__(256) void k_cast(const float* __restrict__ w1,
                                              const float* __restrict__ w2,
                                              const float* __restrict__ w3, int heads, int d,
                                              int h, WSet out) {
  const int64_t total = (int64_t)heads * h * d;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  out.w1b[i] = to_bf16(kNegLog2e * w1[i]);
  out.w3b[i] = to_bf16(w3[i]);
  out.w2b[i] = to_bf16(kNegInvLog2e * w2[i]);  // same element count, [H][d][h] order
  const int64_t hd = i / ((int64_t)h * d);
  const int64_t rem = i - hd * h * d;
  const int64_t j = rem / d, c = rem - j * d;
  out.w2tb[i] = to_bf16(w2[(hd * d + c) * h + j]);  // w2tb[hd][j][c] = W2[hd][c][j]
}

hipError_t launch_cast(const float* w1, const float* w2, const float* w3, int heads, int d, int h,
                       WSet out, hipStream_t st) {
  const int64_t total = (int64_t)heads * h * d;
  const unsigned blocks = (unsigned)ceil_div(total, 256);
  hipLaunchKernelGGL(k_cast, dim3(blocks), dim3(256), 0, st, w1, w2, w3, heads, d, h, out);
  return hipGetLastError();
}

__device__ __forceinline__ float wave_sum(float x) {
  // Butterfly: every lane ends with the same bits (each step adds the same
  // pair of operands on both partner lanes).
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// One wave per weight row.  Rows of a head: h rows of W1 (length d), h rows
// of W3 (length d), d rows of W2 (length h).  part: [S][H][3][h*d] with the
// three matrices in their natural layouts ([h][d], [h][d], [d][h]).
template <int MAXE>
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int splits,
                                                int heads, int d, int h,
                                                const float* w1, const float* w2,
                                                const float* w3, float* o1, float* o2,
                                                float* o3, int renorm, WSet ob, int emit_bf16) {
  const int rows_per_head = 2 * h + d;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= heads * rows_per_head) return;
  const int head = wave / rows_per_head;
  const int r = wave - head * rows_per_head;
  int mat, row, len;
  if (r < h) {
    mat = 0; row = r; len = d;
  } else if (r < 2 * h) {
    mat = 1; row = r - h; len = d;
  } else {
    mat = 2; row = r - 2 * h; len = h;
  }
  const float* win = mat == 0 ? w1 : (mat == 1 ? w3 : w2);
  float* wout = mat == 0 ? o1 : (mat == 1 ? o3 : o2);
  const int64_t hd_elems = (int64_t)h * d;
  const int64_t base = (int64_t)head * hd_elems + (int64_t)row * len;
  const float* pbase = part + ((int64_t)head * 3 + mat) * hd_elems + (int64_t)row * len;
  const int64_t pstride = (int64_t)heads * 3 * hd_elems;
  const int ne = len / 64;

  float wv[MAXE], nv[MAXE];
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    wv[e] = 0.f;
    nv[e] = 0.f;
    if (e < ne) {
      const int col = lane + 64 * e;
      float s = 0.f;
      for (int si = 0; si < splits; ++si) s += pbase[si * pstride + col];  // fixed order
      wv[e] = win[base + col];
      nv[e] = wv[e] + s;
    }
  }
  if (renorm) {
    float so = 0.f, sn = 0.f;
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
      so = fmaf(wv[e], wv[e], so);
      sn = fmaf(nv[e], nv[e], sn);
    }
    so = wave_sum(so);
    sn = wave_sum(sn);
    // Same code on identical values: an unchanged row gets scale exactly 1.
    const float scale = sqrtf(so) / fmaxf(sqrtf(sn), 1e-12f);
#pragma unroll
    for (int e = 0; e < MAXE; ++e) nv[e] *= scale;
  }
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    if (e < ne) {
      const int col = lane + 64 * e;
      wout[base + col] = nv[e];
      if (emit_bf16) {
        if (mat == 0) {
          ob.w1b[base + col] = to_bf16(kNegLog2e * nv[e]);
        } else if (mat == 1) {
          ob.w3b[base + col] = to_bf16(nv[e]);
        } else {
          ob.w2b[base + col] = to_bf16(kNegInvLog2e * nv[e]);
          ob.w2tb[((int64_t)head * h + col) * d + row] = to_bf16(nv[e]);
        }
      }
    }
  }
}

hipError_t launch_reduce(const float* part, int splits, int heads, int d, int h,
                         const float* w1, const float* w2, const float* w3, float* o1,
                         float* o2, float* o3, int renorm, const WSet* out_bf16,
                         hipStream_t st) {
  const int rows = heads * (2 * h + d);
  const unsigned blocks = (unsigned)ceil_div(rows, 4);
  WSet ob = out_bf16 ? *out_bf16 : WSet{nullptr, nullptr, nullptr, nullptr};
  const int emit = out_bf16 ? 1 : 0;
  const int maxlen = h > d ? h : d;
  if (maxlen <= 128) {
    hipLaunchKernelGGL(k_reduce<2>, dim3(blocks), dim3(256), 0, st, part, splits, heads, d, h,
                       w1, w2, w3, o1, o2, o3, renorm, ob, emit);
  } else {
    hipLaunchKernelGGL(k_reduce<4>, dim3(blocks), dim3(256), 0, st, part, splits, heads, d, h,
                       w1, w2, w3, o1, o2, o3, renorm, ob, emit);
  }
  return hipGetLastError();
}

}  // namespace zm
