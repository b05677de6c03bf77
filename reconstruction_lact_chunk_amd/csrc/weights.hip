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

// One launch, two kinds of workgroup.  The first n_vec workgroups write the
// scaled copies w1b, w3b, w2b, one thread per 4 consecutive elements (16-byte
// loads, 8-byte stores).  The others write the transposed copy
// w2tb[head][j][c] = W2[head][c][j] in 32 x 32 tiles through LDS, so both the
// reads and the writes are row-contiguous.
__global__ __launch_bounds__(256) void k_cast(const float* __restrict__ w1,
                                              const float* __restrict__ w2,
                                              const float* __restrict__ w3, int heads, int d,
                                              int h, WSet out, int n_vec) {
  if ((int)blockIdx.x < n_vec) {
    const int64_t total = (int64_t)heads * h * d;
    const int64_t i = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= total) return;
    const f32x4 a = *(const f32x4*)(w1 + i), b = *(const f32x4*)(w3 + i), c = *(const f32x4*)(w2 + i);
    *(u32x2*)(out.w1b + i) = u32x2{pack_bf16x2(kNegLog2e * a[0], kNegLog2e * a[1]),
                                   pack_bf16x2(kNegLog2e * a[2], kNegLog2e * a[3])};
    *(u32x2*)(out.w3b + i) = u32x2{pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
    *(u32x2*)(out.w2b + i) = u32x2{pack_bf16x2(kNegInvLog2e * c[0], kNegInvLog2e * c[1]),
                                   pack_bf16x2(kNegInvLog2e * c[2], kNegInvLog2e * c[3])};
    return;
  }
  __shared__ float tile[32][33];
  const int t = blockIdx.x - n_vec;
  const int tj = h / 32, tc = d / 32;
  const int hd = t / (tj * tc), rem = t - hd * tj * tc;
  const int c0 = 32 * (rem / tj), j0 = 32 * (rem % tj);
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const float* src = w2 + (int64_t)hd * d * h;
  for (int r = ty; r < 32; r += 8) tile[r][tx] = src[(int64_t)(c0 + r) * h + j0 + tx];
  __syncthreads();
  uint16_t* dst = out.w2tb + (int64_t)hd * h * d;
  for (int r = ty; r < 32; r += 8) dst[(int64_t)(j0 + r) * d + c0 + tx] = to_bf16(tile[tx][r]);
}

hipError_t launch_cast(const float* w1, const float* w2, const float* w3, int heads, int d, int h,
                       WSet out, hipStream_t st) {
  const int64_t total = (int64_t)heads * h * d;
  const int n_vec = (int)ceil_div(total / 4, 256);
  const int n_tr = heads * (h / 32) * (d / 32);
  hipLaunchKernelGGL(k_cast, dim3(n_vec + n_tr), dim3(256), 0, st, w1, w2, w3, heads, d, h, out,
                     n_vec);
  return hipGetLastError();
}

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

// Each workgroup covers 1024 consecutive elements, which lie in one matrix
// (h d is a multiple of 1024 for every supported shape); the grid has no
// partial workgroup.
template <int D, int HID>
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int splits,
                                                int heads, const float* w1, const float* w2,
                                                const float* w3, float* o1, float* o2, float* o3,
                                                int renorm, WSet ob, int emit_bf16) {
  constexpr int64_t HD = (int64_t)HID * D;
  static_assert(HD % 1024 == 0 && (HID == 128 || HID == 256), "workgroups within one matrix");
  const int64_t e = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);  // element index
  if (e >= (int64_t)heads * 3 * HD) return;
  const int64_t head = e / (3 * HD);
  const int64_t rem = e - head * 3 * HD;
  const int mat = (int)(rem / HD);
  const int64_t local = rem - mat * HD;
  const int64_t off = head * HD + local;  // offset in the weight and bf16 arrays
  const int64_t pstride = (int64_t)heads * 3 * HD;
  f32x4 nv;
  if (mat == 2) {  // W2 rows have length h
    reduce_row4<HID>(part, splits, pstride, e, w2 + off, o2 + off, renorm, nv);
  } else {         // W1 / W3 rows have length d
    reduce_row4<D>(part, splits, pstride, e, (mat == 0 ? w1 : w3) + off, (mat == 0 ? o1 : o3) + off,
                   renorm, nv);
  }
  if (emit_bf16) {
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
      // workgroup's 1024 elements are RW whole rows c0 .. c0 + RW - 1 of W2
      // (a row block starts on a multiple of 1024 elements), so thread j
      // writes rows' column j as one RW-element piece of w2tb row j.
      constexpr int RW = 1024 / HID;
      __shared__ float tr[1024];
      *(f32x4*)&tr[4 * threadIdx.x] = nv;
      __syncthreads();
      if ((int)threadIdx.x < HID) {
        const int64_t c0 = (local - 4 * (int64_t)threadIdx.x) / HID;
        unsigned pk2[RW / 2];
#pragma unroll
        for (int r = 0; r < RW; r += 2)
          pk2[r / 2] = (unsigned)to_bf16(tr[r * HID + threadIdx.x]) |
                       ((unsigned)to_bf16(tr[(r + 1) * HID + threadIdx.x]) << 16);
        uint16_t* dst = ob.w2tb + (head * HID + threadIdx.x) * D + c0;
        if constexpr (RW == 4) {
          *(u32x2*)dst = u32x2{pk2[0], pk2[1]};
        } else {
          *(u32x4*)dst = u32x4{pk2[0], pk2[1], pk2[2], pk2[3]};
        }
      }
    }
  }
}

hipError_t launch_reduce(const float* part, int splits, int heads, int d, int h,
                         const float* w1, const float* w2, const float* w3, float* o1,
                         float* o2, float* o3, int renorm, const WSet* out_bf16,
                         hipStream_t st) {
  const int64_t threads = (int64_t)heads * 3 * h * d / 4;
  const unsigned blocks = (unsigned)ceil_div(threads, 256);
  WSet ob = out_bf16 ? *out_bf16 : WSet{nullptr, nullptr, nullptr, nullptr};
  const int emit = out_bf16 ? 1 : 0;
#define ZM_LAUNCH_RED(DD, HH)                                                                   \
  hipLaunchKernelGGL((k_reduce<DD, HH>), dim3(blocks), dim3(256), 0, st, part, splits, heads, w1, \
                     w2, w3, o1, o2, o3, renorm, ob, emit)
  if (d == 128 && h == 256) ZM_LAUNCH_RED(128, 256);
  else if (d == 128 && h == 128) ZM_LAUNCH_RED(128, 128);
  else if (d == 64 && h == 256) ZM_LAUNCH_RED(64, 256);
  else if (d == 64 && h == 128) ZM_LAUNCH_RED(64, 128);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH_RED
  return hipGetLastError();
}

}  // namespace zm
