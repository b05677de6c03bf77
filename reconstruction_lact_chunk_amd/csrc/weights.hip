// Weight-side kernels: the fp32 -> bf16 operand cast of a fast-weight set,
// and the deterministic reduction of the per-chunk partial gradients into
// the stepped, optionally row-renormalised weights.
//
// The step follows the review of ZipMap (kimjy99.github.io), Method 2:
// W' = W - g with g the chunk gradient of Eq. (3) (the partials hold -g), and
// the norm-preserving rescale shown after Eq. (3), read per row: row r of W'
// is scaled by ||W_r|| / max(||W'_r||, 1e-12).  The LaCT summary (mhpn.cn,
// part 二, 2、架构) likewise normalises after summing the chunk's gradients.
#include "reduce_rows.h"

namespace zm {

// One launch, two kinds of workgroup.  The first n_vec workgroups write the
// scaled copies w1b, w3b, w2b, one thread per 4 consecutive elements (16-byte
// loads, 8-byte stores).  The others write the transposed copy
// w2tb[head][j][c] = W2[head][c][j] in 32 x 32 tiles through LDS, so both the
// reads and the writes are row-contiguous.  Block 0 also clears `zero`.
__global__ __launch_bounds__(256) void k_cast(const float* __restrict__ w1,
                                              const float* __restrict__ w2,
                                              const float* __restrict__ w3, int heads, int d,
                                              int h, WSet out, int n_vec, unsigned* zero,
                                              int nzero) {
  if (blockIdx.x == 0 && zero != nullptr)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0u;
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
                       WSet out, hipStream_t st, unsigned* zero, int nzero) {
  const int64_t total = (int64_t)heads * h * d;
  const int n_vec = (int)ceil_div(total / 4, 256);
  const int n_tr = heads * (h / 32) * (d / 32);
  hipLaunchKernelGGL(k_cast, dim3(n_vec + n_tr), dim3(256), 0, st, w1, w2, w3, heads, d, h, out,
                     n_vec, zero, nzero);
  return hipGetLastError();
}

// Each workgroup covers 1024 consecutive elements, which lie in one matrix
// (h d is a multiple of 1024 for every supported shape); the grid has no
// partial workgroup.
template <int D, int HID>
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int splits,
                                                int heads, ReduceOut r) {
  __shared__ float tr[1024];
  const RowPos p[1] = {row_pos<D, HID>(1024 * (int64_t)blockIdx.x, threadIdx.x)};
  const f32x4 wv[1] = {load_w(p[0], r)};
  reduce_groups<D, HID, 1>(part, splits, heads, p, wv, 1, threadIdx.x, r, tr, 1024);
}

hipError_t launch_reduce(const float* part, int splits, int heads, int d, int h,
                         const float* w1, const float* w2, const float* w3, float* o1,
                         float* o2, float* o3, int renorm, const WSet* out_bf16,
                         hipStream_t st) {
  const int64_t threads = (int64_t)heads * 3 * h * d / 4;
  const unsigned blocks = (unsigned)ceil_div(threads, 256);
  const ReduceOut r{w1, w2, w3, o1, o2, o3,
                    out_bf16 ? *out_bf16 : WSet{nullptr, nullptr, nullptr, nullptr}, renorm,
                    out_bf16 ? 1 : 0};
#define ZM_LAUNCH_RED(DD, HH) \
  hipLaunchKernelGGL((k_reduce<DD, HH>), dim3(blocks), dim3(256), 0, st, part, splits, heads, r)
  if (d == 128 && h == 256) ZM_LAUNCH_RED(128, 256);
  else if (d == 128 && h == 128) ZM_LAUNCH_RED(128, 128);
  else if (d == 64 && h == 256) ZM_LAUNCH_RED(64, 256);
  else if (d == 64 && h == 128) ZM_LAUNCH_RED(64, 128);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH_RED
  return hipGetLastError();
}

}  // namespace zm
