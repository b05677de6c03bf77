// Kernel entry and launcher of the chunk-gradient update; the work of one
// workgroup is update_tiles in update_bf16.h.
#include "update_bf16.h"

namespace zm {

template <int D, int HID, int TG>
__global__ __launch_bounds__(512) void k_update_bf16(
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const float* __restrict__ eta, int64_t n, int64_t ld, int heads,
    const uint16_t* __restrict__ w1b, const uint16_t* __restrict__ w3b,
    const uint16_t* __restrict__ w2tb, float* __restrict__ part, int splits, int64_t chunk) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[UpdCfg<D, HID, TG>::LDS_ELEMS];
  update_tiles<D, HID, false, TG>(blockIdx.x, lds, kp, vp, eta, n, ld, heads, w1b, w3b, w2tb,
                                  part, splits, chunk);
}

// The same update, also summing the virtual loss into loss_part (one value per
// workgroup; see update_tiles).
template <int D, int HID, int TG>
__global__ __launch_bounds__(512) void k_update_loss_bf16(
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const float* __restrict__ eta, int64_t n, int64_t ld, int heads,
    const uint16_t* __restrict__ w1b, const uint16_t* __restrict__ w3b,
    const uint16_t* __restrict__ w2tb, float* __restrict__ part, int splits, int64_t chunk,
    float* __restrict__ loss_part) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[UpdCfg<D, HID, TG>::LDS_ELEMS];
  update_tiles<D, HID, true, TG>(blockIdx.x, lds, kp, vp, eta, n, ld, heads, w1b, w3b, w2tb,
                                 part, splits, chunk, loss_part);
}

// loss[head] = ln(2) x the block sums of that head, chunks then slices in
// order (fixed order: bitwise reproducible).  One thread per head.
__global__ __launch_bounds__(64) void k_loss_sum(const float* __restrict__ loss_part, int splits,
                                                 int heads, int nsl, float* __restrict__ loss) {
  const int head = blockIdx.x * blockDim.x + threadIdx.x;
  if (head >= heads) return;
  float sum = 0.f;
  for (int c = 0; c < splits; ++c)
    for (int sl = 0; sl < nsl; ++sl) sum += loss_part[((int64_t)c * heads + head) * nsl + sl];
  loss[head] = -kNegInvLog2e * sum;
}

hipError_t launch_update_bf16(const uint16_t* k, const uint16_t* v, const float* eta, int64_t n,
                              int64_t ld, int heads, int d, int h, WSet w, float* part,
                              UpdatePlan plan, hipStream_t st, float* loss_part) {
  if (plan.splits <= 0) return hipSuccess;
  if (plan.tg != 1 && plan.tg != 2) return hipErrorInvalidValue;
  const int nsl = plan_slices(plan, h);
  const int64_t pairs = (int64_t)heads * plan.splits;
  const unsigned blocks = (unsigned)(ceil_div(pairs, 8) * 8 * nsl);
#define ZM_LAUNCH_UPD_TG(DD, HH, TT)                                                               \
  do {                                                                                             \
    if (loss_part)                                                                                 \
      hipLaunchKernelGGL((k_update_loss_bf16<DD, HH, TT>), dim3(blocks), dim3(512), 0, st, k, v,   \
                         eta, n, ld, heads, w.w1b, w.w3b, w.w2tb, part, plan.splits, plan.chunk,   \
                         loss_part);                                                               \
    else                                                                                           \
      hipLaunchKernelGGL((k_update_bf16<DD, HH, TT>), dim3(blocks), dim3(512), 0, st, k, v, eta,   \
                         n, ld, heads, w.w1b, w.w3b, w.w2tb, part, plan.splits, plan.chunk);       \
  } while (0)
#define ZM_LAUNCH_UPD(DD, HH)              \
  do {                                     \
    if (plan.tg == 2)                      \
      ZM_LAUNCH_UPD_TG(DD, HH, 2);         \
    else                                   \
      ZM_LAUNCH_UPD_TG(DD, HH, 1);         \
  } while (0)
  if (d == 128 && h == 256) ZM_LAUNCH_UPD(128, 256);
  else if (d == 128 && h == 128) ZM_LAUNCH_UPD(128, 128);
  else if (d == 64 && h == 256) ZM_LAUNCH_UPD(64, 256);
  else if (d == 64 && h == 128) ZM_LAUNCH_UPD(64, 128);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH_UPD
#undef ZM_LAUNCH_UPD_TG
  return hipGetLastError();
}

hipError_t launch_loss_sum(const float* loss_part, int splits, int heads, int nsl, float* loss,
                           hipStream_t st) {
  hipLaunchKernelGGL(k_loss_sum, dim3((unsigned)ceil_div(heads, 64)), dim3(64), 0, st, loss_part,
                     splits, heads, nsl, loss);
  return hipGetLastError();
}

}  // namespace zm
