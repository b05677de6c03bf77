// Kernel entry and launcher of the chunk-gradient update; the work of one
// workgroup is update_tiles in update_bf16.h.
#include "update_bf16.h"

namespace zm {

template <int D, int HID>
__global__ __launch_bounds__(512) void k_update_bf16(
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const float* __restrict__ eta, int64_t n, int64_t ld, int heads,
    const uint16_t* __restrict__ w1b, const uint16_t* __restrict__ w3b,
    const uint16_t* __restrict__ w2tb, float* __restrict__ part, int splits, int64_t chunk) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[UpdCfg<D, HID>::LDS_ELEMS];
  update_tiles<D, HID>(blockIdx.x, lds, kp, vp, eta, n, ld, heads, w1b, w3b, w2tb, part, splits,
                       chunk);
}

hipError_t launch_update_bf16(const uint16_t* k, const uint16_t* v, const float* eta, int64_t n,
                              int64_t ld, int heads, int d, int h, WSet w, float* part,
                              UpdatePlan plan, hipStream_t st) {
  if (plan.splits <= 0) return hipSuccess;
  const int nsl = h / kHidPerWg;
  const int64_t pairs = (int64_t)heads * plan.splits;
  const unsigned blocks = (unsigned)(ceil_div(pairs, 8) * 8 * nsl);
#define ZM_LAUNCH_UPD(DD, HH)                                                                  \
  hipLaunchKernelGGL((k_update_bf16<DD, HH>), dim3(blocks), dim3(512), 0, st, k, v, eta, n, ld, \
                     heads, w.w1b, w.w3b, w.w2tb, part, plan.splits, plan.chunk)
  if (d == 128 && h == 256) ZM_LAUNCH_UPD(128, 256);
  else if (d == 128 && h == 128) ZM_LAUNCH_UPD(128, 128);
  else if (d == 64 && h == 256) ZM_LAUNCH_UPD(64, 256);
  else if (d == 64 && h == 128) ZM_LAUNCH_UPD(64, 128);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH_UPD
  return hipGetLastError();
}

}  // namespace zm
