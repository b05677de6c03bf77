// Kernel entry and launcher of the apply; the work of one workgroup is
// apply_tiles in apply_bf16.h.
#include "apply_bf16.h"

namespace zm {

template <int D, int HID>
__global__ __launch_bounds__(512) void k_apply_bf16(
    const uint16_t* __restrict__ qp, uint16_t* __restrict__ op, int64_t n, int64_t ld, int heads,
    const uint16_t* __restrict__ w1b, const uint16_t* __restrict__ w3b,
    const uint16_t* __restrict__ w2b, int64_t chunk) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[AppCfg<D, HID>::LDS_ELEMS];
  apply_tiles<D, HID>(blockIdx.x, lds, qp, op, n, ld, heads, w1b, w3b, w2b, chunk);
}

hipError_t launch_apply_bf16(const uint16_t* q, uint16_t* o, int64_t n, int64_t ld, int heads,
                             int d, int h, WSet w, hipStream_t st) {
  const ApplyPlan plan = plan_apply(n, heads);
  if (plan.splits <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((int64_t)heads * plan.splits);
#define ZM_LAUNCH_APP(DD, HH)                                                                   \
  hipLaunchKernelGGL((k_apply_bf16<DD, HH>), dim3(blocks), dim3(512), 0, st, q, o, n, ld, heads, \
                     w.w1b, w.w3b, w.w2b, plan.chunk)
  if (d == 128 && h == 256) ZM_LAUNCH_APP(128, 256);
  else if (d == 128 && h == 128) ZM_LAUNCH_APP(128, 128);
  else if (d == 64 && h == 256) ZM_LAUNCH_APP(64, 256);
  else if (d == 64 && h == 128) ZM_LAUNCH_APP(64, 128);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH_APP
  return hipGetLastError();
}

}  // namespace zm
