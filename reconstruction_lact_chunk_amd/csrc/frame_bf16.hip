// One launch for a chunk that is read before it is written (the
// apply-then-update order of a streaming frame; LaCT summary, mhpn.cn,
// part 二, 3、应用场景, order (c)): the read o = f_W(q) and the chunk-gradient
// partial sums both use only the incoming W, so they can run side by side as
// two kinds of workgroup of one kernel.  This saves a launch and lets the
// shorter read fill the compute units the update leaves free, instead of
// running after it.  Update blocks come first (they take longer) and keep
// their XCD mapping (block index % 8); the apply blocks follow.  Results are
// those of the two separate kernels, bit for bit: each block runs the same
// code on the same tokens.
#include "apply_bf16.h"
#include "update_bf16.h"

namespace zm {

template <int D, int HID>
__global__ __launch_bounds__(512) void k_frame_bf16(
    const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vp, const float* __restrict__ eta, uint16_t* __restrict__ op,
    int64_t n, int64_t ld, int heads, const uint16_t* __restrict__ w1b,
    const uint16_t* __restrict__ w3b, const uint16_t* __restrict__ w2b,
    const uint16_t* __restrict__ w2tb, float* __restrict__ part, int splits, int64_t chunk_u,
    int upd_blocks, int64_t chunk_a) {
  constexpr int LU = UpdCfg<D, HID>::LDS_ELEMS, LA = AppCfg<D, HID>::LDS_ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LU > LA ? LU : LA];
  if ((int)blockIdx.x < upd_blocks)
    update_tiles<D, HID>(blockIdx.x, lds, kp, vp, eta, n, ld, heads, w1b, w3b, w2tb, part, splits,
                         chunk_u);
  else
    apply_tiles<D, HID>(blockIdx.x - upd_blocks, lds, qp, op, n, ld, heads, w1b, w3b, w2b,
                        chunk_a);
}

hipError_t launch_frame_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const float* eta, uint16_t* o, int64_t n, int64_t ld, int heads,
                             int d, int h, WSet w, float* part, UpdatePlan plan, hipStream_t st) {
  if (plan.splits <= 0 || n <= 0) return hipSuccess;
  const int nsl = h / kHidPerWg;
  const int64_t pairs = (int64_t)heads * plan.splits;
  const int upd_blocks = (int)(ceil_div(pairs, 8) * 8 * nsl);
  const ApplyPlan ap = plan_apply(n, heads, kTargetWgs - upd_blocks);
  const unsigned blocks = (unsigned)(upd_blocks + (int64_t)heads * ap.splits);
#define ZM_LAUNCH_FRAME(DD, HH)                                                                 \
  hipLaunchKernelGGL((k_frame_bf16<DD, HH>), dim3(blocks), dim3(512), 0, st, q, k, v, eta, o, n, \
                     ld, heads, w.w1b, w.w3b, w.w2b, w.w2tb, part, plan.splits, plan.chunk,      \
                     upd_blocks, ap.chunk)
  if (d == 128 && h == 256) ZM_LAUNCH_FRAME(128, 256);
  else if (d == 128 && h == 128) ZM_LAUNCH_FRAME(128, 128);
  else if (d == 64 && h == 256) ZM_LAUNCH_FRAME(64, 256);
  else if (d == 64 && h == 128) ZM_LAUNCH_FRAME(64, 128);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH_FRAME
  return hipGetLastError();
}

}  // namespace zm
