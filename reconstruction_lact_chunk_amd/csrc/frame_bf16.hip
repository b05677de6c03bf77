// One launch for a read and an update step that use the same weights W: the
// read o = f_W(q) of n_q queries and the chunk-gradient partial sums over
// n_kv tokens run side by side as two kinds of workgroup of one kernel.  Two
// schedules of the LaCT summary (mhpn.cn, part 二, 3、应用场景) have such
// pairs: a chunk read before it is written (order (c), the default streaming
// frame: the same chunk's q and k), and in the block-causal order (b) the
// read of chunk c after its update together with the update of chunk c + 1.  This saves a launch and lets the
// shorter read fill the compute units the update leaves free, instead of
// running after it.  Update blocks come first (they take longer) and keep
// their XCD mapping (block index % 8); the apply blocks follow.  Results are
// those of the two separate kernels, bit for bit: each block runs the same
// code on the same tokens.
#include "apply_bf16.h"
#include "update_bf16.h"

namespace zm {

template <int D, int HID, int TG>
__global__ __launch_bounds__(512) void k_frame_bf16(
    const uint16_t* __restrict__ qp, uint16_t* __restrict__ op, int64_t n_q,
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const float* __restrict__ eta, int64_t n_kv, int64_t ld, int heads,
    const uint16_t* __restrict__ w1b,
    const uint16_t* __restrict__ w3b, const uint16_t* __restrict__ w2b,
    const uint16_t* __restrict__ w2tb, float* __restrict__ part, int splits, int64_t chunk_u,
    int upd_blocks, int64_t chunk_a) {
  constexpr int LU = UpdCfg<D, HID, TG>::LDS_ELEMS, LA = AppCfg<D, HID>::LDS_ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LU > LA ? LU : LA];
  if ((int)blockIdx.x < upd_blocks)
    update_tiles<D, HID, false, TG>(blockIdx.x, lds, kp, vp, eta, n_kv, ld, heads, w1b, w3b,
                                    w2tb, part, splits, chunk_u);
  else
    apply_tiles<D, HID>(blockIdx.x - upd_blocks, lds, qp, op, n_q, ld, heads, w1b, w3b, w2b,
                        chunk_a);
}

hipError_t launch_frame_bf16(const uint16_t* q, uint16_t* o, int64_t n_q, const uint16_t* k,
                             const uint16_t* v, const float* eta, int64_t n_kv, int64_t ld,
                             int heads, int d, int h, WSet w, float* part, UpdatePlan plan,
                             hipStream_t st) {
  if (plan.splits <= 0 || n_kv <= 0 || n_q <= 0) return hipErrorInvalidValue;
  if (plan.tg != 1 && plan.tg != 2) return hipErrorInvalidValue;
  const int nsl = plan_slices(plan, h);
  const int64_t pairs = (int64_t)heads * plan.splits;
  const int upd_blocks = (int)(ceil_div(pairs, 8) * 8 * nsl);
  ApplyPlan ap = plan_apply(n_q, heads, kTargetWgs - upd_blocks);
  // With few compute units left over, the read's workgroups would get long
  // runs and finish last: then they take the usual plan and queue behind
  // the update's workgroups instead.
  if (ap.chunk > 2 * plan.chunk) ap = plan_apply(n_q, heads);
  const unsigned blocks = (unsigned)(upd_blocks + (int64_t)heads * ap.splits);
#define ZM_LAUNCH_FRAME_TG(DD, HH, TT)                                                          \
  hipLaunchKernelGGL((k_frame_bf16<DD, HH, TT>), dim3(blocks), dim3(512), 0, st, q, o, n_q, k,  \
                     v, eta, n_kv, ld, heads, w.w1b, w.w3b, w.w2b, w.w2tb, part, plan.splits,    \
                     plan.chunk, upd_blocks, ap.chunk)
#define ZM_LAUNCH_FRAME(DD, HH)          \
  do {                                   \
    if (plan.tg == 2)                    \
      ZM_LAUNCH_FRAME_TG(DD, HH, 2);     \
    else                                 \
      ZM_LAUNCH_FRAME_TG(DD, HH, 1);     \
  } while (0)
  if (d == 128 && h == 256) ZM_LAUNCH_FRAME(128, 256);
  else if (d == 128 && h == 128) ZM_LAUNCH_FRAME(128, 128);
  else if (d == 64 && h == 256) ZM_LAUNCH_FRAME(64, 256);
  else if (d == 64 && h == 128) ZM_LAUNCH_FRAME(64, 128);
  else return hipErrorInvalidValue;
#undef ZM_LAUNCH_FRAME
#undef ZM_LAUNCH_FRAME_TG
  return hipGetLastError();
}

}  // namespace zm
