// One launch for a read and an update step that use the same weights W: the
// read o = f_W(q) of n_q queries and the chunk-gradient partial sums over
// n_kv tokens run side by side as two kinds of workgroup of one kernel.  Two
// schedules of the LaCT summary (mhpn.cn, part 二, 3、应用场景) have such
// pairs: a chunk read before it is written (order (c), the default streaming
// frame: the same chunk's q and k), and in the block-causal order (b) the
// read of chunk c after its update together with the update of chunk c + 1.
// This saves a launch and lets the shorter read fill the compute units the
// update leaves free, instead of running after it.  Update blocks come
// first (they take longer) and keep their block indices, so their XCD
// grouping (indices that agree mod 8 share an XCD) is that of the update
// kernel; the apply blocks follow.  Results are those of the two separate
// kernels, bit for bit: each block runs the same code on the same tokens.
//
// For short chunks (those that take the two-token-group update) the launch
// can also reduce the partial sums (the step and renorm of the review of
// ZipMap, Method 2, after Eq. (3)).  Reduce blocks come last.  Each waits
// until every update and apply block of its head has finished, then runs the
// reduce kernel's per-element code (reduce_rows.h) on its share of the head.
// Results again equal the separate kernels bit for bit.  This removes the reduce's launch and the wait between
// the two launches; the partial sums are written and read back within one
// XCD, where most of the reads hit its L2.
//
// How the wait works.  Blocks are dispatched round-robin over the 8 XCDs:
// block b runs on XCD (b + s) mod 8, where the offset s is the same for every
// block of a launch but changes from launch to launch (it continues from the
// launches before; measured with eager launches and graph replays alike).
// With heads a multiple of 8, every update and apply block of head j has a
// block index of j's residue mod 8, and the reduce blocks of head j are
// placed the same way, so all of them run on one XCD, whatever s is.  That
// XCD's L2 is the point where its compute units see each other's stores.  A
// finishing update block waits for its own stores to complete (vmcnt 0:
// written into the L2), then one thread adds to its head's arrival counter
// with a device-scope atomic; a read block only has to be past its reads of
// W (the bf16 copies that the reduce may rewrite), which its results already
// depend on.  A reduce block's first thread polls that counter until all of
// the head's blocks have arrived; its loads of the partial sums come after a
// workgroup barrier, and no block of the launch has read those addresses
// before, so none can hit a stale line in a compute unit's L1.
//
// The one-XCD premise is checked, not assumed.  Every block reads the XCD it
// runs on (the hardware XCC_ID register) and derives its offset s; the
// arrival counter is 64 bits with one 8-bit field per offset, and a block
// adds 1 to its own offset's field.  A reduce block trusts the partial sums
// only if every arrival of its head sits in the field of its own offset
// (then all ran on its XCD); otherwise it writes NaN rather than a value it
// cannot trust.
//
// Progress.  Update and apply blocks never wait, and reduce blocks have the
// highest indices, so every block a reduce block waits for is dispatched no
// later than the reduce block itself and finishes on its own; the reduce
// blocks also stay fewer than the compute units of an XCD.  The poll is
// bounded in time all the same (kSpinTicks of the 100 MHz real-time clock,
// far beyond the longest chunk that takes this launch, a few thousand tokens):
// a reduce block that runs out sets a sticky error word and writes NaN, and
// so does every later fused launch on this workspace until a cast clears the
// word.
//
// Each reduce block counts itself past the wait in another word of its
// head; the last one to count clears the counter and that word once its own
// items are done, so each launch leaves the sync region as it found it
// (zero).
//
// Measured on 1374-token frames (8 heads of 128 / 256): the reduce blocks
// read about 86% of their requests from the L2, yet the launch fetches as
// many bytes from memory as the two separate launches did (the W rows and
// the partial sums the L2 could not keep); the gain is the reduce's launch
// and the wait between the launches, about 2.5 us of a 28 us frame.
#include "apply_bf16.h"
#include "reduce_rows.h"
#include "update_bf16.h"

namespace zm {

namespace {

// Arrival counter of a head: the first 64 bits of its kSyncWords block, 8
// bits per dispatch offset; word 2 counts the reduce blocks past the wait.
constexpr unsigned kMaxArrivals = 255;
// 2 s of the 100 MHz real-time clock: a legitimate wait lasts microseconds,
// and the bound also covers time the process spends switched off the GPU.
constexpr uint64_t kSpinTicks = 200000000;
constexpr int kRedPerXcd = 24;               // at most this many reduce blocks per XCD
constexpr int kRedU = 2;                     // items a reduce block loads at once

// The XCD this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ unsigned hw_xcd() {
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 7u;
}

// This launch's dispatch offset as seen by block blk: XCD = (blk + s) mod 8.
__device__ __forceinline__ unsigned dispatch_offset(int blk) {
  return (hw_xcd() - (unsigned)blk) & 7u;
}

// Sum of the 8 one-byte fields of an arrival counter.
__device__ __forceinline__ unsigned field_sum(unsigned long long v) {
  unsigned t = 0;
#pragma unroll
  for (int f = 0; f < 8; ++f) t += (unsigned)(v >> (8 * f)) & 0xffu;
  return t;
}

// Called by every thread of a block at its end.  stores: the block's global
// stores must be in the L2 before the count (update blocks: the partial
// sums); a read block only has to be past its reads of W, which its results
// already depend on.
__device__ __forceinline__ void arrive(unsigned* ctr, int blk, bool stores) {
  if (stores) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(reinterpret_cast<unsigned long long*>(ctr),
                           1ull << (8 * dispatch_offset(blk)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 polls the head's arrival counter until `arrivals` blocks have
// counted; true if the reduce may trust the partial sums: no time-out, every
// arrival from the dispatch offset `offset` of this block (so from its XCD),
// no sticky error from an earlier launch (sticky_ok).  flag: one int of LDS.
// No global memory wait comes after the poll, so the caller's loads issue at
// once.
__device__ __forceinline__ bool wait_head(unsigned* ctr, unsigned* err, unsigned arrivals,
                                          unsigned offset, bool sticky_ok, int* flag) {
  if (threadIdx.x == 0) {
    unsigned long long* const c = reinterpret_cast<unsigned long long*>(ctr);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long v;
    bool timeout = false;
    while (field_sum(v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) <
           arrivals) {
      if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
        timeout = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (timeout) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = !timeout && ((unsigned)(v >> (8 * offset)) & 0xffu) == arrivals && sticky_ok;
  }
  __syncthreads();
  return *flag != 0;
}

// Reduce block rb (0-based; rb % 8 picks the XCD's heads, since rb and the
// block index agree mod 8): items of 2048 weight elements,
// the P2 items of each head of this XCD in turn, every per_xcd-th one from
// rb / 8.  per_xcd <= P2, so each of the XCD's reduce blocks waits once on
// every head of the XCD.  The two halves of the workgroup take the two
// 1024-element halves of an item (one matrix: h d is a multiple of 2048).
// Items go in groups of up to U of one head: W for a group is loaded before
// the head's wait and the partial sums of the whole group after it, all
// loads in flight together.  After the wait thread 0 counts the block as
// past it; the head's last block to count clears the head's counters once
// its own items are done (every block of the head is past its wait by then).
template <int D, int HID>
__device__ __forceinline__ void reduce_blocks(int rb, uint16_t* lds, const float* part,
                                              int splits, int heads, unsigned* sync,
                                              unsigned arrivals, int per_xcd,
                                              ReduceOut ro) {
  constexpr int U = kRedU;
  constexpr int P2 = 3 * HID * D / 2048;
  constexpr int64_t HD3 = 3 * (int64_t)HID * D;
  const int xcd = rb & 7, idx = rb >> 3;
  const int items = (heads / 8) * P2;
  // a wave lies in one half: its half index is a scalar
  const int half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8), t = threadIdx.x & 255;
  float* const tr = reinterpret_cast<float*>(lds) + 1024 * half;  // U x 2 x 1024 floats
  int* const flag = reinterpret_cast<int*>(lds) + 2048 * U;
  unsigned* const err = sync + kSyncWords * heads;
  const unsigned offset = dispatch_offset(blockIdx.x);
  bool sticky_ok = true;
  if (threadIdx.x == 0)
    sticky_ok = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
  bool ok = true;
  int cur = -1;
  unsigned passed = 0;  // thread 0: blocks of the current head past the wait before this one
  auto finish_head = [&](int hl) {
    if (threadIdx.x == 0 && passed == (unsigned)per_xcd - 1) {
      unsigned* ctr = sync + kSyncWords * (xcd + 8 * hl);
      __hip_atomic_store(reinterpret_cast<unsigned long long*>(ctr), 0ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctr + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  for (int i = idx; i < items;) {
    const int hl = i / P2, hd = xcd + 8 * hl;
    int nu = 1;  // items of this head in the group: i, i + per_xcd, ...
    while (nu < U && i + nu * per_xcd < items && (i + nu * per_xcd) / P2 == hl) ++nu;
    RowPos p[U];
    f32x4 wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // unused slots repeat item i (loaded, not used)
      const int j = u < nu ? i + u * per_xcd : i;
      p[u] = row_pos<D, HID>(hd * HD3 + (int64_t)(j - hl * P2) * 2048 + 1024 * half, t);
      wv[u] = load_w(p[u], ro);
    }
    if (hl != cur) {
      if (cur >= 0) finish_head(cur);
      cur = hl;
      unsigned* ctr = sync + kSyncWords * hd;
      ok = wait_head(ctr, err, arrivals, offset, sticky_ok, flag);
      if (threadIdx.x == 0) {
        // The lane index (0 here) keeps the address lane-varying to the
        // compiler: a uniform one gets a wave-wide scan around the atomic
        // that waits for its result at once, while only finish_head needs it.
        unsigned* done = ctr + 2 + __builtin_amdgcn_mbcnt_lo(~0u, 0u);
        passed = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    reduce_groups<D, HID, U>(part, splits, heads, p, wv, nu, t, ro, tr, 2048, !ok);
    __syncthreads();  // tr and flag are rewritten for the next group
    i += nu * per_xcd;
  }
  if (cur >= 0) finish_head(cur);
}

}  // namespace

template <int D, int HID, int TG>
__global__ __launch_bounds__(512) void k_frame_bf16(
    const uint16_t* __restrict__ qp, uint16_t* __restrict__ op, int64_t n_q,
    const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const float* __restrict__ eta, int64_t n_kv, int64_t ld, int heads,
    const uint16_t* __restrict__ w1b,
    const uint16_t* __restrict__ w3b, const uint16_t* __restrict__ w2b,
    const uint16_t* __restrict__ w2tb, float* __restrict__ part, int splits, int64_t chunk_u,
    int upd_blocks, int64_t chunk_a, int app_blocks, unsigned* sync, int red_base,
    int red_per_xcd, unsigned arrivals, ReduceOut ro) {
  using UC = UpdCfg<D, HID, TG>;
  constexpr int LU = UC::LDS_ELEMS, LA = AppCfg<D, HID>::LDS_ELEMS;
  static_assert(sizeof(uint16_t) * (LU > LA ? LU : LA) >= sizeof(float) * (2048 * kRedU + 1),
                "reduce scratch fits the LDS");
  __shared__ __attribute__((aligned(16))) uint16_t lds[LU > LA ? LU : LA];
  const int b = blockIdx.x;
  if (b < upd_blocks) {
    update_tiles<D, HID, false, TG>(b, lds, kp, vp, eta, n_kv, ld, heads, w1b, w3b, w2tb, part,
                                    splits, chunk_u);
    if (sync) {
      const int pair = upd_block_pair<UC::NSL>(b);
      if (pair < heads * splits) arrive(sync + kSyncWords * (pair % heads), b, true);
    }
  } else if (sync == nullptr || b < red_base) {
    // blocks past the apply's (padding before the reduce blocks) find no tokens
    apply_tiles<D, HID>(b - upd_blocks, lds, qp, op, n_q, ld, heads, w1b, w3b, w2b, chunk_a);
    if (sync && b - upd_blocks < app_blocks)
      arrive(sync + kSyncWords * ((b - upd_blocks) % heads), b, false);
  } else {
    reduce_blocks<D, HID>(b - red_base, lds, part, splits, heads, sync, arrivals, red_per_xcd,
                          ro);
  }
}

hipError_t launch_frame_bf16(const uint16_t* q, uint16_t* o, int64_t n_q, const uint16_t* k,
                             const uint16_t* v, const float* eta, int64_t n_kv, int64_t ld,
                             int heads, int d, int h, WSet w, float* part, UpdatePlan plan,
                             hipStream_t st, const FrameReduce* fr) {
  // n_q = 0 (no read) only with the reduce: an update step in one launch
  if (plan.splits <= 0 || n_kv <= 0 || n_q < 0 || (n_q == 0 && fr == nullptr))
    return hipErrorInvalidValue;
  if (plan.tg != 1 && plan.tg != 2) return hipErrorInvalidValue;
  if (fr && (!frame_fuses_reduce(heads, plan, n_q) || fr->sync == nullptr))
    return hipErrorInvalidValue;
  const int nsl = plan_slices(plan, h);
  const int64_t pairs = (int64_t)heads * plan.splits;
  const int upd_blocks = (int)(ceil_div(pairs, 8) * 8 * nsl);
  ApplyPlan ap = plan_apply(n_q, heads, kTargetWgs - upd_blocks);
  // With few compute units left over, the read's workgroups would get long
  // runs and finish last: then they take the usual plan and queue behind
  // the update's workgroups instead.
  if (ap.chunk > 2 * plan.chunk) ap = plan_apply(n_q, heads);
  const int app_blocks = heads * ap.splits;
  // Reduce blocks: from the first multiple of 8 after the apply blocks, at
  // most kRedPerXcd and at most one head's items per XCD.
  int red_base = upd_blocks + app_blocks, red_per_xcd = 0;
  unsigned arrivals = 0;
  ReduceOut ro{};
  unsigned* sync = nullptr;
  if (fr) {
    red_base = (int)(ceil_div(red_base, 8) * 8);
    const int p2 = 3 * h * d / 2048;
    red_per_xcd = p2 < kRedPerXcd ? p2 : kRedPerXcd;
    arrivals = (unsigned)(plan.splits * nsl + ap.splits);
    if (arrivals > kMaxArrivals) return hipErrorInvalidValue;  // one byte per offset
    ro = fr->out;
    sync = fr->sync;
  }
  const unsigned blocks = (unsigned)(red_base + 8 * red_per_xcd);
#define ZM_LAUNCH_FRAME_TG(DD, HH, TT)                                                          \
  hipLaunchKernelGGL((k_frame_bf16<DD, HH, TT>), dim3(blocks), dim3(512), 0, st, q, o, n_q, k,  \
                     v, eta, n_kv, ld, heads, w.w1b, w.w3b, w.w2b, w.w2tb, part, plan.splits,    \
                     plan.chunk, upd_blocks, ap.chunk, app_blocks, sync, red_base, red_per_xcd,  \
                     arrivals, ro)
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
