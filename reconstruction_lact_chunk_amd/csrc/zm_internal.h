// Internal declarations of the TTT library: vector types, bf16 helpers, the
// split plan shared by the host planner and the kernels, and the launchers
// each kernel translation unit exports to the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // MFMA A/B operand (16x16x32)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;     // MFMA accumulator (16x16)
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;  // 16 raw bytes
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// ---- tiling constants shared by planner and kernels -----------------------
constexpr int kTok = 32;          // tokens per LDS tile (bf16 kernels); chunks are multiples
constexpr int kWaves = 8;         // waves per workgroup of the bf16 kernels
constexpr int kHidPerWg = 128;    // hidden units of a bf16 update workgroup (half with two token groups)
constexpr int kHidPerWgF32 = 64;  // hidden units owned by one fp32 update workgroup
constexpr int kTargetWgs = 256;   // MI355X compute units: one workgroup each
constexpr int kMinTilesPerChunk = 4;

// bf16 operand copies of one weight set, [H][h][d] except w2b [H][d][h].
// Two copies carry a constant so that the kernels save a multiply per
// (token, hidden unit): W1 is stored times -log2(e), so W1 x comes out of the
// matrix core as the exponent of the sigmoid's exp2, and the apply's W2 is
// stored times -1/log2(e) to undo that factor in SiLU(a) = a sig(a).
constexpr float kNegLog2e = -1.44269504088896341f;
constexpr float kNegInvLog2e = -0.693147180559945309f;
struct WSet {
  uint16_t* w1b;   // -log2(e) W1 rows (hidden-major)
  uint16_t* w3b;   // W3 rows
  uint16_t* w2b;   // -W2 / log2(e), as stored: [d][h]
  uint16_t* w2tb;  // W2 transposed: [h][d]
};

// Where a reduce writes the stepped weights: fp32 W' (may alias the inputs w*:
// every element is read and written by the same thread) and, with emit, its
// bf16 copies into ob.
struct ReduceOut {
  const float* w1;
  const float* w2;
  const float* w3;
  float* o1;
  float* o2;
  float* o3;
  WSet ob;
  int renorm;
  int emit;
};

// Keeps a computed value in place: an empty volatile asm that takes the value
// as a register in/out operand, so the compiler must compute it before this
// point and cannot sink the computation towards its later uses.  Emits no
// instruction.  Used to interleave independent VALU work with matrix-core
// work in software-pipelined loops.
// Wave priority from progress through the N slots of a pipelined iteration,
// changed at each quarter.  Two waves share a SIMD and the older one
// otherwise always wins issue, finishing early and idling at the barrier
// while the other runs alone; with priority falling as a wave advances, the
// wave that is behind is preferred and both arrive together.  The older wave
// of each pair (waves 0..3 of 8) steps 3, 2, 1, 0; the younger one (waves
// 4..7) steps 3, Y1, Y2, Y3, tuned per kernel.
template <int N, int Y1, int Y2, int Y3>
__device__ __forceinline__ void set_progress_priority(int slot) {
  const bool young = (threadIdx.x >> 6) >= 4;
  if (slot == 0) __builtin_amdgcn_s_setprio(3);
  if (slot == N / 4) {
    if (young) __builtin_amdgcn_s_setprio(Y1);
    else __builtin_amdgcn_s_setprio(2);
  }
  if (slot == N / 2) {
    if (young) __builtin_amdgcn_s_setprio(Y2);
    else __builtin_amdgcn_s_setprio(1);
  }
  if (slot == (3 * N) / 4) {
    if (young) __builtin_amdgcn_s_setprio(Y3);
    else __builtin_amdgcn_s_setprio(0);
  }
}

__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(unsigned& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ float bf16lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (round to nearest even) and pack them, lo first.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(unsigned, b);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// p[0] + p[stride] + ... + p[(splits - 1) stride] for 16-byte values, added in
// slot order from zero (fixed order: bitwise reproducible).  The loads go out
// in groups of eight before their adds: a plain loop waits for each load
// before the next add, which makes the partial-sum reduction a chain of
// dependent memory round trips.
__device__ __forceinline__ f32x4 sum_slots(const float* __restrict__ p, int64_t stride,
                                           int splits) {
  constexpr int G = 8;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += G) {
    f32x4 v[G];
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (s0 + i < splits) v[i] = *(const f32x4*)(p + (int64_t)(s0 + i) * stride);
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (s0 + i < splits) sum += v[i];
  }
  return sum;
}

// Records a description of the last failure on this thread (read back through
// zm_ttt_last_error); printf-style.
void set_last_error(const char* fmt, ...);

// ---- split plan ------------------------------------------------------------
struct UpdatePlan {
  int splits;        // S: token chunks (partial sums) per head
  int64_t chunk;     // tokens per chunk, a multiple of tg * kTok
  int tg = 1;        // token groups per workgroup of the bf16 update (1 or 2)
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The split is a pure function of (n, heads, d_hidden): results never depend
// on the device or on occupancy.  Workgroups of 128 hidden units (tg = 1)
// get chunks of at least kMinTilesPerChunk 32-token tiles, as many chunks as
// fill the GPU.  When even that leaves compute units idle (a short chunk such
// as a streamed frame), workgroups of 64 hidden units and two token groups
// (tg = 2, 64-token tiles) take the same per-wave work with half the partial
// sums per workgroup.  Hidden widths below 128 keep tg = 1.
inline UpdatePlan plan_update(int64_t n, int heads, int d_hidden) {
  UpdatePlan p{0, 0, 1};
  if (n <= 0) return p;
  const int nsl = d_hidden / kHidPerWg > 0 ? d_hidden / kHidPerWg : 1;
  int64_t target = kTargetWgs / (int64_t)(heads * nsl);
  if (target < 1) target = 1;
  const int64_t tiles = ceil_div(n, kTok);
  int64_t s = ceil_div(tiles, kMinTilesPerChunk);
  if (s < target && d_hidden >= kHidPerWg) {
    // two token groups: 2 nsl slices per head, 64-token tiles
    int64_t target2 = target / 2;
    if (target2 < 1) target2 = 1;
    const int64_t tiles2 = ceil_div(n, 2 * kTok);
    int64_t s2 = ceil_div(tiles2, kMinTilesPerChunk);
    if (s2 > target2) s2 = target2;
    if (s2 < 1) s2 = 1;
    p.tg = 2;
    p.chunk = ceil_div(tiles2, s2) * 2 * kTok;
    p.splits = (int)ceil_div(n, p.chunk);
    return p;
  }
  if (s > target) s = target;
  if (s < 1) s = 1;
  p.chunk = ceil_div(tiles, s) * kTok;
  p.splits = (int)ceil_div(n, p.chunk);
  return p;
}

// Hidden slices (update workgroups per head and chunk) of a plan.
inline int plan_slices(const UpdatePlan& p, int d_hidden) {
  const int hpw = kHidPerWg / p.tg;
  return d_hidden / hpw > 0 ? d_hidden / hpw : 1;
}

// Partial-sum slots a workspace reserves for an update over n tokens: the
// planned split count of the tg = 1 plan before rounding.  It never decreases
// with n and bounds the realized count plan_update(n').splits of every
// n' <= n (that count is ceil(n' / chunk') with chunk' >= n' / s', so at most
// s', and a tg = 2 plan's s' is at most the tg = 1 count of the same n'),
// which is what lets one workspace, sized for the longest chunk, serve every
// shorter chunk.
// The realized count alone is not monotonic: 1058 tokens over 16 heads of
// hidden 256 realize 7 splits, 949 tokens 8.
inline int update_slots(int64_t n, int heads, int d_hidden) {
  if (n <= 0) return 0;
  const int nsl = d_hidden / kHidPerWg > 0 ? d_hidden / kHidPerWg : 1;
  int64_t target = kTargetWgs / (int64_t)(heads * nsl);
  if (target < 1) target = 1;
  int64_t s = ceil_div(ceil_div(n, kTok), kMinTilesPerChunk);
  if (s > target) s = target;
  if (s < 1) s = 1;
  return (int)s;
}

struct ApplyPlan {
  int splits;
  int64_t chunk;
};

// Up to `wgs` workgroups (by default one per compute unit).  A launch shared
// with update workgroups passes the compute units those leave free; fewer
// than one per head falls back to the default.  The apply is per token, so
// its output does not depend on the split.
inline ApplyPlan plan_apply(int64_t n, int heads, int64_t wgs = kTargetWgs) {
  ApplyPlan p{0, 0};
  if (n <= 0) return p;
  if (wgs < heads) wgs = kTargetWgs;
  int64_t target = wgs / heads;
  if (target < 1) target = 1;
  const int64_t tiles = ceil_div(n, kTok);
  int64_t s = tiles < target ? tiles : target;
  p.chunk = ceil_div(tiles, s) * kTok;
  p.splits = (int)ceil_div(n, p.chunk);
  return p;
}

// ---- launchers (each returns hipSuccess or the launch error) --------------
// zero non-null: the same launch also clears nzero words there.
hipError_t launch_cast(const float* w1, const float* w2, const float* w3, int heads, int d, int h,
                       WSet out, hipStream_t st, unsigned* zero = nullptr, int nzero = 0);

// loss_part non-null: also the virtual loss's per-workgroup sums (splits x
// heads x plan_slices floats) for launch_loss_sum.
hipError_t launch_update_bf16(const uint16_t* k, const uint16_t* v, const float* eta, int64_t n,
                              int64_t ld, int heads, int d, int h, WSet w, float* part,
                              UpdatePlan plan, hipStream_t st, float* loss_part = nullptr);
// loss[head] from the per-workgroup sums of launch_update_bf16 (splits may be
// 0: zeros); nsl = plan_slices of the update's plan.
hipError_t launch_loss_sum(const float* loss_part, int splits, int heads, int nsl, float* loss,
                           hipStream_t st);

hipError_t launch_reduce(const float* part, int splits, int heads, int d, int h,
                         const float* w1, const float* w2, const float* w3,
                         float* o1, float* o2, float* o3, int renorm, const WSet* out_bf16,
                         hipStream_t st);
// Sums the split slots of part into slot 0 and replaces each matrix there by
// its Newton-Schulz orthonormalisation (in place).  f32: fp32 products,
// else split-bf16 products.
hipError_t launch_newton_schulz(float* part, int splits, int heads, int d, int h, bool f32,
                                hipStream_t st);
// Adds the partial-sum slots of part ([splits][heads][3][h d]) into slot 0.
hipError_t launch_sum_splits(float* part, int splits, int heads, int d, int h, hipStream_t st);

hipError_t launch_apply_bf16(const uint16_t* q, uint16_t* o, int64_t n, int64_t ld, int heads,
                             int d, int h, WSet w, hipStream_t st);

// The reduce inside the shared read-and-update launch (frame_bf16.hip): the
// launch's last workgroups wait for the update and read workgroups of their
// head, then reduce its partial sums, which are still in that XCD's L2.  It
// needs every workgroup of a head on one XCD (heads a multiple of 8), and it
// pays only where the partial sums are few: chunks short enough for the
// two-token-group update (plan.tg == 2), whose partial sums are halved and
// mostly stay in the L2.  For longer chunks (16 slots of 3.1 MB per 8 heads of
// 128 / 256) the reduce reads them from memory either way, and in one launch it
// ran no faster than as a launch of its own.  The sync region holds
// kSyncWords words per head and one more block for a sticky error word; it
// must be zero before the first such launch (launch_cast clears it) and each
// launch leaves it zero.
constexpr int kSyncWords = 64;                  // 256 bytes: one head's counters
// Longest read that may share a launch with an in-launch reduce: its blocks
// must finish well within the reduce blocks' 2 s wait bound (a million
// queries take about 1.5 ms at 8 heads, 12 ms at 64).
constexpr int64_t kFuseMaxRead = (int64_t)1 << 20;
inline size_t frame_sync_words(int heads) { return (size_t)kSyncWords * (heads + 1); }
// n_q: the queries read in the same launch (0 for an update alone).
inline bool frame_fuses_reduce(int heads, const UpdatePlan& plan, int64_t n_q) {
  return heads % 8 == 0 && plan.tg == 2 && plan.splits > 0 && n_q >= 0 && n_q <= kFuseMaxRead;
}
struct FrameReduce {
  unsigned* sync;   // frame_sync_words(heads) words
  ReduceOut out;
};

// The apply of n_q queries and the update partial sums over n_kv tokens
// (plan = plan_update(n_kv, ...)), both through the bf16 set w, in one launch
// (frame_bf16.hip).  n_kv > 0; q / o and k / v rows share the stride ld.
// fr non-null (frame_fuses_reduce must hold): the launch also reduces the
// partial sums into fr->out, as launch_reduce would; then n_q may be 0 (a
// whole update step in one launch), else n_q > 0.
hipError_t launch_frame_bf16(const uint16_t* q, uint16_t* o, int64_t n_q, const uint16_t* k,
                             const uint16_t* v, const float* eta, int64_t n_kv, int64_t ld,
                             int heads, int d, int h, WSet w, float* part, UpdatePlan plan,
                             hipStream_t st, const FrameReduce* fr = nullptr);

hipError_t launch_update_f32(const float* k, const float* v, const float* eta, int64_t n,
                             int64_t ld, int heads, int d, int h, const float* w1,
                             const float* w2, const float* w3, float* part, UpdatePlan plan,
                             hipStream_t st);

hipError_t launch_apply_f32(const float* q, float* o, int64_t n, int64_t ld, int heads, int d,
                            int h, const float* w1, const float* w2, const float* w3,
                            hipStream_t st);

}  // namespace zm
