// Hand-written token-row products of the full-width fast weight (one head of
// d = 1024, hidden h = 2048: the 6 d^2 state of the ZipMap paper-reading
// notes' state-size paragraph), with the SwiGLU gate fused into the product
// that feeds it (review of ZipMap, kimjy99.github.io, Method 2, Eq. (1)-(4)).
// One kernel template, two epilogues:
//   kRead:   for query rows q, x = -log2(e) W1 q and b = W3 q, written as
//            U' = x sig(a) b = -log2(e) SiLU(a) b (the bf16 W2 copy of the
//            read's last product carries -1 / log2(e));
//   kUpdate: for key rows k, x = -log2(e) W1 k and b = W3 k; with e = W2^T v
//            (bf16, a plain library product) and the rate eta of the token,
//            the gate backward ga = eta e b SiLU'(a), gb = eta e SiLU(a) and
//            u_eta = eta SiLU(a) b, the operands of the chunk-reduction
//            products (u_eta overwrites e in place).
// x and b never leave registers.
//
// Tiling: a workgroup of 8 waves owns TM = 256 tokens x TN = 128 hidden units
// of both W1 and W3 and runs the whole contraction in k-steps of 32.  The
// products are taken transposed (rows = hidden units, columns = tokens), so
// each lane's four accumulator rows are four consecutive units of one token:
// the gate pairs x and b from the same lane.  Waves form a 4 x 2 grid over the
// tile; each holds, per product, 4 x 4 blocks of v_mfma_f32_16x16x32_bf16.
//
// Operands go global -> LDS with the gfx950 direct loads (16 bytes per lane,
// no register staging) into a ring of four stages: per stage the 256 token
// rows and the 2 TN weight rows, 64 bytes (one k-step) per row.  The four
// 16-byte chunks of a row are stored XOR-swizzled by (row >> 1) & 3: the
// direct load writes a wave's 64 lanes to 1 KB of consecutive LDS, so each
// lane fetches the chunk that belongs at its slot, and the fragment reads (16
// rows x one chunk per 16 lanes) are free of bank conflicts.  One barrier per
// k-step; fragments of the next k-step are read while the current one's MFMAs
// run.
//
// Measured on this shape: the global -> LDS traffic of the 256 x 256 output
// tile is what holds the loop below the matrix rate (a copy of the kernel
// that never refills the ring runs 14 % faster); a fifth stage (160 KB) or
// two 4-wave workgroups per compute unit are slower, and a larger tile does
// not fit the registers of 8 waves.
#include "wide_path.h"

namespace zm {
namespace {

constexpr int kKStep = 32;   // contraction per stage (elements)
constexpr int kRowBytes = kKStep * 2;
constexpr int TN = 128, WN = 2;   // hidden units per tile; waves across them

// Workgroup shape: TM tokens per tile over WM x 2 waves, a ring of STAGES
// stages, BLOCKS workgroups per compute unit.  (A 4-wave shape of 128 tokens
// and 3 stages, two workgroups per compute unit, measured slower: its smaller
// tile costs more LDS writes and L2 traffic per product than the overlap of
// the two workgroups recovers.)
template <int TM_, int WM_, int STAGES_, int BLOCKS_>
struct Shape {
  static constexpr int TM = TM_, WM = WM_, STAGES = STAGES_, BLOCKS = BLOCKS_;
  static constexpr int NW = WM * WN;                        // waves
  static constexpr int ROWS = TM + 2 * TN;                  // rows per stage
  static constexpr int STAGE = ROWS * kRowBytes;
  static constexpr int LOADS = ROWS / (NW * 16);            // direct loads per wave per stage
  static constexpr int LDS = STAGES * STAGE;
  static_assert(ROWS % (NW * 16) == 0, "whole loads");
  static_assert(TM / WM == 64 && TN / WN == 64, "64 x 64 units per wave");
  static_assert(STAGES >= 4 && (STAGES - 2) * LOADS + 8 < 64, "wait counts");
  // epilogue: 4 KB of the update's e per wave in each of two ring buffers, 8 KB
  // of output staging per wave in two others
  static_assert(NW * 8192 <= 2 * STAGE && NW * 4096 <= STAGE, "epilogue staging");
  static_assert(BLOCKS * LDS <= 160 * 1024, "LDS");
};
using Cfg = Shape<256, 4, 4, 1>;   // 8 waves, 128 KB: one workgroup per CU
constexpr int HB = 4, TB = 4;         // 16-unit / 16-token blocks per wave
constexpr int kHidGroups = 4;         // XCD groups over the hidden tiles (a divisor of 8; 4
                                      // measured best: each token tile is fetched by 2 XCDs)

enum Mode { kRead = 0, kUpdate = 1 };

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate: vmcnt(n) (6 bits, split over [3:0] and [15:14]),
// expcnt untouched, lgkmcnt(0).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

// s_waitcnt vmcnt(n) lgkmcnt(0) for an n that is a constant after unrolling.
__device__ __forceinline__ void wait_vm_lgkm0(int n) {
  switch (n) {
#define ZM_WAIT_CASE(N) \
  case N: __builtin_amdgcn_s_waitcnt(waitcnt_vm(N)); break;
    ZM_WAIT_CASE(1) ZM_WAIT_CASE(2) ZM_WAIT_CASE(3) ZM_WAIT_CASE(4) ZM_WAIT_CASE(5)
    ZM_WAIT_CASE(6) ZM_WAIT_CASE(7) ZM_WAIT_CASE(8) ZM_WAIT_CASE(9) ZM_WAIT_CASE(10)
    ZM_WAIT_CASE(11) ZM_WAIT_CASE(12) ZM_WAIT_CASE(13) ZM_WAIT_CASE(14) ZM_WAIT_CASE(15)
    ZM_WAIT_CASE(16) ZM_WAIT_CASE(17) ZM_WAIT_CASE(18) ZM_WAIT_CASE(19) ZM_WAIT_CASE(20)
    ZM_WAIT_CASE(21) ZM_WAIT_CASE(22) ZM_WAIT_CASE(23) ZM_WAIT_CASE(24)
#undef ZM_WAIT_CASE
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
  }
}

// Byte offset, inside a stage, of logical 16-byte chunk c of row r.
__device__ __forceinline__ int swz_off(int r, int c) {
  return r * kRowBytes + 16 * (c ^ ((r >> 1) & 3));
}

}  // namespace

// x: token rows ([n] rows of stride ld, D elements used); w0, w1: the W1 and
// W3 copies [ncols][D] (ncols = h hidden units).  Outputs as in the header;
// eta [n] with stride eta_ld (kUpdate only); out1 holds e on entry and u_eta
// on exit (kUpdate only).
template <class S, int MODE, int D>
__global__ __launch_bounds__(S::NW * 64, S::BLOCKS) void k_wide_rows(
    const uint16_t* __restrict__ x, int64_t ld, int64_t n, const uint16_t* __restrict__ w0,
    const uint16_t* __restrict__ w1, int ncols, const float* __restrict__ eta, int64_t eta_ld,
    uint16_t* __restrict__ out0, int64_t ldo0, uint16_t* __restrict__ out1, int64_t ldo1) {
  constexpr int NK = D / kKStep;
  constexpr int TM = S::TM, WM = S::WM, kStages = S::STAGES, kStage = S::STAGE;
  constexpr int kLoads = S::LOADS;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS];

  // Block -> tile: the 8 XCDs take blocks round-robin.  They form kHidGroups
  // groups of hidden tiles x 8 / kHidGroups groups of token tiles: XCD x owns
  // hidden tiles (x % kHidGroups) * per_xcd .. (their weight rows stay in its
  // L2) and the token tiles t with t % (8 / kHidGroups) == x / kHidGroups,
  // its hidden tiles of one token tile next to each other.
  constexpr int kTokGroups = 8 / kHidGroups;
  const int per_xcd = ncols / TN / kHidGroups;
  const int b = blockIdx.x;
  const int xcd = b & 7, i = b >> 3;
  const int ht = (xcd % kHidGroups) * per_xcd + i % per_xcd;
  const int64_t t0 = ((int64_t)(i / per_xcd) * kTokGroups + xcd / kHidGroups) * TM;
  if (t0 >= n) return;
  const int j0 = ht * TN;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int wm = w % WM, wn = w / WM;

  // ---- direct loads: wave w fills stage rows w * kLoads * 16 .., 16 per load;
  // lane l of a load: row base + l / 4, physical chunk l % 4.  Rows 0..TM-1
  // are tokens, then TN rows of W1 and TN of W3.
  const uint16_t* src[kLoads];
#pragma unroll
  for (int ii = 0; ii < kLoads; ++ii) {
    const int r = (w * kLoads + ii) * 16 + (l >> 2);
    const int c = (l & 3) ^ ((r >> 1) & 3);   // logical chunk stored at this slot
    if (r < TM) {
      int64_t tok = t0 + r;
      if (tok >= n) tok = n - 1;             // rows past the end: any valid row
      src[ii] = x + tok * ld + 8 * c;
    } else {
      const int p = (r - TM) / TN, rr = (r - TM) % TN;
      src[ii] = (p == 0 ? w0 : w1) + (int64_t)(j0 + rr) * D + 8 * c;
    }
  }
  auto load_stage = [&](int k) {
    unsigned char* dst = smem + (k % kStages) * kStage + w * kLoads * 16 * kRowBytes;
#pragma unroll
    for (int ii = 0; ii < kLoads; ++ii)
      __builtin_amdgcn_global_load_lds((const void*)(src[ii] + k * kKStep),
                                       (lds_void*)(dst + ii * 16 * kRowBytes), 16, 0, 0);
  };

  // ---- fragment reads: weight rows (A operand), token rows (B operand), chunk l / 16
  const int rl = l & 15, cl = l >> 4;
  const int off_w = swz_off(TM + (TN / WN) * wn + rl, cl);   // + (p TN + 16 hb) rows
  const int off_x = swz_off((TM / WM) * wm + rl, cl);        // + 16 tb rows
  struct Frags {
    bf16x8 w[2][HB], x[TB];
  };
  auto read_frags = [&](int k, Frags& f) {
    const unsigned char* s = smem + (k % kStages) * kStage;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        f.w[p][hb] = as_bf16x8(*(const u32x4*)(s + off_w + (p * TN + 16 * hb) * kRowBytes));
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
      f.x[tb] = as_bf16x8(*(const u32x4*)(s + off_x + 16 * tb * kRowBytes));
  };

  f32x4 acc[2][HB][TB];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[p][hb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          acc[p][hb][tb] = mfma_bf16(f.w[p][hb], f.x[tb], acc[p][hb][tb]);
  };

  // ---- the update's e tile, prefetched during the last k-steps.  Once there
  // is no stage left to load, the k-step that would have refilled the buffer
  // of stage NK - kStages + hf (the barrier of k-step NK - kStages + 1 + hf
  // has retired every read of it) loads instead the wave's rows 32 hf ..
  // 32 hf + 31 of e (its 64 token rows x 64 units) there by direct loads, 4 KB
  // per wave, laid out as the staging tiles of the epilogue (row r of 128
  // bytes, 16-byte chunk c at slot c ^ (r & 7)).
  const int row0 = (TM / WM) * wm, col0 = (TN / WN) * wn;
  auto e_tile = [&](int hf) {
    return smem + ((NK - kStages + hf) % kStages) * kStage + w * 4096;
  };
  auto load_e = [&](int hf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * hf + 8 * i + (l >> 3);
      int64_t tok = t0 + row0 + r;
      if (tok >= n) tok = n - 1;
      const int c = (l & 7) ^ (r & 7);
      __builtin_amdgcn_global_load_lds((const void*)(out1 + tok * ldo1 + j0 + col0 + 8 * c),
                                       (lds_void*)(e_tile(hf) + i * 1024), 16, 0, 0);
    }
  };

  // ---- pipeline: stages k + 1 .. k + kStages - 2 in flight while stage k is
  // read and k - 1 multiplied.  Direct loads count on vmcnt and complete in
  // order.  Each wave waits for its own loads of stage k (the loads issued
  // after them may stay outstanding: kLoads per later stage, 4 per half of the
  // update's e) and its own LDS reads (the buffer refilled next was read in
  // the previous iteration); the barrier then makes every wave's part of stage
  // k visible and every read of that buffer retired, and the workgroup acquire
  // fence on LDS keeps the next reads below it.  A release fence would also be
  // correct, but the compiler answers it by draining every direct load, which
  // undoes the prefetch.
  constexpr int kEFirst = NK - kStages + 1;   // k-step that issues e's first half
  auto wait_stage = [&](int k) {
    const int later = (kStages - 2 < NK - 1 - k ? kStages - 2 : NK - 1 - k) * kLoads;
    const int halves = MODE != kUpdate ? 0 : (k - kEFirst < 0 ? 0 : (k - kEFirst > 2 ? 2 : k - kEFirst));
    wait_vm_lgkm0(later + 4 * halves);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  auto issue = [&](int k) {   // the loads that follow the wait of k-step k
    if (k + kStages - 1 < NK) load_stage(k + kStages - 1);
    else if (MODE == kUpdate && k == kEFirst) load_e(0);
    else if (MODE == kUpdate && k == kEFirst + 1) load_e(1);
  };
#pragma unroll
  for (int k = 0; k < kStages - 1; ++k) load_stage(k);
  Frags fa, fb;
  wait_stage(0);
  issue(0);
  read_frags(0, fa);
#pragma unroll   // fully: every wait count and ring offset is then a constant
  for (int k = 1; k < NK; k += 2) {
    wait_stage(k);
    issue(k);
    read_frags(k, fb);
    mma(fa);
    if (k + 1 < NK) {
      wait_stage(k + 1);
      issue(k + 1);
      read_frags(k + 1, fa);
    }
    mma(fb);
  }
  if (NK % 2 == 1) mma(fa);

  // ---- epilogue.  Lane holds units 64 wn + 16 hb + 4 (l / 16) + 0..3 of
  // token row 64 wm + 16 tb + l % 16 of the tile.  Global traffic goes through
  // per-wave LDS staging tiles of the wave's 64 token rows x 64 units (bf16,
  // rows of 128 bytes, 16-byte chunk c of row r at slot c ^ (r & 7)): memory is
  // touched in whole 128-byte row segments (8 lanes x 16 bytes, 8 rows per
  // instruction), registers in the accumulator layout, both free of bank
  // conflicts.  Token rows past the end are clamped for loads and skipped for
  // stores.
  //
  // The scheduling barrier keeps the epilogue out of the unrolled main loop's
  // scheduling region (mixed in, its addresses are computed early and spilled).
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();   // every wave is done with the ring; the e loads have landed
  // output staging: two ring buffers other than e's, 4 waves in each
  unsigned char* out_tile =
      smem + ((NK + 2 + w / 4) % kStages) * kStage + (w % 4) * 8192;
  auto out_row = [&](int r) { return out_tile + r * 128; };
  auto e_row = [&](int r) { return e_tile(r >> 5) + (r & 31) * 128; };
  auto frag_at = [&](auto row, int tb, int hb) {   // this lane's 8 bytes of block (tb, hb)
    const int r = 16 * tb + rl, c = 2 * hb + (cl >> 1);
    return row(r) + 16 * (c ^ (r & 7)) + 8 * (cl & 1);
  };
  const int lrow = l >> 3, lchunk = l & 7;   // row-segment role: rows lrow + 8 i
  auto lds_sync = [] {   // the wave's own LDS accesses are complete and ordered
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  };
  auto stage = [&](const u32x2 (&pk)[TB][HB]) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) *(u32x2*)frag_at(out_row, tb, hb) = pk[tb][hb];
  };
  // a staged tile (after lds_sync) to rows of dst; the stores are
  // non-temporal (measured faster: the tile is read back only by the next
  // kernel, after much other traffic)
  auto flush = [&](auto row, uint16_t* dst, int64_t ldd) {
    u32x4 seg[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = lrow + 8 * i;
      seg[i] = *(const u32x4*)(row(r) + 16 * (lchunk ^ (r & 7)));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t tok = t0 + row0 + lrow + 8 * i;
      if (tok < n)
        __builtin_nontemporal_store(seg[i], (u32x4*)(dst + tok * ldd + j0 + col0 + 8 * lchunk));
    }
  };

  if constexpr (MODE == kRead) {
    u32x2 pk[TB][HB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float v0[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xx = acc[0][hb][tb][r], bb = acc[1][hb][tb][r];
          v0[r] = xx * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(xx)) * bb;
        }
        pk[tb][hb] = u32x2{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3])};
      }
    stage(pk);
    lds_sync();
    flush(out_row, out0, ldo0);
  } else {
    float et[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      int64_t tok = t0 + row0 + 16 * tb + rl;
      if (tok >= n) tok = n - 1;
      et[tb] = eta[tok * eta_ld];
    }
    // ga to the output staging, eta u over e in its tile (each lane rewrites
    // the slot it read), gb held in registers
    u32x2 pb[TB][HB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        unsigned char* pe = frag_at(e_row, tb, hb);
        const u32x2 ev = *(const u32x2*)pe;
        float v0[4], v1[4], v2[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const unsigned wv = ev[r >> 1];
          const float xx = acc[0][hb][tb][r], bb = acc[1][hb][tb][r];
          const float ee = et[tb] * ((r & 1) ? bf16hi(wv) : bf16lo(wv));
          const float a = xx * kNegInvLog2e;
          const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(xx));
          const float sl = a * sg;
          v0[r] = ee * bb * (sg + sl * (1.f - sg));
          v1[r] = ee * sl;
          v2[r] = et[tb] * sl * bb;
        }
        *(u32x2*)frag_at(out_row, tb, hb) =
            u32x2{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3])};
        *(u32x2*)pe = u32x2{pack_bf16x2(v2[0], v2[1]), pack_bf16x2(v2[2], v2[3])};
        pb[tb][hb] = u32x2{pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
      }
    lds_sync();
    flush(out_row, out0, ldo0);
    flush(e_row, out1, ldo1);
    lds_sync();   // the output staging's reads are done before it is written again
    stage(pb);
    lds_sync();
    flush(out_row, out0 + ncols, ldo0);
  }
}

namespace {

// One block per (token tile, hidden tile).
template <class S>
unsigned rows_grid(int64_t n, int ncols) {
  constexpr int kTokGroups = 8 / kHidGroups;
  return (unsigned)(ceil_div(ceil_div(n, S::TM), kTokGroups) * kTokGroups * (ncols / TN));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

hipError_t launch_wide_fwd_gate_apply(const uint16_t* q, int64_t ldq, int64_t n,
                                      const uint16_t* w1, const uint16_t* w3, int d, int h,
                                      uint16_t* u, int64_t ldu, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d != kWideD || h % (8 * TN) != 0 || ldq % 8 || ldu % 8 || !aligned16(q) ||
      !aligned16(w1) || !aligned16(w3) || !aligned16(u))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_wide_rows<Cfg, kRead, kWideD>), dim3(rows_grid<Cfg>(n, h)),
                     dim3(Cfg::NW * 64), 0, st,
                     q, ldq, n, w1, w3, h, nullptr, 0, u, ldu, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_wide_fwd_gate_update(const uint16_t* k, int64_t ldk, int64_t n,
                                       const uint16_t* w1, const uint16_t* w3, int d, int h,
                                       const float* eta, int64_t eta_ld, uint16_t* gab,
                                       int64_t ldab, uint16_t* e, int64_t lde, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d != kWideD || h % (8 * TN) != 0 || ldk % 8 || ldab % 8 || lde % 8 || !aligned16(k) ||
      !aligned16(w1) || !aligned16(w3) || !aligned16(gab) || !aligned16(e))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_wide_rows<Cfg, kUpdate, kWideD>), dim3(rows_grid<Cfg>(n, h)),
                     dim3(Cfg::NW * 64), 0, st,
                     k, ldk, n, w1, w3, h, eta, eta_ld, gab, ldab, e, lde);
  return hipGetLastError();
}

}  // namespace zm
