// Apply kernel: o_i = f_W(q_i) = W2 [SiLU(W1 q_i) (*) (W3 q_i)] for every query
// token and head (review of ZipMap, kimjy99.github.io, Method 2, Eq. (1) and
// Eq. (4); target-view ray queries use the same read).  bf16 operands on the
// gfx950 matrix cores, fp32 accumulation, bf16 output.
//
// A workgroup owns (head, contiguous run of query tiles); per tile of 32
// tokens:
//   phase 1  each wave computes A^T = W1[J] Q^T and B^T = W3[J] Q^T for its
//            own h/8 hidden units J (its W1/W3 rows live in registers), then
//            U = SiLU(A) (*) B, written to LDS as bf16 [token][hidden];
//   phase 2  each wave computes O^T = W2[Dw, :] U^T for its own output rows
//            Dw (its W2 rows live in registers), K = all h hidden units.
// The tiles are software-pipelined (see the main loop) so that MFMA work of
// two tiles is interleaved with the gate's VALU / transcendental work of a
// third.
#pragma once

#include "zm_internal.h"

namespace zm {

template <int D, int HID>
struct AppCfg {
  static constexpr int T = kTok;
  // LDS layouts, each free of bank conflicts on gfx950 (64 four-byte banks
  // for reads: a 16-byte read serves 16 lanes per cycle, grouped by half-wave
  // and by the parity of the lane's quad index, an 8-byte read 32 lanes;
  // writes go 128 bytes per cycle):
  //   Q tile: rows padded by 32 bytes (row reads, 16-byte staging writes);
  //   U tile: unpadded rows, 16-byte chunk ch of row r stored at ch ^ (r % 16)
  //           (16-byte writes of 8 rows, row reads of 16 rows);
  //   O tile: rows padded by 8 bytes, so the 8-byte writes of 16 rows and the
  //           8-byte reads of the store both spread over all banks.
  static constexpr int DP = D + 16;           // Q tile row pitch (elements)
  static constexpr int UP = HID;              // U tile row pitch
  static constexpr int OP = D + 4;            // output tile row pitch
  static constexpr int HPW = HID / kWaves;    // phase-1 hidden units per wave (16 or 32)
  static constexpr int MB1 = HPW / 16;        // phase-1 row blocks per wave
  static constexpr int KS1 = D / 32;          // phase-1 k-steps
  static constexpr int NB = T / 16;           // token blocks per tile
  static constexpr int DB = D / 16;           // phase-2 row blocks (16 output dims each)
  static constexpr int WPD = kWaves / DB;     // waves sharing one phase-2 row block
  static constexpr int TBW = NB / WPD;        // token blocks per wave in phase 2
  static constexpr int KS2 = HID / 32;        // phase-2 k-steps
  static constexpr int CPT = D / 8;           // 16-byte chunks per query row
  static constexpr int ITEMS = T * CPT;
  // one LDS buffer: Q tiles [2][T * DP], then U tiles [2][T * UP], then O
  // tiles [2][T * OP] (each part a multiple of 16 bytes)
  static constexpr int US_OFF = 2 * T * DP;
  static constexpr int OS_OFF = US_OFF + 2 * T * UP;
  static constexpr int LDS_ELEMS = OS_OFF + 2 * T * OP;
  static_assert(US_OFF % 8 == 0 && OS_OFF % 8 == 0, "16-byte aligned parts");
  static_assert(MB1 >= 1 && MB1 <= 2, "hidden width per wave");
  static_assert(WPD >= 1 && TBW >= 1, "phase-2 split");
  static_assert(ITEMS <= kWaves * 64, "staging");
};

// SiLU(a) b up to the factor -log2(e): x = -log2(e) a comes out of the
// matrix core (the bf16 W1 copy carries the factor) and the bf16 W2 copy
// carries -1/log2(e), so x sig(a) b is what the second product needs.
__device__ __forceinline__ float silu_gate(float x, float b) {
  const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x));
  return x * sg * b;
}

// Element offset of U(r, col) in its tile (col a multiple of 4).
template <int HID>
__device__ __forceinline__ int u_off(int r, int col) {
  return r * HID + (((col >> 3) ^ (r & 15)) << 3) + (col & 7);
}

// The work of apply block `blk` (one workgroup of 512 threads): the kernels
// that run it pass their block index and a 16-byte-aligned LDS buffer of
// AppCfg::LDS_ELEMS elements, viewed here as the Q, U and O tile pairs.
template <int D, int HID>
__device__ __forceinline__ void apply_tiles(
    int blk, uint16_t* __restrict__ lds, const uint16_t* __restrict__ qp,
    uint16_t* __restrict__ op, int64_t n, int64_t ld, int heads,
    const uint16_t* __restrict__ w1b, const uint16_t* __restrict__ w3b,
    const uint16_t* __restrict__ w2b, int64_t chunk) {
  using C = AppCfg<D, HID>;
  constexpr int T = C::T, DP = C::DP, UP = C::UP, MB1 = C::MB1, KS1 = C::KS1, NB = C::NB,
                DB = C::DB, TBW = C::TBW, KS2 = C::KS2, CPT = C::CPT;
  uint16_t(*const qs)[T * DP] = reinterpret_cast<uint16_t(*)[T * DP]>(lds);
  uint16_t(*const us)[T * UP] = reinterpret_cast<uint16_t(*)[T * UP]>(lds + C::US_OFF);
  uint16_t(*const os)[T * C::OP] = reinterpret_cast<uint16_t(*)[T * C::OP]>(lds + C::OS_OFF);

  const unsigned ublk = (unsigned)blk;
  const int head = (int)(ublk % (unsigned)heads);
  const int64_t t_begin = (int64_t)(ublk / (unsigned)heads) * chunk;
  const int64_t t_end = (t_begin + chunk < n) ? t_begin + chunk : n;
  if (t_begin >= t_end) return;
  const int ntiles = (int)ceil_div(t_end - t_begin, T);

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
  const int j0 = w * C::HPW;

  // Phase-1 A operands: lane holds W[j0 + perm(mb, c)][32 ks + 8 g .. +7].
  // With two row blocks, row m of block mb is hidden unit 8 (m/4) + 4 mb + m%4,
  // so accumulator rows 4g..4g+3 of both blocks are hidden j0 + 8g .. 8g+7.
  bf16x8 w1f[MB1][KS1], w3f[MB1][KS1];
#pragma unroll
  for (int mb = 0; mb < MB1; ++mb) {
    const int hrow = MB1 == 2 ? 8 * (c >> 2) + 4 * mb + (c & 3) : c;
    const int64_t off = ((int64_t)head * HID + j0 + hrow) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks) {
      w1f[mb][ks] = as_bf16x8(*(const u32x4*)(w1b + off + 32 * ks));
      w3f[mb][ks] = as_bf16x8(*(const u32x4*)(w3b + off + 32 * ks));
    }
  }
  // Phase-2 A operands: lane holds W2[16 db + c][32 ks + 8 g .. +7].
  const int db = w % DB;
  const int tb0 = (w / DB) * TBW;
  bf16x8 w2f[KS2];
  {
    const int64_t off = ((int64_t)head * D + 16 * db + c) * HID + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks) w2f[ks] = as_bf16x8(*(const u32x4*)(w2b + off + 32 * ks));
  }

  const bool has_item = tid < C::ITEMS;
  const int s_tok = tid / CPT, s_ch = tid - (tid / CPT) * CPT;
  // Query rows past the end are fetched from a valid row (the tile's first)
  // and their outputs are never stored, so no zeroing is needed.
  const int lane_off = has_item ? s_tok * (int)ld + head * D + 8 * s_ch : head * D;
  auto fetch = [&](int it) {
    const int64_t t0 = t_begin + (int64_t)it * T;
    // queries are read once and outputs written once: non-temporal, so the L2
    // keeps the weights (and, in the shared launch, the partial sums) instead
    if (t0 + T <= t_end) return __builtin_nontemporal_load((const u32x4*)(qp + t0 * ld + lane_off));
    const int64_t tc = (has_item && t0 < t_end && t0 + s_tok < t_end) ? t0 + s_tok
                       : (t0 < t_end ? t0 : t_begin);
    return *(const u32x4*)(qp + tc * ld + head * D + (has_item ? 8 * s_ch : 0));
  };
  auto stage = [&](int buf, const u32x4& qr) {
    if constexpr (C::ITEMS < kWaves * 64) {
      if (!has_item) return;
    }
    *(u32x4*)(&qs[buf & 1][s_tok * DP + 8 * s_ch]) = qr;
  };

  struct Acc1 {
    f32x4 a[MB1][NB], b[MB1][NB];
  };
  // phase-1 slot (ks, nb): one Q^T operand, 2 * MB1 MFMAs
  auto p1_frag = [&](int buf, int ks, int nb) {
    return as_bf16x8(*(const u32x4*)(&qs[buf & 1][(16 * nb + c) * DP + 32 * ks + 8 * g]));
  };
  auto p1_mma = [&](Acc1& x, int ks, int nb, const bf16x8& qf) {
#pragma unroll
    for (int mb = 0; mb < MB1; ++mb) {
      if (ks == 0) {
        x.a[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        x.b[mb][nb] = x.a[mb][nb];
      }
      x.a[mb][nb] = mfma_bf16(w1f[mb][ks], qf, x.a[mb][nb]);
      x.b[mb][nb] = mfma_bf16(w3f[mb][ks], qf, x.b[mb][nb]);
    }
  };
  auto phase1 = [&](int buf) {
    Acc1 x;
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) p1_mma(x, ks, nb, p1_frag(buf, ks, nb));
    return x;
  };
  // Phase-2 slot k: two U^T operands and two MFMAs.  With two token blocks
  // per wave the slot is k-step k of both blocks (independent accumulators);
  // with one block it is k-steps 2 k and 2 k + 1 of that block.
  struct Frag2 {
    bf16x8 x, y;
  };
  auto p2_frag = [&](int buf, int k) {
    const uint16_t* ub = us[buf & 1];
    if constexpr (TBW == 2) {
      const int r = 16 * tb0 + c;
      return Frag2{as_bf16x8(*(const u32x4*)(ub + u_off<HID>(r, 8 * g + 32 * k))),
                   as_bf16x8(*(const u32x4*)(ub + u_off<HID>(r + 16, 8 * g + 32 * k)))};
    } else {
      const int r = 16 * tb0 + c;
      return Frag2{as_bf16x8(*(const u32x4*)(ub + u_off<HID>(r, 8 * g + 64 * k))),
                   as_bf16x8(*(const u32x4*)(ub + u_off<HID>(r, 8 * g + 64 * k + 32)))};
    }
  };
  // q selects the slot's first (0) or second (1) MFMA
  auto p2_mma1 = [&](f32x4* acc, int k, int q, const Frag2& fr) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    if constexpr (TBW == 2) {
      acc[q] = mfma_bf16(w2f[k], q == 0 ? fr.x : fr.y, k == 0 ? z : acc[q]);
    } else {
      acc[0] = mfma_bf16(w2f[2 * k + q], q == 0 ? fr.x : fr.y, (k == 0 && q == 0) ? z : acc[0]);
    }
  };
  auto p2_mma = [&](f32x4* acc, int k, const Frag2& fr) {
    p2_mma1(acc, k, 0, fr);
    p2_mma1(acc, k, 1, fr);
  };
  // Outputs go through LDS so that each output row leaves as one coalesced
  // 16-byte-per-lane store: phase 2 of tile it writes its results (lane holds
  // O[token 16 tb + c][16 db + 4 g + i]) into os[it % 2], and the next
  // iteration, after the barrier, stores the tile to memory at its end.
  auto o_to_lds = [&](const f32x4* acc, int it) {
#pragma unroll
    for (int tbi = 0; tbi < TBW; ++tbi) {
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[tbi][0], acc[tbi][1]);
      pk[1] = pack_bf16x2(acc[tbi][2], acc[tbi][3]);
      *(u32x2*)(&os[it & 1][(16 * (tb0 + tbi) + c) * C::OP + 16 * db + 4 * g]) = pk;
    }
  };
  const int o_lane_off = has_item ? s_tok * (int)ld + head * D + 8 * s_ch : 0;
  // Reading an output tile back from LDS and storing it are separate steps,
  // so the read can be issued early in an iteration and the store late.
  // The two 8-byte halves are read as two instructions.  Merged into one
  // ds_read2_b64 (what the compiler does with adjacent reads) they are served
  // like a 16-byte read, 16 lanes per cycle, where two rows of the tile meet in
  // every bank group: 1.5e7 bank-conflict cycles per f700 launch, against none
  // with the reads apart.  The offset of the second half is hidden from the
  // compiler so that it keeps them apart.
  auto o_read = [&](int it) {
    const uint16_t* src = &os[it & 1][(has_item ? s_tok : 0) * C::OP + 8 * s_ch];
    const u32x2 lo = *(const u32x2*)(src);
    unsigned half = 4;
    asm volatile("" : "+v"(half));
    const u32x2 hi = *(const u32x2*)(src + half);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  auto o_store = [&](int it, const u32x4& v) {
    if constexpr (C::ITEMS < kWaves * 64) {
      if (!has_item) return;
    }
    const int64_t tile0 = t_begin + (int64_t)it * T;
    if (tile0 + s_tok < t_end) __builtin_nontemporal_store(v, (u32x4*)(op + tile0 * ld + o_lane_off));
  };
  auto o_from_lds = [&](int it) { o_store(it, o_read(it)); };
  // SiLU gate of element e (= (mb * NB + nb) * 4 + i) into the packed U rows
  constexpr int NE = MB1 * NB * 4;
  auto gate_elem = [&](const Acc1& x, int e, float* uv) {
    const int i = e & 3, nb = (e >> 2) % NB, mb = (e >> 2) / NB;
    uv[e] = silu_gate(x.a[mb][nb][i], x.b[mb][nb][i]);
  };
  // U row nb of this wave: hidden j0 + 8 g .. (two row blocks) or j0 + 4 g ..;
  // upk[e / 2] holds elements e, e + 1 (element e = (mb * NB + nb) * 4 + i)
  // packed as bf16.
  auto write_u = [&](int buf, const unsigned* upk) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint16_t* ub = us[buf & 1];
      const int r = 16 * nb + c;
      if constexpr (MB1 == 2) {
        u32x4 pk;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int e0 = (mb * NB + nb) * 4;
          pk[2 * mb] = upk[e0 / 2];
          pk[2 * mb + 1] = upk[e0 / 2 + 1];
        }
        *(u32x4*)(ub + u_off<HID>(r, j0 + 8 * g)) = pk;
      } else {
        const int e0 = nb * 4;
        u32x2 pk;
        pk[0] = upk[e0 / 2];
        pk[1] = upk[e0 / 2 + 1];
        *(u32x2*)(ub + u_off<HID>(r, j0 + 4 * g)) = pk;
      }
    }
  };
  auto gate_all = [&](const Acc1& x, unsigned* upk) {
    float uv[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) gate_elem(x, e, uv);
#pragma unroll
    for (int e = 0; e < NE; e += 2) upk[e / 2] = pack_bf16x2(uv[e], uv[e + 1]);
  };

  // Software pipeline: iteration i gates tile i (VALU), multiplies tile i - 1
  // through W2 (phase 2) and tile i + 1 through W1, W3 (phase 1), as slots of
  // MFMAs whose LDS operands are fetched two slots ahead; one gate micro-step
  // follows each MFMA.  Then U(i) goes to LDS, O(i - 1) to LDS, Q(i + 2) is
  // staged and O(i - 2) leaves for memory.  Two Q, U and O buffers; one
  // barrier per iteration; wave priority follows progress through the slots.
  constexpr int NS2 = TBW * KS2 / 2;   // phase-2 slots
  constexpr int NS1 = KS1 * NB;        // phase-1 slots
  constexpr int NSLOT = NS1 + NS2;
  // The prologue's three tiles are fetched together, so that their memory
  // round trips overlap.
  const u32x4 q0 = fetch(0), q1 = fetch(1), q2 = fetch(2);
  stage(0, q0);
  stage(1, q1);
  __syncthreads();
  Acc1 cur = phase1(0);
  __syncthreads();  // every wave is done with Q(0) before Q(2) reuses its buffer
  f32x4 acc2[TBW];
  {  // i = 0: no phase 2 yet
    unsigned upk[NE / 2];
    gate_all(cur, upk);
    if (ntiles > 1) cur = phase1(1);
    write_u(0, upk);
    stage(2, q2);
    __syncthreads();
  }
  // Slots alternate phase 2 (two MFMAs) and phase 1 (2 * MB1 MFMAs) while
  // both last; the gate runs as a rolling three-stage pipeline over the
  // elements: in slot j, exp2 for element j, reciprocal for j - 1 and the
  // products for j - 2, so each slot holds independent work.
  auto slot_is_p2 = [&](int j) {
    constexpr int both = 2 * (NS1 < NS2 ? NS1 : NS2);
    return j < both ? (j & 1) == 0 : NS2 > NS1;
  };
  auto slot_idx = [&](int j) {  // index within its phase
    constexpr int both = 2 * (NS1 < NS2 ? NS1 : NS2);
    return j < both ? (j >> 1) : (j - both / 2);
  };
  // Gate micro-steps: elements in groups of four chains, 15 micro-steps per
  // group (four exp2, two steps of two adds, four reciprocals, two steps of
  // two products with x, two with b, one pair of bf16 packs), each at most
  // two plain VALU operations or one transcendental, so that one fits in the
  // shadow of one MFMA.
  constexpr int NMICRO = (NE / 4) * 15;
  auto step = [&](int it, const Acc1& cur, Acc1& nxt) __attribute__((always_inline)) {
    const u32x4 qn = fetch(it + 2);
    Frag2 f2[NSLOT];
    bf16x8 f1[NSLOT];
    auto load_slot = [&](int j) {
      const int k = slot_idx(j);
      if (slot_is_p2(j)) f2[j] = p2_frag(it - 1, k);
      else f1[j] = p1_frag(it + 1, k / NB, k % NB);
    };
    float gt[4], gy[4];
    unsigned upk[NE / 2];
    auto micro = [&](int m) __attribute__((always_inline)) {
      if (m >= NMICRO) return;
      const int grp = m / 15, k = m % 15;
      auto xv = [&](int h) {
        const int e = 4 * grp + h, i = e & 3, nb = (e >> 2) % NB, mb = (e >> 2) / NB;
        return cur.a[mb][nb][i];
      };
      auto bv = [&](int h) {
        const int e = 4 * grp + h, i = e & 3, nb = (e >> 2) % NB, mb = (e >> 2) / NB;
        return cur.b[mb][nb][i];
      };
      if (k < 4) {
        gt[k] = __builtin_amdgcn_exp2f(xv(k));
        pin(gt[k]);
      } else if (k < 6) {
        const int h = 2 * (k - 4);
        gt[h] = 1.f + gt[h];
        gt[h + 1] = 1.f + gt[h + 1];
        pin(gt[h]);
        pin(gt[h + 1]);
      } else if (k < 10) {
        gt[k - 6] = __builtin_amdgcn_rcpf(gt[k - 6]);
        pin(gt[k - 6]);
      } else if (k < 12) {
        const int h = 2 * (k - 10);
        gy[h] = xv(h) * gt[h];
        gy[h + 1] = xv(h + 1) * gt[h + 1];
        pin(gy[h]);
        pin(gy[h + 1]);
      } else if (k < 14) {
        const int h = 2 * (k - 12);
        gy[h] = gy[h] * bv(h);
        gy[h + 1] = gy[h + 1] * bv(h + 1);
        pin(gy[h]);
        pin(gy[h + 1]);
      } else {
        unsigned p0 = pack_bf16x2(gy[0], gy[1]), p1 = pack_bf16x2(gy[2], gy[3]);
        pin(p0);
        pin(p1);
        upk[2 * grp] = p0;
        upk[2 * grp + 1] = p1;
      }
    };
    constexpr int LA = 2;  // LDS operand lookahead, in slots
#pragma unroll
    for (int j = 0; j < LA; ++j) load_slot(j);
    int mi = 0;
    u32x4 ov = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
      set_progress_priority<NSLOT, 3, 1, 0>(j);
      if (j == 2 && it >= 2) ov = o_read(it - 2);  // output tile it - 2, stored at the end
      if (j + LA < NSLOT) load_slot(j + LA);
      const int k = slot_idx(j);
      if (slot_is_p2(j)) {
        p2_mma1(acc2, k, 0, f2[j]);
        micro(mi++);
        __builtin_amdgcn_sched_barrier(0);
        p2_mma1(acc2, k, 1, f2[j]);
        micro(mi++);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        const int ks = k / NB, nb = k % NB;
#pragma unroll
        for (int mb = 0; mb < MB1; ++mb) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          nxt.a[mb][nb] = mfma_bf16(w1f[mb][ks], f1[j], ks == 0 ? z : nxt.a[mb][nb]);
          micro(mi++);
          __builtin_amdgcn_sched_barrier(0);
          nxt.b[mb][nb] = mfma_bf16(w3f[mb][ks], f1[j], ks == 0 ? z : nxt.b[mb][nb]);
          micro(mi++);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int m = 0; m < NMICRO; ++m)
      if (m >= mi) micro(m);
    write_u(it, upk);
    o_to_lds(acc2, it - 1);
    stage(it + 2, qn);
    // Output tile it - 2 (in LDS since the previous iteration) leaves last,
    // so that its store has a whole iteration to complete before the next
    // wait on the memory counter.
    if (it >= 2) o_store(it - 2, ov);
    __syncthreads();
  };
  Acc1 alt;
  int it = 1;
  for (; it + 2 < ntiles; it += 2) {  // two steady iterations per trip
    step(it, cur, alt);
    step(it + 1, alt, cur);
  }
  if (it + 1 < ntiles) {
    step(it, cur, alt);
    cur = alt;
  }
  if (ntiles > 1) {  // i = ntiles - 1: no phase 1
    if (ntiles >= 3) o_from_lds(ntiles - 3);
    unsigned upk[NE / 2];
    gate_all(cur, upk);
#pragma unroll
    for (int k = 0; k < NS2; ++k) p2_mma(acc2, k, p2_frag(ntiles - 2, k));
    write_u(ntiles - 1, upk);
    o_to_lds(acc2, ntiles - 2);
    __syncthreads();
    o_from_lds(ntiles - 2);
  }
#pragma unroll
  for (int k = 0; k < NS2; ++k) p2_mma(acc2, k, p2_frag(ntiles - 1, k));
  o_to_lds(acc2, ntiles - 1);
  __syncthreads();
  o_from_lds(ntiles - 1);
}

}  // namespace zm
