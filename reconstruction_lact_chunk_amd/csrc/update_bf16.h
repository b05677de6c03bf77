// Chunk-gradient kernel of the large-chunk TTT update, bf16 operands on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation.
//
// What it computes (review of ZipMap, kimjy99.github.io, Method 2, Eq. (1)-(3);
// LaCT summary, mhpn.cn part 二 2、架构): for the SwiGLU fast weight
// f(x) = W2 [SiLU(W1 x) (*) (W3 x)] and the per-token loss -eta_i f(k_i)^T v_i,
// minus the gradient summed over a chunk of tokens is
//     D1 = sum_i  ga_i k_i^T,   D3 = sum_i gb_i k_i^T,   D2 = sum_i eta_i v_i u_i^T
// with a = W1 k, b = W3 k, s = SiLU(a), u = s (*) b, e = W2^T (eta v) and
//     ga = e (*) b (*) SiLU'(a),   gb = e (*) s,   SiLU'(a) = sig(a) + s (1 - sig(a)).
// eta is folded into v once per token (V_eta = eta v), so e, ga, gb carry it
// and D2 = sum_i u_i (eta_i v_i)^T needs no extra scaling.
//
// Work split: a workgroup owns (head, 128 hidden units, one chunk of tokens);
// each of its 8 waves owns 16 hidden units and keeps, for the whole chunk, its
// slice of D1^T, D3^T (d x 16) and D2^T (16 x d) in registers, plus its bf16
// slices of W1, W3, W2^T as MFMA operands.  Per tile of 32 tokens:
//   forward   A = K W1^T, B = K W3^T, E = V_eta W2   (M = tokens, K = d)
//   pointwise SiLU / gate backward in registers
//   backward  D1^T += K^T Ga, D3^T += K^T Gb, D2^T += U^T V_eta  (K = tokens)
// software-pipelined over tiles (see the main loop).  For short chunks the
// planner picks a second shape (TG = 2, UpdCfg): 64 hidden units per
// workgroup, its waves 4 hidden-unit groups x 2 token groups over 64-token
// tiles, whose accumulators are added in the workgroup before the partial
// sums are written (half the partial sums per workgroup).
// The backward contracts over tokens, so its K / V_eta operands are read
// from the token-major LDS tile with the gfx950 transposing LDS load
// (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
// i % 4 of the 8-byte words loaded by lanes 4e + i / 4 (e = 0..3), which turns
// four 4-column row pieces into four 4-row column pieces.  The forward's
// token rows are permuted (token map tau below) so that each lane's forward
// accumulators are exactly the tokens its backward operand slots hold, and
// the tile rows are XOR-swizzled in 16-byte chunks so that both the forward
// row reads and the transposing reads are free of LDS bank conflicts.
// The chunk's partial sums go to workspace; a second kernel adds them in a
// fixed order (no atomics, bitwise reproducible).
#pragma once

#include "zm_internal.h"

namespace zm {

// TG token groups: with TG = 1 the 8 waves of a workgroup own 8 x 16 hidden
// units and share every 32-token tile; with TG = 2 they are 4 hidden-unit
// groups x 2 token groups, a "tile" is 64 tokens (32 per token group) and the
// workgroup owns 64 hidden units.  TG = 2 writes half the partial sums per
// workgroup (the two token groups' accumulators are added in the workgroup
// first), which pays on short chunks such as a streamed frame, where writing
// and re-reading the partial sums is a large part of the time.
template <int D, int HID, int TG = 1>
struct UpdCfg {
  static constexpr int T = kTok;                // tokens per token group and tile
  static constexpr int HPW = 16 * kWaves / TG;  // hidden units per workgroup
  static constexpr int NSL = HID / HPW;         // hidden slices (workgroups) per head and chunk
  static constexpr int KS = D / 32;             // forward k-steps
  static constexpr int MB = D / 16;             // 16-row blocks along d
  static constexpr int CPT = D / 8;             // 16-byte chunks per token row
  static constexpr int ITEMS = TG * T * CPT;    // staging items per tile
  static constexpr int TILE = T * (D + 16);     // elements per padded 32-token tile
  static constexpr int SUB = 2 * TILE;          // one token group's K and V_eta tiles
  static constexpr int BUF = TG * SUB;          // elements per LDS buffer
  static constexpr int NBUF = TG == 1 ? 8 : 4;  // LDS buffers (tile t in buffer t % NBUF)
  static constexpr int LOOK = TG == 1 ? 3 : 2;  // tile t + LOOK is staged in iteration t
  static constexpr int LDS_ELEMS = NBUF * BUF;
  static constexpr int IPT = (ITEMS + kWaves * 64 - 1) / (kWaves * 64);  // staging items per thread
  static_assert(TG == 1 || TG == 2, "token groups");
  static_assert(HID % HPW == 0, "hidden slices");
  static_assert(IPT <= TG, "staging items per thread");
  // TG = 2 epilogue: one token group's three accumulator sets pass through LDS
  static_assert(TG == 1 || (kWaves / TG) * 3 * (D / 16) * 64 * 16 <= LDS_ELEMS * 2,
                "accumulator exchange fits the LDS buffer");
};

// Tile layout: row r (token) of D bf16, rows padded by 32 bytes.  gfx950 LDS
// reads see 64 four-byte banks; a 16-byte read is served 16 lanes per cycle
// (each half-wave split by the parity of the lane's quad index), an 8-byte
// read 32 lanes per cycle, and writes go 128 bytes per cycle.  With this
// pitch and the token map tau below, the forward row reads, the transposing
// reads and the staging writes are all free of bank conflicts, and every
// operand address of a slot is a per-lane base plus a constant, so the
// addresses cost no VALU work inside the loop.
template <int D>
__device__ __forceinline__ constexpr int tile_pitch() {
  return D + 16;
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * tile_pitch<D>() + col;
}
// Token held in operand slot j (0..7) by the lanes of 16-lane group g; the
// forward's MFMA row m = 4 g' + i of block mb reads token tau(g', 4 mb + i).
__device__ __forceinline__ int tau(int g, int j) {
  return 16 * (g >> 1) + 4 * (g & 1) + 8 * (j >> 2) + (j & 3);
}

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) void*)(p)));
}

// SiLU / gate backward for one (token, hidden) element.  x = -log2(e) W1 k
// (the bf16 W1 copy carries the factor), b = W3 k, e = W2^T (eta v).
// Returns ga, gb and u = SiLU(a) b, each scaled by -log2(e); the kernel undoes
// that scale on the partial sums.  With s' = x sig = -log2(e) SiLU(a):
//   sig = 1 / (1 + 2^x),  u' = s' b,  gb' = e s',
//   ga' = e (u' + sig (-log2(e) b - u')),
// the last from ga = e b (sig + s (1 - sig)) = e (u + sig (b - u)), which
// takes one operation fewer per element than the product form.
__device__ __forceinline__ void gate_backward(float x, float b, float e, float& ga, float& gb,
                                              float& u) {
  const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x));
  const float sp = x * sg;
  u = sp * b;
  gb = e * sp;
  ga = e * fmaf(sg, fmaf(kNegLog2e, b, -u), u);
}

// Block -> (pair, slice) of the update: blocks are dispatched round-robin
// over the 8 XCDs (block b on XCD (b + s) mod 8, s fixed within a launch);
// the NSL hidden slices of one (head, chunk) pair get ids 8 apart, so they
// run on the same XCD at about the same time and share K/V through its L2.
// Pair p is head p % heads of token chunk p / heads; p >= heads * splits
// marks a block without work.  With heads a multiple of 8, every block of
// head j has an id of j's residue mod 8.
template <int NSL>
__device__ __forceinline__ int upd_block_pair(int blk) {
  const int lane8 = blk & 7, r = blk >> 3;
  return (r / NSL) * 8 + lane8;
}

// The work of update block `blk` (one workgroup of 512 threads): the kernels
// that run it pass their block index (offset by a multiple of 8, so that
// blocks whose indices agree mod 8 still share an XCD) and a 16-byte-aligned
// LDS buffer of UpdCfg::LDS_ELEMS elements.
// With LOSS, the block also sums u' . e over its tokens and hidden units (u'
// = -log2(e) u and e = W2^T (eta v) are both in registers for the gate
// backward) and writes the sum to loss_part[(chunk * heads + head) * NSL +
// slice]: the per-token loss -eta_i f(k_i)^T v_i = -eta_i u_i . W2^T v_i of
// the review of ZipMap, Method 2, Eq. (2), summed, is ln(2) times the sum of
// those block values.
template <int D, int HID, bool LOSS = false, int TG = 1>
__device__ __forceinline__ void update_tiles(
    int blk, uint16_t* __restrict__ lds, const uint16_t* __restrict__ kp,
    const uint16_t* __restrict__ vp, const float* __restrict__ eta, int64_t n, int64_t ld,
    int heads, const uint16_t* __restrict__ w1b, const uint16_t* __restrict__ w3b,
    const uint16_t* __restrict__ w2tb, float* __restrict__ part, int splits, int64_t chunk,
    float* __restrict__ loss_part = nullptr) {
  using C = UpdCfg<D, HID, TG>;
  constexpr int T = C::T, KS = C::KS, MB = C::MB, CPT = C::CPT, IPT = C::IPT;

  const int slice = (blk >> 3) % C::NSL;
  const int pair = upd_block_pair<C::NSL>(blk);
  if (pair >= heads * splits) return;
  const int head = pair % heads, chunk_id = pair / heads;
  const int64_t t_begin = (int64_t)chunk_id * chunk;
  const int64_t t_end = (t_begin + chunk < n) ? t_begin + chunk : n;
  const int ntiles = t_end > t_begin ? (int)ceil_div(t_end - t_begin, TG * T) : 0;  // tiles of TG * T tokens

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
  constexpr int WPG = kWaves / TG;            // waves per token group
  const int tg = w / WPG;                     // this wave's token group
  const int j0 = slice * C::HPW + (w % WPG) * 16;  // first hidden unit of this wave

  // Forward B operands: lane holds W[j0 + c][32 ks + 8 g .. +7].
  bf16x8 w1f[KS], w3f[KS], w2f[KS];
  {
    const int64_t off = ((int64_t)head * HID + j0 + c) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      w1f[ks] = as_bf16x8(*(const u32x4*)(w1b + off + 32 * ks));
      w3f[ks] = as_bf16x8(*(const u32x4*)(w3b + off + 32 * ks));
      w2f[ks] = as_bf16x8(*(const u32x4*)(w2tb + off + 32 * ks));
    }
  }

  f32x4 acc1[MB], acc3[MB], acc2[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    acc1[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc3[m] = acc1[m];
    acc2[m] = acc1[m];
  }
  float lacc = 0.f;   // LOSS: this lane's sum of u' e

  // ---- staging: IPT 16-byte chunks of k and of v per thread -------------
  // Item i = tid + 512 q of a tile is token row i / CPT (row r of token group
  // r / 32) and 16-byte chunk i % CPT.
  struct Staged {
    u32x4 k[IPT], v[IPT];
    float e[IPT];
  };
  bool has_item[IPT];
  int s_tok[IPT], s_ch[IPT], lane_tok_off[IPT], lane_eta_off[IPT];
#pragma unroll
  for (int q = 0; q < IPT; ++q) {
    const int it_ = tid + q * kWaves * 64;
    has_item[q] = it_ < C::ITEMS;
    s_tok[q] = it_ / CPT;
    s_ch[q] = it_ - (it_ / CPT) * CPT;
    // Per-lane element offsets of this thread's staging chunk inside a tile;
    // the tile base is uniform, so loads use a scalar base + vector offset.
    lane_tok_off[q] = has_item[q] ? s_tok[q] * (int)ld + head * D + 8 * s_ch[q] : head * D;
    lane_eta_off[q] = (has_item[q] ? s_tok[q] : 0) * heads + head;
  }
  constexpr int TT = TG * T;  // tokens per tile
  constexpr int QROWS = kWaves * 64 / CPT;  // token rows between a thread's staging items
  static_assert(IPT == 1 || C::ITEMS % (kWaves * 64) == 0, "every thread has all its items");
  auto fetch = [&](int it) {
    const int64_t t0 = t_begin + (int64_t)it * TT;
    Staged r;
    if (t0 + TT <= t_end) {  // whole tile in range (uniform branch)
      // item q is item 0 moved by q * QROWS token rows: one per-lane offset,
      // the rest in the uniform base
#pragma unroll
      for (int q = 0; q < IPT; ++q) {
        const int64_t tq = t0 + (int64_t)q * QROWS;
        // Tokens are streamed (read by the NSL slices of one XCD, then dead):
        // non-temporal loads let the L2 evict them first, which keeps more of
        // a short chunk's partial sums there for the in-launch reduce.
        r.k[q] = __builtin_nontemporal_load((const u32x4*)(kp + tq * ld + lane_tok_off[0]));
        r.v[q] = __builtin_nontemporal_load((const u32x4*)(vp + tq * ld + lane_tok_off[0]));
        r.e[q] = eta[tq * heads + lane_eta_off[0]];
      }
    } else if (TG == 2 && t0 >= t_end) {
      // a tile past the last one (prefetch overrun): staged, never read
#pragma unroll
      for (int q = 0; q < IPT; ++q) {
        r.k[q] = u32x4{0u, 0u, 0u, 0u};
        r.v[q] = r.k[q];
        r.e[q] = 0.f;
      }
    } else {
      // Tail tile: out-of-range tokens get eta = 0 and a real token's k and v
      // (finite values; eta = 0 zeroes their contribution, since e, ga, gb
      // and V_eta all carry eta).
      // Tiles past the last one (prefetch overrun) read the chunk's first
      // token, so every load stays inside the token array.
#pragma unroll
      for (int q = 0; q < IPT; ++q) {
        const bool ok = has_item[q] && t0 + s_tok[q] < t_end;
        const int64_t tc = ok ? t0 + s_tok[q] : (t0 < t_end ? t0 : t_begin);
        const int col = has_item[q] ? 8 * s_ch[q] : 0;
        r.k[q] = *(const u32x4*)(kp + tc * ld + head * D + col);
        r.v[q] = *(const u32x4*)(vp + tc * ld + head * D + col);
        const float e0 = eta[tc * heads + head];
        r.e[q] = ok ? e0 : 0.f;
      }
    }
    return r;
  };
  auto stage = [&](int buf, const Staged& r) {
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
      if (C::ITEMS < (q + 1) * kWaves * 64 && !has_item[q]) continue;  // folds per q
      // token row s_tok lies in token group s_tok / T
      const int grp = TG == 1 ? 0 : s_tok[q] / T;
      uint16_t* ktm = lds + (buf & (C::NBUF - 1)) * C::BUF + grp * C::SUB;
      uint16_t* vtm = ktm + C::TILE;
      u32x4 vs;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vs[i] = pack_bf16x2(bf16lo(r.v[q][i]) * r.e[q], bf16hi(r.v[q][i]) * r.e[q]);
      const int off = tile_off<D>(TG == 1 ? s_tok[q] : s_tok[q] % T, 8 * s_ch[q]);
      *(u32x4*)(ktm + off) = r.k[q];
      *(u32x4*)(vtm + off) = vs;
    }
  };
  // this wave's K tile in buffer buf (its V_eta tile follows at + TILE)
  auto tile_base = [&](int buf) -> uint16_t* {
    return lds + (buf & (C::NBUF - 1)) * C::BUF + (TG == 1 ? 0 : tg * C::SUB);
  };

  // Transposing-read addresses: lane (g, s) loads 4 columns 16 m + 4 (s % 4)
  // of rows tau(g, s / 4) (slots 0..3) and tau(g, 4 + s / 4) (slots 4..7).
  const int row_a = tau(g, c >> 2), row_b = row_a + 8;

  struct Fwd {
    f32x4 a[2], b[2], e[2];
  };
  struct Grad {
    bf16x8 ga, gb, u;
  };

  // forward A = K W1^T, B = K W3^T, E = V_eta W2 on one tile (24 MFMAs)
  auto forward = [&](int buf) {
    const uint16_t* ktm = tile_base(buf);
    const uint16_t* vtm = ktm + C::TILE;
    Fwd f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f.a[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      f.b[mb] = f.a[mb];
      f.e[mb] = f.a[mb];
      // MFMA row m = 4 g' + i of block mb holds token tau(g', 4 mb + i), so a
      // lane's accumulator rows are the tokens of its backward slots.
      const int row = tau(c >> 2, 4 * mb + (c & 3));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = tile_off<D>(row, 32 * ks + 8 * g);
        const bf16x8 ka = as_bf16x8(*(const u32x4*)(ktm + off));
        const bf16x8 va = as_bf16x8(*(const u32x4*)(vtm + off));
        f.a[mb] = mfma_bf16(ka, w1f[ks], f.a[mb]);
        f.b[mb] = mfma_bf16(ka, w3f[ks], f.b[mb]);
        f.e[mb] = mfma_bf16(va, w2f[ks], f.e[mb]);
      }
    }
    return f;
  };

  // pointwise SiLU / gate backward (VALU); slot j of each operand is token tau(g, j)
  auto pointwise = [&](const Fwd& f) {
    u32x4 gap, gbp, up;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        float ga0, gb0, u0, ga1, gb1, u1;
        gate_backward(f.a[mb][i], f.b[mb][i], f.e[mb][i], ga0, gb0, u0);
        gate_backward(f.a[mb][i + 1], f.b[mb][i + 1], f.e[mb][i + 1], ga1, gb1, u1);
        if constexpr (LOSS) {
          lacc = fmaf(u0, f.e[mb][i], lacc);
          lacc = fmaf(u1, f.e[mb][i + 1], lacc);
        }
        gap[2 * mb + i / 2] = pack_bf16x2(ga0, ga1);
        gbp[2 * mb + i / 2] = pack_bf16x2(gb0, gb1);
        up[2 * mb + i / 2] = pack_bf16x2(u0, u1);
      }
    }
    return Grad{as_bf16x8(gap), as_bf16x8(gbp), as_bf16x8(up)};
  };

  // backward D1^T += K^T Ga, D3^T += K^T Gb, D2^T += U^T V_eta (24 MFMAs)
  auto backward = [&](int buf, const Grad& gr) {
    const uint16_t* ktm = tile_base(buf);
    const uint16_t* vtm = ktm + C::TILE;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int col = 16 * m + 4 * (c & 3);
      const int oa = tile_off<D>(row_a, col), ob = tile_off<D>(row_b, col);
      // A = K^T: rows d = 16 m + c, slots = tokens tau(g, 0..7); B = Ga / Gb
      const bf16x8 kt = __builtin_shufflevector(lds_read_tr(ktm + oa), lds_read_tr(ktm + ob),
                                                0, 1, 2, 3, 4, 5, 6, 7);
      acc1[m] = mfma_bf16(kt, gr.ga, acc1[m]);
      acc3[m] = mfma_bf16(kt, gr.gb, acc3[m]);
      // A = U^T (hidden x tokens); B = V_eta (tokens x d = 16 m + c)
      const bf16x8 vt = __builtin_shufflevector(lds_read_tr(vtm + oa), lds_read_tr(vtm + ob),
                                                0, 1, 2, 3, 4, 5, 6, 7);
      acc2[m] = mfma_bf16(gr.u, vt, acc2[m]);
    }
  };

  // ---- one "slot" = one operand fetch from LDS + 3 MFMAs ------------------
  struct Frag2 {
    bf16x8 x, y;
  };
  auto fwd_frag = [&](int buf, int mb, int ks) {  // K and V_eta rows (A operands)
    const uint16_t* ktm = tile_base(buf);
    const int off = tile_off<D>(tau(c >> 2, 4 * mb + (c & 3)), 32 * ks + 8 * g);
    return Frag2{as_bf16x8(*(const u32x4*)(ktm + off)),
                 as_bf16x8(*(const u32x4*)(ktm + C::TILE + off))};
  };
  auto bwd_frag = [&](int buf, int m) {  // K^T and V_eta^T column pieces
    const uint16_t* ktm = tile_base(buf);
    const int col = 16 * m + 4 * (c & 3);
    const int oa = tile_off<D>(row_a, col), ob = tile_off<D>(row_b, col);
    return Frag2{__builtin_shufflevector(lds_read_tr(ktm + oa), lds_read_tr(ktm + ob),
                                         0, 1, 2, 3, 4, 5, 6, 7),
                 __builtin_shufflevector(lds_read_tr(ktm + C::TILE + oa),
                                         lds_read_tr(ktm + C::TILE + ob), 0, 1, 2, 3, 4, 5, 6, 7)};
  };

  constexpr int NBS = MB;            // backward slots
  constexpr int NSLOT = NBS + 2 * KS;
  constexpr int LA = 1;              // LDS operand lookahead, in slots (2 spills)
  auto load_slot = [&](int t, int j) __attribute__((always_inline)) {
    return j < NBS ? bwd_frag(t - 1, j) : fwd_frag(t + 1, (j - NBS) / KS, (j - NBS) % KS);
  };
  // Steady iteration t: backward(t - 1) in slots 0..NBS-1 and forward(t + 1)
  // in slots NBS..NSLOT-1, three MFMAs per slot, each slot's LDS operands
  // fetched LA slots ahead.  The gate backward of tile t is cut into
  // micro-steps of at most two plain VALU operations or one transcendental,
  // and one micro-step follows each MFMA: on gfx950 about that much VALU work
  // issues in the shadow of a 16x16x32 MFMA, while longer VALU runs stall
  // the matrix core.  Element rows are processed in pairs (two independent
  // chains), 13 micro-steps per pair; the steps left over after the last
  // MFMA, then staging of tile t + 2 and one barrier close the iteration.
  // Every gate value is pinned where it is computed so that the compiler
  // keeps this placement.  The loop is unrolled by two so the carried state
  // alternates between two register sets instead of being copied.
  constexpr int NMICRO = 4 * 13;
  auto step = [&](int t, const Fwd& f, const Grad& prev, Fwd& fn, Grad& cur, bool barrier)
      __attribute__((always_inline)) {
    const Staged nx = fetch(t + C::LOOK);
    Frag2 fr[NSLOT];
#pragma unroll
    for (int j = 0; j < LA; ++j) fr[j] = load_slot(t, j);
    float g_t[2], g_sg[2], g_sp[2], g_u[2], g_gb[2], g_w[2], g_ga[2];
    u32x4 gap, gbp, up;
    auto micro = [&](int i) __attribute__((always_inline)) {
      if (i >= NMICRO) return;
      const int pr = i / 13, k = i % 13;
      auto el = [&](int h, auto&& fn2) __attribute__((always_inline)) {
        const int r = 2 * pr + h, mb = r >> 2, q = r & 3;
        fn2(h, f.a[mb][q], f.b[mb][q], f.e[mb][q]);
      };
      switch (k) {
        case 0:
        case 1:
          el(k, [&](int h, float x, float, float) { g_t[h] = __builtin_amdgcn_exp2f(x); pin(g_t[h]); });
          break;
        case 2:
          el(0, [&](int h, float, float, float) { g_t[h] = 1.f + g_t[h]; pin(g_t[h]); });
          el(1, [&](int h, float, float, float) { g_t[h] = 1.f + g_t[h]; pin(g_t[h]); });
          break;
        case 3:
        case 4:
          el(k - 3, [&](int h, float, float, float) { g_sg[h] = __builtin_amdgcn_rcpf(g_t[h]); pin(g_sg[h]); });
          break;
        case 5:
          for (int h = 0; h < 2; ++h)
            el(h, [&](int hh, float x, float, float) { g_sp[hh] = x * g_sg[hh]; pin(g_sp[hh]); });
          break;
        case 6:
          for (int h = 0; h < 2; ++h)
            el(h, [&](int hh, float, float b, float) { g_u[hh] = g_sp[hh] * b; pin(g_u[hh]); });
          break;
        case 7:
          for (int h = 0; h < 2; ++h)
            el(h, [&](int hh, float, float, float e) { g_gb[hh] = e * g_sp[hh]; pin(g_gb[hh]); });
          break;
        case 8:
          for (int h = 0; h < 2; ++h)
            el(h, [&](int hh, float, float b, float) {
              g_w[hh] = fmaf(kNegLog2e, b, -g_u[hh]);
              pin(g_w[hh]);
            });
          break;
        case 9:
          for (int h = 0; h < 2; ++h)
            el(h, [&](int hh, float, float, float) {
              g_w[hh] = fmaf(g_sg[hh], g_w[hh], g_u[hh]);
              pin(g_w[hh]);
            });
          break;
        case 10:
          for (int h = 0; h < 2; ++h)
            el(h, [&](int hh, float, float, float e) { g_ga[hh] = e * g_w[hh]; pin(g_ga[hh]); });
          break;
        case 11: {
          unsigned pa = pack_bf16x2(g_ga[0], g_ga[1]), pb = pack_bf16x2(g_gb[0], g_gb[1]);
          pin(pa);
          pin(pb);
          gap[pr] = pa;
          gbp[pr] = pb;
          break;
        }
        default: {
          unsigned pu = pack_bf16x2(g_u[0], g_u[1]);
          pin(pu);
          up[pr] = pu;
          if constexpr (LOSS) {
            el(0, [&](int, float, float, float e) { lacc = fmaf(g_u[0], e, lacc); });
            el(1, [&](int, float, float, float e) { lacc = fmaf(g_u[1], e, lacc); });
          }
          break;
        }
      }
    };
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
      set_progress_priority<NSLOT, 3, 2, 1>(j);
      if (j + LA < NSLOT) fr[j + LA] = load_slot(t, j + LA);
      const Frag2& c = fr[j];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        if (j < NBS) {
          if (q == 0) acc1[j] = mfma_bf16(c.x, prev.ga, acc1[j]);
          if (q == 1) acc3[j] = mfma_bf16(c.x, prev.gb, acc3[j]);
          if (q == 2) acc2[j] = mfma_bf16(prev.u, c.y, acc2[j]);
        } else {
          const int mb = (j - NBS) / KS, ks = (j - NBS) % KS;
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          if (q == 0) fn.a[mb] = mfma_bf16(c.x, w1f[ks], ks == 0 ? z : fn.a[mb]);
          if (q == 1) fn.b[mb] = mfma_bf16(c.x, w3f[ks], ks == 0 ? z : fn.b[mb]);
          if (q == 2) fn.e[mb] = mfma_bf16(c.y, w2f[ks], ks == 0 ? z : fn.e[mb]);
        }
        micro(3 * j + q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 3 * NSLOT; i < NMICRO; ++i) micro(i);
    stage(t + C::LOOK, nx);
    if (barrier) __syncthreads();
    cur = Grad{as_bf16x8(gap), as_bf16x8(gbp), as_bf16x8(up)};
  };

  // TG = 1: tile t is staged in iteration t - 3 (the prologue stages tiles
  // 0..3), read by the forward in iteration t - 1 and by the backward in
  // iteration t + 1.  A barrier closes every even iteration only: a staged
  // tile is first read two iterations later, and a buffer is rewritten
  // (NBUF = 8) four iterations after its last read, so a barrier always lies
  // between.  The prologue's four tiles are fetched together, so that their
  // memory round trips overlap (on a short chunk the prologue is a large part
  // of the block's time).
  // TG = 2 (tiles twice as large, NBUF = 4): tile t is staged in iteration
  // t - 2 and a barrier closes every iteration; a buffer is rewritten two
  // iterations after its last read.
  if (ntiles > 0) {
    Fwd fa, fb;
    Grad ga_, gb_;
    if constexpr (TG == 1) {
      const Staged s0 = fetch(0), s1 = fetch(1), s2 = fetch(2), s3 = fetch(3);
      stage(0, s0);
      stage(1, s1);
      stage(2, s2);
      __syncthreads();
      fa = forward(0);
      ga_ = pointwise(fa);
      // t = 0: no backward yet
      if (ntiles > 1) fa = forward(1);
      stage(3, s3);
      __syncthreads();
    } else {
      const Staged s0 = fetch(0), s1 = fetch(1);
      stage(0, s0);
      stage(1, s1);
      const Staged s2 = fetch(2);
      __syncthreads();
      fa = forward(0);
      ga_ = pointwise(fa);
      if (ntiles > 1) fa = forward(1);
      stage(2, s2);
      __syncthreads();
    }
    int t = 1;
    for (; t + 2 < ntiles; t += 2) {  // steady state, two iterations per trip
      step(t, fa, ga_, fb, gb_, TG == 2);
      step(t + 1, fb, gb_, fa, ga_, true);
    }
    if (t + 1 < ntiles) {  // one steady iteration left
      step(t, fa, ga_, fb, gb_, true);
      fa = fb;
      ga_ = gb_;
      ++t;
    }
    if (ntiles > 1) {  // t = ntiles - 1: no forward
      const Grad cur = pointwise(fa);
      backward(ntiles - 2, ga_);
      ga_ = cur;
    }
    backward(ntiles - 1, ga_);
  }
  if constexpr (LOSS) {
    // lanes in butterfly order, then the 8 wave sums in wave order (fixed)
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) lacc += __shfl_xor(lacc, m, 64);
    __syncthreads();   // the tile ring is no longer read
    float* red = (float*)lds;
    if (l == 0) red[w] = lacc;
    __syncthreads();
    if (tid == 0) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) sum += red[i];
      loss_part[((int64_t)chunk_id * heads + head) * C::NSL + slice] = sum;
    }
  }
  // TG = 2: the two token groups' accumulators are added (group 0 + group 1:
  // one fixed order), each group combining and writing half of the 16-row
  // blocks m of all three sums (group 0 the first half).
  constexpr int MH = TG == 2 ? MB / 2 : MB;
  if constexpr (TG == 2) {
    static_assert(MB % 2 == 0, "blocks split between the token groups");
    __syncthreads();   // the tile ring (and the loss scratch) is no longer read
    f32x4* xch = reinterpret_cast<f32x4*>(lds);
    const int hg = w % WPG;
    // slot of (hidden group, receiving token group, sum, block m' < MH, lane)
    auto slot = [&](int to, int mat, int mm) { return (((hg * 2 + to) * 3 + mat) * MH + mm) * 64 + l; };
    if (tg == 0) {   // hands over blocks MH.., keeps 0..MH-1
#pragma unroll
      for (int mm = 0; mm < MH; ++mm) {
        xch[slot(1, 0, mm)] = acc1[MH + mm];
        xch[slot(1, 1, mm)] = acc3[MH + mm];
        xch[slot(1, 2, mm)] = acc2[MH + mm];
      }
    } else {         // hands over blocks 0..MH-1, keeps MH..
#pragma unroll
      for (int mm = 0; mm < MH; ++mm) {
        xch[slot(0, 0, mm)] = acc1[mm];
        xch[slot(0, 1, mm)] = acc3[mm];
        xch[slot(0, 2, mm)] = acc2[mm];
      }
    }
    __syncthreads();
    if (tg == 0) {
#pragma unroll
      for (int mm = 0; mm < MH; ++mm) {
        acc1[mm] = acc1[mm] + xch[slot(0, 0, mm)];
        acc3[mm] = acc3[mm] + xch[slot(0, 1, mm)];
        acc2[mm] = acc2[mm] + xch[slot(0, 2, mm)];
      }
    } else {
#pragma unroll
      for (int mm = 0; mm < MH; ++mm) {
        acc1[MH + mm] = xch[slot(1, 0, mm)] + acc1[MH + mm];
        acc3[MH + mm] = xch[slot(1, 1, mm)] + acc3[MH + mm];
        acc2[MH + mm] = xch[slot(1, 2, mm)] + acc2[MH + mm];
      }
    }
  }
  // all three partial sums were accumulated from ga', gb', u', which carry -log2(e)
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    acc1[m] *= kNegInvLog2e;
    acc3[m] *= kNegInvLog2e;
    acc2[m] *= kNegInvLog2e;
  }

  // Partial sums in natural weight layouts: [3][h*d] per (chunk, head).
  const int64_t hd_elems = (int64_t)HID * D;
  float* P = part + ((int64_t)chunk_id * heads + head) * 3 * hd_elems;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (TG == 2 && (m < MH) != (tg == 0)) continue;   // the other token group writes it
    // acc1/acc3 lane values: D1[j0 + c][16 m + 4 g + i], i = 0..3
    *(f32x4*)(P + (int64_t)(j0 + c) * D + 16 * m + 4 * g) = acc1[m];
    *(f32x4*)(P + hd_elems + (int64_t)(j0 + c) * D + 16 * m + 4 * g) = acc3[m];
    // acc2 lane values: D2^T[j0 + 4 g + i][16 m + c] = D2[16 m + c][j0 + 4 g + i]
    *(f32x4*)(P + 2 * hd_elems + (int64_t)(16 * m + c) * HID + j0 + 4 * g) = acc2[m];
  }
}

}  // namespace zm
