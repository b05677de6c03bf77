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
// Phase 1 of tile i and phase 2 of tile i-1 run between the same pair of
// barriers, so the MFMA work of one phase overlaps the pointwise work of the
// other.
#include "zm_internal.h"

namespace zm {

template <int D, int HID>
struct AppCfg {
  static constexpr int T = kTok;
  static constexpr int DP = D + 8;            // Q tile row pitch (elements)
  static constexpr int UP = HID + 8;          // U tile row pitch
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
  static_assert(MB1 >= 1 && MB1 <= 2, "hidden width per wave");
  static_assert(WPD >= 1 && TBW >= 1, "phase-2 split");
  static_assert(ITEMS <= kWaves * 64, "staging");
};

__device__ __forceinline__ float silu_gate(float a, float b) {
  const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504088896341f * a));
  return a * sg * b;
}

template <int D, int HID>
__global__ __launch_bounds__(512) void k_apply_bf16(
    const uint16_t* __restrict__ qp, uint16_t* __restrict__ op, int64_t n, int64_t ld, int heads,
    const uint16_t* __restrict__ w1b, const uint16_t* __restrict__ w3b,
    const uint16_t* __restrict__ w2b, int64_t chunk) {
  using C = AppCfg<D, HID>;
  constexpr int T = C::T, DP = C::DP, UP = C::UP, MB1 = C::MB1, KS1 = C::KS1, NB = C::NB,
                DB = C::DB, TBW = C::TBW, KS2 = C::KS2, CPT = C::CPT;
  __shared__ __attribute__((aligned(16))) uint16_t qs[2][T * DP];
  __shared__ __attribute__((aligned(16))) uint16_t us[2][T * UP];

  const int head = blockIdx.x % heads;
  const int64_t t_begin = (int64_t)(blockIdx.x / heads) * chunk;
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
  u32x4 qr = {0u, 0u, 0u, 0u};
  auto fetch = [&](int it) {
    qr = u32x4{0u, 0u, 0u, 0u};
    const int64_t t = t_begin + (int64_t)it * T + s_tok;
    if (has_item && t < t_end) qr = *(const u32x4*)(qp + t * ld + (int64_t)head * D + 8 * s_ch);
  };
  auto stage = [&](int buf) {
    if (has_item) *(u32x4*)(&qs[buf][s_tok * DP + 8 * s_ch]) = qr;
  };

  auto phase1 = [&](int buf) {
    f32x4 aa[MB1][NB], bb[MB1][NB];
#pragma unroll
    for (int mb = 0; mb < MB1; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        aa[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        bb[mb][nb] = aa[mb][nb];
      }
#pragma unroll
    for (int ks = 0; ks < KS1; ++ks) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        // B = Q^T: lane holds Q[16 nb + c][32 ks + 8 g .. +7]
        const bf16x8 qf = as_bf16x8(*(const u32x4*)(&qs[buf][(16 * nb + c) * DP + 32 * ks + 8 * g]));
#pragma unroll
        for (int mb = 0; mb < MB1; ++mb) {
          aa[mb][nb] = mfma_bf16(w1f[mb][ks], qf, aa[mb][nb]);
          bb[mb][nb] = mfma_bf16(w3f[mb][ks], qf, bb[mb][nb]);
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint16_t* dst = &us[buf][(16 * nb + c) * UP + j0];
      if constexpr (MB1 == 2) {
        u32x4 pk;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          pk[2 * mb] = pack_bf16x2(silu_gate(aa[mb][nb][0], bb[mb][nb][0]),
                                   silu_gate(aa[mb][nb][1], bb[mb][nb][1]));
          pk[2 * mb + 1] = pack_bf16x2(silu_gate(aa[mb][nb][2], bb[mb][nb][2]),
                                       silu_gate(aa[mb][nb][3], bb[mb][nb][3]));
        }
        *(u32x4*)(dst + 8 * g) = pk;
      } else {
        u32x2 pk;
        pk[0] = pack_bf16x2(silu_gate(aa[0][nb][0], bb[0][nb][0]), silu_gate(aa[0][nb][1], bb[0][nb][1]));
        pk[1] = pack_bf16x2(silu_gate(aa[0][nb][2], bb[0][nb][2]), silu_gate(aa[0][nb][3], bb[0][nb][3]));
        *(u32x2*)(dst + 4 * g) = pk;
      }
    }
  };

  auto phase2 = [&](int buf, int it) {
    const int64_t tile0 = t_begin + (int64_t)it * T;
#pragma unroll
    for (int tbi = 0; tbi < TBW; ++tbi) {
      const int tb = tb0 + tbi;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS2; ++ks) {
        // B = U^T: lane holds U[16 tb + c][32 ks + 8 g .. +7]
        const bf16x8 uf = as_bf16x8(*(const u32x4*)(&us[buf][(16 * tb + c) * UP + 32 * ks + 8 * g]));
        acc = mfma_bf16(w2f[ks], uf, acc);
      }
      // lane holds O[token 16 tb + c][16 db + 4 g + i]
      const int64_t t = tile0 + 16 * tb + c;
      if (t < t_end) {
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[0], acc[1]);
        pk[1] = pack_bf16x2(acc[2], acc[3]);
        *(u32x2*)(op + t * ld + (int64_t)head * D + 16 * db + 4 * g) = pk;
      }
    }
  };

  fetch(0);
  stage(0);
  __syncthreads();
  for (int it = 0; it <= ntiles; ++it) {
    const bool more = it + 1 < ntiles;
    if (more) fetch(it + 1);
    if (it < ntiles) phase1(it & 1);
    if (it > 0) phase2((it - 1) & 1, it - 1);
    if (more) stage((it + 1) & 1);
    __syncthreads();
  }
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
