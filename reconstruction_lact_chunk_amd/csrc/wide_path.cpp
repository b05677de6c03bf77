// Full-width fast weight: one head of d = 1024 with hidden width h = 2048
// (the single full-width SwiGLU whose 6 d^2 state the ZipMap paper-reading
// notes size in their state-size paragraph).  Its weights (12 MB in bf16) do
// not fit a compute unit, so the fused register-resident kernels of the
// narrow heads do not apply.  The layer runs per token block of at most
// kWideBlock tokens as
//   update: E = V W2                                  (library GEMM, bf16 out)
//           [Ga Gb], eta U from K W1^T, K W3^T, E and eta: the two products
//           with the gate backward in their epilogue   (k_wide_rows, update)
//           D13^T = K^T [Ga Gb], D2^T = (eta U)^T V    (library GEMMs, fp32 partials)
//           then the fixed-order slot sum into natural layouts, and the
//           reduce / step / renorm;
//   apply:  U' = -log2(e) SiLU(Q W1^T) (*) Q W3^T: the two products with the
//           gate in their epilogue                     (k_wide_rows, read)
//           O = U' W2'^T                               (library GEMM).
// The products that feed a gate are hand-written (wide_gemm.hip: the gate
// runs on the accumulators, so x and b never reach memory); the plain
// products go to hipBLASLt (gemm_lt.cpp: bf16 operands, fp32 accumulation).
// The token sum is combined in a fixed order (bitwise reproducible).
#include "wide_path.h"

#include "gemm_lt.h"

namespace zm {
namespace {

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool rm_nt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
           int64_t ldb, void* C, int64_t ldc, bool out_f32, const WideBufs& w, hipStream_t st) {
  return lt_rm_nt(M, N, K, A, lda, B, ldb, C, ldc, out_f32, LtWs{w.lt_ws, w.lt_ws_bytes}, st);
}

bool rm_tn(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
           int64_t ldb, void* C, int64_t ldc, bool out_f32, const WideBufs& w, hipStream_t st,
           int count = 1, int64_t sa = 0, int64_t sb = 0, int64_t sc = 0, float beta = 0.f) {
  return lt_rm_tn(M, N, K, A, lda, B, ldb, C, ldc, out_f32, LtWs{w.lt_ws, w.lt_ws_bytes}, st,
                  count, sa, sb, sc, beta);
}

}  // namespace

bool wide_shape(int d, int h) { return d == kWideD && h == kWideH; }

// Partial slots of an update over n_kv tokens: kWideSub, or one when there are
// fewer tokens than sub-blocks (then every product adds into slot 0).
int64_t wide_splits(int64_t n_kv) { return n_kv >= kWideSub ? kWideSub : (n_kv > 0 ? 1 : 0); }

size_t wide_extra_bytes(int heads, int d, int h, int64_t n_kv, int64_t n_q, bool ns) {
  const int64_t rows_kv = n_kv < kWideBlock ? n_kv : kWideBlock;
  const int64_t rows_q = n_q < kWideBlock ? n_q : kWideBlock;
  const int64_t rows = rows_kv > rows_q ? rows_kv : rows_q;
  const size_t bufs = round_up((size_t)rows * 3 * h * sizeof(uint16_t), 256);
  const size_t slot = (size_t)heads * 3 * (size_t)h * d * sizeof(float);
  const size_t part = round_up((size_t)wide_splits(n_kv) * slot, 256);
  const size_t sum = n_kv > 0 ? round_up(slot, 256) : 0;
  return kWideLtWorkspace + (ns ? round_up(wide_ns_bytes(heads, d, h), 256) : 0) + sum + bufs +
         part;
}

WideBufs wide_bufs(void* ws, size_t ws_bytes, size_t base, int heads, int d, int h, int64_t n_kv,
                   int64_t n_q, bool ns) {
  WideBufs w;
  char* p = (char*)ws + base;
  w.lt_ws = p;
  w.lt_ws_bytes = kWideLtWorkspace;
  const size_t ns_bytes = ns ? round_up(wide_ns_bytes(heads, d, h), 256) : 0;
  w.ns = ns ? p + kWideLtWorkspace : nullptr;
  const size_t sum_bytes =
      n_kv > 0 ? round_up((size_t)heads * 3 * (size_t)h * d * sizeof(float), 256) : 0;
  w.sum = n_kv > 0 ? (float*)(p + kWideLtWorkspace + ns_bytes) : nullptr;
  w.ab = (uint16_t*)(p + kWideLtWorkspace + ns_bytes + sum_bytes);
  const size_t part = (size_t)wide_splits(n_kv) * heads * 3 * (size_t)h * d * sizeof(float);
  // partial sums at the end of the workspace, so the token-block buffers can
  // be sized by the larger of the update and apply counts
  const size_t part_off = part <= ws_bytes ? ((ws_bytes - part) / 256) * 256 : 0;
  w.part = (float*)((char*)ws + part_off);
  const int64_t rows_kv = n_kv < kWideBlock ? n_kv : kWideBlock;
  const int64_t rows_q = n_q < kWideBlock ? n_q : kWideBlock;
  const int64_t rows = rows_kv > rows_q ? rows_kv : rows_q;
  const size_t ab_end =
      base + kWideLtWorkspace + ns_bytes + sum_bytes + (size_t)rows * 3 * h * sizeof(uint16_t);
  w.fits = part <= ws_bytes && ab_end <= part_off;
  return w;
}

int wide_update(int heads, int d, int h, int64_t ld, int64_t n, const uint16_t* k,
                const uint16_t* v, const float* eta, const WSet& wb, const WideBufs& w,
                hipStream_t st) {
  const int64_t hd_elems = (int64_t)h * d;
  const int64_t rows = n < kWideBlock ? n : kWideBlock;
  uint16_t* ab = w.ab;                 // [rows][2 h]
  uint16_t* e = w.ab + rows * 2 * h;   // [rows][h]
  const int64_t pstride = (int64_t)heads * 3 * hd_elems;
  const int64_t blocks = ceil_div(n, kWideBlock);
  for (int hd = 0; hd < heads; ++hd) {
    for (int64_t blk = 0; blk < blocks; ++blk) {
      const int64_t s0 = blk * kWideBlock;
      const int64_t len = (n - s0) < kWideBlock ? (n - s0) : kWideBlock;
      const uint16_t* kb = k + s0 * ld + (int64_t)hd * d;
      const uint16_t* vb = v + s0 * ld + (int64_t)hd * d;
      float* slot = w.part + (int64_t)hd * 3 * hd_elems;
      // forward on the values, e = W2^T v (bf16, a plain library product),
      // then the W1 / W3 products on the keys with the gate backward in their
      // epilogue: ga, gb into ab, eta u over e
      if (!rm_nt(len, h, d, vb, ld, wb.w2tb + hd * hd_elems, d, e, h, false, w, st))
        return ZM_ERR_HIP;
      const hipError_t ge = launch_wide_fwd_gate_update(kb, ld, len, wb.w1b + hd * hd_elems,
                                                        wb.w3b + hd * hd_elems, d, h,
                                                        eta + s0 * heads + hd, heads, ab, 2 * h,
                                                        e, h, st);
      if (ge != hipSuccess) {
        set_last_error("wide forward+gate (update) launch: %s", hipGetErrorString(ge));
        return ZM_ERR_HIP;
      }
      // minus the gradient over this block, transposed: [D1; D3]^T = K^T [Ga Gb]
      // (d x 2h) and D2^T = (eta U)^T V (h x d); the library runs these
      // orientations faster than [Ga Gb]^T K and V^T (eta U).  The block's
      // tokens go to kWideSub sub-blocks as one batched product, each adding
      // into its own partial slot (slot i holds sub-block i of every block,
      // added in block order): enough output tiles to fill the GPU, and a
      // fixed summation order.
      const float beta = blk == 0 ? 0.f : 1.f;
      const int64_t sub = len / kWideSub, rest = len - sub * kWideSub;
      if (sub > 0) {
        if (!rm_tn(d, 2 * h, sub, kb, ld, ab, 2 * h, slot, 2 * h, true, w, st, kWideSub,
                   sub * ld, sub * 2 * h, pstride, beta) ||
            !rm_tn(h, d, sub, e, h, vb, ld, slot + 2 * hd_elems, d, true, w, st, kWideSub,
                   sub * h, sub * ld, pstride, beta))
          return ZM_ERR_HIP;
      }
      if (rest > 0) {  // the remainder tokens add into slot 0
        const int64_t r0 = sub * kWideSub;
        const float rb = (sub > 0 || blk > 0) ? 1.f : 0.f;
        if (!rm_tn(d, 2 * h, rest, kb + r0 * ld, ld, ab + r0 * 2 * h, 2 * h, slot, 2 * h, true, w,
                   st, 1, 0, 0, 0, rb) ||
            !rm_tn(h, d, rest, e + r0 * h, h, vb + r0 * ld, ld, slot + 2 * hd_elems, d, true, w,
                   st, 1, 0, 0, 0, rb))
          return ZM_ERR_HIP;
      }
    }
  }
  return ZM_OK;
}

int wide_apply(int heads, int d, int h, int64_t ld, int64_t n, const uint16_t* q, uint16_t* o,
               const WSet& wb, const WideBufs& w, hipStream_t st) {
  const int64_t hd_elems = (int64_t)h * d;
  for (int hd = 0; hd < heads; ++hd) {
    for (int64_t s0 = 0; s0 < n; s0 += kWideBlock) {
      const int64_t len = (n - s0) < kWideBlock ? (n - s0) : kWideBlock;
      const uint16_t* qb = q + s0 * ld + (int64_t)hd * d;
      uint16_t* ob = o + s0 * ld + (int64_t)hd * d;
      // U' = -log2(e) SiLU(W1 q) (*) W3 q in one kernel, into the block buffer
      const hipError_t ge = launch_wide_fwd_gate_apply(qb, ld, len, wb.w1b + hd * hd_elems,
                                                       wb.w3b + hd * hd_elems, d, h, w.ab, 2 * h,
                                                       st);
      if (ge != hipSuccess) {
        set_last_error("wide forward+gate (apply) launch: %s", hipGetErrorString(ge));
        return ZM_ERR_HIP;
      }
      // O = U' (-W2 / log2(e))^T with U' = -log2(e) U
      if (!rm_nt(len, d, h, w.ab, 2 * h, wb.w2b + hd * hd_elems, h, ob, ld, false, w, st))
        return ZM_ERR_HIP;
    }
  }
  return ZM_OK;
}

}  // namespace zm
