// Full-width fast weight: one head of d = 1024 with hidden width h = 2048
// (the single full-width SwiGLU whose 6 d^2 state the ZipMap paper-reading
// notes size in their state-size paragraph).  Its weights (12 MB in bf16) do
// not fit a compute unit, so the fused register-resident kernels of the
// narrow heads do not apply.  The layer runs per token block of at most
// kWideBlock tokens as
//   update: A = K W1^T, B = K W3^T, E = V W2        (library GEMMs, bf16 out)
//           gate backward in place                   (k_wide_gate_update)
//           D13 = [Ga Gb]^T K, D2 = V^T (eta U)      (library GEMMs, fp32 partials)
//           then the fixed-order reduce / step / renorm over the blocks;
//   apply:  A = Q W1^T, B = Q W3^T; U = SiLU(A) (*) B; O = U W2^T.
// The dense products are plain GEMMs and go to hipBLASLt (gemm_lt.cpp: bf16
// operands, fp32 accumulation); the token sum is combined in a fixed order
// (bitwise reproducible).
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

// [x | b] rows of the token-block buffer: x = tokens (-log2(e) W1)^T and
// b = tokens W3^T, [len][2 h].  With one head the bf16 W1 and W3 copies are
// adjacent in the workspace, i.e. [W1; W3] is one [2 h][d] operand and the
// two products are one GEMM.
bool forward_w13(int64_t len, int h, int d, const uint16_t* tok, int64_t ld, const WSet& wb,
                 int hd, int heads, uint16_t* ab, const WideBufs& w, hipStream_t st) {
  const int64_t hd_elems = (int64_t)h * d;
  if (heads == 1 && wb.w3b == wb.w1b + hd_elems)
    return rm_nt(len, 2 * h, d, tok, ld, wb.w1b, d, ab, 2 * h, false, w, st);
  return rm_nt(len, h, d, tok, ld, wb.w1b + hd * hd_elems, d, ab, 2 * h, false, w, st) &&
         rm_nt(len, h, d, tok, ld, wb.w3b + hd * hd_elems, d, ab + h, 2 * h, false, w, st);
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
  const size_t part = round_up((size_t)wide_splits(n_kv) * heads * 3 * (size_t)h * d * sizeof(float),
                               256);
  return kWideLtWorkspace + (ns ? round_up(wide_ns_bytes(heads, d, h), 256) : 0) + bufs + part;
}

WideBufs wide_bufs(void* ws, size_t ws_bytes, size_t base, int heads, int d, int h, int64_t n_kv,
                   bool ns) {
  WideBufs w;
  char* p = (char*)ws + base;
  w.lt_ws = p;
  w.lt_ws_bytes = kWideLtWorkspace;
  const size_t ns_bytes = ns ? round_up(wide_ns_bytes(heads, d, h), 256) : 0;
  w.ns = ns ? p + kWideLtWorkspace : nullptr;
  w.ab = (uint16_t*)(p + kWideLtWorkspace + ns_bytes);
  const size_t part = (size_t)wide_splits(n_kv) * heads * 3 * (size_t)h * d * sizeof(float);
  // partial sums at the end of the workspace, so the token-block buffers can
  // be sized by the larger of the update and apply counts
  w.part = (float*)((char*)ws + ((ws_bytes - part) / 256) * 256);
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
      // forward on the keys: x = -log2(e) W1 k, b = W3 k, e = W2^T v
      if (!forward_w13(len, h, d, kb, ld, wb, hd, heads, ab, w, st) ||
          !rm_nt(len, h, d, vb, ld, wb.w2tb + hd * hd_elems, d, e, h, false, w, st))
        return ZM_ERR_HIP;
      const hipError_t ge = launch_wide_gate_update(ab, e, eta + s0 * heads + hd, heads, len, h, st);
      if (ge != hipSuccess) {
        set_last_error("wide gate (update) launch: %s", hipGetErrorString(ge));
        return ZM_ERR_HIP;
      }
      // minus the gradient over this block: [D1; D3] = [Ga Gb]^T K, D2 = V^T (eta U).
      // The block's tokens go to kWideSub sub-blocks as one batched product,
      // each adding into its own partial slot (slot i holds sub-block i of
      // every block, added in block order): enough output tiles to fill the
      // GPU, and a fixed summation order.
      const float beta = blk == 0 ? 0.f : 1.f;
      const int64_t sub = len / kWideSub, rest = len - sub * kWideSub;
      if (sub > 0) {
        if (!rm_tn(2 * h, d, sub, ab, 2 * h, kb, ld, slot, d, true, w, st, kWideSub,
                   sub * 2 * h, sub * ld, pstride, beta) ||
            !rm_tn(d, h, sub, vb, ld, e, h, slot + 2 * hd_elems, h, true, w, st, kWideSub,
                   sub * ld, sub * h, pstride, beta))
          return ZM_ERR_HIP;
      }
      if (rest > 0) {  // the remainder tokens add into slot 0
        const int64_t r0 = sub * kWideSub;
        const float rb = (sub > 0 || blk > 0) ? 1.f : 0.f;
        if (!rm_tn(2 * h, d, rest, ab + r0 * 2 * h, 2 * h, kb + r0 * ld, ld, slot, d, true, w, st,
                   1, 0, 0, 0, rb) ||
            !rm_tn(d, h, rest, vb + r0 * ld, ld, e + r0 * h, h, slot + 2 * hd_elems, h, true, w,
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
      if (!forward_w13(len, h, d, qb, ld, wb, hd, heads, w.ab, w, st)) return ZM_ERR_HIP;
      const hipError_t ge = launch_wide_gate_apply(w.ab, len, h, st);
      if (ge != hipSuccess) {
        set_last_error("wide gate (apply) launch: %s", hipGetErrorString(ge));
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
