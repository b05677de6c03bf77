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
// The dense products are plain GEMMs and go to hipBLASLt (bf16 operands, fp32
// accumulation); each block writes its own partial slot, so the token sum is
// combined in a fixed order (bitwise reproducible).
#include "wide_path.h"

#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

namespace zm {
namespace {

constexpr int kMaxDevices = 16;
hipblasLtHandle_t g_lt[kMaxDevices] = {};
std::once_flag g_lt_once[kMaxDevices];
hipblasStatus_t g_lt_status[kMaxDevices];

// One hipBLASLt handle per device, created on first use and kept for the
// process (creating it loads the library's kernels).
hipblasLtHandle_t lt_handle(int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_lt_once[dev], [dev] { g_lt_status[dev] = hipblasLtCreate(&g_lt[dev]); });
  *dev_out = dev;
  return g_lt_status[dev] == HIPBLAS_STATUS_SUCCESS ? g_lt[dev] : nullptr;
}

typedef std::tuple<int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int, int,
                   int64_t, int64_t, int64_t>
    GemmKey;

// Strided batch of a GEMM: `count` products, operand and result pointers
// advancing by the given element strides; beta = 1 adds to D.
struct Batch {
  int count = 1;
  int64_t sa = 0, sb = 0, sd = 0;
  float beta = 0.f;
};
std::mutex g_algo_mu;
std::map<GemmKey, hipblasLtMatmulAlgo_t> g_algos;

struct LtObjs {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  ~LtObjs() {
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (d) hipblasLtMatrixLayoutDestroy(d);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

#define LT_TRY(expr)                                                                    \
  do {                                                                                  \
    const hipblasStatus_t _s = (expr);                                                  \
    if (_s != HIPBLAS_STATUS_SUCCESS) {                                                 \
      set_last_error("hipBLASLt %s failed (status %d) for m=%lld n=%lld k=%lld", #expr, \
                     (int)_s, (long long)m, (long long)n, (long long)k);               \
      return false;                                                                     \
    }                                                                                   \
  } while (0)

// Column-major D (m x n, ldd) = op(A) op(B): bf16 A and B, fp32 accumulation,
// D in bf16 or fp32.  The algorithm from the library's heuristic is cached
// per problem shape.
bool gemm(hipblasOperation_t ta, hipblasOperation_t tb, int64_t m, int64_t n, int64_t k,
          const void* A, int64_t lda, const void* B, int64_t ldb, void* D, int64_t ldd,
          bool out_f32, void* ws, size_t ws_bytes, hipStream_t st, const Batch& bt = Batch()) {
  if (m == 0 || n == 0) return true;
  int dev = 0;
  hipblasLtHandle_t h = lt_handle(&dev);
  if (!h) {
    set_last_error("hipBLASLt handle creation failed");
    return false;
  }
  const hipDataType dt = out_f32 ? HIP_R_32F : HIP_R_16BF;
  LtObjs o;
  LT_TRY(hipblasLtMatmulDescCreate(&o.op, HIPBLAS_COMPUTE_32F, HIP_R_32F));
  const int32_t opa = ta, opb = tb;
  LT_TRY(hipblasLtMatmulDescSetAttribute(o.op, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)));
  LT_TRY(hipblasLtMatmulDescSetAttribute(o.op, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)));
  const bool an = ta == HIPBLAS_OP_N, bn = tb == HIPBLAS_OP_N;
  LT_TRY(hipblasLtMatrixLayoutCreate(&o.a, HIP_R_16BF, an ? m : k, an ? k : m, lda));
  LT_TRY(hipblasLtMatrixLayoutCreate(&o.b, HIP_R_16BF, bn ? k : n, bn ? n : k, ldb));
  LT_TRY(hipblasLtMatrixLayoutCreate(&o.d, dt, m, n, ldd));
  if (bt.count > 1) {
    const int32_t cnt = bt.count;
    const hipblasLtMatrixLayoutAttribute_t kc = HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT;
    const hipblasLtMatrixLayoutAttribute_t ks = HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET;
    LT_TRY(hipblasLtMatrixLayoutSetAttribute(o.a, kc, &cnt, sizeof(cnt)));
    LT_TRY(hipblasLtMatrixLayoutSetAttribute(o.b, kc, &cnt, sizeof(cnt)));
    LT_TRY(hipblasLtMatrixLayoutSetAttribute(o.d, kc, &cnt, sizeof(cnt)));
    LT_TRY(hipblasLtMatrixLayoutSetAttribute(o.a, ks, &bt.sa, sizeof(bt.sa)));
    LT_TRY(hipblasLtMatrixLayoutSetAttribute(o.b, ks, &bt.sb, sizeof(bt.sb)));
    LT_TRY(hipblasLtMatrixLayoutSetAttribute(o.d, ks, &bt.sd, sizeof(bt.sd)));
  }
  const GemmKey key{dev, opa, opb, m, n, k, lda, ldb, ldd, out_f32 ? 1 : 0, bt.count,
                    bt.sa, bt.sb, bt.sd};
  hipblasLtMatmulAlgo_t algo;
  bool have = false;
  {
    std::lock_guard<std::mutex> lock(g_algo_mu);
    auto it = g_algos.find(key);
    if (it != g_algos.end()) {
      algo = it->second;
      have = true;
    }
  }
  if (!have) {
    LT_TRY(hipblasLtMatmulPreferenceCreate(&o.pref));
    const uint64_t cap = ws_bytes;
    LT_TRY(hipblasLtMatmulPreferenceSetAttribute(o.pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                 &cap, sizeof(cap)));
    // the library's ranking, first candidate whose workspace fits
    constexpr int kCand = 8;
    hipblasLtMatmulHeuristicResult_t res[kCand];
    int count = 0;
    LT_TRY(hipblasLtMatmulAlgoGetHeuristic(h, o.op, o.a, o.b, o.d, o.d, o.pref, kCand, res,
                                           &count));
    int pick = -1;
    for (int i = 0; i < count && pick < 0; ++i)
      if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= ws_bytes) pick = i;
    if (pick < 0) {
      set_last_error("hipBLASLt found no algorithm within %zu workspace bytes for m=%lld n=%lld "
                     "k=%lld (%d candidates)", ws_bytes, (long long)m, (long long)n,
                     (long long)k, count);
      return false;
    }
    algo = res[pick].algo;
    std::lock_guard<std::mutex> lock(g_algo_mu);
    g_algos[key] = algo;
  }
  const float alpha = 1.f, beta = bt.beta;
  LT_TRY(hipblasLtMatmul(h, o.op, &alpha, A, o.a, B, o.b, &beta, D, o.d, D, o.d, &algo, ws,
                         ws_bytes, st));
  return true;
}

// Row-major C (M x N, ldc) = A (M x K, lda) B (N x K, ldb)^T.
bool rm_nt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
           int64_t ldb, void* C, int64_t ldc, bool out_f32, const WideBufs& w, hipStream_t st) {
  return gemm(HIPBLAS_OP_T, HIPBLAS_OP_N, N, M, K, B, ldb, A, lda, C, ldc, out_f32, w.lt_ws,
              w.lt_ws_bytes, st);
}

// Row-major C (M x N, ldc) = A (K x M, lda)^T B (K x N, ldb) (+ C with beta 1),
// batched: operand strides sa (A), sb (B), sc (C).
bool rm_tn(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
           int64_t ldb, void* C, int64_t ldc, bool out_f32, const WideBufs& w, hipStream_t st,
           int count = 1, int64_t sa = 0, int64_t sb = 0, int64_t sc = 0, float beta = 0.f) {
  Batch bt;
  bt.count = count;
  bt.sa = sb;  // the column-major call swaps the operands
  bt.sb = sa;
  bt.sd = sc;
  bt.beta = beta;
  return gemm(HIPBLAS_OP_N, HIPBLAS_OP_T, N, M, K, B, ldb, A, lda, C, ldc, out_f32, w.lt_ws,
              w.lt_ws_bytes, st, bt);
}

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

bool wide_shape(int d, int h) { return d == kWideD && h == kWideH; }

// Partial slots of an update over n_kv tokens: kWideSub, or one when there are
// fewer tokens than sub-blocks (then every product adds into slot 0).
int64_t wide_splits(int64_t n_kv) { return n_kv >= kWideSub ? kWideSub : (n_kv > 0 ? 1 : 0); }

size_t wide_extra_bytes(int heads, int d, int h, int64_t n_kv, int64_t n_q) {
  const int64_t rows_kv = n_kv < kWideBlock ? n_kv : kWideBlock;
  const int64_t rows_q = n_q < kWideBlock ? n_q : kWideBlock;
  const int64_t rows = rows_kv > rows_q ? rows_kv : rows_q;
  const size_t bufs = round_up((size_t)rows * 3 * h * sizeof(uint16_t), 256);
  const size_t part = round_up((size_t)wide_splits(n_kv) * heads * 3 * (size_t)h * d * sizeof(float),
                               256);
  return kWideLtWorkspace + bufs + part;
}

WideBufs wide_bufs(void* ws, size_t ws_bytes, size_t base, int heads, int d, int h, int64_t n_kv) {
  WideBufs w;
  char* p = (char*)ws + base;
  w.lt_ws = p;
  w.lt_ws_bytes = kWideLtWorkspace;
  w.ab = (uint16_t*)(p + kWideLtWorkspace);
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
      if (!rm_nt(len, h, d, kb, ld, wb.w1b + hd * hd_elems, d, ab, 2 * h, false, w, st) ||
          !rm_nt(len, h, d, kb, ld, wb.w3b + hd * hd_elems, d, ab + h, 2 * h, false, w, st) ||
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
      if (!rm_nt(len, h, d, qb, ld, wb.w1b + hd * hd_elems, d, w.ab, 2 * h, false, w, st) ||
          !rm_nt(len, h, d, qb, ld, wb.w3b + hd * hd_elems, d, w.ab + h, 2 * h, false, w, st))
        return ZM_ERR_HIP;
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
