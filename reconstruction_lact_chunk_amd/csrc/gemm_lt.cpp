// Plain GEMMs through hipBLASLt: bf16 operands, fp32 accumulation, bf16 or
// fp32 results, row-major helpers over the library's column-major interface.
// One library handle per device, created on first use; the algorithm the
// library's heuristic picks is cached per problem shape.
#include "gemm_lt.h"

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

}  // namespace

bool lt_rm_nt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb, void* C, int64_t ldc, bool out_f32, LtWs ws, hipStream_t st, int count,
              int64_t sa, int64_t sb, int64_t sc, float beta) {
  Batch bt;
  bt.count = count;
  bt.sa = sb;  // the column-major call swaps the operands
  bt.sb = sa;
  bt.sd = sc;
  bt.beta = beta;
  return gemm(HIPBLAS_OP_T, HIPBLAS_OP_N, N, M, K, B, ldb, A, lda, C, ldc, out_f32, ws.p,
              ws.bytes, st, bt);
}

bool lt_rm_tn(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb, void* C, int64_t ldc, bool out_f32, LtWs ws, hipStream_t st, int count,
              int64_t sa, int64_t sb, int64_t sc, float beta) {
  Batch bt;
  bt.count = count;
  bt.sa = sb;  // the column-major call swaps the operands
  bt.sb = sa;
  bt.sd = sc;
  bt.beta = beta;
  return gemm(HIPBLAS_OP_N, HIPBLAS_OP_T, N, M, K, B, ldb, A, lda, C, ldc, out_f32, ws.p, ws.bytes,
              st, bt);
}

}  // namespace zm
