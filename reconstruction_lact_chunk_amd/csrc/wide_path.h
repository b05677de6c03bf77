// Full-width fast weight (d = 1024, h = 2048): token-block orchestration of
// the hand-written forward + gate kernels (wide_gemm.hip), the plain library
// GEMMs and the reduce kernel (wide_kernels.hip).  Used by the C-ABI layer
// when the descriptor names that shape.
#pragma once

#include "zm_ttt.h"
#include "zm_internal.h"

namespace zm {

constexpr int kWideD = 1024;
constexpr int kWideH = 2048;
constexpr int64_t kWideBlock = 131072;              // tokens per block of the token buffers
constexpr int kWideSub = 8;                         // partial slots: sub-blocks of each block
constexpr size_t kWideLtWorkspace = (size_t)64 << 20;  // GEMM library workspace (= kLtWorkspace)

struct WideBufs {
  void* lt_ws;        // GEMM library workspace
  size_t lt_ws_bytes;
  void* ns;           // Newton-Schulz buffers (with that step rule), else null
  float* sum;         // the slots' sum [heads][3][h d] in natural layouts (with an update)
  uint16_t* ab;       // token-block buffers: [rows][2 h] then [rows][h], bf16
  float* part;        // partial sums [kWideSub][heads][3 h d] (transposed; see launch_wide_tsum),
                      // at the end of the workspace
  bool fits;          // every buffer above lies inside the workspace, block buffers below part
};

bool wide_shape(int d, int h);
int64_t wide_splits(int64_t n_kv);
// Workspace bytes beyond the two bf16 weight sets (ns: with the Newton-Schulz
// step rule).
size_t wide_extra_bytes(int heads, int d, int h, int64_t n_kv, int64_t n_q, bool ns);
// The buffers of a call with an update over n_kv tokens and an apply over n_q
// queries (either may be 0) inside the caller's workspace of ws_bytes; `fits`
// says whether they all lie inside it (checked on the host before any launch).
WideBufs wide_bufs(void* ws, size_t ws_bytes, size_t base, int heads, int d, int h, int64_t n_kv,
                   int64_t n_q, bool ns);

// Newton-Schulz of every matrix of the summed partials part0 ([heads][3][h d],
// natural layouts), in place; ns_ws holds wide_ns_bytes().
size_t wide_ns_bytes(int heads, int d, int h);
int wide_newton_schulz(float* part0, int heads, int d, int h, void* ns_ws, void* lt_ws,
                       size_t lt_bytes, hipStream_t st);

// Minus the chunk gradient over n tokens into the kWideSub partial slots of
// w.part (sub-block i of every block adds into slot i), each slot transposed:
// per head [D1; D3]^T (d x 2h, row-major), then D2^T (h x d).
int wide_update(int heads, int d, int h, int64_t ld, int64_t n, const uint16_t* k,
                const uint16_t* v, const float* eta, const WSet& wb, const WideBufs& w,
                hipStream_t st);
// o = f_W(q) through the bf16 set wb.
int wide_apply(int heads, int d, int h, int64_t ld, int64_t n, const uint16_t* q, uint16_t* o,
               const WSet& wb, const WideBufs& w, hipStream_t st);

// U' = -log2(e) SiLU(W1 q) (*) W3 q for n query rows (stride ldq), W1 copy w1
// (carrying -log2(e)) and w3 [h][d] bf16, into u (rows of stride ldu), as one
// hand-written product with the gate in its epilogue (wide_gemm.hip).
hipError_t launch_wide_fwd_gate_apply(const uint16_t* q, int64_t ldq, int64_t n,
                                      const uint16_t* w1, const uint16_t* w3, int d, int h,
                                      uint16_t* u, int64_t ldu, hipStream_t st);
// The update's W1 / W3 products on key rows k (stride ldk) with the gate
// backward in their epilogue: from the bf16 W1 (carrying -log2(e)) and W3
// copies [h][d], e = W2^T v in e[t][j] (stride lde, bf16) and rates eta [n]
// (stride eta_ld), writes ga to gab[t][j], gb to gab[t][h + j] (rows of stride
// ldab) and eta u over e (wide_gemm.hip).
hipError_t launch_wide_fwd_gate_update(const uint16_t* k, int64_t ldk, int64_t n,
                                       const uint16_t* w1, const uint16_t* w3, int d, int h,
                                       const float* eta, int64_t eta_ld, uint16_t* gab,
                                       int64_t ldab, uint16_t* e, int64_t lde, hipStream_t st);
// sum = the `splits` transposed slots of part added in slot order, in the
// natural layouts [heads][3][h d] (W1, W3 as [h][d], W2 as [d][h]).
hipError_t launch_wide_tsum(const float* part, int splits, int heads, int d, int h, float* sum,
                            hipStream_t st);
hipError_t launch_wide_reduce(const float* part, int splits, int heads, int d, int h,
                              const float* w1, const float* w2, const float* w3, float* o1,
                              float* o2, float* o3, int renorm, const WSet* out_bf16,
                              hipStream_t st);

}  // namespace zm
