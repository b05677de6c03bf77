// Full-width fast weight (d = 1024, h = 2048): token-block orchestration of
// library GEMMs and the wide elementwise / reduce kernels.  Used by the C-ABI
// layer when the descriptor names that shape.
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
  uint16_t* ab;       // token-block buffers: [rows][2 h] then [rows][h], bf16
  float* part;        // partial sums [kWideSub][heads][3][h d], at the end of the workspace
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

// Newton-Schulz of every matrix of the summed partials part0 ([heads][3][h d]),
// in place; ns_ws holds wide_ns_bytes().
size_t wide_ns_bytes(int heads, int d, int h);
int wide_newton_schulz(float* part0, int heads, int d, int h, void* ns_ws, void* lt_ws,
                       size_t lt_bytes, hipStream_t st);

// Minus the chunk gradient over n tokens into w.part (one slot per block).
int wide_update(int heads, int d, int h, int64_t ld, int64_t n, const uint16_t* k,
                const uint16_t* v, const float* eta, const WSet& wb, const WideBufs& w,
                hipStream_t st);
// o = f_W(q) through the bf16 set wb.
int wide_apply(int heads, int d, int h, int64_t ld, int64_t n, const uint16_t* q, uint16_t* o,
               const WSet& wb, const WideBufs& w, hipStream_t st);

hipError_t launch_wide_gate_update(uint16_t* ab, uint16_t* e, const float* eta,
                                   int64_t eta_stride, int64_t tokens, int h, hipStream_t st);
hipError_t launch_wide_gate_apply(uint16_t* ab, int64_t tokens, int h, hipStream_t st);
hipError_t launch_wide_reduce(const float* part, int splits, int heads, int d, int h,
                              const float* w1, const float* w2, const float* w3, float* o1,
                              float* o2, float* o3, int renorm, const WSet* out_bf16,
                              hipStream_t st);

}  // namespace zm
