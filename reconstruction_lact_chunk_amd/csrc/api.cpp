// C-ABI layer of the TTT library: argument validation (host only, before any
// HIP call), workspace carving and the kernel sequence of each entry point.
// The entry points, their arguments and error behaviour are specified in
// include/zm_ttt.h.
#include "zm_ttt.h"

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "gemm_lt.h"
#include "layer_kernels.h"
#include "wide_path.h"
#include "zm_internal.h"

namespace zm {

thread_local char g_last_error[512] = "";

void set_last_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

}  // namespace zm

using namespace zm;

namespace {

constexpr int kVersion = 10400;  // 1.4.0
constexpr int64_t kMaxChunks = (int64_t)1 << 24;
constexpr int kMaxInnerSteps = 64;

constexpr int kMaxProfEvents = 14;
// Widest layer (H d) whose output-gate rows a wave holds in registers.
constexpr int64_t kMaxLayerWidth = 8192;
constexpr int64_t kMaxLdTok = (int64_t)1 << 24;  // elements between token rows
void* g_prof[kMaxProfEvents] = {};
bool g_prof_on = false;

enum Stage {
  kStageCast = 0,
  kStageUpdate = 1,
  kStageReduce = 2,
  kStageApply = 3,
  kStageNewtonSchulz = 4,
  kStageProject = 5,
  kStageOutputGate = 6
};

inline void prof_mark(int slot, hipStream_t st) {
  if (g_prof_on && g_prof[slot]) (void)hipEventRecord((hipEvent_t)g_prof[slot], st);
}

struct Scoped {
  int stage;
  hipStream_t st;
  Scoped(int s, hipStream_t stream) : stage(s), st(stream) { prof_mark(2 * s, st); }
  ~Scoped() { prof_mark(2 * stage + 1, st); }
};

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_desc(const zm_ttt_desc* d) {
  if (!d) return ZM_ERR_INVALID_ARG;
  if (d->heads < 1 || d->d_head < 1 || d->d_hidden < 1) return ZM_ERR_INVALID_ARG;
  if (d->io_dtype != ZM_BF16 && d->io_dtype != ZM_F32) return ZM_ERR_INVALID_ARG;
  if (d->renorm != ZM_RENORM_NONE && d->renorm != ZM_RENORM_ROW) return ZM_ERR_INVALID_ARG;
  if (d->step_rule != ZM_STEP_GRADIENT && d->step_rule != ZM_STEP_NEWTON_SCHULZ)
    return ZM_ERR_INVALID_ARG;
  if (d->ld_tok < (int64_t)d->heads * d->d_head || d->ld_tok % 8 != 0) return ZM_ERR_INVALID_ARG;
  // the bf16 kernels form a token's offset inside a 32-token tile in 32 bits
  if (d->ld_tok > kMaxLdTok) return ZM_ERR_INVALID_ARG;
  if (d->heads > 64) return ZM_ERR_UNSUPPORTED;
  if (wide_shape(d->d_head, d->d_hidden)) {
    // full width: bf16 io only
    if (d->io_dtype != ZM_BF16) return ZM_ERR_UNSUPPORTED;
    return ZM_OK;
  }
  const bool ok_shape = (d->d_head == 64 || d->d_head == 128) &&
                        (d->d_hidden == 128 || d->d_hidden == 256);
  if (!ok_shape) return ZM_ERR_UNSUPPORTED;
  return ZM_OK;
}

inline bool is_wide(const zm_ttt_desc* d) { return wide_shape(d->d_head, d->d_hidden); }

// Caller's workspace.
struct Ws {
  void* p;
  size_t bytes;
};

struct Layout {
  size_t set_a, set_b, sync, part, loss, total;   // loss: virtual-loss block sums (narrow heads)
  UpdatePlan plan;
};

// Workspace: two bf16 weight sets (4 arrays each), then for the narrow heads
// the shared launch's sync words (frame_sync_words) and the partial sums (for
// the full width: the token-block buffers and the partial sums).  Offsets up
// to the partial sums do not depend on the token counts.
Layout layout(const zm_ttt_desc* d, int64_t n_kv, int64_t n_q) {
  Layout L{};
  const size_t welems = (size_t)d->heads * d->d_hidden * d->d_head;
  const size_t set_bytes = round_up(4 * welems * sizeof(uint16_t), 256);
  L.set_a = 0;
  L.set_b = set_bytes;
  L.sync = L.part = 2 * set_bytes;
  if (is_wide(d)) {
    L.plan = UpdatePlan{(int)wide_splits(n_kv), kWideBlock, 1};
    L.total = L.part + wide_extra_bytes(d->heads, d->d_head, d->d_hidden, n_kv, n_q,
                                        d->step_rule == ZM_STEP_NEWTON_SCHULZ);
    return L;
  }
  L.part = L.sync + round_up(frame_sync_words(d->heads) * sizeof(unsigned), 256);
  L.plan = plan_update(n_kv, d->heads, d->d_hidden);
  // slots for any update of at most n_kv tokens (see update_slots), then one
  // float per update workgroup for the virtual loss
  const int slots = update_slots(n_kv, d->heads, d->d_hidden);
  // the loss's block sums: one per (slot, head, hidden slice), slices of a
  // two-token-group plan (64 hidden units) included
  const int nsl = d->d_hidden / (kHidPerWg / 2) > 0 ? d->d_hidden / (kHidPerWg / 2) : 1;
  L.loss = L.part + round_up((size_t)slots * 3 * welems * sizeof(float), 256);
  L.total = L.loss + round_up((size_t)slots * d->heads * nsl * sizeof(float), 256);
  return L;
}

WSet carve_set(void* ws, size_t off, size_t welems) {
  uint16_t* p = (uint16_t*)((char*)ws + off);
  return WSet{p, p + welems, p + 2 * welems, p + 3 * welems};
}

// Host-side bound of the partial-sum slots a launch is about to write:
// `splits` slots of 3 h d fp32 per head from byte offset part_off.  The
// workspace size check at entry already covers every planned count; this
// check turns a planner slip into a status code instead of a write past the
// caller's allocation.
int check_part_range(size_t part_off, int splits, size_t welems, size_t ws_bytes) {
  const size_t need = part_off + (size_t)splits * 3 * welems * sizeof(float);
  if (splits < 0 || need > ws_bytes) {
    set_last_error("partial sums of %d slots need %zu workspace bytes, %zu given", splits, need,
                   ws_bytes);
    return ZM_ERR_WORKSPACE;
  }
  return ZM_OK;
}

int check_wide_bufs(const WideBufs& wb, size_t ws_bytes) {
  if (!wb.fits) {
    set_last_error("full-width token-block buffers and partial sums exceed the %zu-byte workspace",
                   ws_bytes);
    return ZM_ERR_WORKSPACE;
  }
  return ZM_OK;
}

int check_counts(int64_t n_kv, int64_t n_q) {
  const int64_t kMax = (int64_t)1 << 31;  // token indices fit 32-bit tile counts
  if (n_kv < 0 || n_q < 0 || n_kv > kMax || n_q > kMax) return ZM_ERR_INVALID_ARG;
  return ZM_OK;
}

int check_tokens(const void* p, int64_t n) {
  if (n == 0) return ZM_OK;
  if (!p || !aligned(p, 16)) return ZM_ERR_INVALID_ARG;
  return ZM_OK;
}

int check_eta(const float* p, int64_t n) {
  if (n == 0) return ZM_OK;
  if (!p || !aligned(p, 4)) return ZM_ERR_INVALID_ARG;
  return ZM_OK;
}

int check_weights(const float* a, const float* b, const float* c) {
  if (!a || !b || !c) return ZM_ERR_INVALID_ARG;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16)) return ZM_ERR_INVALID_ARG;
  return ZM_OK;
}

int check_ws(const zm_ttt_desc* d, int64_t n_kv, int64_t n_q, void* ws, size_t ws_bytes) {
  const Layout L = layout(d, n_kv, n_q);
  if (!ws) return ZM_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return ZM_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return ZM_ERR_WORKSPACE;
  return ZM_OK;
}

#define ZM_TRY(expr)            \
  do {                          \
    const int _s = (expr);      \
    if (_s != ZM_OK) return _s; \
  } while (0)

#define ZM_HIP(expr)                                                                \
  do {                                                                              \
    const hipError_t _e = (expr);                                                   \
    if (_e != hipSuccess) {                                                         \
      zm::set_last_error("%s: %s (%d)", #expr, hipGetErrorString(_e), (int)_e);     \
      return ZM_ERR_HIP;                                                            \
    }                                                                               \
  } while (0)

int finish_update(const zm_ttt_desc* d, int64_t n, const float* w1, const float* w2,
                  const float* w3, float* o1, float* o2, float* o3, float* part, int splits,
                  const WSet* emit, hipStream_t st);

// The update part shared by update, update_apply and stream_step: partial
// sums over n_kv tokens, then the reduce/step/renorm into w*_out.  When
// emit is non-null the reduce also writes the bf16 copies of W_hat there.
int run_update(const zm_ttt_desc* d, int64_t n, const void* k, const void* v, const float* eta,
               const float* w1, const float* w2, const float* w3, float* o1, float* o2,
               float* o3, Ws wsp, const WSet* emit, bool cast_done, hipStream_t st,
               float* loss = nullptr) {
  void* const ws = wsp.p;
  const Layout L = layout(d, n, 0);
  const size_t welems = (size_t)d->heads * d->d_hidden * d->d_head;
  const WSet a = carve_set(ws, L.set_a, welems);
  if (is_wide(d)) {
    const bool ns = d->step_rule == ZM_STEP_NEWTON_SCHULZ;
    const WideBufs wb = wide_bufs(ws, wsp.bytes, L.part, d->heads, d->d_head, d->d_hidden, n, 0,
                                  ns);
    ZM_TRY(check_wide_bufs(wb, wsp.bytes));
    const int splits = L.plan.splits;
    if (n > 0) {
      if (!cast_done) {
        Scoped s(kStageCast, st);
        ZM_HIP(launch_cast(w1, w2, w3, d->heads, d->d_head, d->d_hidden, a, st));
      }
      Scoped s(kStageUpdate, st);
      ZM_TRY(wide_update(d->heads, d->d_head, d->d_hidden, d->ld_tok, n, (const uint16_t*)k,
                         (const uint16_t*)v, eta, a, wb, st));
    }
    // The slots are transposed: launch_wide_tsum adds them in slot order into
    // wb.sum in natural layouts, which the Newton-Schulz step and the reduce
    // read as a single slot.
    if (n > 0 && ns) {
      Scoped s(kStageNewtonSchulz, st);
      ZM_HIP(launch_wide_tsum(wb.part, splits, d->heads, d->d_head, d->d_hidden, wb.sum, st));
      ZM_TRY(wide_newton_schulz(wb.sum, d->heads, d->d_head, d->d_hidden, wb.ns, wb.lt_ws,
                                wb.lt_ws_bytes, st));
    }
    Scoped s(kStageReduce, st);
    if (n > 0 && !ns)
      ZM_HIP(launch_wide_tsum(wb.part, splits, d->heads, d->d_head, d->d_hidden, wb.sum, st));
    ZM_HIP(launch_wide_reduce(n > 0 ? wb.sum : wb.part, n > 0 ? 1 : 0, d->heads, d->d_head,
                              d->d_hidden, w1, w2, w3, o1, o2, o3, d->renorm, emit, st));
    return ZM_OK;
  }
  float* part = (float*)((char*)ws + L.part);
  ZM_TRY(check_part_range(L.part, L.plan.splits, welems, wsp.bytes));
  // the virtual loss's block sums (bf16 narrow path only; the entry point checks)
  float* const loss_part = loss ? (float*)((char*)ws + L.loss) : nullptr;
  unsigned* const sync = (unsigned*)((char*)ws + L.sync);
  if (n > 0) {
    if (d->io_dtype == ZM_BF16) {
      if (!cast_done) {
        Scoped s(kStageCast, st);
        ZM_HIP(launch_cast(w1, w2, w3, d->heads, d->d_head, d->d_hidden, a, st, sync,
                           (int)frame_sync_words(d->heads)));
      }
      Scoped s(kStageUpdate, st);
      if (!loss && d->step_rule == ZM_STEP_GRADIENT && frame_fuses_reduce(d->heads, L.plan, 0)) {
        // short chunk: partial sums and reduce in one launch
        Scoped r(kStageReduce, st);
        const FrameReduce fr{sync, ReduceOut{w1, w2, w3, o1, o2, o3,
                                             emit ? *emit : WSet{nullptr, nullptr, nullptr, nullptr},
                                             d->renorm, emit ? 1 : 0}};
        ZM_HIP(launch_frame_bf16(nullptr, nullptr, 0, (const uint16_t*)k, (const uint16_t*)v, eta,
                                 n, d->ld_tok, d->heads, d->d_head, d->d_hidden, a, part, L.plan,
                                 st, &fr));
        return ZM_OK;
      }
      ZM_HIP(launch_update_bf16((const uint16_t*)k, (const uint16_t*)v, eta, n, d->ld_tok,
                                d->heads, d->d_head, d->d_hidden, a, part, L.plan, st, loss_part));
    } else {
      Scoped s(kStageUpdate, st);
      ZM_HIP(launch_update_f32((const float*)k, (const float*)v, eta, n, d->ld_tok, d->heads,
                               d->d_head, d->d_hidden, w1, w2, w3, part, L.plan, st));
    }
  }
  if (loss)  // n = 0: zeros
    ZM_HIP(launch_loss_sum(loss_part, n > 0 ? L.plan.splits : 0, d->heads,
                           plan_slices(L.plan, d->d_hidden), loss, st));
  return finish_update(d, n, w1, w2, w3, o1, o2, o3, part, L.plan.splits, emit, st);
}

// The rest of a narrow-head update once the partial sums of n tokens are in
// part ([splits][heads][3][h d]): the Newton-Schulz step if asked for, then
// the reduce/step/renorm into o*.
int finish_update(const zm_ttt_desc* d, int64_t n, const float* w1, const float* w2,
                  const float* w3, float* o1, float* o2, float* o3, float* part, int splits,
                  const WSet* emit, hipStream_t st) {
  if (n > 0 && d->step_rule == ZM_STEP_NEWTON_SCHULZ) {
    // partials -> slot 0 -> NewtonSchulz(minus the gradient), in place
    Scoped ns(kStageNewtonSchulz, st);
    ZM_HIP(launch_newton_schulz(part, splits, d->heads, d->d_head, d->d_hidden,
                                d->io_dtype == ZM_F32, st));
    splits = 1;
  }
  Scoped s(kStageReduce, st);
  ZM_HIP(launch_reduce(part, splits, d->heads, d->d_head, d->d_hidden, w1, w2, w3, o1, o2, o3,
                       d->renorm, emit, st));
  return ZM_OK;
}

// Apply through fp32 weights w* (fp32 path) or through the bf16 set `set`
// (bf16 path; the caller has filled it).
int run_apply(const zm_ttt_desc* d, int64_t n, const void* q, void* o, const float* w1,
              const float* w2, const float* w3, const WSet& set, Ws wsp, hipStream_t st) {
  if (n == 0) return ZM_OK;
  Scoped s(kStageApply, st);
  if (is_wide(d)) {
    const Layout L = layout(d, 0, n);
    const WideBufs wb = wide_bufs(wsp.p, wsp.bytes, L.part, d->heads, d->d_head, d->d_hidden, 0,
                                  n, d->step_rule == ZM_STEP_NEWTON_SCHULZ);
    ZM_TRY(check_wide_bufs(wb, wsp.bytes));
    return wide_apply(d->heads, d->d_head, d->d_hidden, d->ld_tok, n, (const uint16_t*)q,
                      (uint16_t*)o, set, wb, st);
  }
  if (d->io_dtype == ZM_BF16) {
    ZM_HIP(launch_apply_bf16((const uint16_t*)q, (uint16_t*)o, n, d->ld_tok, d->heads, d->d_head,
                             d->d_hidden, set, st));
  } else {
    ZM_HIP(launch_apply_f32((const float*)q, (float*)o, n, d->ld_tok, d->heads, d->d_head,
                            d->d_hidden, w1, w2, w3, st));
  }
  return ZM_OK;
}

// One chunk of a sequence read and written in the given order (streaming
// frame or chunk of zm_ttt_chunked): with APPLY_THEN_UPDATE o = f_W(q), then
// W <- Update(W; chunk) `inner` times; with UPDATE_THEN_APPLY the updates come
// first.  do_update = false only reads.  W is updated in place.  With bf16 io,
// reuse says that set a of the workspace already holds the bf16 copies of the
// incoming W (no cast), and emit that set a must hold those of the outgoing W
// on return (the last reduce writes them).
int run_chunk(const zm_ttt_desc* d, int order, bool do_update, int inner, int64_t n,
              const void* q, const void* k, const void* v, const float* eta, float* w1, float* w2,
              float* w3, void* o, Ws ws, hipStream_t st, bool reuse = false, bool emit = false) {
  const size_t welems = (size_t)d->heads * d->d_hidden * d->d_head;
  const Layout L = layout(d, n, n);
  const WSet a = carve_set(ws.p, L.set_a, welems);
  const WSet b = carve_set(ws.p, L.set_b, welems);
  const bool bf16 = d->io_dtype == ZM_BF16;
  reuse = reuse && bf16;
  emit = emit && bf16;
  const int updates = do_update ? inner : 0;
  unsigned* const sync = is_wide(d) ? nullptr : (unsigned*)((char*)ws.p + L.sync);
  if (order == ZM_APPLY_THEN_UPDATE || updates == 0) {
    // Read the chunk with the incoming W; the first update shares that cast.
    if (bf16 && !reuse) {
      Scoped s(kStageCast, st);
      ZM_HIP(launch_cast(w1, w2, w3, d->heads, d->d_head, d->d_hidden, a, st, sync,
                         sync ? (int)frame_sync_words(d->heads) : 0));
    }
    int first = 0;
    if (bf16 && !is_wide(d) && updates > 0 && n > 0) {
      // The read and the first update's partial sums use only the incoming W:
      // one launch for both (both stages' profile events bracket it), which
      // for short frames also reduces them.
      float* part = (float*)((char*)ws.p + L.part);
      ZM_TRY(check_part_range(L.part, L.plan.splits, welems, ws.bytes));
      const WSet* out = (emit && updates == 1) ? &a : nullptr;
      const bool fuse = d->step_rule == ZM_STEP_GRADIENT && frame_fuses_reduce(d->heads, L.plan, n);
      const FrameReduce fr{sync, ReduceOut{w1, w2, w3, w1, w2, w3,
                                           out ? *out : WSet{nullptr, nullptr, nullptr, nullptr},
                                           d->renorm, out ? 1 : 0}};
      {
        Scoped su(kStageUpdate, st);
        Scoped sa(kStageApply, st);
        ZM_HIP(launch_frame_bf16((const uint16_t*)q, (uint16_t*)o, n, (const uint16_t*)k,
                                 (const uint16_t*)v, eta, n, d->ld_tok, d->heads, d->d_head,
                                 d->d_hidden, a, part, L.plan, st, fuse ? &fr : nullptr));
      }
      // the frame kernel has read set a before the reduce rewrites it
      if (!fuse)
        ZM_TRY(finish_update(d, n, w1, w2, w3, w1, w2, w3, part, L.plan.splits, out, st));
      first = 1;
    } else {
      ZM_TRY(run_apply(d, n, q, o, w1, w2, w3, a, ws, st));
    }
    for (int i = first; i < updates; ++i)
      ZM_TRY(run_update(d, n, k, v, eta, w1, w2, w3, w1, w2, w3, ws,
                        (emit && i == updates - 1) ? &a : nullptr, bf16 && i == 0, st));
    return ZM_OK;
  }
  // The last update also writes the bf16 copies the read uses (into set a
  // when they must outlive the call).
  for (int i = 0; i < updates; ++i) {
    const WSet* out = nullptr;
    if (bf16 && i == updates - 1) out = emit ? &a : (n > 0 ? &b : nullptr);
    ZM_TRY(run_update(d, n, k, v, eta, w1, w2, w3, w1, w2, w3, ws, out, reuse && i == 0, st));
  }
  return run_apply(d, n, q, o, w1, w2, w3, emit ? a : b, ws, st);
}

inline size_t io_bytes(const zm_ttt_desc* d) { return d->io_dtype == ZM_BF16 ? 2 : 4; }

// zm_ttt_chunked for the narrow heads with bf16 io.  Between chunks W's bf16
// copy stays current in set a: it is cast once, and every reduce re-emits it
// with the stepped W.  Each read shares a launch with an update step that
// uses the same W.  With APPLY_THEN_UPDATE, chunk c's read goes with its own
// first update.  With UPDATE_THEN_APPLY, chunk c's read waits for the first
// update of the next updated chunk, which starts from the same W.  Reads of
// chunks without an update run alone.  Every kernel sees the inputs of the
// per-chunk routine, so the results are bitwise those of run_chunk.
int run_chunked_bf16(const zm_ttt_desc* d, int order, int64_t n_chunks, const int64_t* offsets,
                     const uint8_t* update_mask, int inner, const char* q, const char* k,
                     const char* v, const float* eta, float* w1, float* w2, float* w3, char* o,
                     Ws ws, hipStream_t st) {
  const Layout L0 = layout(d, 0, 0);  // set and partial-sum offsets do not depend on n
  const WSet a = carve_set(ws.p, L0.set_a, (size_t)d->heads * d->d_hidden * d->d_head);
  float* part = (float*)((char*)ws.p + L0.part);
  unsigned* const sync = (unsigned*)((char*)ws.p + L0.sync);
  const size_t row = (size_t)d->ld_tok * sizeof(uint16_t);
  const int hd = d->heads, dh = d->d_head, hh = d->d_hidden;
  auto tok = [&](const char* base, int64_t c) { return (const uint16_t*)(base + offsets[c] * row); };
  auto len = [&](int64_t c) { return offsets[c + 1] - offsets[c]; };
  auto read = [&](int64_t c) {  // o_c = f_W(q_c) through set a
    Scoped s(kStageApply, st);
    return launch_apply_bf16(tok(q, c), (uint16_t*)(o + offsets[c] * row), len(c), d->ld_tok, hd,
                             dh, hh, a, st);
  };
  // One update step on chunk c from the W in set a (W <- step, a <- bf16(W)),
  // with chunk rc's read in the same launch when rc >= 0.
  auto step = [&](int64_t c, int64_t rc) -> int {
    const UpdatePlan plan = plan_update(len(c), hd, hh);
    ZM_TRY(check_part_range(L0.part, plan.splits, (size_t)hd * hh * dh, ws.bytes));
    const float* e = eta + offsets[c] * hd;
    const bool fuse = rc >= 0 && d->step_rule == ZM_STEP_GRADIENT &&
                      frame_fuses_reduce(hd, plan, len(rc));
    const bool fuse_alone = rc < 0 && d->step_rule == ZM_STEP_GRADIENT &&
                            frame_fuses_reduce(hd, plan, 0);
    {
      Scoped su(kStageUpdate, st);
      if (rc >= 0) {
        Scoped sa(kStageApply, st);
        const FrameReduce fr{sync, ReduceOut{w1, w2, w3, w1, w2, w3, a, d->renorm, 1}};
        ZM_HIP(launch_frame_bf16(tok(q, rc), (uint16_t*)(o + offsets[rc] * row), len(rc), tok(k, c),
                                 tok(v, c), e, len(c), d->ld_tok, hd, dh, hh, a, part, plan, st,
                                 fuse ? &fr : nullptr));
      } else if (fuse_alone) {
        const FrameReduce fr{sync, ReduceOut{w1, w2, w3, w1, w2, w3, a, d->renorm, 1}};
        ZM_HIP(launch_frame_bf16(nullptr, nullptr, 0, tok(k, c), tok(v, c), e, len(c), d->ld_tok,
                                 hd, dh, hh, a, part, plan, st, &fr));
      } else {
        ZM_HIP(launch_update_bf16(tok(k, c), tok(v, c), e, len(c), d->ld_tok, hd, dh, hh, a, part,
                                  plan, st));
      }
    }
    if (fuse || fuse_alone) return ZM_OK;
    return finish_update(d, len(c), w1, w2, w3, w1, w2, w3, part, plan.splits, &a, st);
  };
  bool cast = false;
  int64_t pending = -1;  // UPDATE_THEN_APPLY: a chunk whose read is still to run
  for (int64_t c = 0; c < n_chunks; ++c) {
    if (len(c) == 0) continue;
    const bool upd = update_mask == nullptr || update_mask[c] != 0;
    if (!cast) {
      Scoped s(kStageCast, st);
      ZM_HIP(launch_cast(w1, w2, w3, hd, dh, hh, a, st, sync, (int)frame_sync_words(hd)));
      cast = true;
    }
    if (order == ZM_APPLY_THEN_UPDATE) {
      if (!upd) {
        ZM_HIP(read(c));
        continue;
      }
      ZM_TRY(step(c, c));
      for (int i = 1; i < inner; ++i) ZM_TRY(step(c, -1));
      continue;
    }
    if (!upd) {  // W does not change: the waiting read and this one use it as it is
      if (pending >= 0) ZM_HIP(read(pending));
      pending = c;
      continue;
    }
    ZM_TRY(step(c, pending));
    for (int i = 1; i < inner; ++i) ZM_TRY(step(c, -1));
    pending = c;
  }
  if (pending >= 0) ZM_HIP(read(pending));
  return ZM_OK;
}

// Workspace of zm_ttt_layer: the projection rows Y [n][ldy] bf16 (q | k | v |
// rate logits; later o' in the k columns and W_g o' in the v columns), eta,
// the GEMM library workspace, then the TTT workspace (last, so the full-width
// path's partial sums at its end stay inside it).
struct LayerLayout {
  int64_t width, ncols, ldy;
  size_t off_eta, off_lt, off_ttt, total;
  zm_ttt_desc tdesc;  // the TTT call's descriptor: q / k / v rows of stride ldy
};

LayerLayout layer_layout(const zm_ttt_desc* d, int64_t n) {
  LayerLayout L;
  L.width = (int64_t)d->heads * d->d_head;
  L.ncols = 3 * L.width + d->heads;
  // Rows start on 128-byte boundaries: a 2-KiB head-row read then spans 16
  // cache lines, not 17 (measured: the whole layer 4.7% faster than with
  // rows rounded to 8 elements only).
  L.ldy = (L.ncols + 63) / 64 * 64;
  L.off_eta = round_up((size_t)n * L.ldy * sizeof(uint16_t), 256);
  L.off_lt = L.off_eta + round_up((size_t)n * d->heads * sizeof(float), 256);
  L.off_ttt = L.off_lt + kLtWorkspace;
  L.tdesc = *d;
  L.tdesc.ld_tok = L.ldy;
  L.total = L.off_ttt + layout(&L.tdesc, n, n).total;
  return L;
}

int check_layer_args(const zm_ttt_desc* d, const zm_layer_weights* lw, int64_t n) {
  ZM_TRY(check_desc(d));
  if (d->io_dtype != ZM_BF16) return ZM_ERR_UNSUPPORTED;
  if ((int64_t)d->heads * d->d_head > kMaxLayerWidth) return ZM_ERR_UNSUPPORTED;
  if (!lw || lw->reserved != 0) return ZM_ERR_INVALID_ARG;
  if (lw->d_in < 8 || lw->d_in % 8 != 0 || lw->d_in > (1 << 20)) return ZM_ERR_INVALID_ARG;
  if (!(lw->eta_scale >= 0.f) || !(lw->rms_eps > 0.f)) return ZM_ERR_INVALID_ARG;
  if (!lw->w_in || !lw->w_gate || !lw->gamma) return ZM_ERR_INVALID_ARG;
  if (!aligned(lw->w_in, 16) || !aligned(lw->w_gate, 16) || !aligned(lw->gamma, 16))
    return ZM_ERR_INVALID_ARG;
  return check_counts(n, n);
}

// ---- library-owned scratch for zm_ttt_update_apply_scratch -----------------
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops) run update + apply in this fixed device array instead
// of a workspace they pass in.  Every GPU the library runs on holds one copy
// of it, at its own address, from module load until the process ends.  In
// host code the array's name is not a device address: kernels get the
// address hipGetSymbolAddress returns for the current device, taken once per
// device and kept below.
constexpr size_t kScratchBytes = ZM_TTT_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of the current device's copy of `scratch` (looked up on the
// first call for each device, with that device current).
int scratch_for_current_device(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_last_error("hipGetDevice: %s (%d)", hipGetErrorString(e), (int)e);
    return ZM_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) {
    set_last_error("device %d beyond the %d devices the scratch table covers", dev,
                   kMaxScratchDevices);
    return ZM_ERR_UNSUPPORTED;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (es != hipSuccess || p == nullptr) {
        set_last_error("hipGetSymbolAddress(scratch): %s (%d)", hipGetErrorString(es), (int)es);
        return ZM_ERR_HIP;
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ZM_OK;
}

}  // namespace

extern "C" {

int zm_ttt_version(void) { return kVersion; }

const char* zm_ttt_last_error(void) { return g_last_error; }

const char* zm_status_string(int status) {
  switch (status) {
    case ZM_OK: return "ok";
    case ZM_ERR_INVALID_ARG: return "invalid argument";
    case ZM_ERR_UNSUPPORTED: return "unsupported shape";
    case ZM_ERR_WORKSPACE: return "workspace missing or too small";
    case ZM_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int zm_ttt_set_profile_events(void* const* events, int n_events) {
  if (events == nullptr) {
    if (n_events != 0) return ZM_ERR_INVALID_ARG;
    for (int i = 0; i < kMaxProfEvents; ++i) g_prof[i] = nullptr;
    g_prof_on = false;
    return ZM_OK;
  }
  if (n_events != 8 && n_events != 10 && n_events != kMaxProfEvents) return ZM_ERR_INVALID_ARG;
  for (int i = 0; i < kMaxProfEvents; ++i) g_prof[i] = i < n_events ? events[i] : nullptr;
  g_prof_on = true;
  return ZM_OK;
}

int zm_ttt_workspace_size(const zm_ttt_desc* desc, int64_t n_kv, int64_t n_q, size_t* bytes) {
  ZM_TRY(check_desc(desc));
  ZM_TRY(check_counts(n_kv, n_q));
  if (!bytes) return ZM_ERR_INVALID_ARG;
  *bytes = layout(desc, n_kv, n_q).total;
  return ZM_OK;
}

int zm_ttt_update(const zm_ttt_desc* desc, int64_t n_kv, const void* k, const void* v,
                  const float* eta, const float* w1, const float* w2, const float* w3,
                  float* w1_out, float* w2_out, float* w3_out, void* workspace,
                  size_t workspace_bytes, void* stream) {
  ZM_TRY(check_desc(desc));
  ZM_TRY(check_counts(n_kv, 0));
  ZM_TRY(check_tokens(k, n_kv));
  ZM_TRY(check_tokens(v, n_kv));
  ZM_TRY(check_eta(eta, n_kv));
  ZM_TRY(check_weights(w1, w2, w3));
  ZM_TRY(check_weights(w1_out, w2_out, w3_out));
  ZM_TRY(check_ws(desc, n_kv, 0, workspace, workspace_bytes));
  hipStream_t st = (hipStream_t)stream;
  return run_update(desc, n_kv, k, v, eta, w1, w2, w3, w1_out, w2_out, w3_out,
                    Ws{workspace, workspace_bytes}, nullptr, false, st);
}

int zm_ttt_update_loss(const zm_ttt_desc* desc, int64_t n_kv, const void* k, const void* v,
                       const float* eta, const float* w1, const float* w2, const float* w3,
                       float* w1_out, float* w2_out, float* w3_out, float* loss, void* workspace,
                       size_t workspace_bytes, void* stream) {
  ZM_TRY(check_desc(desc));
  if (is_wide(desc) || desc->io_dtype != ZM_BF16) {
    set_last_error("the virtual loss is computed by the bf16 narrow-head update only");
    return ZM_ERR_UNSUPPORTED;
  }
  if (loss == nullptr || !aligned(loss, 4)) return ZM_ERR_INVALID_ARG;
  ZM_TRY(check_counts(n_kv, 0));
  ZM_TRY(check_tokens(k, n_kv));
  ZM_TRY(check_tokens(v, n_kv));
  ZM_TRY(check_eta(eta, n_kv));
  ZM_TRY(check_weights(w1, w2, w3));
  ZM_TRY(check_weights(w1_out, w2_out, w3_out));
  ZM_TRY(check_ws(desc, n_kv, 0, workspace, workspace_bytes));
  hipStream_t st = (hipStream_t)stream;
  return run_update(desc, n_kv, k, v, eta, w1, w2, w3, w1_out, w2_out, w3_out,
                    Ws{workspace, workspace_bytes}, nullptr, false, st, loss);
}

int zm_ttt_apply(const zm_ttt_desc* desc, int64_t n_q, const void* q, const float* w1,
                 const float* w2, const float* w3, void* o, void* workspace,
                 size_t workspace_bytes, void* stream) {
  ZM_TRY(check_desc(desc));
  ZM_TRY(check_counts(0, n_q));
  ZM_TRY(check_tokens(q, n_q));
  ZM_TRY(check_tokens(o, n_q));
  ZM_TRY(check_weights(w1, w2, w3));
  ZM_TRY(check_ws(desc, 0, n_q, workspace, workspace_bytes));
  if (n_q == 0) return ZM_OK;
  hipStream_t st = (hipStream_t)stream;
  const size_t welems = (size_t)desc->heads * desc->d_hidden * desc->d_head;
  const Layout L = layout(desc, 0, n_q);
  const WSet a = carve_set(workspace, L.set_a, welems);
  if (desc->io_dtype == ZM_BF16) {
    Scoped s(kStageCast, st);
    ZM_HIP(launch_cast(w1, w2, w3, desc->heads, desc->d_head, desc->d_hidden, a, st));
  }
  return run_apply(desc, n_q, q, o, w1, w2, w3, a, Ws{workspace, workspace_bytes}, st);
}

int zm_ttt_update_apply(const zm_ttt_desc* desc, int64_t n_kv, const void* k, const void* v,
                        const float* eta, int64_t n_q, const void* q, const float* w1,
                        const float* w2, const float* w3, float* w1_out, float* w2_out,
                        float* w3_out, void* o, void* workspace, size_t workspace_bytes,
                        void* stream) {
  ZM_TRY(check_desc(desc));
  ZM_TRY(check_counts(n_kv, n_q));
  ZM_TRY(check_tokens(k, n_kv));
  ZM_TRY(check_tokens(v, n_kv));
  ZM_TRY(check_eta(eta, n_kv));
  ZM_TRY(check_tokens(q, n_q));
  ZM_TRY(check_tokens(o, n_q));
  ZM_TRY(check_weights(w1, w2, w3));
  ZM_TRY(check_weights(w1_out, w2_out, w3_out));
  ZM_TRY(check_ws(desc, n_kv, n_q, workspace, workspace_bytes));
  hipStream_t st = (hipStream_t)stream;
  const size_t welems = (size_t)desc->heads * desc->d_hidden * desc->d_head;
  const Layout L = layout(desc, n_kv, n_q);
  const WSet b = carve_set(workspace, L.set_b, welems);
  const bool bf16 = desc->io_dtype == ZM_BF16;
  const Ws ws{workspace, workspace_bytes};
  ZM_TRY(run_update(desc, n_kv, k, v, eta, w1, w2, w3, w1_out, w2_out, w3_out, ws,
                    (bf16 && n_q > 0) ? &b : nullptr, false, st));
  return run_apply(desc, n_q, q, o, w1_out, w2_out, w3_out, b, ws, st);
}

int zm_ttt_update_apply_scratch(const zm_ttt_desc* desc, int64_t n_kv, const void* k,
                                const void* v, const float* eta, int64_t n_q, const void* q,
                                const float* w1, const float* w2, const float* w3,
                                float* w1_out, float* w2_out, float* w3_out, void* o,
                                void* stream) {
  ZM_TRY(check_desc(desc));
  ZM_TRY(check_counts(n_kv, n_q));
  // the full-width shape needs GEMM-library handles and token-block buffers
  // far beyond the scratch
  if (is_wide(desc)) {
    set_last_error("the full-width head has no scratch variant");
    return ZM_ERR_UNSUPPORTED;
  }
  const size_t need = layout(desc, n_kv, n_q).total;
  if (need > kScratchBytes) {
    set_last_error("update over %lld tokens needs %zu bytes of scratch, the library holds %zu",
                   (long long)n_kv, need, kScratchBytes);
    return ZM_ERR_WORKSPACE;
  }
  ZM_TRY(check_tokens(k, n_kv));
  ZM_TRY(check_tokens(v, n_kv));
  ZM_TRY(check_eta(eta, n_kv));
  ZM_TRY(check_tokens(q, n_q));
  ZM_TRY(check_tokens(o, n_q));
  ZM_TRY(check_weights(w1, w2, w3));
  ZM_TRY(check_weights(w1_out, w2_out, w3_out));
  void* ws = nullptr;
  ZM_TRY(scratch_for_current_device(&ws));
  return zm_ttt_update_apply(desc, n_kv, k, v, eta, n_q, q, w1, w2, w3, w1_out, w2_out, w3_out,
                             o, ws, kScratchBytes, stream);
}

int zm_ttt_stream_step(const zm_ttt_desc* desc, int order, int64_t n_frame, const void* q,
                       const void* k, const void* v, const float* eta, float* w1, float* w2,
                       float* w3, void* o, void* workspace, size_t workspace_bytes,
                       void* stream) {
  ZM_TRY(check_desc(desc));
  const int flags = order & (ZM_STREAM_EMIT_BF16 | ZM_STREAM_REUSE_BF16);
  order &= ~(ZM_STREAM_EMIT_BF16 | ZM_STREAM_REUSE_BF16);
  if (order != ZM_APPLY_THEN_UPDATE && order != ZM_UPDATE_THEN_APPLY) return ZM_ERR_INVALID_ARG;
  ZM_TRY(check_counts(n_frame, n_frame));
  ZM_TRY(check_tokens(q, n_frame));
  ZM_TRY(check_tokens(k, n_frame));
  ZM_TRY(check_tokens(v, n_frame));
  ZM_TRY(check_eta(eta, n_frame));
  ZM_TRY(check_tokens(o, n_frame));
  ZM_TRY(check_weights(w1, w2, w3));
  ZM_TRY(check_ws(desc, n_frame, n_frame, workspace, workspace_bytes));
  return run_chunk(desc, order, true, 1, n_frame, q, k, v, eta, w1, w2, w3, o,
                   Ws{workspace, workspace_bytes}, (hipStream_t)stream,
                   (flags & ZM_STREAM_REUSE_BF16) != 0, (flags & ZM_STREAM_EMIT_BF16) != 0);
}

int zm_ttt_layer_workspace_size(const zm_ttt_desc* desc, const zm_layer_weights* lw, int64_t n,
                                size_t* bytes) {
  ZM_TRY(check_layer_args(desc, lw, n));
  if (!bytes) return ZM_ERR_INVALID_ARG;
  *bytes = layer_layout(desc, n).total;
  return ZM_OK;
}

int zm_ttt_layer(const zm_ttt_desc* desc, const zm_layer_weights* lw, int64_t n, const void* x,
                 int64_t ld_x, const float* w1, const float* w2, const float* w3, float* w1_out,
                 float* w2_out, float* w3_out, void* o, void* workspace, size_t workspace_bytes,
                 void* stream) {
  ZM_TRY(check_layer_args(desc, lw, n));
  if (ld_x < lw->d_in || ld_x % 8 != 0) return ZM_ERR_INVALID_ARG;
  ZM_TRY(check_tokens(x, n));
  ZM_TRY(check_tokens(o, n));
  ZM_TRY(check_weights(w1, w2, w3));
  ZM_TRY(check_weights(w1_out, w2_out, w3_out));
  const LayerLayout LL = layer_layout(desc, n);
  if (desc->ld_tok < LL.width) return ZM_ERR_INVALID_ARG;
  if (!workspace) return ZM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return ZM_ERR_INVALID_ARG;
  if (workspace_bytes < LL.total) return ZM_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  uint16_t* y = (uint16_t*)ws;
  float* eta = (float*)(ws + LL.off_eta);
  const LtWs lt{ws + LL.off_lt, kLtWorkspace};
  const Ws tws{ws + LL.off_ttt, workspace_bytes - LL.off_ttt};
  const zm_ttt_desc* td = &LL.tdesc;
  const int64_t W = LL.width;
  if (n > 0) {
    Scoped s(kStageProject, st);
    if (!lt_rm_nt(n, LL.ncols, lw->d_in, x, ld_x, lw->w_in, lw->d_in, y, LL.ldy, false, lt, st))
      return ZM_ERR_HIP;
    ZM_HIP(launch_eta_from_logits(y, LL.ldy, 3 * W, desc->heads, lw->eta_scale, eta, n, st));
  }
  // update on k, v (columns W .. 3W), then o' = f_W_hat(q) into the k columns
  const size_t welems = (size_t)desc->heads * desc->d_hidden * desc->d_head;
  const WSet b = carve_set(tws.p, layout(td, n, n).set_b, welems);
  ZM_TRY(run_update(td, n, y + W, y + 2 * W, eta, w1, w2, w3, w1_out, w2_out, w3_out, tws,
                    n > 0 ? &b : nullptr, false, st));
  if (n == 0) return ZM_OK;
  ZM_TRY(run_apply(td, n, y, y + W, w1_out, w2_out, w3_out, b, tws, st));
  // g = W_g o' into the v columns, then o = RMSNorm(o') * SiLU(g)
  Scoped s(kStageOutputGate, st);
  if (!lt_rm_nt(n, W, W, y + W, LL.ldy, lw->w_gate, W, y + 2 * W, LL.ldy, false, lt, st))
    return ZM_ERR_HIP;
  ZM_HIP(launch_rmsnorm_gate(y + W, LL.ldy, y + 2 * W, LL.ldy, lw->gamma, lw->rms_eps,
                             (uint16_t*)o, desc->ld_tok, (int)W, n, st));
  return ZM_OK;
}

int zm_ttt_chunked(const zm_ttt_desc* desc, int order, int64_t n_chunks, const int64_t* offsets,
                   const uint8_t* update_mask, int inner_steps, const void* q, const void* k,
                   const void* v, const float* eta, float* w1, float* w2, float* w3, void* o,
                   void* workspace, size_t workspace_bytes, void* stream) {
  ZM_TRY(check_desc(desc));
  if (order != ZM_APPLY_THEN_UPDATE && order != ZM_UPDATE_THEN_APPLY) return ZM_ERR_INVALID_ARG;
  if (n_chunks < 0 || n_chunks > kMaxChunks) return ZM_ERR_INVALID_ARG;
  if (inner_steps < 1 || inner_steps > kMaxInnerSteps) return ZM_ERR_INVALID_ARG;
  if (n_chunks > 0 && !offsets) return ZM_ERR_INVALID_ARG;
  int64_t longest = 0;
  if (n_chunks > 0) {
    if (offsets[0] != 0) return ZM_ERR_INVALID_ARG;
    for (int64_t c = 0; c < n_chunks; ++c) {
      const int64_t len = offsets[c + 1] - offsets[c];
      if (len < 0) return ZM_ERR_INVALID_ARG;
      if (len > longest) longest = len;
    }
  }
  const int64_t n = n_chunks > 0 ? offsets[n_chunks] : 0;
  ZM_TRY(check_counts(n, n));
  ZM_TRY(check_tokens(q, n));
  ZM_TRY(check_tokens(k, n));
  ZM_TRY(check_tokens(v, n));
  ZM_TRY(check_eta(eta, n));
  ZM_TRY(check_tokens(o, n));
  ZM_TRY(check_weights(w1, w2, w3));
  ZM_TRY(check_ws(desc, longest, longest, workspace, workspace_bytes));
  hipStream_t st = (hipStream_t)stream;
  if (desc->io_dtype == ZM_BF16 && !is_wide(desc))
    return run_chunked_bf16(desc, order, n_chunks, offsets, update_mask, inner_steps,
                            (const char*)q, (const char*)k, (const char*)v, eta, w1, w2, w3,
                            (char*)o, Ws{workspace, workspace_bytes}, st);
  const size_t row = (size_t)desc->ld_tok * io_bytes(desc);  // bytes per token row
  for (int64_t c = 0; c < n_chunks; ++c) {
    const int64_t s0 = offsets[c], len = offsets[c + 1] - s0;
    if (len == 0) continue;  // nothing to read; an update on no tokens is the identity
    const size_t tok = (size_t)s0 * row;
    const bool upd = update_mask == nullptr || update_mask[c] != 0;
    ZM_TRY(run_chunk(desc, order, upd, inner_steps, len, (const char*)q + tok,
                     (const char*)k + tok, (const char*)v + tok, eta + s0 * desc->heads, w1, w2,
                     w3, (char*)o + tok, Ws{workspace, workspace_bytes}, st));
  }
  return ZM_OK;
}

}  // extern "C"
