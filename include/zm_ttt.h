/*
 * zm_ttt.h - C ABI of the large-chunk test-time-training (TTT) layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer keeps, per head, a SwiGLU fast weight
 *     f_W(x) = W2 [ SiLU(W1 x) (*) (W3 x) ]          (elementwise product (*))
 * with W1, W3 of shape [h, d] and W2 of shape [d, h].  An update takes one
 * gradient step on the virtual loss  -sum_i eta_i f_W(k_i)^T v_i  summed over
 * every token of a chunk, optionally renormalises each row of the updated
 * weights to its pre-update L2 norm, and an apply reads queries through the
 * weights.
 *   Sources: "[논문리뷰] ZipMap: Linear-Time Stateful 3D Reconstruction via
 *   Test-Time Training" (kimjy99.github.io), Method 2. Feature Backbone,
 *   Eq. (1) (SwiGLU), Eq. (2) (loss), Eq. (3) (chunk gradient with per-token
 *   rate), the renormalised update display, Eq. (4) (apply), and 3. Streaming
 *   Reconstruction, Eq. (6); the ZipMap paper-reading notes (67656.sbs),
 *   sections on Eq. 2 / Eq. 3 and streaming; the mhpn.cn LaCT summary, part
 *   2、架构 (gradients summed over the whole chunk, L2 normalisation) and
 *   3、应用场景 (apply/update orders).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Memory: every pointer is device memory owned by the caller.  The library
 *    allocates nothing, keeps no state between calls (apart from the optional
 *    profiling events below) and never synchronises the stream.  Exception:
 *    the full-width shape (d_head 1024, d_hidden 2048) runs its dense products
 *    through hipBLASLt, whose handle the library creates on the first such
 *    call on a device (the GEMM library then holds its own resources until the
 *    process ends) and whose chosen algorithm per problem shape it caches.
 *  - Token tensors q, k, v, o: [n, heads, d_head] with a token stride of
 *    desc->ld_tok elements (heads * d_head <= ld_tok <= 2^24, multiple of 8;
 *    a larger stride is rejected with ZM_ERR_INVALID_ARG).  Element
 *    type: bf16 or fp32 (desc->io_dtype).  Base pointers 16-byte aligned.
 *  - eta: fp32 [n, heads], contiguous (token-major), 4-byte aligned.
 *  - Weights: fp32, contiguous, 16-byte aligned; W1 and W3 [heads, h, d],
 *    W2 [heads, d, h].  The weights are always fp32; with bf16 io the kernels
 *    round them to bf16 operands and accumulate in fp32.
 *  - Workspace: device scratch of at least zm_ttt_workspace_size() bytes,
 *    256-byte aligned.  Calls sharing one workspace must not overlap in time;
 *    calls on distinct workspaces and streams are independent.  For short
 *    chunks (bf16 io, heads a multiple of 8, the gradient step) an update
 *    reduces its partial sums inside its own launch, whose workgroups meet
 *    at counters kept in the workspace; should that ever fail (a wait past
 *    its 2 s bound), the stepped weights come out NaN, never plausible wrong
 *    values.
 *  - stream: a hipStream_t passed as void*; NULL is the default stream.
 *    Every entry point only enqueues work and returns.
 *  - Errors: arguments are checked on the host before any HIP call; a failed
 *    check returns a negative zm_status and enqueues nothing.  A failed
 *    launch returns ZM_ERR_HIP.  Faults inside kernels surface at the
 *    caller's next synchronisation.  NaN/Inf inputs propagate (one NaN token
 *    poisons the chunk sum); they are not checked.
 *  - Supported shapes: (d_head, d_hidden) in {(64,128), (64,256), (128,128),
 *    (128,256)}, and the full-width (1024, 2048) with bf16 io (the ZipMap
 *    notes' single full-width fast weight with a 6 d^2 state, d = 1024);
 *    heads in [1, 64]; others return ZM_ERR_UNSUPPORTED.
 *  - Results are deterministic: the split of the token sum depends only on
 *    (n, heads, d_head, d_hidden), and partial sums are combined in a fixed
 *    order without atomics.
 */
#ifndef ZM_TTT_H
#define ZM_TTT_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define ZM_API __attribute__((visibility("default")))
#else
#define ZM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Size of the device scratch array behind zm_ttt_update_apply_scratch. */
#define ZM_TTT_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum zm_status {
  ZM_OK = 0,
  ZM_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size or enum */
  ZM_ERR_UNSUPPORTED = -2,   /* valid but unsupported shape */
  ZM_ERR_WORKSPACE = -3,     /* workspace missing or too small */
  ZM_ERR_HIP = -4            /* a HIP launch or runtime call failed */
} zm_status;

typedef enum zm_dtype { ZM_BF16 = 0, ZM_F32 = 1 } zm_dtype;

/* Row renormalisation after the step: each row r (the fan-in vector of one
 * output unit: a row of W1 or W3 of length d, a row of W2 of length h) is
 * rescaled to ||W_r|| / max(||W'_r||, 1e-12) times itself, ||W_r|| being the
 * norm before the update (review, renormalised update display). */
typedef enum zm_renorm { ZM_RENORM_NONE = 0, ZM_RENORM_ROW = 1 } zm_renorm;

/* Per-frame order of the streaming step (LaCT summary, 3、应用场景):
 * APPLY_THEN_UPDATE reads frame t with W(t-1) and then writes it;
 * UPDATE_THEN_APPLY writes frame t first and reads it with W(t). */
typedef enum zm_order { ZM_APPLY_THEN_UPDATE = 0, ZM_UPDATE_THEN_APPLY = 1 } zm_order;

/* Flags OR-ed into the order argument of zm_ttt_stream_step, for a caller that
 * streams frames through one workspace: the bf16 operand copies of W that a
 * frame's reduce writes serve the next frame, which then skips its separate
 * rounding launch (bf16 io; with fp32 io the flags have no effect):
 *   ZM_STREAM_EMIT_BF16:  on return the workspace holds the bf16 operand
 *     copies of the state the call leaves in w1, w2, w3;
 *   ZM_STREAM_REUSE_BF16: the workspace already holds the bf16 operand copies
 *     of the incoming state, left by the previous call on this workspace with
 *     ZM_STREAM_EMIT_BF16; the call does not round w1, w2, w3 again.
 * A stream passes EMIT on its first frame and EMIT | REUSE on the others.
 * With REUSE the caller guarantees that since that previous call neither the
 * workspace nor w1, w2, w3 changed and the descriptor is the same; otherwise
 * the results are undefined (the library keeps no state to check it).  The
 * results are bitwise those of calls without the flags. */
typedef enum zm_stream_flags {
  ZM_STREAM_EMIT_BF16 = 0x100,
  ZM_STREAM_REUSE_BF16 = 0x200
} zm_stream_flags;

/* The step taken with the chunk gradient g of one weight matrix (review, the
 * update display after Eq. (3)):
 *   ZM_STEP_GRADIENT:      W' = W - g;
 *   ZM_STEP_NEWTON_SCHULZ: W' = W - NewtonSchulz(g), the orthonormalisation of
 *     the Muon optimizer that the review names.  The pages give neither its
 *     polynomial nor its step count; the library runs Muon's published odd
 *     quintic: five steps of X <- a X + b (X X^T) X + c (X X^T)^2 X with
 *     (a, b, c) = (3.4445, -4.7750, 2.0315) from X = g / max(||g||_F, 1e-12),
 *     per head and per matrix.  Its products run in split-bf16 (hi + lo
 *     parts, three bf16 matrix-core products each, fp32 accumulation) with bf16
 *     io and in fp32 with fp32 io (at the full-width shape as batched library
 *     GEMMs, three per product).  The result no longer scales with eta: the
 *     step has singular values near 1 whatever the gradient's size, so it is
 *     meant to be used with ZM_RENORM_ROW.  n_kv = 0 leaves W unchanged. */
typedef enum zm_step_rule { ZM_STEP_GRADIENT = 0, ZM_STEP_NEWTON_SCHULZ = 1 } zm_step_rule;

typedef struct zm_ttt_desc {
  int32_t heads;      /* independent fast weights */
  int32_t d_head;     /* d: width of q, k, v, o per head */
  int32_t d_hidden;   /* h: SwiGLU hidden width */
  int32_t io_dtype;   /* zm_dtype of q, k, v, o */
  int32_t renorm;     /* zm_renorm */
  int32_t step_rule;  /* zm_step_rule (0: plain gradient step) */
  int64_t ld_tok;     /* elements between consecutive tokens of q/k/v/o */
} zm_ttt_desc;

/* Bytes of workspace needed by any entry point below for an update over
 * n_kv tokens and an apply over n_q queries (either may be 0).  Writes the
 * size to *bytes.  Returns ZM_OK or a validation error.  The size never
 * decreases as n_kv or n_q grows, so a workspace sized for (n_kv, n_q) also
 * serves every call over at most n_kv tokens and n_q queries. */
ZM_API int zm_ttt_workspace_size(const zm_ttt_desc* desc, int64_t n_kv, int64_t n_q, size_t* bytes);

/* Update (review Eq. (2)-(3) and the renormalised update display):
 *   g = grad_W sum_{i<n_kv} eta_i L(f_W(k_i), v_i),  L(f, v) = -f^T v,
 *   W' = W - g  (or W - NewtonSchulz(g), see zm_step_rule),
 *   W_hat = renorm(W, W') if desc->renorm else W'.
 * k, v: [n_kv, heads, d_head] tokens; eta: [n_kv, heads].
 * w1, w2, w3: the current fast weights (read only).
 * w1_out, w2_out, w3_out: receive W_hat; they may alias w1, w2, w3 (in-place
 * update).  n_kv = 0 is valid and gives W_hat = W. */
ZM_API int zm_ttt_update(const zm_ttt_desc* desc, int64_t n_kv,
                  const void* k, const void* v, const float* eta,
                  const float* w1, const float* w2, const float* w3,
                  float* w1_out, float* w2_out, float* w3_out,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Update and its virtual loss (review Eq. (2)): as zm_ttt_update, and
 * loss[h] = sum_{i<n_kv} eta_i L(f_W(k_i), v_i) = -sum_i eta_i f_W(k_i)^T v_i
 * of head h at the incoming W (the loss whose gradient the step follows).
 * It is read from the update's own registers: f^T v = u . (W2^T v) with
 * u = SiLU(W1 k) (*) W3 k and W2^T v both formed for the gradient, so the
 * loss costs one multiply-add per (token, hidden unit) and a fixed-order
 * sum.  loss: device pointer to heads floats (fp32; operands as the update's
 * bf16 ones).  n_kv = 0 writes zeros.  Bitwise reproducible; W_hat is
 * bitwise that of zm_ttt_update.  The bf16 narrow heads only: fp32 io and the
 * full-width shape return ZM_ERR_UNSUPPORTED.  Workspace as zm_ttt_update. */
ZM_API int zm_ttt_update_loss(const zm_ttt_desc* desc, int64_t n_kv,
                  const void* k, const void* v, const float* eta,
                  const float* w1, const float* w2, const float* w3,
                  float* w1_out, float* w2_out, float* w3_out, float* loss,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Apply (review Eq. (4)): o_i = f_W(q_i) for i < n_q, per head.
 * q, o: [n_q, heads, d_head] in desc->io_dtype; o must not overlap q. */
ZM_API int zm_ttt_apply(const zm_ttt_desc* desc, int64_t n_q, const void* q,
                 const float* w1, const float* w2, const float* w3,
                 void* o, void* workspace, size_t workspace_bytes, void* stream);

/* Bidirectional single chunk (review of ZipMap, Method 2: the chunk update of
 * Eq. (3) over all image tokens, then the read of Eq. (4) with the updated
 * weights; the ZipMap notes' TTT-module section describes the same write-then-
 * read of one chunk; a ray-map target view only reads): the update over all
 * n_kv tokens, then the apply of all n_q queries through W_hat (the queries
 * may include extra target-view rows beyond the image tokens).  Outputs W_hat
 * to w*_out (may alias w*) and o.  Equivalent to zm_ttt_update followed by
 * zm_ttt_apply on W_hat, without re-reading W_hat from fp32. */
ZM_API int zm_ttt_update_apply(const zm_ttt_desc* desc, int64_t n_kv,
                        const void* k, const void* v, const float* eta,
                        int64_t n_q, const void* q,
                        const float* w1, const float* w2, const float* w3,
                        float* w1_out, float* w2_out, float* w3_out, void* o,
                        void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * update and apply as zm_ttt_update_apply, run in a scratch array the library
 * holds in device memory (ZM_TTT_SCRATCH_BYTES = 64 MiB, one copy per GPU
 * from module load to process end) instead of a caller workspace.  The
 * call allocates nothing; on its first use on a device it looks up that
 * device's scratch address.  Results are bitwise those of
 * zm_ttt_update_apply.  Narrow heads only: a call whose workspace need
 * (zm_ttt_workspace_size(desc, n_kv, n_q)) exceeds the scratch returns
 * ZM_ERR_WORKSPACE, and the full-width shape ZM_ERR_UNSUPPORTED.  Every
 * kernel writes what the next one reads, except the counters of the
 * in-launch reduce (see Workspace above), which must start at zero: the
 * call's first kernel clears them (a kernel, not a memset, so the call can
 * be captured).  A call leaves its last contents there.  All calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (two streams, two threads)
 * race and give undefined results; order them on one stream. */
ZM_API int zm_ttt_update_apply_scratch(const zm_ttt_desc* desc, int64_t n_kv,
                                const void* k, const void* v, const float* eta,
                                int64_t n_q, const void* q,
                                const float* w1, const float* w2, const float* w3,
                                float* w1_out, float* w2_out, float* w3_out, void* o,
                                void* stream);

/* One streaming step on one frame of n_frame tokens (review 3. Streaming
 * Reconstruction, Eq. (6)).  order: a zm_order, optionally OR-ed with
 * zm_stream_flags.  w1, w2, w3 hold the state W(t-1) on entry and
 * W(t) on return (updated in place).  q, k, v: [n_frame, heads, d_head];
 * eta: [n_frame, heads]; o receives f_{W(t-1)}(q) (APPLY_THEN_UPDATE) or
 * f_{W(t)}(q) (UPDATE_THEN_APPLY).  o must not overlap q, k, v or eta: with
 * APPLY_THEN_UPDATE and bf16 io the read and the update's partial sums run
 * side by side in one launch. */
ZM_API int zm_ttt_stream_step(const zm_ttt_desc* desc, int order, int64_t n_frame,
                       const void* q, const void* k, const void* v, const float* eta,
                       float* w1, float* w2, float* w3, void* o,
                       void* workspace, size_t workspace_bytes, void* stream);

/* A sequence of n = offsets[n_chunks] tokens cut into consecutive chunks
 * [offsets[c], offsets[c+1]), read and written chunk after chunk with the
 * orders of the LaCT summary (mhpn.cn, part 二, 3、应用场景):
 *   ZM_UPDATE_THEN_APPLY: block-causal, W <- Update(W; chunk c), then
 *     o_c = f_W(q_c) (order (b));
 *   ZM_APPLY_THEN_UPDATE: shifted block-causal, o_c = f_W(q_c), then
 *     W <- Update(W; chunk c) (order (c)).
 * update_mask (host memory, n_chunks bytes, or NULL for all): a zero entry
 * skips chunk c's update, so that chunk is only read (updates on selected
 * chunks and reads on all, order (d)).  inner_steps (1..64) repeats the
 * update on the same chunk, each step taking the gradient at the weights the
 * previous one produced.  A per-chunk rate is a scaling of that chunk's eta
 * rows.
 * offsets: host memory, n_chunks + 1 int64, offsets[0] = 0, non-decreasing;
 * n_chunks in [0, 2^24].  Empty chunks are skipped.
 * q, k, v, o: [n, heads, d_head]; eta: [n, heads]; o must not overlap q, k,
 * v or eta (as for zm_ttt_stream_step).  w1, w2, w3 hold the state and are
 * updated in place.  The workspace must hold
 * zm_ttt_workspace_size(desc, L, L) bytes, L the longest chunk.  Equivalent to
 * one zm_ttt_stream_step per chunk (extended by the mask and inner steps). */
ZM_API int zm_ttt_chunked(const zm_ttt_desc* desc, int order, int64_t n_chunks,
                   const int64_t* offsets, const uint8_t* update_mask, int inner_steps,
                   const void* q, const void* k, const void* v, const float* eta,
                   float* w1, float* w2, float* w3, void* o,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
ZM_API const char* zm_status_string(int status);

/* The slow weights around the layer: the projections of an input token x
 * (width d_in) to q, k, v (ZipMap notes, q / k / v 投影) and to the per-token
 * rate (review, note under Eq. (3): a linear layer of the token), and the
 * output gate of review Eq. (5).  Readings where the pages are silent: the
 * rate is eta = eta_scale * sigmoid(W_eta x); RMSNorm runs over the whole
 * width H * d_head with a learnable scale gamma and epsilon rms_eps. */
typedef struct zm_layer_weights {
  const void* w_in;     /* bf16 [3 H d + H][d_in]: rows of W_Q, W_K, W_V (H d each,
                           head-major, d_head consecutive rows per head), then W_eta (H) */
  const void* w_gate;   /* bf16 [H d][H d]: W_g */
  const float* gamma;   /* fp32 [H d]: RMSNorm scale, 16-byte aligned */
  int32_t d_in;         /* input width, a multiple of 8 */
  float eta_scale;      /* >= 0 */
  float rms_eps;        /* > 0 */
  int32_t reserved;     /* must be 0 */
} zm_layer_weights;

/* Bytes of workspace zm_ttt_layer needs for n tokens. */
ZM_API int zm_ttt_layer_workspace_size(const zm_ttt_desc* desc, const zm_layer_weights* lw,
                                int64_t n, size_t* bytes);

/* The whole TTT layer on one bidirectional chunk of n tokens x (bf16 rows of
 * stride ld_x, ld_x >= d_in, a multiple of 8):
 *   [q | k | v | z] = W_in x,  eta = eta_scale * sigmoid(z),
 *   W_hat = update(W; k, v, eta) (+ renorm, desc->step_rule),
 *   o' = f_{W_hat}(q),  o = RMSNorm(o') * SiLU(W_g o')  (review Eq. (5)).
 * desc: heads, d_head, d_hidden, renorm and step_rule as for the other entry
 * points, with a layer width H d of at most 8192 (wider: ZM_ERR_UNSUPPORTED);
 * io_dtype must be ZM_BF16; desc->ld_tok is the row stride of o
 * (>= H d, a multiple of 8).  w1..w3 are read, W_hat goes to w*_out (may
 * alias).  o: bf16 [n][H d].  The projections and W_g o' run as library GEMMs
 * (bf16 operands, fp32 accumulation, bf16 results); the rate, the gate and the
 * TTT steps run in the library's kernels. */
ZM_API int zm_ttt_layer(const zm_ttt_desc* desc, const zm_layer_weights* lw, int64_t n,
                 const void* x, int64_t ld_x, const float* w1, const float* w2, const float* w3,
                 float* w1_out, float* w2_out, float* w3_out, void* o,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Description of the last ZM_ERR_HIP failure on the calling thread (the HIP
 * call or GEMM-library call that failed and its status), or "" if none.
 * The string stays valid until the thread's next failing call. */
ZM_API const char* zm_ttt_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
ZM_API int zm_ttt_version(void);

/* Profiling aid: when events != NULL, every later launch of kernel stage s
 * (0 weight cast, 1 update partial sums, 2 reduce/step/renorm, 3 apply,
 * 4 Newton-Schulz, 5 input projections and rate, 6 output gate) records
 * events[2s] before and events[2s+1] after itself on the launch stream, for
 * each non-NULL slot.  Where a chunk's read and its update's partial sums
 * share one launch (bf16 APPLY_THEN_UPDATE), the events of stages 1 and 3
 * both bracket that launch; where the reduce runs inside the update's launch
 * (short chunks, see Workspace above), so do those of stage 2.  The events are hipEvent_t handles passed as void*;
 * n_events must be 8 (stages 0-3), 10 (0-4) or 14 (0-6) (or 0 with
 * events == NULL to switch off).  Process-wide setting; not for concurrent use
 * from several threads. */
ZM_API int zm_ttt_set_profile_events(void* const* events, int n_events);

#ifdef __cplusplus
}
#endif

#endif /* ZM_TTT_H */
