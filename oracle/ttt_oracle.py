"""fp64 CPU oracle of the large-chunk test-time-training (TTT) layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It is deliberately
plain and slow: NumPy float64, one head at a time, tokens summed in blocks
only to bound memory.  It shares no code with the HIP library.

Sources (web pages describing ZipMap and LaCT):
  [notes]  "ZipMap：基于 Test-Time Training 的线性时间有状态 3D 重建"
           (67656.sbs paper-reading notes), section "TTT 模块：核心公式与
           fast-weight 使用过程".
  [review] "[논문리뷰] ZipMap: Linear-Time Stateful 3D Reconstruction via
           Test-Time Training" (kimjy99.github.io), Method, 2. Feature
           Backbone and 3. Streaming Reconstruction.
  [lact]   mhpn.cn blog post on TTSA3R / LaCT / ZipMap / LoGeR, part 二
           (LaCT), 2、架构 and 3、应用场景.

Conventions (per head): d = head width, h = hidden width.
  W1, W3 have shape [h, d] and W2 has shape [d, h], so f_W(x) = W x acts on
  column vectors as the pages write it.  Token arrays are row-major [n, d],
  so applying a matrix to every token is ``x @ W.T``.
  Multi-head arrays: q, k, v [n, H, d]; eta [n, H]; W1, W3 [H, h, d];
  W2 [H, d, h].

Readings taken where the pages leave a step open:
  * one gradient step on the chunk; the step is W - g by default, or
    W - NewtonSchulz(g) when asked for ([review] the update display after
    Eq. (3)): the pages name the Muon optimizer's Newton-Schulz
    orthonormalisation but give neither its polynomial nor its step count,
    so the reading is Muon's published odd quintic iteration (K. Jordan,
    "Muon: An optimizer for hidden layers in neural networks", 2024),
    coefficients (3.4445, -4.7750, 2.0315), five steps, started from
    g / max(||g||_F, 1e-12);
  * the chunk gradient is a sum over tokens, no 1/n;
  * eta is one scalar per token and head;
  * the optional renormalisation is per row (the fan-in vector of one output
    unit), with the pre-update row norm and a max(., 1e-12) guard;
  * bidirectional chunk: update first, then read with the updated weights;
    streaming: apply-then-update per frame by default;
  * around the layer ([notes] q / k / v 投影; [review] the rate note under
    Eq. (3) and Eq. (5)): q, k, v are linear projections of the input token;
    the per-token rate comes from a linear layer, read as
    eta = eta_scale * sigmoid(W_eta x) (positive and bounded; the pages name no
    activation); the output gate is RMSNorm(o') * SiLU(W_g o') with RMSNorm
    over the whole width (all heads), a learnable scale gamma and
    eps = 1e-6 (the pages give neither), and it is the layer's output.
"""
from __future__ import annotations

import numpy as np

TOKEN_BLOCK = 65536
RENORM_EPS = 1e-12
MUON_NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
STEP_RULES = ("gradient", "newton_schulz")


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _blocks(n, block=None):
    block = TOKEN_BLOCK if block is None else int(block)
    for s in range(0, n, block):
        yield s, min(n, s + block)


# ---------------------------------------------------------------------------
# Elementwise functions
# ---------------------------------------------------------------------------
def sigmoid(x):
    """Logistic function 1 / (1 + exp(-x)), in the form exp(-|x|) / (1 + exp(-|x|))
    for negative x so that no exponential overflows."""
    x = _f64(x)
    z = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + z), z / (1.0 + z))


def silu(x):
    """SiLU(x) = x * sigmoid(x), the gate nonlinearity of the SwiGLU fast
    weight ([review] Eq. (1); [notes] "Fast-weight MLP：SwiGLU")."""
    x = _f64(x)
    return x * sigmoid(x)


def silu_grad(x):
    """d SiLU / dx = sigmoid(x) * (1 + x * (1 - sigmoid(x)))  (calculus on the
    definition above)."""
    x = _f64(x)
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


# ---------------------------------------------------------------------------
# Fast-weight functions
# ---------------------------------------------------------------------------
def _swiglu_parts(x, w1, w3):
    a = x @ w1.T          # W1 x for every token, [n, h]
    b = x @ w3.T          # W3 x, [n, h]
    sg = sigmoid(a)
    u = (a * sg) * b      # SiLU(W1 x) ⊙ (W3 x)
    return a, b, u, sg


def swiglu(x, w1, w2, w3, block=None):
    """f_W(x) = W2 [SiLU(W1 x) ⊙ (W3 x)] for every row of x.

    [review] Method 2, Eq. (1); [notes] "Fast-weight MLP：SwiGLU".
    x: [n, d]; returns [n, d_out] with d_out = W2.shape[0].
    """
    x, w1, w2, w3 = map(_f64, (x, w1, w2, w3))
    out = np.empty((x.shape[0], w2.shape[0]))
    for s, e in _blocks(x.shape[0], block):
        _, _, u, _ = _swiglu_parts(x[s:e], w1, w3)
        out[s:e] = u @ w2.T
    return out


def linear_fw(x, w):
    """The linear fast weight f_W(x) = W x of the pages' linear-case
    derivation ([notes] "为什么它像 attention（线性情形的直观推导）")."""
    return _f64(x) @ _f64(w).T


# ---------------------------------------------------------------------------
# Vector-Jacobian products: sum over tokens of J_i^T cot_i w.r.t. the weights
# ---------------------------------------------------------------------------
def vjp_swiglu(params, x, cot, block=None):
    """Pull a per-token cotangent on f_W(x_i) back to (W1, W2, W3), summed
    over the tokens.  Chain rule through Eq. (1) of [review]:
        f = W2 u,  u = SiLU(a) ⊙ b,  a = W1 x,  b = W3 x.
    Returns (gW1 [h, d], gW2 [d_out, h], gW3 [h, d]).
    """
    w1, w2, w3 = map(_f64, params)
    x, cot = _f64(x), _f64(cot)
    g1 = np.zeros_like(w1)
    g2 = np.zeros_like(w2)
    g3 = np.zeros_like(w3)
    for s, e in _blocks(x.shape[0], block):
        xb, cb = x[s:e], cot[s:e]
        a, b, u, sg = _swiglu_parts(xb, w1, w3)
        g2 += cb.T @ u                    # f = W2 u  ->  dW2 = cot u^T
        du = cb @ w2                      # cotangent on u, [n, h]
        db = du * (a * sg)                # u = SiLU(a) ⊙ b
        da = du * b * (sg * (1.0 + a * (1.0 - sg)))   # SiLU'(a), see silu_grad
        g1 += da.T @ xb                   # a = W1 x  ->  dW1 = da x^T
        g3 += db.T @ xb                   # b = W3 x  ->  dW3 = db x^T
    return g1, g2, g3


def vjp_linear(params, x, cot, block=None):
    """Same pull-back for the linear fast weight f_W(x) = W x: dW = cot x^T."""
    (w,) = params
    x, cot = _f64(x), _f64(cot)
    g = np.zeros_like(_f64(w))
    for s, e in _blocks(x.shape[0], block):
        g += cot[s:e].T @ x[s:e]
    return (g,)


# ---------------------------------------------------------------------------
# The update: virtual loss, chunk gradient, one step, optional renorm
# ---------------------------------------------------------------------------
def chunk_gradient(vjp, params, k, v, eta, block=None):
    """g = grad_W  sum_i eta_i L(f_W(k_i), v_i)  with  L(f, v) = -f^T v.

    Loss: [review] Eq. (2), [notes] Eq. 2.  Per-token rate inside the sum:
    [review] Eq. (3), [notes] Eq. 3.  The sum covers every token of the chunk
    ([lact] 2、架构, update part).  Since d(eta_i L_i)/d f_i = -eta_i v_i, the
    chunk gradient is the VJP of f_W with cotangent -eta_i v_i per token.
    """
    k, v, eta = _f64(k), _f64(v), _f64(eta)
    cot = -(eta[:, None] * v)
    return vjp(params, k, cot, block=block)


def gradient_step(params, grads):
    """W_hat = W - g, one plain gradient step ([notes] Eq. 3; [review] the
    fast weights are adapted with a single gradient-descent step)."""
    return tuple(_f64(w) - _f64(g) for w, g in zip(params, grads))


def newton_schulz(g, steps=NS_STEPS, coeffs=MUON_NS_COEFFS, eps=RENORM_EPS):
    """Newton-Schulz orthonormalisation of one gradient matrix.

    [review] the update display after Eq. (3): Delta <- NewtonSchulz(g),
    following the Muon optimizer.  Each step applies the odd matrix
    polynomial X <- a X + b (X X^T) X + c (X X^T)^2 X to
    X_0 = g / max(||g||_F, eps); it maps every singular value s of X to
    a s + b s^3 + c s^5 and keeps the singular vectors, so the result
    approaches U V^T (g = U S V^T) for coefficients that drive the
    normalised singular values towards 1 (the textbook cubic (1.5, -0.5, 0)
    converges to U V^T exactly; Muon's quintic lands them near 1 in five
    steps).  g = 0 gives 0.
    """
    x = _f64(g)
    nrm = np.sqrt((x * x).sum())
    x = x / max(nrm, eps)
    a, b, c = coeffs
    for _ in range(steps):
        gram = x @ x.T
        gx = gram @ x
        x = a * x + b * gx + c * (gram @ gx)
    return x


def renorm_rows(w_old, w_new, eps=RENORM_EPS):
    """Norm-preserving L2 renormalisation of the updated weight.

    [review] the update display after Eq. (3) rescales W - Delta to the norm of
    W; [lact] 2、架构 applies an L2 normalisation after the step.  Reading:
    per row (the fan-in vector of one output unit of W x), the norm of the
    row before the update, and max(norm, eps) as a guard (not an offset), so a
    row the update left unchanged comes back bit-for-bit unchanged.
    """
    w_old, w_new = _f64(w_old), _f64(w_new)
    n_old = np.sqrt((w_old * w_old).sum(axis=1, keepdims=True))
    n_new = np.sqrt((w_new * w_new).sum(axis=1, keepdims=True))
    scale = n_old / np.maximum(n_new, eps)
    return w_new * scale


def update_head(k, v, eta, w1, w2, w3, renorm=False, block=None, step="gradient"):
    """One head: W -> W_hat on one chunk of n tokens.
    k, v: [n, d]; eta: [n]; returns (W1_hat, W2_hat, W3_hat).
    step = "gradient": W' = W - g;  step = "newton_schulz": W' = W -
    NewtonSchulz(g) per matrix ([review] the update display after Eq. (3))."""
    if step not in STEP_RULES:
        raise ValueError(step)
    params = tuple(map(_f64, (w1, w2, w3)))
    grads = chunk_gradient(vjp_swiglu, params, k, v, eta, block=block)
    if step == "newton_schulz":
        grads = tuple(newton_schulz(g) for g in grads)
    new = gradient_step(params, grads)
    if renorm:
        new = tuple(renorm_rows(p, q) for p, q in zip(params, new))
    return new


def apply_head(q, w1, w2, w3, block=None):
    """Read the fast weight with the queries: o'_i = f_W(q_i)
    ([review] Eq. (4); target-ray queries use the same read)."""
    return swiglu(q, w1, w2, w3, block=block)


def virtual_loss(k, v, eta, w1, w2, w3):
    """Per-head value of sum_i eta_i L(f_W(k_i), v_i), L = -f^T v
    ([review] Eq. (2)-(3)).  k, v [n, H, d]; eta [n, H]; returns [H]."""
    k, v, eta = _f64(k), _f64(v), _f64(eta)
    out = np.zeros(k.shape[1])
    for hd in range(k.shape[1]):
        f = swiglu(k[:, hd], w1[hd], w2[hd], w3[hd])
        out[hd] = -(eta[:, hd] * (f * v[:, hd]).sum(axis=1)).sum()
    return out


# ---------------------------------------------------------------------------
# Multi-head entry points (heads are independent fast weights)
# ---------------------------------------------------------------------------
def update(k, v, eta, w1, w2, w3, renorm=False, block=None, step="gradient"):
    """All heads: k, v [n, H, d]; eta [n, H]; W1, W3 [H, h, d]; W2 [H, d, h].
    Returns float64 (W1_hat, W2_hat, W3_hat)."""
    k, v, eta = _f64(k), _f64(v), _f64(eta)
    w1, w2, w3 = map(_f64, (w1, w2, w3))
    heads = w1.shape[0]
    o1, o2, o3 = np.empty_like(w1), np.empty_like(w2), np.empty_like(w3)
    for hd in range(heads):
        o1[hd], o2[hd], o3[hd] = update_head(
            k[:, hd], v[:, hd], eta[:, hd], w1[hd], w2[hd], w3[hd],
            renorm=renorm, block=block, step=step)
    return o1, o2, o3


def apply(q, w1, w2, w3, block=None):
    """All heads: q [m, H, d] -> o [m, H, d_out] (float64)."""
    q = _f64(q)
    w1, w2, w3 = map(_f64, (w1, w2, w3))
    out = np.empty((q.shape[0], q.shape[1], w2.shape[1]))
    for hd in range(q.shape[1]):
        out[:, hd] = apply_head(q[:, hd], w1[hd], w2[hd], w3[hd], block=block)
    return out


def update_apply(k, v, eta, q, w1, w2, w3, renorm=False, block=None, step="gradient"):
    """Bidirectional single chunk: update on all tokens, then read every
    query through the updated weights ([notes] write/read flow; [review]
    Eq. (3) then Eq. (4)).  Returns ((W1_hat, W2_hat, W3_hat), o)."""
    new = update(k, v, eta, w1, w2, w3, renorm=renorm, block=block, step=step)
    return new, apply(q, *new, block=block)


def stream(frames, w1, w2, w3, renorm=False, order="apply_then_update", step="gradient"):
    """Streaming: W(t) = Update(W(t-1); frame t) frame after frame
    ([review] 3. Streaming Reconstruction, Eq. (6); [notes] 流式更新).
    Each frame is a dict with q, k, v [p, H, d] and eta [p, H].
    order = "apply_then_update": o_t = f_{W(t-1)}(q_t), then update
            ([lact] 3、应用场景, shifted block-causal order);
    order = "update_then_apply": update, then o_t = f_{W(t)}(q_t)
            ([lact] 3、应用场景, block-causal order).
    Returns (final weights, list of o_t)."""
    if order not in ("apply_then_update", "update_then_apply"):
        raise ValueError(order)
    w = tuple(map(_f64, (w1, w2, w3)))
    outs = []
    for fr in frames:
        if order == "apply_then_update":
            outs.append(apply(fr["q"], *w))
            w = update(fr["k"], fr["v"], fr["eta"], *w, renorm=renorm, step=step)
        else:
            w = update(fr["k"], fr["v"], fr["eta"], *w, renorm=renorm, step=step)
            outs.append(apply(fr["q"], *w))
    return w, outs


def chunked(q, k, v, eta, offsets, w1, w2, w3, order="update_then_apply", update_mask=None,
            inner_steps=1, renorm=False, step="gradient"):
    """A token sequence cut into consecutive chunks [offsets[c], offsets[c+1]),
    read and written chunk after chunk ([lact] 3、应用场景, orders (b)-(d)):
      order "update_then_apply" (block-causal, (b)): W <- Update(W; chunk c),
            then o_c = f_W(q_c);
      order "apply_then_update" (shifted block-causal, (c)): o_c = f_W(q_c),
            then W <- Update(W; chunk c);
      update_mask[c] False skips the update of chunk c, which is then only
            read (selective update, (d): writes on some chunks, reads on all);
      inner_steps > 1 repeats the update on the same chunk, each step taking
            the gradient at the weights the previous step produced.
    A per-chunk rate is a scaling of that chunk's eta rows.  q, k, v [n, H, d];
    eta [n, H].  Returns (final weights, o [n, H, d_out])."""
    if order not in ("apply_then_update", "update_then_apply"):
        raise ValueError(order)
    if inner_steps < 1:
        raise ValueError(inner_steps)
    offsets = [int(x) for x in offsets]
    n_chunks = len(offsets) - 1
    if n_chunks < 0 or offsets[0] != 0 or any(b < a for a, b in zip(offsets, offsets[1:])):
        raise ValueError("offsets must start at 0 and not decrease")
    mask = [True] * n_chunks if update_mask is None else [bool(m) for m in update_mask]
    w = tuple(map(_f64, (w1, w2, w3)))
    q = _f64(q)
    out = np.zeros((q.shape[0], q.shape[1], w[1].shape[1]))
    for c in range(n_chunks):
        s, e = offsets[c], offsets[c + 1]
        if order == "apply_then_update":
            out[s:e] = apply(q[s:e], *w)
        if mask[c]:
            for _ in range(inner_steps):
                w = update(k[s:e], v[s:e], eta[s:e], *w, renorm=renorm, step=step)
        if order == "update_then_apply":
            out[s:e] = apply(q[s:e], *w)
    return w, out


# ---------------------------------------------------------------------------
# Around the layer: input projections and the output gate
# ---------------------------------------------------------------------------
RMS_EPS = 1e-6


def rmsnorm(x, gamma, eps=RMS_EPS):
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis ([review] Eq. (5))."""
    x = _f64(x)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * _f64(gamma)


def output_gate(o_prime, w_gate, gamma, eps=RMS_EPS):
    """o = RMSNorm(o') * SiLU(W_g o') per token ([review] Eq. (5)).
    o_prime: [n, width] (all heads side by side); w_gate: [width, width]."""
    o_prime = _f64(o_prime)
    return rmsnorm(o_prime, gamma, eps) * silu(o_prime @ _f64(w_gate).T)


def project(x, w_in, heads, d, eta_scale):
    """q, k, v = W_Q x, W_K x, W_V x ([notes] q / k / v 投影) and the rate
    eta = eta_scale * sigmoid(W_eta x) ([review] note under Eq. (3)).
    x: [n, d_in]; w_in: [3 H d + H, d_in] (rows W_Q, W_K, W_V, W_eta).
    Returns q, k, v [n, H, d] and eta [n, H]."""
    y = _f64(x) @ _f64(w_in).T
    hd = heads * d
    q, k, v = (y[:, i * hd:(i + 1) * hd].reshape(-1, heads, d) for i in range(3))
    eta = eta_scale * sigmoid(y[:, 3 * hd:3 * hd + heads])
    return q, k, v, eta


def layer(x, w_in, w_gate, gamma, w1, w2, w3, eta_scale, renorm=False, eps=RMS_EPS,
          step="gradient"):
    """The whole TTT layer on one bidirectional chunk: projections, update on
    every token, apply to every token, output gate.  Returns
    ((W1_hat, W2_hat, W3_hat), o [n, H d])."""
    heads, d = _f64(w1).shape[0], _f64(w1).shape[2]
    q, k, v, eta = project(x, w_in, heads, d, eta_scale)
    new, o_prime = update_apply(k, v, eta, q, w1, w2, w3, renorm=renorm, step=step)
    return new, output_gate(o_prime.reshape(o_prime.shape[0], -1), w_gate, gamma, eps)


def update_rows_sampled(k, v, eta, w1, w2, w3, hidden_idx, block=None):
    """Unrenormalised W_hat restricted to a subset J of hidden units of one
    head: (W1_hat[J, :], W2_hat[:, J], W3_hat[J, :]).

    f_W is a sum over hidden units of W2[:, j] * SiLU(W1[j] x) * (W3[j] x),
    so the gradient with respect to unit j's weights involves unit j alone.
    The restriction is therefore exactly the update of the sub-network made of
    the units in J, computed by the same chunk_gradient / gradient_step.
    """
    j = np.asarray(hidden_idx)
    params = (_f64(w1)[j], _f64(w2)[:, j], _f64(w3)[j])
    grads = chunk_gradient(vjp_swiglu, params, k, v, eta, block=block)
    return gradient_step(params, grads)
