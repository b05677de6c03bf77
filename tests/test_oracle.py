"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test checks the oracle against one of: a closed form printed on the
pages (the linear case), calculus done independently (central finite
differences, torch autograd), hand-derived scalar values, invariants of the
update (eta = 0, permutation, chunk additivity, linearity, row norms) or a
pure-Python per-token brute force.  The mutation tests at the bottom plant
plausible mistakes in the oracle and check that some pin catches each one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ttt_oracle as O

RNG = np.random.default_rng(1234)


def rand_problem(n=7, d=3, h=4, seed=0, heads=None):
    r = np.random.default_rng(seed)
    if heads is None:
        k = r.normal(size=(n, d)) / math.sqrt(d)
        v = r.normal(size=(n, d)) / math.sqrt(d)
        q = r.normal(size=(n, d)) / math.sqrt(d)
        eta = 0.5 * r.random(n)
        w1 = r.normal(size=(h, d)) / math.sqrt(d)
        w2 = r.normal(size=(d, h)) / math.sqrt(h)
        w3 = r.normal(size=(h, d)) / math.sqrt(d)
    else:
        k = r.normal(size=(n, heads, d)) / math.sqrt(d)
        v = r.normal(size=(n, heads, d)) / math.sqrt(d)
        q = r.normal(size=(n, heads, d)) / math.sqrt(d)
        eta = 0.5 * r.random((n, heads))
        w1 = r.normal(size=(heads, h, d)) / math.sqrt(d)
        w2 = r.normal(size=(heads, d, h)) / math.sqrt(h)
        w3 = r.normal(size=(heads, h, d)) / math.sqrt(d)
    return dict(k=k, v=v, q=q, eta=eta, w1=w1, w2=w2, w3=w3)


def rel(x, ref):
    x, ref = np.asarray(x), np.asarray(ref)
    return np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300)


# ---------------------------------------------------------------------------
# Elementwise functions and the forward
# ---------------------------------------------------------------------------
def test_sigmoid_silu_values():
    assert O.sigmoid(np.array([0.0]))[0] == 0.5
    assert O.silu(np.array([0.0]))[0] == 0.0
    e1 = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(O.silu(np.array([1.0]))[0] - e1) < 1e-16
    x = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(O.sigmoid(-x), 1.0 - O.sigmoid(x), atol=1e-15)
    # SiLU tends to x for large x and to 0 for very negative x
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15
    # no overflow warnings at extreme inputs
    with np.errstate(over="raise"):
        O.sigmoid(np.array([-1000.0, 1000.0]))


def test_silu_grad_matches_central_difference():
    x = np.linspace(-6, 6, 49)
    hstep = 1e-5
    num = (O.silu(x + hstep) - O.silu(x - hstep)) / (2 * hstep)
    np.testing.assert_allclose(O.silu_grad(x), num, atol=1e-9)


def test_swiglu_two_by_two_hand_values():
    """f_W(x) = W2 [SiLU(W1 x) * (W3 x)] on a 2x2 instance, worked by hand.
    Non-symmetric W1, W2, W3 so that any transposed operand changes the result."""
    x = np.array([[1.0, 2.0]])
    w1 = np.array([[1.0, 0.0], [1.0, 1.0]])      # a = W1 x = (1, 3)
    w3 = np.array([[0.0, 1.0], [2.0, 0.0]])      # b = W3 x = (2, 2)
    w2 = np.array([[1.0, 2.0], [0.0, 3.0]])
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    s3 = 1.0 / (1.0 + math.exp(-3.0))
    u = np.array([1.0 * s1 * 2.0, 3.0 * s3 * 2.0])
    expect = np.array([u[0] + 2.0 * u[1], 3.0 * u[1]])
    got = O.swiglu(x, w1, w2, w3)[0]
    np.testing.assert_allclose(got, expect, rtol=1e-15)


def test_swiglu_block_invariance():
    p = rand_problem(n=50, d=5, h=6)
    a = O.swiglu(p["q"], p["w1"], p["w2"], p["w3"])
    b = O.swiglu(p["q"], p["w1"], p["w2"], p["w3"], block=7)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# The gradient
# ---------------------------------------------------------------------------
def _loss(k, v, eta, w1, w2, w3):
    return O.virtual_loss(k[:, None], v[:, None], eta[:, None], w1[None], w2[None], w3[None])[0]


def test_gradient_matches_central_finite_differences():
    p = rand_problem(n=5, d=4, h=8, seed=3)
    k, v, eta = p["k"], p["v"], p["eta"]
    w = [p["w1"].copy(), p["w2"].copy(), p["w3"].copy()]
    g = O.chunk_gradient(O.vjp_swiglu, tuple(w), k, v, eta)
    step = 1e-6
    for m in range(3):
        num = np.zeros_like(w[m])
        for idx in np.ndindex(*w[m].shape):
            wp = [x.copy() for x in w]
            wm = [x.copy() for x in w]
            wp[m][idx] += step
            wm[m][idx] -= step
            num[idx] = (_loss(k, v, eta, *wp) - _loss(k, v, eta, *wm)) / (2 * step)
        assert rel(g[m], num) < 1e-7, (m, rel(g[m], num))


def _check_autograd(d, h):
    p = rand_problem(n=33, d=d, h=h, seed=4)
    t = {kk: torch.tensor(vv, dtype=torch.float64) for kk, vv in p.items()}
    w1 = t["w1"].clone().requires_grad_(True)
    w2 = t["w2"].clone().requires_grad_(True)
    w3 = t["w3"].clone().requires_grad_(True)
    f = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(t["k"], w1))
        * torch.nn.functional.linear(t["k"], w3), w2)
    loss = -(t["eta"] * (f * t["v"]).sum(dim=1)).sum()
    loss.backward()
    g = O.chunk_gradient(O.vjp_swiglu, (p["w1"], p["w2"], p["w3"]), p["k"], p["v"], p["eta"])
    for gm, tm in zip(g, (w1.grad, w2.grad, w3.grad)):
        assert rel(gm, tm.numpy()) < 1e-12
    # and the loss value itself
    assert abs(_loss(p["k"], p["v"], p["eta"], p["w1"], p["w2"], p["w3"]) - loss.item()) < 1e-12


@pytest.mark.parametrize("d,h", [(6, 10), (5, 5)])
def test_gradient_matches_torch_autograd(d, h):
    _check_autograd(d, h)


def test_update_is_one_step_against_the_gradient():
    p = rand_problem(n=9, d=4, h=5, seed=5)
    g = O.chunk_gradient(O.vjp_swiglu, (p["w1"], p["w2"], p["w3"]), p["k"], p["v"], p["eta"])
    new = O.update_head(p["k"], p["v"], p["eta"], p["w1"], p["w2"], p["w3"], renorm=False)
    for w, gm, nm in zip((p["w1"], p["w2"], p["w3"]), g, new):
        np.testing.assert_array_equal(nm, w - gm)


# ---------------------------------------------------------------------------
# Linear case: the closed form the pages print
# ---------------------------------------------------------------------------
def test_linear_case_closed_form_update():
    """f_W(k) = W k gives W_hat = W + sum_i eta_i v_i k_i^T (ZipMap notes,
    linear-case derivation)."""
    p = rand_problem(n=11, d=5, h=5, seed=6)
    w = RNG.normal(size=(5, 5))
    g = O.chunk_gradient(O.vjp_linear, (w,), p["k"], p["v"], p["eta"])
    (w_hat,) = O.gradient_step((w,), g)
    expect = w.copy()
    for i in range(p["k"].shape[0]):
        expect += p["eta"][i] * np.outer(p["v"][i], p["k"][i])
    np.testing.assert_allclose(w_hat, expect, rtol=0, atol=1e-14)


def test_linear_case_read_is_unnormalised_linear_attention():
    """Reading the updated linear weight with q gives W q + sum_i eta_i v_i (k_i^T q)."""
    p = rand_problem(n=13, d=4, h=4, seed=7)
    w = RNG.normal(size=(4, 4))
    g = O.chunk_gradient(O.vjp_linear, (w,), p["k"], p["v"], p["eta"])
    (w_hat,) = O.gradient_step((w,), g)
    out = O.linear_fw(p["q"], w_hat)
    for j in range(p["q"].shape[0]):
        qj = p["q"][j]
        expect = w @ qj
        for i in range(p["k"].shape[0]):
            expect = expect + p["eta"][i] * p["v"][i] * float(p["k"][i] @ qj)
        np.testing.assert_allclose(out[j], expect, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Invariants of the step
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("renorm", [False, True])
def test_zero_eta_leaves_weights_bitwise_unchanged(renorm):
    p = rand_problem(n=20, d=6, h=8, seed=8, heads=3)
    eta = np.zeros_like(p["eta"])
    new = O.update(p["k"], p["v"], eta, p["w1"], p["w2"], p["w3"], renorm=renorm)
    for w, nm in zip((p["w1"], p["w2"], p["w3"]), new):
        np.testing.assert_array_equal(nm, w)


def test_empty_chunk_leaves_weights_unchanged():
    p = rand_problem(n=0, d=6, h=8, seed=8, heads=2)
    new = O.update(p["k"], p["v"], p["eta"], p["w1"], p["w2"], p["w3"], renorm=True)
    for w, nm in zip((p["w1"], p["w2"], p["w3"]), new):
        np.testing.assert_array_equal(nm, w)


@pytest.mark.parametrize("renorm", [False, True])
def test_permutation_invariance(renorm):
    p = rand_problem(n=40, d=6, h=8, seed=9, heads=2)
    perm = np.random.default_rng(1).permutation(40)
    a, oa = O.update_apply(p["k"], p["v"], p["eta"], p["q"], p["w1"], p["w2"], p["w3"], renorm=renorm)
    b, ob = O.update_apply(p["k"][perm], p["v"][perm], p["eta"][perm], p["q"],
                           p["w1"], p["w2"], p["w3"], renorm=renorm)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oa, ob, rtol=0, atol=1e-13)


def test_chunk_additivity():
    """Delta W over a union of two token sets is the sum of the two Deltas
    (the update is a sum over tokens), which also pins any split of the sum."""
    p = rand_problem(n=30, d=5, h=7, seed=10, heads=2)
    w = (p["w1"], p["w2"], p["w3"])
    full = O.update(p["k"], p["v"], p["eta"], *w)
    a = O.update(p["k"][:13], p["v"][:13], p["eta"][:13], *w)
    b = O.update(p["k"][13:], p["v"][13:], p["eta"][13:], *w)
    for wm, f, x, y in zip(w, full, a, b):
        np.testing.assert_allclose(f - wm, (x - wm) + (y - wm), rtol=0, atol=1e-14)


def test_linearity_in_eta_and_v():
    p = rand_problem(n=25, d=5, h=6, seed=11, heads=2)
    w = (p["w1"], p["w2"], p["w3"])

    def delta(k, v, eta):
        return [n - o for n, o in zip(O.update(k, v, eta, *w), w)]

    d1 = delta(p["k"], p["v"], p["eta"])
    d2 = delta(p["k"], p["v"], 2.5 * p["eta"])
    for x, y in zip(d1, d2):
        np.testing.assert_allclose(y, 2.5 * x, rtol=1e-12, atol=1e-15)
    v2 = np.random.default_rng(5).normal(size=p["v"].shape)
    da = delta(p["k"], v2, p["eta"])
    dsum = delta(p["k"], p["v"] + v2, p["eta"])
    for x, y, z in zip(d1, da, dsum):
        np.testing.assert_allclose(z, x + y, rtol=1e-12, atol=1e-15)


def test_renorm_preserves_row_norms_and_direction():
    p = rand_problem(n=25, d=6, h=9, seed=12, heads=2)
    eta = 50.0 * p["eta"]          # a large step so the renorm matters
    off = O.update(p["k"], p["v"], eta, p["w1"], p["w2"], p["w3"], renorm=False)
    on = O.update(p["k"], p["v"], eta, p["w1"], p["w2"], p["w3"], renorm=True)
    for w, x, y in zip((p["w1"], p["w2"], p["w3"]), off, on):
        nw = np.linalg.norm(w, axis=2)
        ny = np.linalg.norm(y, axis=2)
        np.testing.assert_allclose(ny, nw, rtol=1e-13)
        # same direction as the unnormalised update, row by row
        cos = (x * y).sum(axis=2) / (np.linalg.norm(x, axis=2) * ny)
        np.testing.assert_allclose(cos, 1.0, rtol=1e-13)
        assert rel(x, w) > 1e-3   # the step did change the weights


def test_renorm_zero_row_guard():
    w_old = np.array([[0.0, 0.0], [3.0, 4.0]])
    w_new = np.array([[0.0, 0.0], [6.0, 8.0]])
    out = O.renorm_rows(w_old, w_new)
    np.testing.assert_array_equal(out, [[0.0, 0.0], [3.0, 4.0]])


def test_sampled_hidden_units_match_full_update():
    p = rand_problem(n=31, d=5, h=12, seed=13)
    full = O.update_head(p["k"], p["v"], p["eta"], p["w1"], p["w2"], p["w3"])
    j = np.array([0, 5, 11])
    s1, s2, s3 = O.update_rows_sampled(p["k"], p["v"], p["eta"], p["w1"], p["w2"], p["w3"], j)
    np.testing.assert_allclose(s1, full[0][j], rtol=0, atol=1e-15)
    np.testing.assert_allclose(s2, full[1][:, j], rtol=0, atol=1e-15)
    np.testing.assert_allclose(s3, full[2][j], rtol=0, atol=1e-15)


def test_block_size_does_not_change_the_update():
    p = rand_problem(n=100, d=5, h=6, seed=14, heads=2)
    a = O.update(p["k"], p["v"], p["eta"], p["w1"], p["w2"], p["w3"], renorm=True)
    b = O.update(p["k"], p["v"], p["eta"], p["w1"], p["w2"], p["w3"], renorm=True, block=9)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# Brute force: per token, per scalar, pure Python
# ---------------------------------------------------------------------------
def _brute_force_update(k, v, eta, w1, w2, w3):
    n, d = len(k), len(k[0])
    h = len(w1)
    g1 = [[0.0] * d for _ in range(h)]
    g2 = [[0.0] * h for _ in range(d)]
    g3 = [[0.0] * d for _ in range(h)]
    for i in range(n):
        a = [sum(w1[j][c] * k[i][c] for c in range(d)) for j in range(h)]
        b = [sum(w3[j][c] * k[i][c] for c in range(d)) for j in range(h)]
        sg = [1.0 / (1.0 + math.exp(-x)) for x in a]
        u = [a[j] * sg[j] * b[j] for j in range(h)]
        # dL_i/df = -eta_i v_i
        df = [-eta[i] * v[i][r] for r in range(d)]
        for r in range(d):
            for j in range(h):
                g2[r][j] += df[r] * u[j]
        du = [sum(df[r] * w2[r][j] for r in range(d)) for j in range(h)]
        for j in range(h):
            dsilu = sg[j] + a[j] * sg[j] * (1.0 - sg[j])
            da = du[j] * b[j] * dsilu
            db = du[j] * a[j] * sg[j]
            for c in range(d):
                g1[j][c] += da * k[i][c]
                g3[j][c] += db * k[i][c]
    sub = lambda w, g: [[w[r][c] - g[r][c] for c in range(len(w[0]))] for r in range(len(w))]
    return sub(w1, g1), sub(w2, g2), sub(w3, g3)


def test_brute_force_per_token_loop():
    p = rand_problem(n=5, d=4, h=6, seed=15)
    bf = _brute_force_update(*(p[x].tolist() for x in ("k", "v", "eta", "w1", "w2", "w3")))
    new = O.update_head(p["k"], p["v"], p["eta"], p["w1"], p["w2"], p["w3"])
    for x, y in zip(new, bf):
        np.testing.assert_allclose(x, np.array(y), rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# Streaming
# ---------------------------------------------------------------------------
def _frames(n_frames, p_tok, heads, d, seed):
    r = np.random.default_rng(seed)
    return [dict(q=r.normal(size=(p_tok, heads, d)) / math.sqrt(d),
                 k=r.normal(size=(p_tok, heads, d)) / math.sqrt(d),
                 v=r.normal(size=(p_tok, heads, d)) / math.sqrt(d),
                 eta=0.3 * r.random((p_tok, heads))) for _ in range(n_frames)]


def test_stream_single_frame_equals_single_chunk():
    p = rand_problem(n=1, d=5, h=6, seed=16, heads=2)
    fr = _frames(1, 17, 2, 5, 17)
    w = (p["w1"], p["w2"], p["w3"])
    ws, outs = O.stream(fr, *w, renorm=True, order="update_then_apply")
    wc, oc = O.update_apply(fr[0]["k"], fr[0]["v"], fr[0]["eta"], fr[0]["q"], *w, renorm=True)
    for x, y in zip(ws, wc):
        np.testing.assert_array_equal(x, y)
    np.testing.assert_array_equal(outs[0], oc)
    ws2, outs2 = O.stream(fr, *w, renorm=True, order="apply_then_update")
    np.testing.assert_array_equal(outs2[0], O.apply(fr[0]["q"], *w))
    for x, y in zip(ws2, wc):
        np.testing.assert_array_equal(x, y)


def test_stream_composes_frame_updates():
    p = rand_problem(n=1, d=4, h=6, seed=18, heads=2)
    fr = _frames(3, 11, 2, 4, 19)
    w = (p["w1"], p["w2"], p["w3"])
    ws, outs = O.stream(fr, *w, renorm=True, order="apply_then_update")
    cur = w
    for t in range(3):
        np.testing.assert_array_equal(outs[t], O.apply(fr[t]["q"], *cur))
        cur = O.update(fr[t]["k"], fr[t]["v"], fr[t]["eta"], *cur, renorm=True)
    for x, y in zip(ws, cur):
        np.testing.assert_array_equal(x, y)
    # streaming differs from one bidirectional chunk over the same tokens
    k = np.concatenate([f["k"] for f in fr])
    v = np.concatenate([f["v"] for f in fr])
    eta = np.concatenate([f["eta"] for f in fr])
    wc = O.update(k, v, eta, *w, renorm=True)
    assert rel(ws[0], wc[0]) > 1e-6


# ---------------------------------------------------------------------------
# Mutation tests: a planted mistake in the oracle must fail some pin
# ---------------------------------------------------------------------------
def _pins_pass():
    """Run the sign/eta/sum pin and the calculus pins; True if all pass."""
    try:
        test_linear_case_closed_form_update()
        _check_autograd(6, 10)
        _check_autograd(5, 5)
        test_swiglu_two_by_two_hand_values()
        test_renorm_preserves_row_norms_and_direction()
        test_zero_eta_leaves_weights_bitwise_unchanged(True)
    except AssertionError:
        return False
    return True


def test_pins_pass_unmutated():
    assert _pins_pass()


@pytest.mark.parametrize("mutation", [
    "sign_of_cotangent", "eta_dropped", "silu_grad_as_sigmoid", "w2_transposed_in_vjp",
    "forward_uses_w3_for_gate", "renorm_uses_new_norm", "step_adds_gradient", "eta_squared",
])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    if mutation == "sign_of_cotangent":
        def cg(vjp, params, k, v, eta, block=None):
            return vjp(params, O._f64(k), O._f64(eta)[:, None] * O._f64(v), block=block)
        monkeypatch.setattr(O, "chunk_gradient", cg)
    elif mutation == "eta_dropped":
        def cg(vjp, params, k, v, eta, block=None):
            return vjp(params, O._f64(k), -O._f64(v), block=block)
        monkeypatch.setattr(O, "chunk_gradient", cg)
    elif mutation == "eta_squared":
        def cg(vjp, params, k, v, eta, block=None):
            e = O._f64(eta)
            return vjp(params, O._f64(k), -(e * e)[:, None] * O._f64(v), block=block)
        monkeypatch.setattr(O, "chunk_gradient", cg)
    elif mutation == "silu_grad_as_sigmoid":
        orig = O.vjp_swiglu

        def vj(params, x, cot, block=None):
            # recompute the pull-back with SiLU' replaced by sigmoid
            w1, w2, w3 = params
            a, b = x @ w1.T, x @ w3.T
            sg = O.sigmoid(a)
            du = cot @ w2
            return ((du * b * sg).T @ x, cot.T @ (a * sg * b), (du * a * sg).T @ x)
        monkeypatch.setattr(O, "vjp_swiglu", vj)
    elif mutation == "w2_transposed_in_vjp":
        orig = O.vjp_swiglu

        def vj(params, x, cot, block=None):
            w1, w2, w3 = params
            if w2.shape[0] == w2.shape[1]:
                return orig((w1, w2.T, w3), x, cot, block)
            return orig(params, x, cot, block)
        monkeypatch.setattr(O, "vjp_swiglu", vj)
    elif mutation == "forward_uses_w3_for_gate":
        def parts(x, w1, w3):
            a = x @ w3.T
            b = x @ w1.T
            sg = O.sigmoid(a)
            return a, b, a * sg * b, sg
        monkeypatch.setattr(O, "_swiglu_parts", parts)
    elif mutation == "renorm_uses_new_norm":
        def rr(w_old, w_new, eps=O.RENORM_EPS):
            n_new = np.sqrt((w_new * w_new).sum(axis=1, keepdims=True))
            return w_new / np.maximum(n_new, eps)
        monkeypatch.setattr(O, "renorm_rows", rr)
    elif mutation == "step_adds_gradient":
        monkeypatch.setattr(O, "gradient_step",
                            lambda params, grads: tuple(w + g for w, g in zip(params, grads)))
    assert not _pins_pass(), mutation
