"""Pins of the oracle's Newton-Schulz update rule against facts that do not come
from the oracle's own iteration.

The step is W' = W - NewtonSchulz(g) (review of ZipMap, kimjy99.github.io,
the update display after Eq. (3)).  What fixes the iteration independently:
  * an odd matrix polynomial X -> a X + b (X X^T) X + c (X X^T)^2 X keeps the
    singular vectors and maps each singular value s to a s + b s^3 + c s^5,
    so k steps equal U diag(p^k(s / ||s||)) V^T from numpy's SVD;
  * the textbook cubic (1.5, -0.5, 0) converges to the polar factor U V^T;
  * Muon's quintic lands normalised singular values in [1e-2, 1] inside a
    band around 1 after five steps (the reason for its coefficients);
  * sign, scale and transpose invariances, and 0 -> 0;
  * the wiring into the update (sign, which matrix, renorm after the step) is
    checked against a gradient taken by central finite differences of the
    virtual loss, not by the oracle's chain rule.
"""
import math

import numpy as np
import pytest

from oracle import ttt_oracle as O

MUON = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


def rel(x, ref):
    return float(np.abs(np.asarray(x) - ref).max() / max(np.abs(ref).max(), 1e-300))


def ns_by_svd(g, steps, coeffs):
    """k steps of the odd polynomial acting on the singular values only."""
    u, s, vt = np.linalg.svd(np.asarray(g, dtype=np.float64), full_matrices=False)
    a, b, c = coeffs
    x = s / max(math.sqrt(float((s * s).sum())), O.RENORM_EPS)
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return (u * x) @ vt


def matrix_with_singular_values(m, n, svals, seed):
    r = np.random.default_rng(seed)
    u, _ = np.linalg.qr(r.normal(size=(m, m)))
    v, _ = np.linalg.qr(r.normal(size=(n, n)))
    k = min(m, n)
    return (u[:, :k] * np.asarray(svals)) @ v[:, :k].T


@pytest.mark.parametrize("shape", [(12, 5), (5, 12), (7, 7), (1, 6), (6, 1)])
@pytest.mark.parametrize("coeffs", [MUON, CUBIC, (2.0, -1.3, 0.4)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_ns_acts_on_singular_values(shape, coeffs, steps):
    g = np.random.default_rng(hash((shape, steps)) % 1000).normal(size=shape)
    got = O.newton_schulz(g, steps=steps, coeffs=coeffs)
    assert rel(got, ns_by_svd(g, steps, coeffs)) < 1e-12


def test_ns_default_is_five_muon_steps():
    g = np.random.default_rng(5).normal(size=(9, 4))
    np.testing.assert_array_equal(O.newton_schulz(g), O.newton_schulz(g, steps=5, coeffs=MUON))
    assert rel(O.newton_schulz(g), ns_by_svd(g, 5, MUON)) < 1e-12


@pytest.mark.parametrize("shape", [(10, 4), (4, 10), (6, 6)])
def test_cubic_converges_to_the_polar_factor(shape):
    svals = np.linspace(0.2, 1.0, min(shape))
    g = matrix_with_singular_values(*shape, svals, seed=7)
    u, _, vt = np.linalg.svd(g, full_matrices=False)
    got = O.newton_schulz(g, steps=40, coeffs=CUBIC)
    assert rel(got, u @ vt) < 1e-12
    small = got @ got.T if shape[0] <= shape[1] else got.T @ got
    assert np.abs(small - np.eye(min(shape))).max() < 1e-12


def test_muon_quintic_lands_singular_values_near_one():
    # normalised singular values spread over [1e-2, 1] (times the norm)
    svals = np.logspace(-2, 0, 48)
    g = matrix_with_singular_values(48, 96, svals, seed=8)
    s_in = np.linalg.svd(g / np.linalg.norm(g), compute_uv=False)
    out = np.linalg.svd(O.newton_schulz(g), compute_uv=False)
    assert s_in.min() < 0.01
    assert out.min() > 0.6 and out.max() < 1.25


def test_ns_invariances():
    g = np.random.default_rng(9).normal(size=(8, 5))
    x = O.newton_schulz(g)
    assert rel(O.newton_schulz(-g), -x) < 1e-14
    assert rel(O.newton_schulz(3.7 * g), x) < 1e-13
    assert rel(O.newton_schulz(g.T), x.T) < 1e-13
    np.testing.assert_array_equal(O.newton_schulz(np.zeros((8, 5))), np.zeros((8, 5)))


# ---------------------------------------------------------------------------
# The step that uses it
# ---------------------------------------------------------------------------
def _fd_gradient(k, v, eta, w, step=1e-6):
    def loss(ws):
        return O.virtual_loss(k[:, None], v[:, None], eta[:, None], ws[0][None], ws[1][None],
                              ws[2][None])[0]
    out = []
    for m in range(3):
        num = np.zeros_like(w[m])
        for idx in np.ndindex(*w[m].shape):
            wp = [x.copy() for x in w]
            wm = [x.copy() for x in w]
            wp[m][idx] += step
            wm[m][idx] -= step
            num[idx] = (loss(wp) - loss(wm)) / (2 * step)
        out.append(num)
    return out


def _problem(n, d, h, seed):
    r = np.random.default_rng(seed)
    k = r.normal(size=(n, d)) / math.sqrt(d)
    v = r.normal(size=(n, d)) / math.sqrt(d)
    eta = 0.5 * r.random(n)
    w = [r.normal(size=(h, d)) / math.sqrt(d), r.normal(size=(d, h)) / math.sqrt(h),
         r.normal(size=(h, d)) / math.sqrt(d)]
    return k, v, eta, w


def test_ns_step_follows_the_finite_difference_gradient():
    k, v, eta, w = _problem(6, 4, 7, seed=11)
    g = _fd_gradient(k, v, eta, w)
    new = O.update_head(k, v, eta, *w, renorm=False, step="newton_schulz")
    for m in range(3):
        assert new[m].shape == w[m].shape
        assert rel(w[m] - new[m], ns_by_svd(g[m], 5, MUON)) < 1e-6, m


def test_ns_step_then_row_renorm():
    k, v, eta, w = _problem(6, 4, 7, seed=12)
    g = _fd_gradient(k, v, eta, w)
    new = O.update_head(k, v, eta, *w, renorm=True, step="newton_schulz")
    for m in range(3):
        stepped = w[m] - ns_by_svd(g[m], 5, MUON)
        np.testing.assert_allclose(np.linalg.norm(new[m], axis=1), np.linalg.norm(w[m], axis=1),
                                   rtol=1e-12)
        direction = stepped / np.linalg.norm(stepped, axis=1, keepdims=True)
        assert rel(new[m] / np.linalg.norm(new[m], axis=1, keepdims=True), direction) < 1e-6


@pytest.mark.parametrize("renorm", [False, True])
def test_ns_zero_eta_leaves_weights_bitwise_unchanged(renorm):
    k, v, eta, w = _problem(9, 5, 6, seed=13)
    new = O.update_head(k, v, 0.0 * eta, *w, renorm=renorm, step="newton_schulz")
    for x, y in zip(new, w):
        np.testing.assert_array_equal(x, y)


def test_ns_multi_head_matches_per_head():
    r = np.random.default_rng(14)
    n, heads, d, h = 10, 3, 4, 6
    k = r.normal(size=(n, heads, d))
    v = r.normal(size=(n, heads, d))
    eta = r.random((n, heads))
    w1, w3 = r.normal(size=(heads, h, d)), r.normal(size=(heads, h, d))
    w2 = r.normal(size=(heads, d, h))
    allh = O.update(k, v, eta, w1, w2, w3, renorm=True, step="newton_schulz")
    for hd in range(heads):
        one = O.update_head(k[:, hd], v[:, hd], eta[:, hd], w1[hd], w2[hd], w3[hd], renorm=True,
                            step="newton_schulz")
        for x, y in zip(allh, one):
            np.testing.assert_array_equal(x[hd], y)


def test_unknown_step_rule_is_rejected():
    k, v, eta, w = _problem(3, 2, 3, seed=15)
    with pytest.raises(ValueError):
        O.update_head(k, v, eta, *w, step="adam")


# ---------------------------------------------------------------------------
# Planted mistakes in the iteration must fail a pin above
# ---------------------------------------------------------------------------
def _mutant(kind):
    def ns(g, steps=O.NS_STEPS, coeffs=O.MUON_NS_COEFFS, eps=O.RENORM_EPS):
        x = np.asarray(g, dtype=np.float64)
        if kind != "no_normalisation":
            x = x / max(np.sqrt((x * x).sum()), eps)
        a, b, c = coeffs
        if kind == "sign_of_b":
            b = -b
        with np.errstate(all="ignore"):  # the unnormalised mutant overflows
            for _ in range(1 if kind == "one_step_only" else steps):
                gram = x @ x.T
                gx = gram @ x
                x = a * x + b * gx + c * (gram @ gx)
        return x
    return ns


@pytest.mark.parametrize("kind", ["no_normalisation", "sign_of_b", "one_step_only"])
def test_planted_iteration_mistakes_are_caught(monkeypatch, kind):
    monkeypatch.setattr(O, "newton_schulz", _mutant(kind))
    with pytest.raises(AssertionError):
        test_ns_default_is_five_muon_steps()


def test_planted_step_sign_is_caught(monkeypatch):
    orig = O.newton_schulz
    monkeypatch.setattr(O, "newton_schulz", lambda g, **kw: -orig(g, **kw))
    with pytest.raises(AssertionError):
        test_ns_step_follows_the_finite_difference_gradient()
