"""Pins of the oracle's steps around the TTT layer: input projections with the
per-token rate, and the output gate o = RMSNorm(o') * SiLU(W_g o') (review of
ZipMap, Eq. (5)), against hand-computed values, invariants and per-token loops
that do not use the oracle's own code."""
import math

import numpy as np
import pytest

from oracle import ttt_oracle as O


def test_rmsnorm_hand_values():
    # x = (3, 4): mean of squares 12.5
    got = O.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), eps=0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(got, [[3 / r, 8 / r]], rtol=1e-15)
    # eps enters under the root
    got = O.rmsnorm(np.array([[1.0, 1.0]]), np.ones(2), eps=3.0)
    np.testing.assert_allclose(got, [[0.5, 0.5]], rtol=1e-15)


def test_rmsnorm_scale_invariance_and_unit_rms():
    x = np.random.default_rng(0).normal(size=(5, 16))
    a = O.rmsnorm(x, np.ones(16), eps=0.0)
    np.testing.assert_allclose(O.rmsnorm(7.5 * x, np.ones(16), eps=0.0), a, rtol=1e-13)
    np.testing.assert_allclose((a * a).mean(axis=1), 1.0, rtol=1e-13)


def test_output_gate_per_token_loop():
    r = np.random.default_rng(1)
    n, w = 4, 6
    op, wg, gamma = r.normal(size=(n, w)), r.normal(size=(w, w)), r.normal(size=w)
    got = O.output_gate(op, wg, gamma, eps=1e-6)
    for i in range(n):
        rms = math.sqrt(sum(t * t for t in op[i]) / w + 1e-6)
        for j in range(w):
            g = sum(wg[j, c] * op[i, c] for c in range(w))
            want = op[i, j] / rms * gamma[j] * (g / (1.0 + math.exp(-g)))
            assert abs(got[i, j] - want) < 1e-12
    assert np.all(O.output_gate(op, np.zeros((w, w)), gamma) == 0.0)


def test_projection_layout_per_token_loop():
    r = np.random.default_rng(2)
    n, heads, d, d_in = 3, 2, 4, 5
    x = r.normal(size=(n, d_in))
    w_in = r.normal(size=(3 * heads * d + heads, d_in))
    q, k, v, eta = O.project(x, w_in, heads, d, eta_scale=0.01)
    for i in range(n):
        for which, t in enumerate((q, k, v)):
            for hd in range(heads):
                for c in range(d):
                    row = which * heads * d + hd * d + c
                    assert abs(t[i, hd, c] - sum(w_in[row, m] * x[i, m] for m in range(d_in))) < 1e-12
        for hd in range(heads):
            z = sum(w_in[3 * heads * d + hd, m] * x[i, m] for m in range(d_in))
            assert abs(eta[i, hd] - 0.01 / (1.0 + math.exp(-z))) < 1e-15
    assert np.all(eta > 0) and np.all(eta < 0.01)


def test_layer_is_the_composition_of_its_steps():
    r = np.random.default_rng(3)
    n, heads, d, h = 9, 2, 4, 6
    x = r.normal(size=(n, heads * d))
    w_in = r.normal(size=(3 * heads * d + heads, heads * d)) / math.sqrt(heads * d)
    w_gate = r.normal(size=(heads * d, heads * d))
    gamma = r.normal(size=heads * d)
    w1, w3 = r.normal(size=(heads, h, d)), r.normal(size=(heads, h, d))
    w2 = r.normal(size=(heads, d, h))
    new, o = O.layer(x, w_in, w_gate, gamma, w1, w2, w3, eta_scale=0.05, renorm=True)
    q, k, v, eta = O.project(x, w_in, heads, d, 0.05)
    ref_w = O.update(k, v, eta, w1, w2, w3, renorm=True)
    for a, b in zip(new, ref_w):
        np.testing.assert_array_equal(a, b)
    op = O.apply(q, *ref_w).reshape(n, -1)
    np.testing.assert_array_equal(o, O.output_gate(op, w_gate, gamma))
    # heads are laid side by side in o': head hd owns columns hd*d .. hd*d + d - 1
    np.testing.assert_array_equal(op[:, d:2 * d], O.apply(q[:, 1:2], *[w[1:2] for w in ref_w])[:, 0])


@pytest.mark.parametrize("mutation", ["eps_outside_root", "gate_on_input"])
def test_planted_gate_mistakes_are_caught(monkeypatch, mutation):
    if mutation == "eps_outside_root":
        monkeypatch.setattr(O, "rmsnorm", lambda x, g, eps=O.RMS_EPS: x / (
            np.sqrt((x * x).mean(axis=-1, keepdims=True)) + eps) * g)
        with pytest.raises(AssertionError):
            test_rmsnorm_hand_values()
    else:
        monkeypatch.setattr(O, "output_gate", lambda op, wg, gamma, eps=O.RMS_EPS: O.rmsnorm(
            op, gamma, eps) * O.silu(op))
        with pytest.raises(AssertionError):
            test_output_gate_per_token_loop()
