"""GPU parity of the whole layer (input projections with the per-token rate,
update, apply, output gate; zm_ttt_layer) against the fp64 oracle's layer.
Both sides start from the same bf16 input tokens and slow weights; the GPU
rounds q, k, v, o' and W_g o' to bf16 between its steps, which the bf16 bound
(2e-2) covers."""
import numpy as np
import pytest
import torch

import oracle
import reconstruction_lact_chunk_amd as zm
import workloads as WL
from test_parity_gpu import TOL, check, host, sampled_units, say

pytestmark = pytest.mark.gpu
TOLB = TOL["bf16"]


def run(n, heads, d, h, seed, renorm, step="gradient", eta_scale=0.01):
    say(f"  layer n={n} H={heads} d={d} h={h} renorm={renorm} step={step}")
    x, w_in, w_gate, gamma = WL.make_layer_tensors(n, heads, d, seed, "cuda")
    w = WL.make_weights(heads, d, h, seed, "cuda")
    rule = zm.STEP_NEWTON_SCHULZ if step == "newton_schulz" else zm.STEP_GRADIENT
    (g1, g2, g3), o = zm.layer(x, w_in, w_gate, gamma, *w, eta_scale=eta_scale, renorm=renorm,
                               step_rule=rule)
    torch.cuda.synchronize()
    (r1, r2, r3), ro = oracle.layer(host(x), host(w_in), host(w_gate), host(gamma),
                                    *[host(t) for t in w], eta_scale=eta_scale, renorm=renorm,
                                    step=step)
    for nm, a, b, w0 in zip(("W1", "W2", "W3"), (g1, g2, g3), (r1, r2, r3), w):
        check(f"{nm}_hat", host(a), b, TOLB)
        if not renorm:
            check(f"Delta {nm}", host(a) - host(w0), b - host(w0), TOLB)
    check("o", host(o), ro, TOLB)
    return o


@pytest.mark.parametrize("renorm", [False, True])
def test_layer_8_heads(renorm):
    say(f"case layer 8 x 128/256 renorm={renorm}")
    run(2748, 8, 128, 256, seed=51, renorm=renorm, eta_scale=1.0)


@pytest.mark.parametrize("d,h", [(64, 128), (128, 128)])
def test_layer_other_head_shapes(d, h):
    say(f"case layer H=4 d={d} h={h}")
    run(1001, 4, d, h, seed=52, renorm=True, eta_scale=1.0)


def test_layer_newton_schulz():
    say("case layer with the Newton-Schulz rule")
    run(1374, 8, 128, 256, seed=53, renorm=True, step="newton_schulz")


def test_layer_full_width_head():
    say("case layer with one full-width head (1024 / 2048)")
    run(1374, 1, 1024, 2048, seed=54, renorm=True, eta_scale=1.0)


def test_layer_f8_and_empty():
    wl = WL.WORKLOADS["f8"]
    say("case layer f8 (8 frames x 1374)")
    run(wl.n_kv, 8, 128, 256, seed=55, renorm=True)
    say("case layer n=0")
    x, w_in, w_gate, gamma = WL.make_layer_tensors(4, 8, 128, 56, "cuda")
    w = WL.make_weights(8, 128, 256, 56, "cuda")
    new, o = zm.layer(x[:0], w_in, w_gate, gamma, *w, renorm=True)
    torch.cuda.synchronize()
    assert o.shape == (0, 1024)
    for a, b in zip(new, w):
        assert torch.equal(a, b)


def test_layer700_sampled():
    """The benchmark's whole-layer workload (961,800 tokens): the oracle
    recomputes the projections for every token (cheap) and then checks sampled
    hidden units of W_hat and sampled outputs, whose gate needs only the token
    and W_hat."""
    wl = WL.WORKLOADS["layer700"]
    n = wl.n_kv
    say("case layer700 full size (sampled checks)")
    x, w_in, w_gate, gamma = WL.make_layer_tensors(n, 8, 128, 4, "cuda")
    w = WL.make_weights(8, 128, 256, 4, "cuda")
    (g1, g2, g3), o = zm.layer(x, w_in, w_gate, gamma, *w, renorm=False)
    torch.cuda.synchronize()
    xs, wi = host(x), host(w_in)
    q, k, v, eta = oracle.project(xs, wi, 8, 128, 0.01)
    rng = np.random.default_rng(2)
    for hd in range(8):
        J = sampled_units(256, rng)
        w1, w2, w3 = host(w[0][hd]), host(w[1][hd]), host(w[2][hd])
        s1, s2, s3 = oracle.update_rows_sampled(k[:, hd], v[:, hd], eta[:, hd], w1, w2, w3, J)
        check(f"head {hd} Delta W1[J]", host(g1[hd])[J] - w1[J], s1 - w1[J], TOLB)
        check(f"head {hd} Delta W2[:,J]", host(g2[hd])[:, J] - w2[:, J], s2 - w2[:, J], TOLB)
        check(f"head {hd} Delta W3[J]", host(g3[hd])[J] - w3[J], s3 - w3[J], TOLB)
    idx = np.sort(rng.choice(n, 2048, replace=False))
    op = oracle.apply(q[idx], host(g1), host(g2), host(g3)).reshape(len(idx), -1)
    ref = oracle.output_gate(op, host(w_gate), host(gamma))
    check("o sampled (2048 tokens)", host(o[torch.as_tensor(idx, device="cuda")]), ref, TOLB)
