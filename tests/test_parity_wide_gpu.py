"""GPU parity of the full-width fast weight (one head, d = 1024, hidden
h = 2048) against the fp64 oracle, through the C ABI.  The oracle is the same
shape-generic code as for the narrow heads; bounds are the bf16 ones (2e-2).

Gates as for the narrow heads: W_hat and O with renorm on and off, the step
Delta W = W_hat - W (renorm off), and the apply alone on the oracle's W_hat.
Token counts cross the 131,072-token block of the GEMM path (several partial
slots and a ragged last block)."""
import numpy as np
import pytest
import torch

import oracle
import reconstruction_lact_chunk_amd as zm
import workloads as WL
from test_parity_gpu import TOL, Inputs, check, host, sampled_units, say

pytestmark = pytest.mark.gpu
D, H_ = 1024, 2048
TOLB = TOL["bf16"]


def wide_inputs(n, seed, eta_scale=1.0):
    return Inputs(seed=seed, n=n, heads=1, d=D, h=H_, eta_scale=eta_scale)


def wide_parity(inp, check_apply=True, q_rows=None):
    """q_rows: read only the first q_rows queries (bounds the oracle's apply)."""
    t = inp.t
    n = t["k"].shape[0]
    nq = n if q_rows is None else min(n, q_rows)
    w0 = [inp.np("w1"), inp.np("w2"), inp.np("w3")]
    say(f"  wide update_apply n={n} queries={nq}")
    (a1, a2, a3), o_on = zm.update_apply(t["k"], t["v"], t["eta"], t["q"][:nq], t["w1"], t["w2"],
                                         t["w3"], renorm=True)
    (b1, b2, b3), o_off = zm.update_apply(t["k"], t["v"], t["eta"], t["q"][:nq], t["w1"],
                                          t["w2"], t["w3"], renorm=False)
    torch.cuda.synchronize()
    # one oracle gradient step, renorm applied to it for the renorm-on reference
    ref_off = oracle.update(inp.np("k"), inp.np("v"), inp.np("eta"), *w0, renorm=False)
    ref_on = tuple(oracle.renorm_rows(w[0], r[0])[None] for w, r in zip(w0, ref_off))
    for nm, a, b, r_on, r_off, w in zip(("W1", "W2", "W3"), (a1, a2, a3), (b1, b2, b3), ref_on,
                                        ref_off, w0):
        check(f"{nm}_hat renorm=True", host(a), r_on, TOLB)
        check(f"{nm}_hat renorm=False", host(b), r_off, TOLB)
        check(f"Delta {nm}", host(b) - w, r_off - w, TOLB)
    q = inp.np("q")[:nq]
    check("O renorm=True", host(o_on), oracle.apply(q, *ref_on), TOLB)
    check("O renorm=False", host(o_off), oracle.apply(q, *ref_off), TOLB)
    if check_apply:
        wt = [torch.tensor(x, dtype=torch.float32, device="cuda") for x in ref_on]
        og = host(zm.apply(t["q"][:nq], *wt))
        check("O (apply on oracle W_hat)", og, oracle.apply(q, *[host(x) for x in wt]), TOLB)


@pytest.mark.parametrize("n", [1, 1000, 3001])
def test_wide_small(n):
    say(f"case wide n={n}")
    wide_parity(wide_inputs(n, seed=41 + n, eta_scale=10.0))


@pytest.mark.parametrize("n", [131_077, 131_539])
def test_wide_block_boundary(n):
    # second block of 5 tokens (fewer than the 8 sub-blocks: all into slot 0)
    # or of 467 = 8 x 58 + 3 (batched sub-blocks plus a remainder)
    say(f"case wide n={n} (two token blocks, ragged second)")
    wide_parity(wide_inputs(n, seed=42), check_apply=False, q_rows=4096)


def test_wide_zero_eta_and_empty_chunk():
    say("case wide eta=0 / n_kv=0")
    inp = wide_inputs(700, seed=43)
    t = inp.t
    for renorm in (False, True):
        w = zm.update(t["k"], t["v"], torch.zeros_like(t["eta"]), t["w1"], t["w2"], t["w3"],
                      renorm=renorm)
        e = zm.update(t["k"][:0], t["v"][:0], t["eta"][:0], t["w1"], t["w2"], t["w3"],
                      renorm=renorm)
        torch.cuda.synchronize()
        for a, b, c in zip(w, e, (t["w1"], t["w2"], t["w3"])):
            assert torch.equal(a, c) and torch.equal(b, c)


def test_wide_streaming_and_chunked():
    say("case wide streaming 3 frames and chunked")
    inp = wide_inputs(3 * 1374, seed=44, eta_scale=10.0)
    t = inp.t
    offs = [0, 1374, 2748, 4122]
    w = [t["w1"].clone(), t["w2"].clone(), t["w3"].clone()]
    outs = [host(zm.stream_step(t["q"][s:e], t["k"][s:e], t["v"][s:e], t["eta"][s:e], *w,
                                renorm=True, order=zm.APPLY_THEN_UPDATE))
            for s, e in zip(offs, offs[1:])]
    wc = [t["w1"].clone(), t["w2"].clone(), t["w3"].clone()]
    oc = zm.chunked(t["q"], t["k"], t["v"], t["eta"], offs, *wc, renorm=True,
                    order=zm.UPDATE_THEN_APPLY)
    torch.cuda.synchronize()
    frames = [dict(q=inp.np("q")[s:e], k=inp.np("k")[s:e], v=inp.np("v")[s:e],
                   eta=inp.np("eta")[s:e]) for s, e in zip(offs, offs[1:])]
    w0 = (inp.np("w1"), inp.np("w2"), inp.np("w3"))
    rw, routs = oracle.stream(frames, *w0, renorm=True, order="apply_then_update")
    for i, (a, b) in enumerate(zip(outs, routs)):
        check(f"stream O frame {i}", a, b, TOLB)
    for nm, a, b in zip(("W1", "W2", "W3"), w, rw):
        check(f"stream {nm}", host(a), b, TOLB)
    cw, co = oracle.chunked(inp.np("q"), inp.np("k"), inp.np("v"), inp.np("eta"), offs, *w0,
                            order="update_then_apply", renorm=True)
    check("chunked O", host(oc), co, TOLB)
    for nm, a, b in zip(("W1", "W2", "W3"), wc, cw):
        check(f"chunked {nm}", host(a), b, TOLB)


@pytest.mark.parametrize("rule", [zm.STEP_GRADIENT, zm.STEP_NEWTON_SCHULZ])
def test_wide_bitwise_determinism(rule):
    say(f"case wide determinism n=70000 rule={rule}")
    inp = wide_inputs(70_000, seed=45)
    t = inp.t
    a, oa = zm.update_apply(t["k"], t["v"], t["eta"], t["q"], t["w1"], t["w2"], t["w3"],
                            renorm=True, step_rule=rule)
    b, ob = zm.update_apply(t["k"], t["v"], t["eta"], t["q"], t["w1"], t["w2"], t["w3"],
                            renorm=True, step_rule=rule)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(oa, ob)


def test_wide_fw100_full_size_sampled():
    """100 frames through one full-width head (two token blocks), checked on
    sampled hidden units (the oracle's restriction of the update to them) and
    on sampled queries read through the GPU's W_hat."""
    wl = WL.WORKLOADS["fw100"]
    say("case fw100 full size (sampled checks)")
    inp = Inputs(wl, 46)
    t = inp.t
    (g1, g2, g3), og = zm.update_apply(t["k"], t["v"], t["eta"], t["q"], t["w1"], t["w2"],
                                       t["w3"], renorm=True)
    (f1, f2, f3) = zm.update(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], renorm=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    J = sampled_units(H_, rng, blocks=32)   # 32 units, one in each run of 64
    k, v, eta = host(t["k"][:, 0]), host(t["v"][:, 0]), host(t["eta"][:, 0])
    w1, w2, w3 = host(t["w1"][0]), host(t["w2"][0]), host(t["w3"][0])
    s1, s2, s3 = oracle.update_rows_sampled(k, v, eta, w1, w2, w3, J)
    check("Delta W1[J]", host(f1[0])[J] - w1[J], s1 - w1[J], TOLB)
    check("Delta W3[J]", host(f3[0])[J] - w3[J], s3 - w3[J], TOLB)
    check("Delta W2[:,J]", host(f2[0])[:, J] - w2[:, J], s2 - w2[:, J], TOLB)
    check("W1_hat[J]", host(g1[0])[J], oracle.renorm_rows(w1[J], s1), TOLB)
    check("W3_hat[J]", host(g3[0])[J], oracle.renorm_rows(w3[J], s3), TOLB)
    ref = oracle.renorm_rows(host(t["w2"][0]), host(f2[0]))
    check("W2_hat vs renorm(W2')", host(g2[0]), ref, 1e-5)
    idx = torch.as_tensor(np.sort(rng.choice(wl.n_q, 1024, replace=False)), device="cuda")
    ref = oracle.apply(host(t["q"][idx]), host(g1), host(g2), host(g3))
    check("O sampled (1024 queries)", host(og[idx]), ref, TOLB)


@pytest.mark.parametrize("n", [1, 3001, 20_000])
def test_wide_newton_schulz(n):
    """The review's update display after Eq. (3) on the full-width head: the
    orthonormalisation of each 2048 x 1024 gradient as batched split-bf16 GEMMs."""
    say(f"case wide Newton-Schulz n={n}")
    inp = wide_inputs(n, seed=47 + n)
    t = inp.t
    w0 = [inp.np("w1"), inp.np("w2"), inp.np("w3")]
    ns = zm.STEP_NEWTON_SCHULZ
    (a1, a2, a3), o = zm.update_apply(t["k"], t["v"], t["eta"], t["q"], t["w1"], t["w2"], t["w3"],
                                      renorm=True, step_rule=ns)
    (b1, b2, b3) = zm.update(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], renorm=False,
                             step_rule=ns)
    torch.cuda.synchronize()
    ref_off = oracle.update(inp.np("k"), inp.np("v"), inp.np("eta"), *w0, renorm=False,
                            step="newton_schulz")
    ref_on = tuple(oracle.renorm_rows(w[0], r[0])[None] for w, r in zip(w0, ref_off))
    for nm, a, b, r_on, r_off, w in zip(("W1", "W2", "W3"), (a1, a2, a3), (b1, b2, b3), ref_on,
                                        ref_off, w0):
        check(f"Delta {nm} = -NS(g)", host(b) - w, r_off - w, TOLB)
        assert 0.4 < np.linalg.norm((r_off - w)[0], 2) < 1.3
        check(f"{nm}_hat renorm=True", host(a), r_on, TOLB)
    check("O renorm=True", host(o), oracle.apply(inp.np("q"), *ref_on), TOLB)


@pytest.mark.parametrize("rule", ["gradient", "newton_schulz"])
def test_wide_two_heads(rule):
    """Two full-width heads: the forward products per head (the [W1; W3]
    single-GEMM form needs one head) and a batch of six matrices in the
    Newton-Schulz iteration."""
    say(f"case wide two heads rule={rule}")
    inp = Inputs(seed=48, n=900, heads=2, d=D, h=H_, eta_scale=10.0)
    t = inp.t
    code = zm.STEP_NEWTON_SCHULZ if rule == "newton_schulz" else zm.STEP_GRADIENT
    w0 = [inp.np("w1"), inp.np("w2"), inp.np("w3")]
    (a1, a2, a3), o = zm.update_apply(t["k"], t["v"], t["eta"], t["q"], t["w1"], t["w2"], t["w3"],
                                      renorm=False, step_rule=code)
    torch.cuda.synchronize()
    ref, ro = oracle.update_apply(inp.np("k"), inp.np("v"), inp.np("eta"), inp.np("q"), *w0,
                                  renorm=False, step=rule)
    for nm, a, b, w in zip(("W1", "W2", "W3"), (a1, a2, a3), ref, w0):
        check(f"Delta {nm}", host(a) - w, b - w, TOLB)
    check("O", host(o), ro, TOLB)
