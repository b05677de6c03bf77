"""GPU parity of the Newton-Schulz update rule (W' = W - NewtonSchulz(g), then
the optional row renorm) against the fp64 oracle, through the C ABI.

With this rule the step has singular values near 1 whatever the rates, so
Delta W = W_hat - W (renorm off) is of the size of W itself and checks the
orthonormalisation directly.  Bounds as for the plain step: 2e-2 for bf16 io
(split-bf16 products inside the iteration), 1e-4 for fp32 io.
"""
import numpy as np
import pytest
import torch

import oracle
import reconstruction_lact_chunk_amd as zm
import workloads as WL
from test_parity_gpu import TOL, Inputs, check, host, rel, say

pytestmark = pytest.mark.gpu

NS = zm.STEP_NEWTON_SCHULZ


def gpu_update_apply(inp, renorm, q=None):
    t = inp.t
    q = t["q"] if q is None else q
    say(f"  update_apply[NS] n_kv={t['k'].shape[0]} n_q={q.shape[0]} H={t['k'].shape[1]} "
        f"d={t['k'].shape[2]} h={t['w1'].shape[1]} io={t['k'].dtype} renorm={renorm}")
    w, o = zm.update_apply(t["k"], t["v"], t["eta"], q, t["w1"], t["w2"], t["w3"], renorm=renorm,
                           step_rule=NS)
    torch.cuda.synchronize()
    return [host(x) for x in w], host(o)


def oracle_update_apply(inp, renorm):
    return oracle.update_apply(inp.np("k"), inp.np("v"), inp.np("eta"), inp.np("q"),
                               inp.np("w1"), inp.np("w2"), inp.np("w3"), renorm=renorm,
                               step="newton_schulz")


def ns_parity(inp, tol):
    w0 = [inp.np("w1"), inp.np("w2"), inp.np("w3")]
    for renorm in (False, True):
        wg, og = gpu_update_apply(inp, renorm)
        ref, ro = oracle_update_apply(inp, renorm)
        for nm, a, b, w in zip(("W1", "W2", "W3"), wg, ref, w0):
            check(f"{nm}_hat renorm={renorm}", a, b, tol)
            if not renorm:
                check(f"Delta {nm} = -NS(g)", a - w, b - w, tol)
                # the step's nonzero singular values sit near 1 (Muon's quintic
                # puts them in [0.47, 1.2]), so the check above is not vacuous
                for step in b - w:    # per head
                    assert 0.4 < np.linalg.norm(step, 2) < 1.3
        check(f"O renorm={renorm}", og, ro, tol)


@pytest.mark.parametrize("d,h", [(64, 128), (64, 256), (128, 128), (128, 256)])
def test_ns_fp32_shapes(d, h):
    say(f"case NS fp32 d={d} h={h} n=777 H=3")
    ns_parity(Inputs(seed=21, n=777, heads=3, d=d, h=h, io="f32"), TOL["f32"])


@pytest.mark.parametrize("d,h", [(64, 128), (64, 256), (128, 128), (128, 256)])
def test_ns_bf16_shapes(d, h):
    say(f"case NS bf16 d={d} h={h} n=1001 H=4")
    ns_parity(Inputs(seed=22, n=1001, heads=4, d=d, h=h), TOL["bf16"])


def test_ns_tiny_fp32():
    say("case NS tiny fp32")
    ns_parity(Inputs(WL.WORKLOADS["tiny"], 23), TOL["f32"])


def test_ns_f8_config():
    say("case NS f8 (8 frames x 1374)")
    ns_parity(Inputs(WL.WORKLOADS["f8"], 24), TOL["bf16"])


@pytest.mark.parametrize("n", [1, 33])
def test_ns_tiny_chunks(n):
    # one or a few tokens: g has rank <= n and most singular values are 0
    say(f"case NS n={n}")
    ns_parity(Inputs(seed=25 + n, n=n, heads=2), TOL["bf16"])


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("renorm", [False, True])
def test_ns_zero_eta_and_empty_chunk_leave_weights_unchanged(io, renorm):
    say(f"case NS eta=0 / n_kv=0 io={io} renorm={renorm}")
    inp = Inputs(seed=27, n=300, io=io)
    t = inp.t
    w = zm.update(t["k"], t["v"], torch.zeros_like(t["eta"]), t["w1"], t["w2"], t["w3"],
                  renorm=renorm, step_rule=NS)
    torch.cuda.synchronize()
    for a, b in zip(w, (t["w1"], t["w2"], t["w3"])):
        assert torch.equal(a, b)
    empty = t["k"][:0]
    w = zm.update(empty, empty, t["eta"][:0], t["w1"], t["w2"], t["w3"], renorm=renorm,
                  step_rule=NS)
    torch.cuda.synchronize()
    for a, b in zip(w, (t["w1"], t["w2"], t["w3"])):
        assert torch.equal(a, b)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_ns_streaming_frames(io):
    wl = WL.Workload("stream3", 3, 518, 8, 128, 256, io, True, streaming=True)
    say(f"case NS streaming 3 frames io={io}")
    inp = Inputs(wl, 28)
    t = inp.t
    w = [t["w1"].clone(), t["w2"].clone(), t["w3"].clone()]
    outs = []
    for (s, e) in WL.frame_slices(wl):
        outs.append(host(zm.stream_step(t["q"][s:e], t["k"][s:e], t["v"][s:e], t["eta"][s:e], *w,
                                        renorm=True, order=zm.APPLY_THEN_UPDATE, step_rule=NS)))
    torch.cuda.synchronize()
    frames = [dict(q=inp.np("q")[s:e], k=inp.np("k")[s:e], v=inp.np("v")[s:e],
                   eta=inp.np("eta")[s:e]) for (s, e) in WL.frame_slices(wl)]
    rw, routs = oracle.stream(frames, inp.np("w1"), inp.np("w2"), inp.np("w3"), renorm=True,
                              order="apply_then_update", step="newton_schulz")
    for i, (a, b) in enumerate(zip(outs, routs)):
        check(f"O frame {i}", a, b, TOL[io])
    for nm, a, b in zip(("W1", "W2", "W3"), w, rw):
        check(f"{nm} after 3 frames", host(a), b, TOL[io])


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_ns_bitwise_determinism(io):
    say(f"case NS determinism io={io}")
    inp = Inputs(seed=29, n=5000, io=io)
    t = inp.t
    a = zm.update(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], renorm=True, step_rule=NS)
    b = zm.update(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], renorm=True, step_rule=NS)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_ns_f700_full_size_one_head():
    """The 700-frame chunk with the Newton-Schulz rule, in the launch
    configuration of the full layer (all 8 heads on the GPU).  The iteration
    mixes every hidden unit, so the oracle recomputes whole heads; head 0 and
    head 7 are checked, with renorm off (the step itself) and on."""
    wl = WL.WORKLOADS["f700"]
    say("case NS f700 full size seed=4 (heads 0 and 7)")
    inp = Inputs(wl, 4)
    t = inp.t
    (f1, f2, f3) = zm.update(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], renorm=False,
                             step_rule=NS)
    (g1, g2, g3) = zm.update(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], renorm=True,
                             step_rule=NS)
    torch.cuda.synchronize()
    for hd in (0, 7):
        k, v, eta = host(t["k"][:, hd]), host(t["v"][:, hd]), host(t["eta"][:, hd])
        w = [host(t["w1"][hd]), host(t["w2"][hd]), host(t["w3"][hd])]
        ref = oracle.update_head(k, v, eta, *w, renorm=False, step="newton_schulz")
        for nm, a, b, w0 in zip(("W1", "W2", "W3"), (f1, f2, f3), ref, w):
            check(f"head {hd} Delta {nm}", host(a[hd]) - w0, b - w0, TOL["bf16"])
        for nm, a, b, w0 in zip(("W1", "W2", "W3"), (g1, g2, g3), ref, w):
            check(f"head {hd} {nm}_hat", host(a[hd]), oracle.renorm_rows(w0, b), TOL["bf16"])
