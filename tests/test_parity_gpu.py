"""GPU parity of the HIP library against the fp64 oracle.

Every case draws seeded inputs from workloads.py on the GPU, runs the C ABI
through the binding, copies the inputs to the host for the oracle and
compares element by element with rel(x, ref) = max|x - ref| / max|ref| per
tensor.  Bounds: 2e-2 for bf16 io, 1e-4 for fp32 io.

Because one update step moves the weights only a little at the workloads'
rates, the updated weights alone would pass even with a wrong step.  So the
step itself, Delta W = W_hat - W with renorm off, is checked to the same
bounds, the apply is also checked on the oracle's weights, and a hot-eta case
(rates x100) makes the step comparable to W.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import reconstruction_lact_chunk_amd as zm
import workloads as WL

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)) / max(den, 1e-300))


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


class Inputs:
    """Seeded inputs on the GPU, either of a named workload or of a custom
    token count (for ragged and edge cases)."""

    def __init__(self, wl=None, seed=1, eta_scale=1.0, n=None, heads=8, d=128, h=256, io="bf16",
                 device="cuda"):
        if wl is not None:
            self.t = WL.make_inputs(wl, seed, device, eta_scale)
            return
        self.t = {
            "q": WL.make_tokens(n, heads, d, io, seed, device, WL.STREAM_Q),
            "k": WL.make_tokens(n, heads, d, io, seed, device, WL.STREAM_K),
            "v": WL.make_tokens(n, heads, d, io, seed, device, WL.STREAM_V),
            "eta": WL.make_eta(n, heads, seed, device, eta_scale),
        }
        self.t["w1"], self.t["w2"], self.t["w3"] = WL.make_weights(heads, d, h, seed, device)

    def __getitem__(self, k):
        return self.t[k]

    def np(self, k):
        return host(self.t[k])


def sampled_units(d_hidden, rng, block=16, blocks=None):
    """Hidden units for a sampled check: one drawn from each run of `block`
    consecutive units (every wave's 16-unit block of both 128-unit workgroup
    slices at hidden 256), or from `blocks` equal runs when given."""
    if blocks is not None:
        block = d_hidden // blocks
    starts = np.arange(0, d_hidden, block)
    return np.sort(starts + rng.integers(0, block, len(starts)))


def check(name, x, ref, tol):
    r = rel(x, ref)
    say(f"    {name}: rel {r:.3e} (tol {tol:.0e})")
    assert r <= tol, (name, r, tol)
    return r


def run_update_apply(inp, renorm, q=None):
    t = inp.t
    q = t["q"] if q is None else q
    say(f"  update_apply n_kv={t['k'].shape[0]} n_q={q.shape[0]} H={t['k'].shape[1]} "
        f"d={t['k'].shape[2]} h={t['w1'].shape[1]} io={t['k'].dtype} renorm={renorm}")
    w, o = zm.update_apply(t["k"], t["v"], t["eta"], q, t["w1"], t["w2"], t["w3"], renorm=renorm)
    torch.cuda.synchronize()
    return [host(x) for x in w], host(o)


def oracle_update_apply(inp, renorm):
    return oracle.update_apply(inp.np("k"), inp.np("v"), inp.np("eta"), inp.np("q"),
                               inp.np("w1"), inp.np("w2"), inp.np("w3"), renorm=renorm)


def full_parity(inp, tol, check_delta=True):
    """W_hat and O with renorm on; Delta W with renorm off; apply on oracle W."""
    w0 = [inp.np("w1"), inp.np("w2"), inp.np("w3")]
    for renorm in (True, False):
        wg, og = run_update_apply(inp, renorm)
        (r1, r2, r3), ro = oracle_update_apply(inp, renorm)
        for nm, a, b in zip(("W1", "W2", "W3"), wg, (r1, r2, r3)):
            check(f"{nm}_hat renorm={renorm}", a, b, tol)
        check(f"O renorm={renorm}", og, ro, tol)
        if check_delta and not renorm:
            for nm, a, b, w in zip(("W1", "W2", "W3"), wg, (r1, r2, r3), w0):
                check(f"Delta {nm}", a - w, b - w, tol)
    # apply alone, through the oracle's updated weights (fp32-rounded)
    (r1, r2, r3), ro = oracle_update_apply(inp, True)
    wt = [torch.tensor(x, dtype=torch.float32, device="cuda") for x in (r1, r2, r3)]
    say("  apply (oracle weights)")
    og = host(zm.apply(inp["q"], *wt))
    ref = oracle.apply(inp.np("q"), *[x.cpu().double().numpy() for x in wt])
    check("O (apply on oracle W_hat)", og, ref, tol)


# ---------------------------------------------------------------------------
def test_tiny_fp32():
    say("case tiny fp32 seed=1")
    full_parity(Inputs(WL.WORKLOADS["tiny"], 1), TOL["f32"])


@pytest.mark.parametrize("d,h", [(64, 128), (64, 256), (128, 128), (128, 256)])
def test_fp32_shapes_multi_head(d, h):
    say(f"case fp32 d={d} h={h} n=777 H=3")
    full_parity(Inputs(seed=11, n=777, heads=3, d=d, h=h, io="f32"), TOL["f32"])


@pytest.mark.parametrize("d,h", [(64, 128), (64, 256), (128, 128), (128, 256)])
def test_bf16_shapes_ragged(d, h):
    say(f"case bf16 d={d} h={h} n=1001 H=4")
    full_parity(Inputs(seed=12, n=1001, heads=4, d=d, h=h), TOL["bf16"])


def test_tiny_shape_bf16():
    say("case tiny shape in bf16")
    wl = WL.Workload("tiny_bf16", 4, 70, 1, 64, 128, "bf16", False)
    full_parity(Inputs(wl, 2), TOL["bf16"])


def test_f8_config():
    say("case f8 (8 frames x 1374) seed=2")
    full_parity(Inputs(WL.WORKLOADS["f8"], 2), TOL["bf16"])


def test_f100_config_with_target_view():
    wl = WL.WORKLOADS["f100"]
    say("case f100 (100 frames + 1374 target-view queries) seed=3")
    inp = Inputs(wl, 3)
    wg, og = run_update_apply(inp, True)
    (r1, r2, r3), ro = oracle_update_apply(inp, True)
    for nm, a, b in zip(("W1", "W2", "W3"), wg, (r1, r2, r3)):
        check(f"{nm}_hat", a, b, TOL["bf16"])
    check("O image queries", og[:wl.n_kv], ro[:wl.n_kv], TOL["bf16"])
    check("O target-view queries", og[wl.n_kv:], ro[wl.n_kv:], TOL["bf16"])
    wg, _ = run_update_apply(inp, False)
    (r1, r2, r3), _ = oracle_update_apply(inp, False)
    for nm, a, b, w in zip(("W1", "W2", "W3"), wg, (r1, r2, r3),
                           (inp.np("w1"), inp.np("w2"), inp.np("w3"))):
        check(f"Delta {nm}", a - w, b - w, TOL["bf16"])


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_hot_eta_stress(io):
    say(f"case hot eta x100 io={io}")
    inp = Inputs(seed=4, n=16_384, io=io, eta_scale=100.0)
    wg, _ = run_update_apply(inp, False)
    (r1, _, _), _ = oracle_update_apply(inp, False)
    w1 = inp.np("w1")
    ratio = np.max(np.abs(r1 - w1)) / np.max(np.abs(w1))
    say(f"    step size max|dW1|/max|W1| = {ratio:.3f}")
    assert ratio > 0.1
    full_parity(inp, TOL[io])


@pytest.mark.parametrize("n", [1, 31, 32, 33, 127])
def test_small_and_ragged_token_counts(n):
    say(f"case ragged n={n}")
    full_parity(Inputs(seed=5 + n, n=n), TOL["bf16"])


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("renorm", [False, True])
def test_zero_eta_and_empty_chunk_leave_weights_unchanged(io, renorm):
    say(f"case eta=0 / n_kv=0 io={io} renorm={renorm}")
    inp = Inputs(seed=6, n=500, io=io)
    t = inp.t
    eta0 = torch.zeros_like(t["eta"])
    w = zm.update(t["k"], t["v"], eta0, t["w1"], t["w2"], t["w3"], renorm=renorm)
    torch.cuda.synchronize()
    for a, b in zip(w, (t["w1"], t["w2"], t["w3"])):
        assert torch.equal(a, b)
    empty = t["k"][:0]
    w, o = zm.update_apply(empty, empty, t["eta"][:0], t["q"], t["w1"], t["w2"], t["w3"],
                           renorm=renorm)
    torch.cuda.synchronize()
    for a, b in zip(w, (t["w1"], t["w2"], t["w3"])):
        assert torch.equal(a, b)
    ref = oracle.apply(inp.np("q"), inp.np("w1"), inp.np("w2"), inp.np("w3"))
    check("O with n_kv = 0", host(o), ref, TOL[io])


def test_empty_queries_and_in_place_update():
    say("case n_q = 0, in-place weights")
    inp = Inputs(seed=7, n=400)
    t = inp.t
    ref, _ = oracle_update_apply(inp, True)
    w = [t["w1"].clone(), t["w2"].clone(), t["w3"].clone()]
    outs, o = zm.update_apply(t["k"], t["v"], t["eta"], t["q"][:0], *w, renorm=True, w_out=w)
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    for nm, a, b in zip(("W1", "W2", "W3"), w, ref):
        check(f"{nm}_hat in place", host(a), b, TOL["bf16"])


def test_strided_tokens_from_fused_projection():
    """q, k, v as views into one [n, 3, H, d] projection output (token stride 3*H*d)."""
    say("case strided qkv views")
    n, H, d, h = 700, 8, 128, 256
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    qkv = (torch.randn(n, 3, H, d, generator=g, device="cuda") / math.sqrt(d)).to(torch.bfloat16)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    eta = WL.make_eta(n, H, 8, "cuda")
    w1, w2, w3 = WL.make_weights(H, d, h, 8, "cuda")
    o_buf = torch.empty(n, 3, H, d, dtype=torch.bfloat16, device="cuda")
    (a1, a2, a3), o = zm.update_apply(k, v, eta, q, w1, w2, w3, renorm=True, out=o_buf[:, 1])
    assert o.stride(0) == 3 * H * d
    torch.cuda.synchronize()
    (r1, r2, r3), ro = oracle.update_apply(host(k), host(v), host(eta), host(q), host(w1),
                                           host(w2), host(w3), renorm=True)
    for nm, a, b in zip(("W1", "W2", "W3"), (a1, a2, a3), (r1, r2, r3)):
        check(f"{nm}_hat strided", host(a), b, TOL["bf16"])
    check("O strided", host(o), ro, TOL["bf16"])


@pytest.mark.parametrize("order", ["apply_then_update", "update_then_apply"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_streaming_frames(order, io):
    wl = WL.Workload("stream4", 4, 518, 8, 128, 256, io, True, streaming=True)
    say(f"case streaming 4 frames order={order} io={io}")
    inp = Inputs(wl, 9)
    t = inp.t
    w = [t["w1"].clone(), t["w2"].clone(), t["w3"].clone()]
    code = zm.APPLY_THEN_UPDATE if order == "apply_then_update" else zm.UPDATE_THEN_APPLY
    outs = []
    for (s, e) in WL.frame_slices(wl):
        outs.append(host(zm.stream_step(t["q"][s:e], t["k"][s:e], t["v"][s:e], t["eta"][s:e], *w,
                                        renorm=True, order=code)))
    torch.cuda.synchronize()
    frames = [dict(q=inp.np("q")[s:e], k=inp.np("k")[s:e], v=inp.np("v")[s:e],
                   eta=inp.np("eta")[s:e]) for (s, e) in WL.frame_slices(wl)]
    rw, routs = oracle.stream(frames, inp.np("w1"), inp.np("w2"), inp.np("w3"), renorm=True,
                              order=order)
    for i, (a, b) in enumerate(zip(outs, routs)):
        check(f"O frame {i}", a, b, TOL[io])
    for nm, a, b in zip(("W1", "W2", "W3"), w, rw):
        check(f"{nm} after 4 frames", host(a), b, TOL[io])
    # the state moved: each frame's step is checked, not just W(0)
    assert rel(rw[0], inp.np("w1")) > 1e-4


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_bitwise_determinism(io):
    say(f"case determinism io={io}")
    inp = Inputs(seed=10, n=20_000, io=io)
    t = inp.t
    a, oa = zm.update_apply(t["k"], t["v"], t["eta"], t["q"], t["w1"], t["w2"], t["w3"], renorm=True)
    b, ob = zm.update_apply(t["k"], t["v"], t["eta"], t["q"], t["w1"], t["w2"], t["w3"], renorm=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(oa, ob)


@pytest.mark.parametrize("layer", [0, 23])
def test_f700_full_size_sampled(layer):
    """The 700-frame workload in the launch configuration the benchmark
    times (layer 23: the last layer of the 24-layer stack, fresh weights),
    checked on every head: 16 sampled hidden units per head (one in each wave's
    16-unit block of both 128-unit workgroup slices) of W_hat, and sampled
    query outputs."""
    wl = WL.WORKLOADS["f700"]
    say(f"case f700 full size seed=4 layer={layer} (sampled checks)")
    inp = Inputs(wl, 4)
    t = inp.t
    if layer:
        t["w1"], t["w2"], t["w3"] = WL.make_weights(wl.heads, wl.d_head, wl.d_hidden, 4, "cuda",
                                                    layer=layer)
    (g1, g2, g3), og = zm.update_apply(t["k"], t["v"], t["eta"], t["q"], t["w1"], t["w2"],
                                       t["w3"], renorm=True)
    (f1, f2, f3), _ = zm.update_apply(t["k"], t["v"], t["eta"], t["q"][:0], t["w1"], t["w2"],
                                      t["w3"], renorm=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    heads = list(range(wl.heads))
    for hd in heads:
        J = sampled_units(wl.d_hidden, rng)   # 16 units: one per wave block, both slices
        k = host(t["k"][:, hd])
        v = host(t["v"][:, hd])
        eta = host(t["eta"][:, hd])
        w1, w2, w3 = host(t["w1"][hd]), host(t["w2"][hd]), host(t["w3"][hd])
        s1, s2, s3 = oracle.update_rows_sampled(k, v, eta, w1, w2, w3, J)
        # renorm-off step on the sampled hidden units
        check(f"head {hd} Delta W1[J]", host(f1[hd])[J] - w1[J], s1 - w1[J], TOL["bf16"])
        check(f"head {hd} Delta W3[J]", host(f3[hd])[J] - w3[J], s3 - w3[J], TOL["bf16"])
        check(f"head {hd} Delta W2[:,J]", host(f2[hd])[:, J] - w2[:, J], s2 - w2[:, J], TOL["bf16"])
        # W1 / W3 rows with renorm are functions of the row alone
        r1 = oracle.renorm_rows(w1[J], s1)
        r3 = oracle.renorm_rows(w3[J], s3)
        check(f"head {hd} W1_hat[J]", host(g1[hd])[J], r1, TOL["bf16"])
        check(f"head {hd} W3_hat[J]", host(g3[hd])[J], r3, TOL["bf16"])
    # W2 renorm consistency: renorm-on rows = oracle renorm of the GPU's renorm-off rows
    for hd in heads:
        ref = oracle.renorm_rows(host(t["w2"][hd]), host(f2[hd]))
        check(f"head {hd} W2_hat vs renorm(W2')", host(g2[hd]), ref, 1e-5)
    # outputs on sampled queries through the GPU's W_hat, all heads
    idx = np.sort(rng.choice(wl.n_q, 4096, replace=False))
    q = host(t["q"][torch.as_tensor(idx, device="cuda")])
    ref = oracle.apply(q, host(g1), host(g2), host(g3))
    check("O sampled (4096 queries)", host(og[torch.as_tensor(idx, device="cuda")]), ref, TOL["bf16"])
    # the last tile of the chunk too
    ref = oracle.apply(host(t["q"][-40:]), host(g1), host(g2), host(g3))
    check("O last 40 queries", host(og[-40:]), ref, TOL["bf16"])


def test_stream256_full_size_per_step():
    """256 frames fed one at a time (the streaming workload the benchmark
    times).  At sampled frames t the GPU's own state W(t-1) is taken as the
    start: the frame's output must be f_{W(t-1)}(q_t) and the state step
    W(t) - W(t-1) must match the oracle's step from W(t-1).  The first four
    frames are also checked as a chain from W(0)."""
    wl = WL.WORKLOADS["stream256"]
    say("case stream256 full size seed=5 (per-step checks)")
    inp = Inputs(wl, 5)
    t = inp.t
    w = [t["w1"].clone(), t["w2"].clone(), t["w3"].clone()]
    sampled = {0, 1, 3, 128, 255}
    before, after, outs = {}, {}, {}
    slices = WL.frame_slices(wl)
    for i, (s, e) in enumerate(slices):
        if i in sampled:
            before[i] = [host(x) for x in w]
        o = zm.stream_step(t["q"][s:e], t["k"][s:e], t["v"][s:e], t["eta"][s:e], *w, renorm=True)
        if i in sampled:
            torch.cuda.synchronize()
            after[i] = [host(x) for x in w]
            outs[i] = host(o)
    torch.cuda.synchronize()
    assert all(torch.isfinite(x).all() for x in w)
    for i in sorted(sampled):
        s, e = slices[i]
        wp = before[i]
        ref_o = oracle.apply(host(t["q"][s:e]), *wp)
        check(f"frame {i} O", outs[i], ref_o, TOL["bf16"])
        ref_w = oracle.update(host(t["k"][s:e]), host(t["v"][s:e]), host(t["eta"][s:e]), *wp,
                              renorm=True)
        for nm, a, b, w0 in zip(("W1", "W2", "W3"), after[i], ref_w, wp):
            check(f"frame {i} step {nm}", a - w0, b - w0, TOL["bf16"])
    # chain of the first frames from the initial state
    frames = [dict(q=host(t["q"][s:e]), k=host(t["k"][s:e]), v=host(t["v"][s:e]),
                   eta=host(t["eta"][s:e])) for (s, e) in slices[:4]]
    rw, routs = oracle.stream(frames, inp.np("w1"), inp.np("w2"), inp.np("w3"), renorm=True)
    check("frame 0 O (chain)", outs[0], routs[0], TOL["bf16"])
    check("frame 3 O (chain)", outs[3], routs[3], TOL["bf16"])
    for nm, a, b in zip(("W1", "W2", "W3"), after[3], rw):
        check(f"{nm} after 4 frames (chain)", a, b, TOL["bf16"])


def test_graph_replay_matches_eager():
    """The library only enqueues kernels on the caller's stream (no allocation,
    no memset, no synchronisation), so a call can be captured in a HIP graph.
    The graph is replayed several times with eager work and synchronisations in
    between, and every replay must equal the eager result bitwise."""
    say("case HIP graph capture and replay of update_apply and stream_step")
    inp = Inputs(seed=61, n=2748)
    t = inp.t
    ws = torch.empty(zm.workspace_size(zm.make_desc(t["w1"], t["w2"], t["w3"], zm.BF16, True,
                                                    t["q"], t["k"]), 2748, 2748),
                     dtype=torch.uint8, device="cuda")
    w_out = [torch.empty_like(w) for w in (t["w1"], t["w2"], t["w3"])]
    o = torch.empty_like(t["q"])

    def call():
        zm.update_apply(t["k"], t["v"], t["eta"], t["q"], t["w1"], t["w2"], t["w3"], renorm=True,
                        w_out=w_out, out=o, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref_w = [x.clone() for x in w_out]
    ref_o = o.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        for x in w_out:
            x.zero_()
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(w_out, ref_w):
            assert torch.equal(x, y), r
        assert torch.equal(o, ref_o), r
        _ = (t["q"].float() * 2).sum().item()  # eager work between replays


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_max_heads(io):
    """64 heads (the largest count accepted) of d 64 / hidden 128."""
    say(f"case 64 heads io={io}")
    full_parity(Inputs(seed=62, n=777, heads=64, d=64, h=128, io=io), TOL[io])
