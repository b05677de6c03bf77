"""Seeded random sweeps on the GPU.

1. Small ragged cases of every entry point that reads and writes (update +
   apply, streaming in both orders, chunked schedules) for every narrow head
   shape, both io dtypes, both step rules and renorm on and off, against the
   fp64 oracle at the bf16 / fp32 bounds.
2. Random chunk schedules (offsets with empty and one-token chunks, update
   masks, inner steps, both orders, both step rules) through zm_ttt_chunked,
   bitwise equal to a loop of separate zm_ttt_update / zm_ttt_apply calls.

The largest fp32 differences come from the Newton-Schulz rule on gradients of
rank at most n (a few tokens): the quintic multiplies rounding noise in the
gradient's null space by up to 3.4445^5 ~ 490 over five steps, which fp32
arithmetic cannot avoid and the fp64 oracle does not see."""
import random

import numpy as np
import pytest
import torch

import oracle
import reconstruction_lact_chunk_amd as zm
import workloads as WL
from test_parity_gpu import TOL, host, say

pytestmark = pytest.mark.gpu
SHAPES = [(64, 128), (64, 256), (128, 128), (128, 256)]


def rel(x, r):
    m = np.max(np.abs(r))
    return float(np.max(np.abs(x - r)) / m) if m > 0 else float(np.max(np.abs(x)))


def tokens(n, heads, d, io, seed):
    return [WL.make_tokens(n, heads, d, io, seed, "cuda", s) for s in (1, 2, 3)]


@pytest.mark.parametrize("seed", range(4))
def test_random_small_cases_against_the_oracle(seed):
    rng = random.Random(1000 + seed)
    worst = {"bf16": 0.0, "f32": 0.0}
    for case in range(20):
        d, h = rng.choice(SHAPES)
        heads = rng.choice([1, 2, 3, 8])
        io = rng.choice(["bf16", "bf16", "f32"])
        rule = rng.choice(["gradient", "gradient", "newton_schulz"])
        zr = zm.STEP_NEWTON_SCHULZ if rule == "newton_schulz" else zm.STEP_GRADIENT
        renorm = rng.random() < 0.6
        kind = rng.choice(["update_apply", "stream_au", "stream_ua", "chunked"])
        s = rng.randint(0, 10 ** 6)
        n = rng.choice([1, 2, 31, 32, 33, 63, 65, rng.randint(1, 700)])
        say(f"  case {seed}.{case}: {kind} H={heads} d={d} h={h} n={n} io={io} rule={rule} "
            f"renorm={renorm}")
        q, k, v = tokens(n, heads, d, io, s)
        eta = WL.make_eta(n, heads, s, "cuda", eta_scale=rng.choice([1.0, 100.0]))
        w = WL.make_weights(heads, d, h, s, "cuda")
        w0 = [host(t) for t in w]
        if kind == "update_apply":
            got_w, got_o = zm.update_apply(k, v, eta, q, *w, renorm=renorm, step_rule=zr)
            ref_w, ref_o = oracle.update_apply(host(k), host(v), host(eta), host(q), *w0,
                                               renorm=renorm, step=rule)
        elif kind.startswith("stream"):
            order_s = "apply_then_update" if kind == "stream_au" else "update_then_apply"
            got_w = [t.clone() for t in w]
            got_o = zm.stream_step(q, k, v, eta, *got_w, renorm=renorm, step_rule=zr,
                                   order=zm.APPLY_THEN_UPDATE if kind == "stream_au"
                                   else zm.UPDATE_THEN_APPLY)
            ref_w, outs = oracle.stream([dict(q=host(q), k=host(k), v=host(v), eta=host(eta))],
                                        *w0, renorm=renorm, order=order_s, step=rule)
            ref_o = outs[0]
        else:
            offs = sorted({0, n, *rng.sample(range(n + 1), min(2, n + 1))})
            order_s = rng.choice(["apply_then_update", "update_then_apply"])
            got_w = [t.clone() for t in w]
            got_o = zm.chunked(q, k, v, eta, offs, *got_w, renorm=renorm, step_rule=zr,
                               order=zm.APPLY_THEN_UPDATE if order_s == "apply_then_update"
                               else zm.UPDATE_THEN_APPLY)
            ref_w, ref_o = oracle.chunked(host(q), host(k), host(v), host(eta), offs, *w0,
                                          order=order_s, renorm=renorm, step=rule)
        torch.cuda.synchronize()
        errs = [rel(host(a), b) for a, b in zip(list(got_w) + [got_o], list(ref_w) + [ref_o])]
        worst[io] = max(worst[io], max(errs))
        assert max(errs) <= TOL[io], (kind, heads, d, h, n, io, rule, renorm, errs)
    say(f"  worst bf16 {worst['bf16']:.2e}, f32 {worst['f32']:.2e}")


@pytest.mark.parametrize("seed", range(3))
def test_random_chunk_schedules_equal_separate_calls(seed):
    rng = random.Random(2000 + seed)
    for case in range(20):
        d, h = rng.choice(SHAPES)
        heads = rng.choice([1, 3, 8, 16])
        lens = [rng.choice([0, 1, 31, 32, 33, rng.randint(1, 1500)])
                for _ in range(rng.randint(1, 5))]
        offs = [0]
        for x in lens:
            offs.append(offs[-1] + x)
        n = offs[-1]
        if n == 0:
            continue
        order = rng.choice([zm.APPLY_THEN_UPDATE, zm.UPDATE_THEN_APPLY])
        mask = None if rng.random() < 0.5 else [rng.random() < 0.7 for _ in lens]
        inner = rng.choice([1, 1, 2])
        zr = zm.STEP_NEWTON_SCHULZ if rng.random() < 0.25 else zm.STEP_GRADIENT
        renorm = rng.random() < 0.7
        say(f"  case {seed}.{case}: H={heads} d={d} h={h} offsets={offs} order={order} "
            f"mask={mask} inner={inner} rule={zr}")
        s = rng.randint(0, 10 ** 6)
        q, k, v = tokens(n, heads, d, "bf16", s)
        eta = WL.make_eta(n, heads, s, "cuda")
        w = WL.make_weights(heads, d, h, s, "cuda")
        state = [t.clone() for t in w]
        o = zm.chunked(q, k, v, eta, offs, *state, renorm=renorm, order=order,
                       update_mask=mask, inner_steps=inner, step_rule=zr)
        ref = [t.clone() for t in w]
        o_ref = torch.zeros_like(o)
        for c in range(len(lens)):
            a, b = offs[c], offs[c + 1]
            if a == b:
                continue
            if order == zm.APPLY_THEN_UPDATE:
                o_ref[a:b] = zm.apply(q[a:b], *ref)
            for _ in range(inner if (mask is None or mask[c]) else 0):
                ref = list(zm.update(k[a:b], v[a:b], eta[a:b], *ref, renorm=renorm,
                                     step_rule=zr))
            if order == zm.UPDATE_THEN_APPLY:
                o_ref[a:b] = zm.apply(q[a:b], *ref)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
        for x, y in zip(state, ref):
            assert torch.equal(x, y)


@pytest.mark.parametrize("heads,d,h", [(16, 64, 256), (8, 128, 256), (3, 128, 128)])
def test_one_workspace_serves_every_smaller_call(heads, d, h):
    """A workspace sized for the largest call, reused for smaller ones (the
    order that once overflowed: 1058 tokens, then 949), gives bitwise the
    results of calls with their own workspace."""
    say(f"  case one workspace H={heads} d={d} h={h}")
    sizes = [1058, 949, 1, 33, 1500, 700]
    big = max(sizes)
    w = WL.make_weights(heads, d, h, 5, "cuda")
    desc = zm.binding.make_desc(*w, zm.BF16, True)
    ws = torch.empty(zm.binding.workspace_size(desc, big, big), dtype=torch.uint8, device="cuda")
    for i, n in enumerate(sizes):
        q, k, v = tokens(n, heads, d, "bf16", 40 + i)
        eta = WL.make_eta(n, heads, 40 + i, "cuda")
        (a1, a2, a3), oa = zm.update_apply(k, v, eta, q, *w, renorm=True, workspace=ws)
        (b1, b2, b3), ob = zm.update_apply(k, v, eta, q, *w, renorm=True)
        sa = [x.clone() for x in w]
        sb = [x.clone() for x in w]
        pa = zm.stream_step(q, k, v, eta, *sa, renorm=True, workspace=ws)
        pb = zm.stream_step(q, k, v, eta, *sb, renorm=True)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob) and torch.equal(pa, pb)
        for x, y in zip((a1, a2, a3, *sa), (b1, b2, b3, *sb)):
            assert torch.equal(x, y)
