"""GPU parity of the multi-chunk schedule (zm_ttt_chunked: block-causal and
shifted orders, updates on selected chunks, repeated inner steps) against the
fp64 oracle's chunked schedule, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import reconstruction_lact_chunk_amd as zm
from test_parity_gpu import TOL, Inputs, check, host, say

pytestmark = pytest.mark.gpu

ORDERS = {"update_then_apply": zm.UPDATE_THEN_APPLY, "apply_then_update": zm.APPLY_THEN_UPDATE}


def run_both(inp, offsets, order, io, mask=None, inner=1, renorm=True, step="gradient"):
    t = inp.t
    say(f"  chunked n={offsets[-1]} chunks={len(offsets) - 1} order={order} mask={mask} "
        f"inner={inner} step={step} io={io}")
    w = [t["w1"].clone(), t["w2"].clone(), t["w3"].clone()]
    rule = zm.STEP_NEWTON_SCHULZ if step == "newton_schulz" else zm.STEP_GRADIENT
    o = zm.chunked(t["q"], t["k"], t["v"], t["eta"], offsets, *w, renorm=renorm,
                   order=ORDERS[order], update_mask=mask, inner_steps=inner, step_rule=rule)
    torch.cuda.synchronize()
    rw, ro = oracle.chunked(inp.np("q"), inp.np("k"), inp.np("v"), inp.np("eta"), offsets,
                            inp.np("w1"), inp.np("w2"), inp.np("w3"), order=order,
                            update_mask=mask, inner_steps=inner, renorm=renorm, step=step)
    tol = TOL[io]
    for c in range(len(offsets) - 1):
        s, e = offsets[c], offsets[c + 1]
        if e > s:
            check(f"O chunk {c}", host(o[s:e]), ro[s:e], tol)
    for nm, a, b in zip(("W1", "W2", "W3"), w, rw):
        check(f"{nm} final", host(a), b, tol)
    return w, o


@pytest.mark.parametrize("order", list(ORDERS))
def test_chunked_orders_bf16(order):
    say(f"case chunked bf16 order={order}")
    inp = Inputs(seed=31, n=4122, eta_scale=10.0)
    run_both(inp, [0, 1374, 2748, 3100, 4122], order, "bf16")


def test_chunked_selective_updates():
    say("case chunked selective updates")
    inp = Inputs(seed=32, n=3000, eta_scale=10.0)
    w, _ = run_both(inp, [0, 700, 1500, 2200, 3000], "update_then_apply", "bf16",
                    mask=[True, False, True, False])


def test_chunked_inner_steps():
    say("case chunked two inner steps")
    inp = Inputs(seed=33, n=2000, eta_scale=10.0)
    run_both(inp, [0, 900, 2000], "apply_then_update", "bf16", inner=2)


def test_chunked_empty_chunks_and_tail():
    say("case chunked empty chunks and ragged tail")
    inp = Inputs(seed=34, n=1061, eta_scale=10.0)
    run_both(inp, [0, 0, 500, 500, 1037, 1061], "update_then_apply", "bf16")


@pytest.mark.parametrize("order", list(ORDERS))
def test_chunked_fp32(order):
    say(f"case chunked fp32 order={order}")
    inp = Inputs(seed=35, n=1500, heads=2, d=64, h=128, io="f32", eta_scale=10.0)
    run_both(inp, [0, 333, 1000, 1500], order, "f32", mask=[True, True, False], inner=2)


def test_chunked_newton_schulz():
    say("case chunked Newton-Schulz")
    inp = Inputs(seed=36, n=2400, heads=4)
    run_both(inp, [0, 800, 1600, 2400], "apply_then_update", "bf16", step="newton_schulz")


def test_chunked_equals_stream_steps_bitwise():
    say("case chunked == stream_step loop")
    inp = Inputs(seed=37, n=2748)
    t = inp.t
    offs = [0, 1000, 1374, 2748]
    wa = [t["w1"].clone(), t["w2"].clone(), t["w3"].clone()]
    oa = zm.chunked(t["q"], t["k"], t["v"], t["eta"], offs, *wa, renorm=True,
                    order=zm.APPLY_THEN_UPDATE)
    wb = [t["w1"].clone(), t["w2"].clone(), t["w3"].clone()]
    ob = torch.empty_like(oa)
    for s, e in zip(offs, offs[1:]):
        zm.stream_step(t["q"][s:e], t["k"][s:e], t["v"][s:e], t["eta"][s:e], *wb, renorm=True,
                       order=zm.APPLY_THEN_UPDATE, out=ob[s:e])
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    for x, y in zip(wa, wb):
        assert torch.equal(x, y)
