"""The one-launch read-and-update of an apply-then-update step (frame_bf16.hip)
against the standalone kernels of the same library: the streaming step's
output must equal zm_ttt_apply on the incoming W and its new W must equal
zm_ttt_update, bit for bit, whatever share of the compute units the two kinds
of workgroup get (including frames large enough that the update alone fills
the GPU and the read's workgroups queue behind it)."""
import pytest
import torch

import reconstruction_lact_chunk_amd as zm
import workloads as WL
from test_parity_gpu import say

pytestmark = pytest.mark.gpu


def tensors(n, heads, d, h, seed):
    q = WL.make_tokens(n, heads, d, "bf16", seed, "cuda", 1)
    k = WL.make_tokens(n, heads, d, "bf16", seed, "cuda", 2)
    v = WL.make_tokens(n, heads, d, "bf16", seed, "cuda", 3)
    eta = WL.make_eta(n, heads, seed, "cuda")
    return q, k, v, eta, WL.make_weights(heads, d, h, seed, "cuda")


@pytest.mark.parametrize("heads,d,h,n,rule", [
    (8, 128, 256, 1374, zm.STEP_GRADIENT),       # one streaming frame: both kinds fit at once
    (8, 128, 256, 100_000, zm.STEP_GRADIENT),    # the update fills the GPU; the read queues
    (64, 64, 256, 1374, zm.STEP_GRADIENT),       # 256 update blocks from many heads
    (1, 64, 128, 777, zm.STEP_GRADIENT),
    (3, 128, 128, 33, zm.STEP_GRADIENT),         # one ragged tile
    (8, 128, 256, 1374, zm.STEP_NEWTON_SCHULZ),
])
def test_frame_launch_equals_separate_kernels(heads, d, h, n, rule):
    say(f"case frame launch H={heads} d={d} h={h} n={n} rule={rule}")
    q, k, v, eta, w = tensors(n, heads, d, h, seed=61)
    state = [t.clone() for t in w]
    o = zm.stream_step(q, k, v, eta, *state, renorm=True, order=zm.APPLY_THEN_UPDATE,
                       step_rule=rule)
    o_ref = zm.apply(q, *w)
    w_ref = zm.update(k, v, eta, *w, renorm=True, step_rule=rule)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for a, b in zip(state, w_ref):
        assert torch.equal(a, b)


def test_chunked_inner_steps_after_the_shared_launch():
    """Two inner steps: the first update shares the read's launch, the second
    runs alone on the weights the first produced."""
    say("case chunked A->U, two inner steps")
    q, k, v, eta, w = tensors(2 * 1374, 8, 128, 256, seed=62)
    state = [t.clone() for t in w]
    o = zm.chunked(q, k, v, eta, [0, 1374, 2748], *state, renorm=True,
                   order=zm.APPLY_THEN_UPDATE, inner_steps=2)
    ref = [t.clone() for t in w]
    outs = []
    for s, e in ((0, 1374), (1374, 2748)):
        outs.append(zm.apply(q[s:e], *ref))
        for _ in range(2):
            ref = list(zm.update(k[s:e], v[s:e], eta[s:e], *ref, renorm=True))
    torch.cuda.synchronize()
    assert torch.equal(o, torch.cat(outs))
    for a, b in zip(state, ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("order", [zm.APPLY_THEN_UPDATE, zm.UPDATE_THEN_APPLY])
@pytest.mark.parametrize("mask,inner,rule", [
    (None, 1, zm.STEP_GRADIENT),
    ([1, 0, 1, 1, 1, 0], 1, zm.STEP_GRADIENT),
    ([0, 1, 1, 0, 1, 1], 2, zm.STEP_GRADIENT),
    ([1, 1, 0, 1, 0, 0], 1, zm.STEP_NEWTON_SCHULZ),
])
def test_chunked_equals_separate_calls(order, mask, inner, rule):
    """zm_ttt_chunked keeps W's bf16 copy across chunks and pairs each read with
    an update step that uses the same W; every result must equal a plain loop
    of zm_ttt_update / zm_ttt_apply calls, bit for bit (ragged chunks, an empty
    chunk, skipped updates, inner steps)."""
    offsets = [0, 1374, 2074, 2074, 2107, 4855, 4984]
    say(f"case chunked vs separate calls order={order} mask={mask} inner={inner} rule={rule}")
    q, k, v, eta, w = tensors(offsets[-1], 8, 128, 256, seed=63)
    state = [t.clone() for t in w]
    o = zm.chunked(q, k, v, eta, offsets, *state, renorm=True, order=order, update_mask=mask,
                   inner_steps=inner, step_rule=rule)
    ref = [t.clone() for t in w]
    o_ref = torch.zeros_like(o)
    for c in range(len(offsets) - 1):
        s, e = offsets[c], offsets[c + 1]
        if s == e:
            continue
        upd = mask is None or mask[c]
        if order == zm.APPLY_THEN_UPDATE:
            o_ref[s:e] = zm.apply(q[s:e], *ref)
        for _ in range(inner if upd else 0):
            ref = list(zm.update(k[s:e], v[s:e], eta[s:e], *ref, renorm=True, step_rule=rule))
        if order == zm.UPDATE_THEN_APPLY:
            o_ref[s:e] = zm.apply(q[s:e], *ref)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for a, b in zip(state, ref):
        assert torch.equal(a, b)
