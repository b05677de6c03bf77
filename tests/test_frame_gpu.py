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
