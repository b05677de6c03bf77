"""zm_ttt_update_apply_scratch (the entry point for callers that cannot
allocate device memory) against zm_ttt_update_apply with a caller workspace:
the same kernels on the same inputs, so W_hat and o must agree bitwise.  Calls
follow one another on the same GPU, so the scratch keeps the previous call's
contents when the next (smaller) one starts; none of it may leak into a result."""
import pytest
import torch

import reconstruction_lact_chunk_amd as zm
import workloads as WL

pytestmark = pytest.mark.gpu


def inputs(n_kv, n_q, heads, d, h, io, seed, eta_scale=1.0):
    x = {"k": WL.make_tokens(n_kv, heads, d, io, seed, "cuda", WL.STREAM_K),
         "v": WL.make_tokens(n_kv, heads, d, io, seed, "cuda", WL.STREAM_V),
         "q": WL.make_tokens(n_q, heads, d, io, seed, "cuda", WL.STREAM_Q),
         "eta": WL.make_eta(n_kv, heads, seed, "cuda", eta_scale)}
    x["w1"], x["w2"], x["w3"] = WL.make_weights(heads, d, h, seed, "cuda")
    return x


def compare(x, renorm, rule=zm.STEP_GRADIENT):
    args = (x["k"], x["v"], x["eta"], x["q"], x["w1"], x["w2"], x["w3"])
    (a1, a2, a3), oa = zm.update_apply_scratch(*args, renorm=renorm, step_rule=rule)
    (b1, b2, b3), ob = zm.update_apply(*args, renorm=renorm, step_rule=rule)
    torch.cuda.synchronize()
    for nm, a, b in (("W1", a1, b1), ("W2", a2, b2), ("W3", a3, b3), ("o", oa, ob)):
        assert torch.equal(a, b), nm
    assert not torch.equal(a1, x["w1"])   # the update did move W


def test_scratch_entry_point_matches_the_workspace_entry_point():
    print("case no-alloc: f8 (10,992 tokens), then 1001 tokens", flush=True)
    compare(inputs(10_992, 10_992, 8, 128, 256, "bf16", 71), renorm=True)
    compare(inputs(1001, 37, 8, 128, 256, "bf16", 72, eta_scale=30.0), renorm=False)


def test_scratch_entry_point_other_shapes_and_rules():
    print("case no-alloc: fp32 io, Newton-Schulz, empty queries", flush=True)
    compare(inputs(3000, 500, 3, 64, 128, "f32", 73, eta_scale=10.0), renorm=True)
    compare(inputs(2000, 2000, 4, 128, 128, "bf16", 74), renorm=True, rule=zm.STEP_NEWTON_SCHULZ)
    compare(inputs(513, 0, 8, 128, 256, "bf16", 75, eta_scale=5.0), renorm=True)
