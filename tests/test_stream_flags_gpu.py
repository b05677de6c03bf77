"""The streaming step's bf16-reuse flags: a chain of frames where each frame's
reduce leaves W's bf16 operand copies in the workspace for the next frame
(EMIT on the first frame, EMIT | REUSE after it) gives bitwise the outputs and
states of the plain chain, in both orders, under both step rules, at the narrow
and full-width head shapes; with fp32 io the flags change nothing."""
import pytest
import torch

import reconstruction_lact_chunk_amd as zm
import workloads as WL
from test_parity_gpu import say

pytestmark = pytest.mark.gpu


def chain(x, frames, order, rule, flags, renorm=True):
    w = [x["w1"].clone(), x["w2"].clone(), x["w3"].clone()]
    p = max(e - s for s, e in frames)
    io = zm.BF16 if x["q"].dtype == torch.bfloat16 else zm.F32
    desc = zm.make_desc(*w, io, renorm, x["q"], x["k"], step_rule=rule)
    ws = torch.empty(zm.workspace_size(desc, p, p), dtype=torch.uint8, device="cuda")
    outs = []
    for i, (s, e) in enumerate(frames):
        outs.append(zm.stream_step(x["q"][s:e], x["k"][s:e], x["v"][s:e], x["eta"][s:e], *w,
                                   renorm=renorm, order=order, workspace=ws, step_rule=rule,
                                   emit_bf16=flags, reuse_bf16=flags and i > 0))
    torch.cuda.synchronize()
    return w, outs


def frames_of(sizes):
    out, s = [], 0
    for n in sizes:
        out.append((s, s + n))
        s += n
    return out, s


@pytest.mark.parametrize("order", [zm.APPLY_THEN_UPDATE, zm.UPDATE_THEN_APPLY])
@pytest.mark.parametrize("rule", [zm.STEP_GRADIENT, zm.STEP_NEWTON_SCHULZ])
@pytest.mark.parametrize("shape", [(8, 128, 256, "bf16"), (3, 64, 128, "bf16"),
                                   (2, 64, 256, "f32"), (1, 1024, 2048, "bf16")])
def test_flagged_chain_is_bitwise_the_plain_chain(order, rule, shape):
    heads, d, h, io = shape
    wide = d == 1024
    if wide and rule == zm.STEP_NEWTON_SCHULZ and order == zm.UPDATE_THEN_APPLY:
        pytest.skip("one Newton-Schulz order suffices at the full width (slow oracle-free case)")
    sizes = [1374, 1001, 0, 33, 1374, 700] if not wide else [600, 0, 257, 600]
    frames, n = frames_of(sizes)
    say(f"case stream flags order={order} rule={rule} shape={shape}")
    g = 60 + heads + d
    x = {"q": WL.make_tokens(n, heads, d, io, g, "cuda", WL.STREAM_Q),
         "k": WL.make_tokens(n, heads, d, io, g, "cuda", WL.STREAM_K),
         "v": WL.make_tokens(n, heads, d, io, g, "cuda", WL.STREAM_V),
         "eta": WL.make_eta(n, heads, g, "cuda", eta_scale=20.0)}
    x["w1"], x["w2"], x["w3"] = WL.make_weights(heads, d, h, g, "cuda")
    w_a, o_a = chain(x, frames, order, rule, flags=False)
    w_b, o_b = chain(x, frames, order, rule, flags=True)
    for a, b in zip(w_a, w_b):
        assert torch.equal(a, b)
    for i, (a, b) in enumerate(zip(o_a, o_b)):
        assert torch.equal(a, b), f"frame {i}"
    assert not torch.equal(w_a[0], x["w1"])
