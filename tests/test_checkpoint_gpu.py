"""Checkpoint and resume of the streaming state.

The scene memory of the streaming recursion is the fast weight W alone (the
ZipMap notes' state-size paragraph: a fixed-size state whatever the number of
frames; review, 3. Streaming Reconstruction, Eq. (6)).  So a stream cut after
any frame, with W written out and read back, must continue exactly: the
resumed run is compared bitwise with the uninterrupted one.  The resumed half
gets a fresh workspace filled with garbage, since nothing of the state may
live there."""
import io

import numpy as np
import pytest
import torch

import reconstruction_lact_chunk_amd as zm
import workloads as WL
from test_parity_gpu import say

pytestmark = pytest.mark.gpu


def _save_load(ws):
    """W through a serialized checkpoint (as a file on disk would hold it)."""
    buf = io.BytesIO()
    torch.save({"w1": ws[0].cpu(), "w2": ws[1].cpu(), "w3": ws[2].cpu()}, buf)
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    return [ck[k].to("cuda") for k in ("w1", "w2", "w3")]


def _garbage_workspace(nbytes):
    return torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("order", [zm.APPLY_THEN_UPDATE, zm.UPDATE_THEN_APPLY])
def test_stream256_resume_after_128_frames_is_bitwise(order):
    wl = WL.WORKLOADS["stream256"]
    say(f"case checkpoint stream256 order={order}")
    x = WL.make_inputs(wl, seed=21, device="cuda")
    frames = WL.frame_slices(wl)
    p = wl.tokens_per_frame
    desc = zm.make_desc(x["w1"], x["w2"], x["w3"], zm.BF16, True, x["q"], x["k"])
    nbytes = zm.workspace_size(desc, p, p)

    def run(w, span, ws):
        outs = []
        for (s, e) in span:
            outs.append(zm.stream_step(x["q"][s:e], x["k"][s:e], x["v"][s:e], x["eta"][s:e], *w,
                                       renorm=True, order=order, workspace=ws))
        return outs

    straight = [t.clone() for t in (x["w1"], x["w2"], x["w3"])]
    o_straight = run(straight, frames, torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
    first = [t.clone() for t in (x["w1"], x["w2"], x["w3"])]
    o_first = run(first, frames[:128], torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
    resumed = _save_load(first)
    del first
    o_second = run(resumed, frames[128:], _garbage_workspace(nbytes))
    torch.cuda.synchronize()
    for a, b in zip(straight, resumed):
        assert torch.equal(a, b)
    for i, (a, b) in enumerate(zip(o_straight, o_first + o_second)):
        assert torch.equal(a, b), f"frame {i}"
    # the state did move over the second half
    assert not torch.equal(straight[0], x["w1"])


def test_chunked_resume_is_bitwise():
    """The same cut through zm_ttt_chunked: chunks 0..127 in one call, then
    chunks 128..255 in another call from the checkpointed W."""
    wl = WL.WORKLOADS["stream256"]
    say("case checkpoint chunked256")
    x = WL.make_inputs(wl, seed=22, device="cuda")
    p = wl.tokens_per_frame
    offs = [i * p for i in range(wl.frames + 1)]
    desc = zm.make_desc(x["w1"], x["w2"], x["w3"], zm.BF16, True, x["q"], x["k"])
    nbytes = zm.workspace_size(desc, p, p)
    straight = [t.clone() for t in (x["w1"], x["w2"], x["w3"])]
    o_straight = zm.chunked(x["q"], x["k"], x["v"], x["eta"], offs, *straight, renorm=True,
                            workspace=torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
    half = 128 * p
    first = [t.clone() for t in (x["w1"], x["w2"], x["w3"])]
    o1 = zm.chunked(x["q"][:half], x["k"][:half], x["v"][:half], x["eta"][:half], offs[:129],
                    *first, renorm=True,
                    workspace=torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
    resumed = _save_load(first)
    o2 = zm.chunked(x["q"][half:], x["k"][half:], x["v"][half:], x["eta"][half:],
                    [o - half for o in offs[128:]], *resumed, renorm=True,
                    workspace=_garbage_workspace(nbytes))
    torch.cuda.synchronize()
    for a, b in zip(straight, resumed):
        assert torch.equal(a, b)
    assert torch.equal(o_straight, torch.cat([o1, o2]))
    assert np.isfinite(o_straight.float().cpu().numpy()).all()
