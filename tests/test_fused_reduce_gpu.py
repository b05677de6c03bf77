"""The reduce inside the shared read-and-update launch (frame_bf16.hip).

For heads a multiple of 8 and chunks short enough for the two-token-group
update, the launch that reads a frame and computes its partial sums also
reduces them: its last
workgroups wait on per-head arrival counters in the workspace, then run the
reduce kernel's code.  An update step without a read (zm_ttt_update,
update_apply, the update-then-read stream order, inner steps) takes the same
launch with no read blocks.  These tests hold it to the separate kernels bit
for bit; the loss variant of the update (zm_ttt_update_loss) is never fused
and serves as the separate-kernel reference where every other entry point
fuses.
The cases cover every narrow shape, 8 to 64 heads, ragged and single-tile
frames, the longest chunk that takes two token groups, and the first that
takes one, which keeps the separate reduce.
The counters must be zero after every launch.  A sticky error word set from
the host must turn the stepped weights into NaN rather than plausible values.
"""
import pytest
import torch

import reconstruction_lact_chunk_amd as zm
import test_tiling_host as TH
import workloads as WL
from test_parity_gpu import say

pytestmark = pytest.mark.gpu


def last_fused(heads, h):
    """The longest chunk whose update takes two token groups (and so the
    in-launch reduce); one token more takes one group and the separate reduce."""
    n = 32
    while TH.plan_update_tg(n + 32, heads, h)[2] == 2:
        n += 32
    while TH.plan_update_tg(n + 1, heads, h)[2] == 2:
        n += 1
    return n


N8 = last_fused(8, 256)


def tensors(n, heads, d, h, seed):
    q = WL.make_tokens(n, heads, d, "bf16", seed, "cuda", 1)
    k = WL.make_tokens(n, heads, d, "bf16", seed, "cuda", 2)
    v = WL.make_tokens(n, heads, d, "bf16", seed, "cuda", 3)
    eta = WL.make_eta(n, heads, seed, "cuda", eta_scale=20.0)
    return q, k, v, eta, WL.make_weights(heads, d, h, seed, "cuda")


def sync_range(heads, d, h):
    """Byte range of the sync words in the workspace: after two bf16 weight
    sets (4 arrays of heads x h x d each, 256-byte rounded)."""
    set_bytes = (4 * heads * h * d * 2 + 255) // 256 * 256
    return 2 * set_bytes, 2 * set_bytes + 256 * (heads + 1)


def separate_update(k, v, eta, w, renorm=True):
    """A step through the separate update and reduce kernels: the loss variant
    of the update is never fused, and its weights equal the plain update's
    bit for bit (tests/test_virtual_loss_gpu.py)."""
    w_new, _ = zm.update_loss(k, v, eta, *w, renorm=renorm)
    return list(w_new)


def workspace(w, q, n):
    desc = zm.make_desc(*w, zm.BF16, True, q, q)
    return torch.zeros(zm.workspace_size(desc, n, n), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("heads,d,h,n", [
    (8, 128, 256, 1374),       # the streamed frame
    (8, 128, 256, 33),         # one ragged tile
    (16, 128, 128, 2000),
    (8, 64, 128, 500),         # 12 reduce blocks per XCD (a head's items)
    (24, 64, 256, 4000),       # three heads per XCD
    (64, 64, 128, 1374),       # eight heads per XCD
    (8, 128, 256, N8),         # the longest fused chunk
    (8, 128, 256, N8 + 1),     # one group: separate reduce
])
def test_fused_reduce_equals_separate_kernels(heads, d, h, n):
    say(f"case fused reduce H={heads} d={d} h={h} n={n}")
    q, k, v, eta, w = tensors(n, heads, d, h, seed=71 + heads + n % 13)
    state = [t.clone() for t in w]
    ws = workspace(w, q, n)
    o = zm.stream_step(q, k, v, eta, *state, renorm=True, order=zm.APPLY_THEN_UPDATE,
                       workspace=ws)
    o_ref = zm.apply(q, *w)
    w_ref = separate_update(k, v, eta, w)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for a, b in zip(state, w_ref):
        assert torch.equal(a, b)
    a, b = sync_range(heads, d, h)
    assert int(ws[a:b].count_nonzero()) == 0


@pytest.mark.parametrize("renorm", [True, False])
def test_emitting_chain_equals_separate_calls(renorm):
    """Frames that keep W's bf16 copies in the workspace (the reduce blocks
    write them while other heads' blocks still read theirs) against a plain
    loop of zm_ttt_apply and separate update kernels."""
    heads, d, h = 8, 128, 256
    sizes = [1374, 1001, 33, 1374, 4096]
    n = sum(sizes)
    say(f"case fused reduce emitting chain renorm={renorm}")
    q, k, v, eta, w = tensors(n, heads, d, h, seed=77)
    state = [t.clone() for t in w]
    ref = [t.clone() for t in w]
    ws = workspace(w, q, max(sizes))
    s = 0
    for i, m in enumerate(sizes):
        sl = slice(s, s + m)
        o = zm.stream_step(q[sl], k[sl], v[sl], eta[sl], *state, renorm=renorm, workspace=ws,
                           emit_bf16=True, reuse_bf16=i > 0)
        o_ref = zm.apply(q[sl], *ref)
        ref = separate_update(k[sl], v[sl], eta[sl], ref, renorm=renorm)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), i
        for a, b in zip(state, ref):
            assert torch.equal(a, b), i
        s += m
    a, b = sync_range(heads, d, h)
    assert int(ws[a:b].count_nonzero()) == 0


def test_sticky_error_word_gives_nan_until_a_cast_clears_it():
    heads, d, h, n = 8, 128, 256, 1374
    say("case fused reduce sticky error word")
    q, k, v, eta, w = tensors(n, heads, d, h, seed=79)
    state = [t.clone() for t in w]
    ws = workspace(w, q, n)
    zm.stream_step(q, k, v, eta, *state, renorm=True, workspace=ws, emit_bf16=True)
    a, _ = sync_range(heads, d, h)
    err = a + 256 * heads
    ws[err] = 1   # as a timed-out wait would leave it
    prev = [t.clone() for t in state]
    o = zm.stream_step(q, k, v, eta, *state, renorm=True, workspace=ws, emit_bf16=True,
                       reuse_bf16=True)
    torch.cuda.synchronize()
    assert torch.equal(o, zm.apply(q, *prev))       # the read still used the incoming W
    for t in state:
        assert bool(torch.isnan(t).all())
    assert int(ws[err]) == 1                         # sticky
    # a call that casts clears the word: fresh weights give the separate result again
    state = [t.clone() for t in w]
    zm.stream_step(q, k, v, eta, *state, renorm=True, workspace=ws)
    w_ref = separate_update(k, v, eta, w)
    torch.cuda.synchronize()
    for x, y in zip(state, w_ref):
        assert torch.equal(x, y)
    assert int(ws[err]) == 0


def test_chunked_block_causal_fuses_every_step():
    """zm_ttt_chunked in the block-causal order pairs chunk c's read with its
    update in one launch; with 8 heads every such step reduces inside it."""
    heads, d, h = 8, 128, 256
    offsets = [0, 1374, 2748, 2781, 4122, 4122, 5496]
    n = offsets[-1]
    say("case fused reduce chunked block-causal")
    q, k, v, eta, w = tensors(n, heads, d, h, seed=81)
    state = [t.clone() for t in w]
    o = zm.chunked(q, k, v, eta, offsets, *state, renorm=True, order=zm.APPLY_THEN_UPDATE)
    ref = [t.clone() for t in w]
    o_ref = torch.zeros_like(o)
    for c in range(len(offsets) - 1):
        s, e = offsets[c], offsets[c + 1]
        if s == e:
            continue
        o_ref[s:e] = zm.apply(q[s:e], *ref)
        ref = separate_update(k[s:e], v[s:e], eta[s:e], ref)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for a, b in zip(state, ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("heads,d,h,n", [
    (8, 128, 256, 1374), (8, 128, 256, 33), (16, 64, 128, 777), (64, 128, 256, 200),
    (8, 64, 256, N8), (8, 128, 128, last_fused(8, 128)), (8, 128, 256, 10_992),
])
def test_update_alone_fuses_and_equals_separate_kernels(heads, d, h, n):
    """zm_ttt_update and zm_ttt_update_apply on short chunks run the update
    and its reduce as one launch (no read blocks)."""
    say(f"case fused update alone H={heads} d={d} h={h} n={n}")
    q, k, v, eta, w = tensors(n, heads, d, h, seed=83 + heads + n % 11)
    ref = separate_update(k, v, eta, w)
    got = zm.update(k, v, eta, *w, renorm=True)
    (w_ua, o_ua) = zm.update_apply(k, v, eta, q, *w, renorm=True)
    o_ref = zm.apply(q, *ref)
    torch.cuda.synchronize()
    for a, b, c in zip(got, w_ua, ref):
        assert torch.equal(a, c)
        assert torch.equal(b, c)
    assert torch.equal(o_ua, o_ref)


def test_update_then_read_stream_equals_separate_kernels():
    """Frames in the update-then-read order with the bf16 flags: each frame's
    update and reduce share a launch, whose reduce also writes the bf16 copies
    the read uses."""
    heads, d, h = 8, 128, 256
    sizes = [1374, 700, 33, 1374]
    say("case fused update-then-read stream")
    q, k, v, eta, w = tensors(sum(sizes), heads, d, h, seed=85)
    state = [t.clone() for t in w]
    ref = [t.clone() for t in w]
    ws = workspace(w, q, max(sizes))
    s = 0
    for i, m in enumerate(sizes):
        sl = slice(s, s + m)
        o = zm.stream_step(q[sl], k[sl], v[sl], eta[sl], *state, renorm=True,
                           order=zm.UPDATE_THEN_APPLY, workspace=ws, emit_bf16=True,
                           reuse_bf16=i > 0)
        ref = separate_update(k[sl], v[sl], eta[sl], ref)
        o_ref = zm.apply(q[sl], *ref)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), i
        for a, b in zip(state, ref):
            assert torch.equal(a, b), i
        s += m
    a, b = sync_range(heads, d, h)
    assert int(ws[a:b].count_nonzero()) == 0


def test_chunked_inner_steps_fuse_every_step():
    """Two inner steps per chunk: the first shares the read's launch, the
    second runs as an update-and-reduce launch of its own."""
    heads, d, h = 8, 128, 256
    offsets = [0, 1374, 2074, 2107]
    say("case fused chunked inner steps")
    q, k, v, eta, w = tensors(offsets[-1], heads, d, h, seed=87)
    state = [t.clone() for t in w]
    o = zm.chunked(q, k, v, eta, offsets, *state, renorm=True, order=zm.APPLY_THEN_UPDATE,
                   inner_steps=2)
    ref = [t.clone() for t in w]
    o_ref = torch.zeros_like(o)
    for c in range(len(offsets) - 1):
        s, e = offsets[c], offsets[c + 1]
        o_ref[s:e] = zm.apply(q[s:e], *ref)
        for _ in range(2):
            ref = separate_update(k[s:e], v[s:e], eta[s:e], ref)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for a, b in zip(state, ref):
        assert torch.equal(a, b)


def test_any_dispatch_offset_gives_the_separate_result():
    """Blocks go to XCD (block + s) mod 8 with an offset s that follows from
    the launches before; a small torch kernel of a varying grid before each
    call moves it.  Every offset must give the separate kernels' result (the
    reduce checks that a head's blocks share an XCD, not which one)."""
    heads, d, h, n = 8, 128, 256, 1374
    say("case fused reduce under varying dispatch offsets")
    q, k, v, eta, w = tensors(n, heads, d, h, seed=89)
    ref = separate_update(k, v, eta, w)
    o_ref = zm.apply(q, *w)
    ws = workspace(w, q, n)
    pad = torch.ones(64 * 1024 * 8, device="cuda")
    for m in range(1, 9):   # elementwise kernels of different grids
        pad[: m * 256 * 4 + 17].mul_(1.0)
        state = [t.clone() for t in w]
        o = zm.stream_step(q, k, v, eta, *state, renorm=True, workspace=ws)
        pad[: m * 512 + 3].add_(0.0)
        got = zm.update(k, v, eta, *w, renorm=True)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), m
        for a, b, c in zip(state, got, ref):
            assert torch.equal(a, c), m
            assert torch.equal(b, c), m


def test_graph_replays_of_fused_launches_equal_eager():
    """Stream frames and an update_apply short enough to reduce inside the
    update's launch, captured in a HIP graph and replayed several times with
    eager work of varying grids in between (which moves the dispatch offset):
    every replay must equal the eager result bitwise.  The graph holds no
    memset: the cast clears the sync words with a kernel."""
    heads, d, h, n = 8, 128, 256, 1374
    say("case fused reduce under HIP graph replay")
    q, k, v, eta, w = tensors(2 * n, heads, d, h, seed=91)
    ws = workspace(w, q, 2 * n)
    state = [t.clone() for t in w]
    w_out = [torch.empty_like(t) for t in w]
    o1, o2, o3 = (torch.empty_like(q[:n]) for _ in range(3))

    def call():
        for t, t0 in zip(state, w):
            t.copy_(t0)
        zm.stream_step(q[:n], k[:n], v[:n], eta[:n], *state, renorm=True, out=o1, workspace=ws,
                       emit_bf16=True)
        zm.stream_step(q[n:], k[n:], v[n:], eta[n:], *state, renorm=True, out=o2, workspace=ws,
                       emit_bf16=True, reuse_bf16=True)
        zm.update_apply(k[:n], v[:n], eta[:n], q[:n], *w, renorm=True, w_out=w_out, out=o3,
                        workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in state + w_out + [o1, o2, o3]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    pad = torch.ones(1 << 20, device="cuda")
    for r in range(4):
        for t in state + w_out + [o1, o2, o3]:
            t.zero_()
        pad[: 1000 * r + 77].mul_(1.0)   # eager work of a varying grid
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(state + w_out + [o1, o2, o3], ref):
            assert torch.equal(a, b), r
    # and the eager result is the separate kernels' one
    w1 = separate_update(k[:n], v[:n], eta[:n], w)
    w2 = separate_update(k[n:], v[n:], eta[n:], w1)
    torch.cuda.synchronize()
    for a, b in zip(ref[:3], w2):
        assert torch.equal(a, b)
    for a, b in zip(ref[3:6], w1):
        assert torch.equal(a, b)


@pytest.mark.parametrize("n_read", [1 << 20, (1 << 20) + 1])
def test_long_paired_read_keeps_the_wait_short(n_read):
    """In the block-causal order chunk c's read shares a launch with chunk
    c + 1's update.  A short update chunk reduces inside that launch only when
    the read is at most 2^20 queries, so the reduce blocks never wait on a
    read long enough to approach their time bound; past it the separate
    reduce runs.  Both sides of the limit equal the separate kernels."""
    heads, d, h, short = 8, 64, 128, 1374
    say(f"case fused reduce beside a long read n_read={n_read}")
    offsets = [0, n_read, n_read + short]
    q, k, v, eta, w = tensors(offsets[-1], heads, d, h, seed=93)
    state = [t.clone() for t in w]
    o = zm.chunked(q, k, v, eta, offsets, *state, renorm=True, order=zm.UPDATE_THEN_APPLY)
    ref = separate_update(k[:n_read], v[:n_read], eta[:n_read], w)
    o_ref0 = zm.apply(q[:n_read], *ref)
    ref = separate_update(k[n_read:], v[n_read:], eta[n_read:], ref)
    o_ref1 = zm.apply(q[n_read:], *ref)
    torch.cuda.synchronize()
    assert torch.equal(o[:n_read], o_ref0)
    assert torch.equal(o[n_read:], o_ref1)
    for a, b in zip(state, ref):
        assert torch.equal(a, b)
