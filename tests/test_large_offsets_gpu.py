"""Token offsets beyond 32 bits in the bf16 kernels.

q, k, v and o are [n, H, d] views into rows of 8192 bf16 elements (the widest
layer the library accepts), with n = 300,000 tokens: the last rows sit about
2.46e9 elements (4.9e9 bytes) from the base pointer, past both 2^31 elements
and 2^32 bytes.  The update + apply is checked against the oracle on sampled
hidden units and sampled queries (the last rows included); the streaming step
(read and update in one launch) and a chunked schedule are checked bitwise
against separate update / apply calls on the same views.
"""
import numpy as np
import pytest
import torch

import oracle
import reconstruction_lact_chunk_amd as zm
import workloads as WL
from test_parity_gpu import TOL, check, host, say

pytestmark = pytest.mark.gpu

N, H, D, HID, LD = 300_000, 8, 128, 256, 8192


def views(buf, cols):
    return [buf[:, c:c + H * D].unflatten(1, (H, D)) for c in cols]


@pytest.fixture(scope="module")
def big():
    assert (N - 1) * LD + 7 * H * D > 2 ** 31
    say(f"case large offsets n={N} ld={LD} (inputs {N * LD * 2 / 1e9:.1f} GB)")
    buf = torch.empty(N, LD, dtype=torch.bfloat16, device="cuda")
    q, k, v = views(buf, (0, 3 * H * D, 7 * H * D))  # v in the last columns of each row
    for x, s in ((q, WL.STREAM_Q), (k, WL.STREAM_K), (v, WL.STREAM_V)):
        x.copy_(WL.make_tokens(N, H, D, "bf16", 12, "cuda", s))
    eta = WL.make_eta(N, H, 12, "cuda")
    w = WL.make_weights(H, D, HID, 12, "cuda")
    obuf = torch.zeros(N, LD, dtype=torch.bfloat16, device="cuda")
    yield dict(q=q, k=k, v=v, eta=eta, w=w, obuf=obuf)
    del buf, obuf
    torch.cuda.empty_cache()


def test_update_apply_against_the_oracle(big):
    q, k, v, eta, w = big["q"], big["k"], big["v"], big["eta"], big["w"]
    (o,) = views(big["obuf"], (4 * H * D,))
    assert o.stride(0) == LD
    (g1, g2, g3), og = zm.update_apply(k, v, eta, q, *w, renorm=False, out=o)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for hd in (0, H - 1):
        J = np.sort(rng.choice(HID, 3, replace=False))
        w1, w2, w3 = (host(x[hd]) for x in w)
        s1, s2, s3 = oracle.update_rows_sampled(host(k[:, hd]), host(v[:, hd]), host(eta[:, hd]),
                                                w1, w2, w3, J)
        check(f"head {hd} Delta W1[J]", host(g1[hd])[J] - w1[J], s1 - w1[J], TOL["bf16"])
        check(f"head {hd} Delta W3[J]", host(g3[hd])[J] - w3[J], s3 - w3[J], TOL["bf16"])
        check(f"head {hd} Delta W2[:,J]", host(g2[hd])[:, J] - w2[:, J], s2 - w2[:, J],
              TOL["bf16"])
    wg = [host(x) for x in (g1, g2, g3)]
    idx = np.sort(rng.choice(N - 64, 2048, replace=False))
    sel = torch.as_tensor(idx, device="cuda")
    check("O sampled (2048 queries)", host(og[sel]), oracle.apply(host(q[sel]), *wg), TOL["bf16"])
    check("O last 64 queries", host(og[-64:]), oracle.apply(host(q[-64:]), *wg), TOL["bf16"])
    # rows outside the output view are untouched
    assert not big["obuf"][:, :4 * H * D].any() and not big["obuf"][:, 5 * H * D:].any()


def test_stream_step_equals_separate_calls(big):
    q, k, v, eta, w = big["q"], big["k"], big["v"], big["eta"], big["w"]
    o_a, o_b = views(big["obuf"], (0, 2 * H * D))
    state = [x.clone() for x in w]
    zm.stream_step(q, k, v, eta, *state, renorm=True, order=zm.APPLY_THEN_UPDATE, out=o_a)
    zm.apply(q, *w, out=o_b)
    ref = zm.update(k, v, eta, *w, renorm=True)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    for a, b in zip(state, ref):
        assert torch.equal(a, b)


def test_chunked_equals_separate_calls(big):
    q, k, v, eta, w = big["q"], big["k"], big["v"], big["eta"], big["w"]
    o_a, o_b = views(big["obuf"], (0, 2 * H * D))
    offs = [0, 123_457, N]
    state = [x.clone() for x in w]
    zm.chunked(q, k, v, eta, offs, *state, renorm=True, order=zm.UPDATE_THEN_APPLY, out=o_a)
    ref = list(w)
    for a, b in zip(offs, offs[1:]):
        ref = list(zm.update(k[a:b], v[a:b], eta[a:b], *ref, renorm=True))
        zm.apply(q[a:b], *ref, out=o_b[a:b])
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b)
    for a, b in zip(state, ref):
        assert torch.equal(a, b)
