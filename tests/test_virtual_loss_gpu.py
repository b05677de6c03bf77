"""The virtual loss read from the update's registers (zm_ttt_update_loss).

Per head, loss = sum_i eta_i L(f_W(k_i), v_i) with L(f, v) = -f^T v (review of
ZipMap, Method 2, Eq. (2)), at the incoming W.  Checked against the oracle's
virtual_loss on the same bf16 tokens and fp32 weights.  The loss is a sum of
terms of both signs, so its error is bounded against the sum of their
magnitudes, S = sum_i eta_i sum_j |u_ij| |(W2^T v_i)_j| (u = SiLU(W1 k) (*)
W3 k), with the bf16 operand bound of the other parity tests: the kernel
forms u and W2^T v from bf16 copies of W and bf16 tokens, as the update does.
The update itself must come out bitwise as zm_ttt_update's, and the loss is
bitwise reproducible and independent of the step rule."""
import numpy as np
import pytest
import torch

import oracle
import reconstruction_lact_chunk_amd as zm
import workloads as WL
from test_parity_gpu import host, say

pytestmark = pytest.mark.gpu

TOL = 2e-2


def inputs(n, heads, d, h, seed):
    t = {"k": WL.make_tokens(n, heads, d, "bf16", seed, "cuda", WL.STREAM_K),
         "v": WL.make_tokens(n, heads, d, "bf16", seed, "cuda", WL.STREAM_V),
         "eta": WL.make_eta(n, heads, seed, "cuda")}
    t["w1"], t["w2"], t["w3"] = WL.make_weights(heads, d, h, seed, "cuda")
    return t


def magnitude(t):
    """S: the loss's terms summed in absolute value, per head (fp64)."""
    k, v, eta = host(t["k"]), host(t["v"]), host(t["eta"])
    w1, w2, w3 = (host(t[n]) for n in ("w1", "w2", "w3"))
    out = np.zeros(k.shape[1])
    for hd in range(k.shape[1]):
        a = k[:, hd] @ w1[hd].T
        u = a / (1.0 + np.exp(-a)) * (k[:, hd] @ w3[hd].T)
        e = v[:, hd] @ w2[hd]
        out[hd] = (eta[:, hd, None] * np.abs(u) * np.abs(e)).sum()
    return out


@pytest.mark.parametrize("heads,d,h", [(8, 128, 256), (3, 64, 128), (2, 128, 128), (1, 64, 256)])
@pytest.mark.parametrize("n", [1, 33, 1000, 5001])
def test_loss_matches_the_oracle(heads, d, h, n):
    say(f"case virtual loss heads={heads} d={d} h={h} n={n}")
    t = inputs(n, heads, d, h, seed=70 + n % 7 + d)
    w, loss = zm.update_loss(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], renorm=True)
    torch.cuda.synchronize()
    ref = oracle.virtual_loss(host(t["k"]), host(t["v"]), host(t["eta"]), host(t["w1"]),
                              host(t["w2"]), host(t["w3"]))
    got = host(loss)
    err = np.abs(got - ref) / magnitude(t)
    assert err.max() <= TOL, (got, ref, err)
    # the update is untouched by the loss
    w_plain = zm.update(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], renorm=True)
    torch.cuda.synchronize()
    for a, b in zip(w, w_plain):
        assert torch.equal(a, b)


def test_loss_at_f8_size_every_head():
    wl = WL.WORKLOADS["f8"]
    say("case virtual loss f8")
    x = WL.make_inputs(wl, seed=9, device="cuda")
    _, loss = zm.update_loss(x["k"], x["v"], x["eta"], x["w1"], x["w2"], x["w3"], renorm=True)
    torch.cuda.synchronize()
    t = {n: x[n] for n in ("k", "v", "eta", "w1", "w2", "w3")}
    ref = oracle.virtual_loss(*(host(t[n]) for n in ("k", "v", "eta", "w1", "w2", "w3")))
    err = np.abs(host(loss) - ref) / magnitude(t)
    assert err.max() <= TOL
    # a loss of sizable magnitude is also close in relative terms
    assert np.abs(host(loss) - ref).max() <= TOL * np.abs(ref).max()


def test_loss_sign_follows_the_rates_and_values():
    """Scaling every rate by 3 scales the loss by 3 (up to the rounding of the
    rate-scaled values to bf16); negating v negates it (up to fp32 rounding:
    the matrix cores' accumulation is not bitwise sign-symmetric)."""
    say("case virtual loss scaling")
    t = inputs(777, 4, 128, 256, seed=5)
    _, l1 = zm.update_loss(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"])
    _, l3 = zm.update_loss(t["k"], t["v"], t["eta"] * 3, t["w1"], t["w2"], t["w3"])
    _, ln = zm.update_loss(t["k"], -t["v"], t["eta"], t["w1"], t["w2"], t["w3"])
    torch.cuda.synchronize()
    a, b, c = host(l1), host(l3), host(ln)
    m = magnitude(t)
    assert np.all(np.abs(b - 3 * a) <= 1e-2 * 3 * m)
    assert np.all(np.abs(c + a) <= 1e-5 * m)


def test_loss_is_reproducible_and_independent_of_the_step_rule():
    say("case virtual loss determinism / step rule")
    t = inputs(2048, 8, 128, 256, seed=11)
    _, l1 = zm.update_loss(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"])
    _, l2 = zm.update_loss(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"])
    _, l3 = zm.update_loss(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], renorm=True,
                           step_rule=zm.STEP_NEWTON_SCHULZ)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2)
    assert torch.equal(l1, l3)


def test_empty_update_gives_zero_loss():
    say("case virtual loss n=0")
    t = inputs(0, 8, 128, 256, seed=3)
    loss = torch.full((8,), float("nan"), device="cuda")
    w, loss = zm.update_loss(t["k"], t["v"], t["eta"], t["w1"], t["w2"], t["w3"], loss=loss)
    torch.cuda.synchronize()
    assert torch.equal(loss, torch.zeros(8, device="cuda"))
    for a, b in zip(w, (t["w1"], t["w2"], t["w3"])):
        assert torch.equal(a, b)
