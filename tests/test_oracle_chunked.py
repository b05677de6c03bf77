"""Pins of the oracle's multi-chunk schedule (LaCT summary, mhpn.cn, part 二,
3、应用场景: block-causal update-then-apply, shifted apply-then-update, updates
on selected chunks only) against compositions of the single-chunk update and
apply, which other tests pin to the pages and to calculus."""
import math

import numpy as np
import pytest

from oracle import ttt_oracle as O


def seq(n, heads, d, h, seed):
    r = np.random.default_rng(seed)
    t = dict(q=r.normal(size=(n, heads, d)) / math.sqrt(d),
             k=r.normal(size=(n, heads, d)) / math.sqrt(d),
             v=r.normal(size=(n, heads, d)) / math.sqrt(d),
             eta=0.3 * r.random((n, heads)))
    w = (r.normal(size=(heads, h, d)) / math.sqrt(d), r.normal(size=(heads, d, h)) / math.sqrt(h),
         r.normal(size=(heads, h, d)) / math.sqrt(d))
    return t, w


def run(t, offsets, w, **kw):
    return O.chunked(t["q"], t["k"], t["v"], t["eta"], offsets, *w, **kw)


def assert_same(ws, ref):
    for x, y in zip(ws, ref):
        np.testing.assert_array_equal(x, y)


def test_one_chunk_update_then_apply_is_the_bidirectional_chunk():
    t, w = seq(23, 2, 4, 6, 1)
    wc, oc = run(t, [0, 23], w, renorm=True)
    wr, orf = O.update_apply(t["k"], t["v"], t["eta"], t["q"], *w, renorm=True)
    assert_same(wc, wr)
    np.testing.assert_array_equal(oc, orf)


def test_apply_then_update_is_the_streaming_recursion():
    t, w = seq(30, 2, 4, 6, 2)
    offs = [0, 7, 19, 30]
    frames = [dict(q=t["q"][s:e], k=t["k"][s:e], v=t["v"][s:e], eta=t["eta"][s:e])
              for s, e in zip(offs, offs[1:])]
    ws, outs = O.stream(frames, *w, renorm=True, order="apply_then_update")
    wc, oc = run(t, offs, w, order="apply_then_update", renorm=True)
    assert_same(wc, ws)
    np.testing.assert_array_equal(oc, np.concatenate(outs))


def test_update_then_apply_reads_each_chunk_after_writing_it():
    t, w = seq(20, 1, 3, 5, 3)
    offs = [0, 8, 20]
    wc, oc = run(t, offs, w)
    w1 = O.update(t["k"][:8], t["v"][:8], t["eta"][:8], *w)
    np.testing.assert_array_equal(oc[:8], O.apply(t["q"][:8], *w1))
    w2 = O.update(t["k"][8:], t["v"][8:], t["eta"][8:], *w1)
    np.testing.assert_array_equal(oc[8:], O.apply(t["q"][8:], *w2))
    assert_same(wc, w2)


def test_no_updates_reads_everything_with_the_initial_weights():
    t, w = seq(17, 2, 4, 6, 4)
    wc, oc = run(t, [0, 5, 17], w, update_mask=[False, False])
    assert_same(wc, w)
    np.testing.assert_array_equal(oc, O.apply(t["q"], *w))


def test_selective_update_skips_masked_chunks():
    t, w = seq(24, 1, 4, 6, 5)
    offs = [0, 6, 12, 24]
    wc, oc = run(t, offs, w, update_mask=[True, False, True])
    w1 = O.update(t["k"][:6], t["v"][:6], t["eta"][:6], *w)
    np.testing.assert_array_equal(oc[6:12], O.apply(t["q"][6:12], *w1))
    w2 = O.update(t["k"][12:], t["v"][12:], t["eta"][12:], *w1)
    assert_same(wc, w2)


def test_inner_steps_repeat_the_update_on_the_chunk():
    t, w = seq(12, 1, 3, 4, 6)
    wc, oc = run(t, [0, 12], w, inner_steps=3, renorm=True)
    cur = w
    for _ in range(3):
        cur = O.update(t["k"], t["v"], t["eta"], *cur, renorm=True)
    assert_same(wc, cur)
    np.testing.assert_array_equal(oc, O.apply(t["q"], *cur))


def test_schedule_composes_over_a_split_of_the_sequence():
    t, w = seq(26, 2, 4, 6, 7)
    wa, oa = run(t, [0, 5, 13, 26], w, order="apply_then_update", renorm=True)
    head = {x: y[:13] for x, y in t.items()}
    tail = {x: y[13:] for x, y in t.items()}
    w1, o1 = run(head, [0, 5, 13], w, order="apply_then_update", renorm=True)
    w2, o2 = run(tail, [0, 13], w1, order="apply_then_update", renorm=True)
    assert_same(wa, w2)
    np.testing.assert_array_equal(oa, np.concatenate([o1, o2]))


def test_empty_chunks_change_nothing():
    t, w = seq(9, 1, 3, 4, 8)
    wa, oa = run(t, [0, 0, 4, 4, 9, 9], w)
    wb, ob = run(t, [0, 4, 9], w)
    assert_same(wa, wb)
    np.testing.assert_array_equal(oa, ob)


def test_newton_schulz_rule_passes_through():
    t, w = seq(14, 1, 4, 6, 9)
    wc, _ = run(t, [0, 14], w, renorm=True, step="newton_schulz")
    assert_same(wc, O.update(t["k"], t["v"], t["eta"], *w, renorm=True, step="newton_schulz"))


@pytest.mark.parametrize("bad", [dict(offsets=[1, 5]), dict(offsets=[0, 5, 3]),
                                 dict(order="both"), dict(inner_steps=0)])
def test_bad_schedules_are_rejected(bad):
    t, w = seq(5, 1, 2, 3, 10)
    offsets = bad.pop("offsets", [0, 5])
    with pytest.raises(ValueError):
        run(t, offsets, w, **bad)
