"""Parity of the two update shapes on both sides of the planner's switch.

Short chunks take the two-token-group update: workgroups of 64 hidden units
whose waves split every 64-token tile between two token groups and add their
accumulators before writing.  Longer chunks take the one-group update.  Both
are checked against the oracle, with the bound of the other bf16 parity tests,
on the last token count that takes two groups, the first that takes one, and
a short count.  The shape each count takes comes from the host model of the
planner (tests/test_tiling_host.py), which mirrors plan_update; the cases
cover d_head 64 (one staging item per thread) and 128 (two), hidden 128 and
256, and 1 to 64 heads.
"""
import pytest

import test_tiling_host as TH
from test_parity_gpu import TOL, Inputs, full_parity, say

pytestmark = pytest.mark.gpu

CASES = [(8, 128, 256), (3, 64, 128), (16, 64, 256), (1, 128, 128), (64, 128, 256)]


def last_two_group_count(heads, h):
    """The largest token count whose plan takes two token groups."""
    n = 32
    while TH.plan_update_tg(n + 32, heads, h)[2] == 2:
        n += 32
    return n


@pytest.mark.parametrize("heads,d,h", CASES)
def test_both_update_shapes_match_the_oracle(heads, d, h):
    n2 = last_two_group_count(heads, h)
    counts = (max(1, n2 // 3 + 5), n2, n2 + 1)
    shapes = [TH.plan_update_tg(n, heads, h)[2] for n in counts]
    assert shapes == [2, 2, 1], (counts, shapes)
    for n, tg in zip(counts, shapes):
        say(f"case token groups {tg}: n={n} heads={heads} d={d} h={h}")
        full_parity(Inputs(seed=400 + n % 97, n=n, heads=heads, d=d, h=h), TOL["bf16"])
