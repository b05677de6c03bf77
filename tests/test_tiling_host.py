"""Host-side model of the bf16 kernels' tiling, fetch rows and LDS buffer
schedule, checked on the CPU.

The model mirrors the index arithmetic of update_bf16.hip and apply_bf16.hip
(split plan, chunk ranges, the tile-fetch fallback rows used for tail tiles
and for the prefetch overrun past the last tile, and which LDS buffer each
pipeline step reads or writes between barriers).  It checks that every global
load row lies inside its chunk, that chunks partition the tokens, and that no
barrier interval both writes and reads one LDS buffer or writes a buffer whose
previous contents are still needed.
"""
import itertools

import pytest

TOK = 32
TARGET_WGS = 256
MIN_TILES = 4


def ceil_div(a, b):
    return (a + b - 1) // b


def plan_update(n, heads, d_hidden):
    if n <= 0:
        return 0, 0
    nsl = max(d_hidden // 128, 1)
    target = max(TARGET_WGS // (heads * nsl), 1)
    tiles = ceil_div(n, TOK)
    s = min(max(ceil_div(tiles, MIN_TILES), 1), target)
    chunk = ceil_div(tiles, s) * TOK
    return ceil_div(n, chunk), chunk


def plan_apply(n, heads):
    if n <= 0:
        return 0, 0
    target = max(TARGET_WGS // heads, 1)
    tiles = ceil_div(n, TOK)
    s = min(tiles, target)
    chunk = ceil_div(tiles, s) * TOK
    return ceil_div(n, chunk), chunk


def fetch_rows_update(t_begin, t_end, it):
    """Token rows loaded by the 32 staging rows of tile `it`."""
    t0 = t_begin + it * TOK
    rows = []
    for s_tok in range(TOK):
        if t0 + TOK <= t_end:
            rows.append(t0 + s_tok)
        else:
            ok = t0 + s_tok < t_end
            rows.append(t0 + s_tok if ok else (t0 if t0 < t_end else t_begin))
    return rows


def fetch_rows_apply(t_begin, t_end, it):
    t0 = t_begin + it * TOK
    rows = []
    for s_tok in range(TOK):
        if t0 + TOK <= t_end:
            rows.append(t0 + s_tok)
        else:
            ok = t0 < t_end and t0 + s_tok < t_end
            rows.append(t0 + s_tok if ok else (t0 if t0 < t_end else t_begin))
    return rows


SIZES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 1000, 1374, 10_992, 137_400, 138_774,
         961_800]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("heads,d_hidden", [(8, 256), (1, 128), (3, 128), (64, 256)])
def test_update_chunks_partition_and_loads_in_bounds(n, heads, d_hidden):
    splits, chunk = plan_update(n, heads, d_hidden)
    assert chunk % TOK == 0 and splits >= 1
    covered = []
    for c in range(splits):
        tb, te = c * chunk, min(n, c * chunk + chunk)
        assert tb < te, "no empty chunk"
        covered.append((tb, te))
        ntiles = ceil_div(te - tb, TOK)
        # the pipeline fetches tiles 0 .. ntiles + 1 (two past the end at most)
        for it in range(ntiles + 2):
            for r in fetch_rows_update(tb, te, it):
                assert tb <= r < te <= n
    assert covered[0][0] == 0 and covered[-1][1] == n
    assert all(a[1] == b[0] for a, b in zip(covered, covered[1:]))


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("heads", [1, 8, 64])
def test_apply_chunks_partition_and_loads_in_bounds(n, heads):
    splits, chunk = plan_apply(n, heads)
    covered = []
    for c in range(splits):
        tb, te = c * chunk, min(n, c * chunk + chunk)
        assert tb < te
        covered.append((tb, te))
        ntiles = ceil_div(te - tb, TOK)
        for it in range(ntiles + 2):
            for r in fetch_rows_apply(tb, te, it):
                assert tb <= r < te <= n
    assert covered[0][0] == 0 and covered[-1][1] == n


def check_schedule(intervals, nbuf):
    """intervals: list of dicts with 'read' and 'write' lists of tile ids.
    A tile t lives in buffer t % nbuf.  Checks: no buffer is read and written
    in one interval; a tile is written before it is read in a later interval;
    a buffer is not overwritten while a tile in it is still to be read."""
    written = {}
    last_read_needed = {}
    for k, iv in enumerate(intervals):
        rb = {t % nbuf for t in iv["read"]}
        wb = {t % nbuf for t in iv["write"]}
        assert not (rb & wb), (k, iv)
        for t in iv["read"]:
            assert written.get(t % nbuf) == t, (k, t, "read before written or overwritten")
        for t in iv["write"]:
            old = written.get(t % nbuf)
            if old is not None:
                later = [j for j in range(k, len(intervals)) if old in intervals[j]["read"]]
                assert not later, (k, t, old, "overwrites a tile still to be read")
            written[t % nbuf] = t
    return True


def update_schedule(ntiles):
    ivs = [{"read": [], "write": [0, 1]}]                       # prologue staging
    ivs.append({"read": [0, 1], "write": [2]})                   # forward(0); t = 0
    for t in range(1, ntiles - 1):
        ivs.append({"read": [t - 1, t + 1], "write": [t + 2]})   # backward, forward, stage
    if ntiles > 1:
        ivs.append({"read": [ntiles - 2, ntiles - 1], "write": []})
    else:
        ivs.append({"read": [0], "write": []})
    return ivs


def apply_q_schedule(ntiles):
    ivs = [{"read": [], "write": [0, 1]},                        # prologue staging
           {"read": [0], "write": []},                           # phase1(0); barrier
           {"read": [1], "write": [2]}]                          # i = 0
    for it in range(1, ntiles - 1):
        ivs.append({"read": [it + 1], "write": [it + 2]})
    return ivs


def apply_u_schedule(ntiles):
    ivs = [{"read": [], "write": [0]}]                           # i = 0 writes U(0)
    for it in range(1, ntiles - 1):
        ivs.append({"read": [it - 1], "write": [it]})
    if ntiles > 1:
        ivs.append({"read": [ntiles - 2], "write": [ntiles - 1]})
    ivs.append({"read": [ntiles - 1], "write": []})
    return ivs


def apply_o_schedule(ntiles):
    """Output tiles staged in LDS: phase 2 of tile t writes it, the next
    barrier interval stores it to memory."""
    ivs = [{"read": [], "write": []}]                            # prologue / i = 0
    for it in range(1, ntiles - 1):
        ivs.append({"read": [it - 2] if it >= 2 else [], "write": [it - 1]})
    if ntiles > 1:
        ivs.append({"read": [ntiles - 3] if ntiles >= 3 else [], "write": [ntiles - 2]})
        ivs.append({"read": [ntiles - 2], "write": [ntiles - 1]})
    else:
        ivs.append({"read": [], "write": [0]})
    ivs.append({"read": [ntiles - 1], "write": []})
    return ivs


@pytest.mark.parametrize("ntiles", list(range(1, 12)))
def test_pipeline_buffer_schedules_are_hazard_free(ntiles):
    # tiles past the last are staged (prefetch overrun) but never read
    check_schedule(update_schedule(ntiles), 4)
    check_schedule(apply_q_schedule(ntiles), 2)
    check_schedule(apply_u_schedule(ntiles), 2)
    sched = apply_o_schedule(ntiles)
    check_schedule(sched, 2)
    # every output tile is written once and stored once
    assert sorted(t for iv in sched for t in iv["write"]) == list(range(ntiles))
    assert sorted(t for iv in sched for t in iv["read"]) == list(range(ntiles))


def test_schedule_checker_catches_a_missing_barrier():
    # the apply prologue without the barrier after phase1(0) stages Q(2) over Q(0)
    bad = [{"read": [], "write": [0, 1]}, {"read": [0, 1], "write": [2]}]
    with pytest.raises(AssertionError):
        check_schedule(bad, 2)


def lds_conflict_degree(byte_addrs, width, group, nbanks=128):
    """Bank-conflict degree of one LDS access: 4-byte banks repeating every
    4 * nbanks bytes, the wave's lanes served `group` at a time.  The default
    (128 banks; 16-byte accesses 32 lanes at a time, 8-byte accesses 64 at a
    time) reproduces the measured cost of strided 16-byte reads; the update
    tile's transposing reads measured faster with a layout that is
    conflict-free under the 64-bank reading (16 and 32 lanes at a time)."""
    worst = 1
    for g0 in range(0, len(byte_addrs), group):
        banks = {}
        for a in byte_addrs[g0:g0 + group]:
            for w in range(width // 4):
                banks.setdefault((a // 4 + w) % nbanks, set()).add(a // 4 + w)
        worst = max(worst, max(len(v) for v in banks.values()))
    return worst


def test_lds_model_reproduces_measured_ordering():
    # measured on the MI355X: pitch 288 B conflict-free, 272 B and 528 B 2-way,
    # 256 B heavily conflicted (cycles per b128 read 5.4 / 9.5 / 9.0 / 32.9)
    pat = lambda pitch: [(l % 16) * pitch + (l // 16) * 16 for l in range(64)]
    assert lds_conflict_degree(pat(288), 16, 32) == 1
    assert lds_conflict_degree(pat(272), 16, 32) == 2
    assert lds_conflict_degree(pat(528), 16, 32) == 2
    assert lds_conflict_degree(pat(256), 16, 32) == 8


def test_tau_and_swizzle_layout():
    """Token map and XOR swizzle of the update tile: a bijection; the forward
    MFMA rows of each lane are the tokens of its backward operand slots; the
    two transposing reads of a lane share one swizzle; forward row reads,
    transposing reads and staging writes are free of bank conflicts under the
    64-bank reading; and the transposing read delivers tokens tau(g, 0..7) of
    column 16 m + i."""
    def tau(g, j):
        return 16 * (g >> 1) + 4 * (g & 1) + 8 * (j >> 2) + (j & 3)

    for D in (64, 128):
        def swz(r):
            sh = 0 if D == 128 else 1
            return 2 * ((r >> sh) & (D // 16 - 1)) + ((r >> 4) & 1)

        def off(r, col):  # element offset
            return r * D + (((col >> 3) ^ swz(r)) << 3) + (col & 7)

        assert sorted(off(r, c) for r in range(TOK) for c in range(D)) == list(range(TOK * D))
        assert sorted(tau(g, j) for g in range(4) for j in range(8)) == list(range(TOK))
        for g, c in itertools.product(range(4), range(16)):
            row_a = tau(g, c >> 2)
            assert row_a + 8 == tau(g, 4 + (c >> 2)) and swz(row_a + 8) == swz(row_a)
        for mb, ks in itertools.product(range(2), range(D // 32)):
            addrs = [2 * off(tau((l % 16) >> 2, 4 * mb + (l % 4)), 32 * ks + 8 * (l // 16))
                     for l in range(64)]
            assert lds_conflict_degree(addrs, 16, 16, 64) == 1
        for h, m in itertools.product(range(2), range(D // 16)):
            addrs = [2 * off(tau(l // 16, 4 * h + (l % 16) // 4), 16 * m + 4 * (l % 4))
                     for l in range(64)]
            assert lds_conflict_degree(addrs, 8, 32, 64) == 1
        cpt = D // 8
        for w in range(8):
            items = [64 * w + l for l in range(64) if 64 * w + l < TOK * cpt]
            if items:
                addrs = [2 * off(i // cpt, 8 * (i % cpt)) for i in items]
                assert lds_conflict_degree(addrs, 16, 16, 64) == 1
        # transposing read: lane i gets element i % 4 of source lanes 4 e + i / 4
        flat = {off(r, c): (r, c) for r in range(TOK) for c in range(D)}
        for h, m, g in itertools.product(range(2), range(D // 16), range(4)):
            src = [[flat[off(tau(g, 4 * h + s // 4), 16 * m + 4 * (s % 4)) + x] for x in range(4)]
                   for s in range(16)]
            for i, e in itertools.product(range(16), range(4)):
                assert src[4 * e + i // 4][i % 4] == (tau(g, 4 * h + e), 16 * m + i)
        # forward accumulator row 4 g + i of block mb is the token of slot 4 mb + i
        for g, i, mb in itertools.product(range(4), range(4), range(2)):
            lane_c = 4 * g + i  # the lane whose A-row is MFMA row 4 g + i
            assert tau(lane_c >> 2, 4 * mb + (lane_c & 3)) == tau(g, 4 * mb + i)


@pytest.mark.parametrize("D,H", [(128, 256), (64, 128), (128, 128), (64, 256)])
def test_apply_tile_reads_conflict_free(D, H):
    DP, UP = D + 16, H + 16   # element pitches of the Q and U tiles
    for ks in range(D // 32):
        assert lds_conflict_degree([2 * ((l % 16) * DP + 32 * ks + 8 * (l // 16))
                                    for l in range(64)], 16, 32) == 1
    for ks in range(H // 32):
        assert lds_conflict_degree([2 * ((l % 16) * UP + 32 * ks + 8 * (l // 16))
                                    for l in range(64)], 16, 32) == 1
