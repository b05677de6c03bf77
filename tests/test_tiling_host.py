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
import math

import numpy as np

import pytest

TOK = 32
TARGET_WGS = 256
MIN_TILES = 4


def ceil_div(a, b):
    return (a + b - 1) // b


def plan_update_tg(n, heads, d_hidden):
    """(splits, chunk, tg): workgroups of 128 hidden units and 32-token tiles
    (tg = 1), or, when chunks of MIN_TILES tiles would not fill the GPU, of
    64 hidden units and two token groups over 64-token tiles (tg = 2)."""
    if n <= 0:
        return 0, 0, 1
    nsl = max(d_hidden // 128, 1)
    target = max(TARGET_WGS // (heads * nsl), 1)
    tiles = ceil_div(n, TOK)
    s = ceil_div(tiles, MIN_TILES)
    if s < target and d_hidden >= 128:
        target2 = max(target // 2, 1)
        tiles2 = ceil_div(n, 2 * TOK)
        s2 = min(max(ceil_div(tiles2, MIN_TILES), 1), target2)
        chunk = ceil_div(tiles2, s2) * 2 * TOK
        return ceil_div(n, chunk), chunk, 2
    s = min(max(s, 1), target)
    chunk = ceil_div(tiles, s) * TOK
    return ceil_div(n, chunk), chunk, 1


def plan_update(n, heads, d_hidden):
    splits, chunk, _ = plan_update_tg(n, heads, d_hidden)
    return splits, chunk


def update_slots(n, heads, d_hidden):
    """Partial-sum slots the workspace reserves for n tokens (planned split count)."""
    if n <= 0:
        return 0
    nsl = max(d_hidden // 128, 1)
    target = max(TARGET_WGS // (heads * nsl), 1)
    return min(max(ceil_div(ceil_div(n, TOK), MIN_TILES), 1), target)


def plan_apply(n, heads):
    if n <= 0:
        return 0, 0
    target = max(TARGET_WGS // heads, 1)
    tiles = ceil_div(n, TOK)
    s = min(tiles, target)
    chunk = ceil_div(tiles, s) * TOK
    return ceil_div(n, chunk), chunk


def fetch_rows_update(t_begin, t_end, it, tile=TOK):
    """Token rows loaded by the staging rows of tile `it` (tile tokens)."""
    t0 = t_begin + it * tile
    rows = []
    for s_tok in range(tile):
        if t0 + tile <= t_end:
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
    splits, chunk, tg = plan_update_tg(n, heads, d_hidden)
    tile = tg * TOK
    assert chunk % tile == 0 and splits >= 1
    covered = []
    for c in range(splits):
        tb, te = c * chunk, min(n, c * chunk + chunk)
        assert tb < te, "no empty chunk"
        covered.append((tb, te))
        ntiles = ceil_div(te - tb, tile)
        # tg = 1: the prologue fetches tiles 0..3 and iteration t tile t + 3;
        # tg = 2: the prologue fetches tiles 0..2 and iteration t tile t + 2
        look = 3 if tg == 1 else 2
        for it in range(max(look + 1, ntiles + look - 1)):
            for r in fetch_rows_update(tb, te, it, tile):
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
    """intervals: list of dicts with 'read' and 'write' lists of tile ids,
    one per stretch between barriers.  A tile t lives in buffer t % nbuf.
    Checks: no buffer is read and written in one interval; a tile is written
    in an earlier interval than any read of it; a buffer is not overwritten
    while a tile in it is still to be read."""
    written = {}
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
    """Barrier intervals of the update kernel: tiles 0..2 staged, barrier;
    forward(0), forward(1) and staging of tile 3, barrier; then iteration t
    reads tiles t - 1 (backward) and t + 1 (forward) and stages tile t + 3,
    with a barrier after every even iteration (and after the last steady
    iteration); the epilogue reads the last two tiles."""
    ivs = [{"read": [], "write": [0, 1, 2]},
           {"read": [0, 1], "write": [3]}]
    cur = {"read": [], "write": []}
    last = ntiles - 2                       # last steady iteration
    for t in range(1, ntiles - 1):
        cur["read"] += [t - 1, t + 1]
        cur["write"] += [t + 3]
        if t % 2 == 0 or t == last:
            ivs.append(cur)
            cur = {"read": [], "write": []}
    assert not cur["read"]
    ivs.append({"read": [ntiles - 2, ntiles - 1] if ntiles > 1 else [0], "write": []})
    return ivs


def update_schedule_tg2(ntiles):
    """Barrier intervals of the two-token-group update (tiles of 64 tokens,
    4 buffers): tiles 0, 1 staged, barrier; forward(0), forward(1) and
    staging of tile 2, barrier; then iteration t reads tiles t - 1
    (backward) and t + 1 (forward) and stages tile t + 2, with a barrier
    after every iteration; the epilogue reads the last two tiles."""
    ivs = [{"read": [], "write": [0, 1]},
           {"read": [0, 1] if ntiles > 1 else [0], "write": [2]}]
    for t in range(1, ntiles - 1):
        ivs.append({"read": [t - 1, t + 1], "write": [t + 2]})
    ivs.append({"read": [ntiles - 2, ntiles - 1] if ntiles > 1 else [0], "write": []})
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


@pytest.mark.parametrize("ntiles", list(range(1, 14)))
def test_pipeline_buffer_schedules_are_hazard_free(ntiles):
    # tiles past the last are staged (prefetch overrun) but never read
    check_schedule(update_schedule(ntiles), 8)
    check_schedule(update_schedule_tg2(ntiles), 4)
    check_schedule(apply_q_schedule(ntiles), 2)
    check_schedule(apply_u_schedule(ntiles), 2)
    sched = apply_o_schedule(ntiles)
    check_schedule(sched, 2)
    # every output tile is written once and stored once
    assert sorted(t for iv in sched for t in iv["write"]) == list(range(ntiles))
    assert sorted(t for iv in sched for t in iv["read"]) == list(range(ntiles))


def test_update_schedule_needs_eight_buffers_or_six():
    # six buffers are the fewest that keep the every-other-iteration barrier
    # scheme hazard free; five let staging overwrite a tile still to be read
    for ntiles in range(6, 14):
        check_schedule(update_schedule(ntiles), 6)
    with pytest.raises(AssertionError):
        for ntiles in range(6, 14):
            check_schedule(update_schedule(ntiles), 5)


def test_two_token_group_schedule_needs_four_buffers():
    for ntiles in range(4, 14):
        check_schedule(update_schedule_tg2(ntiles), 4)
    with pytest.raises(AssertionError):
        for ntiles in range(4, 14):
            check_schedule(update_schedule_tg2(ntiles), 3)


def test_short_chunks_take_two_token_groups():
    # a streamed 1374-token frame, 8 heads of hidden 256: 6 chunks of 256
    # tokens in workgroups of 64 hidden units (192 workgroups)
    assert plan_update_tg(1374, 8, 256) == (6, 256, 2)
    # a chunk long enough to fill the GPU with 4-tile chunks keeps tg = 1
    assert plan_update_tg(2048, 8, 256)[2] == 1
    assert plan_update_tg(961_800, 8, 256)[2] == 1
    # hidden 128 has one 128-unit slice per head: tg = 2 gives two
    assert plan_update_tg(1000, 3, 128)[2] == 2


def test_schedule_checker_catches_a_missing_barrier():
    # the apply prologue without the barrier after phase1(0) stages Q(2) over Q(0)
    bad = [{"read": [], "write": [0, 1]}, {"read": [0, 1], "write": [2]}]
    with pytest.raises(AssertionError):
        check_schedule(bad, 2)


def _parity(x):
    return bin(x).count("1") & 1


def _degree(byte_addrs, width, groups, nbanks):
    worst = 1
    for grp in groups:
        banks = {}
        for lane in grp:
            a = byte_addrs[lane]
            for w in range(width // 4):
                banks.setdefault((a // 4 + w) % nbanks, set()).add(a // 4 + w)
        if banks:
            worst = max(worst, max(len(v) for v in banks.values()))
    return worst


# gfx950 LDS bank model fitted to counter measurements (SQ_LDS_BANK_CONFLICT
# and SQ_LDS_IDX_ACTIVE per instruction on single-pattern probe kernels):
# reads see 64 four-byte banks; a 16-byte read takes 4 cycles, each serving
# the 16 lanes of one half-wave whose quad index (lane / 4 within the half)
# has a given parity; an 8-byte read (plain or transposing) takes 2 cycles of
# 32 lanes.  Writes are served 128 bytes per cycle over 32 banks: 8
# consecutive lanes for 16-byte writes, 16 for 8-byte writes.
def read_b128_degree(addrs):
    groups = {}
    for lane in range(64):
        groups.setdefault((lane >> 5, _parity((lane >> 2) & 7)), []).append(lane)
    return _degree(addrs, 16, groups.values(), 64)


def read_b64_degree(addrs):
    return _degree(addrs, 8, [range(32), range(32, 64)], 64)


def write_degree(addrs, width):
    n = 128 // width
    return _degree(addrs, width, [range(i, i + n) for i in range(0, 64, n)], 32)


def _tr_segments(segs):
    # transposing read: lane 16 g + s loads 8 bytes of segment 4 g + s / 4
    return [segs[4 * (l // 16) + (l % 16) // 4] + 8 * (l % 4) for l in range(64)]


MEASURED = [  # (pattern, kind, LDS cycles per wave instruction measured on the MI355X)
    ([(l % 16) * 256 + (l // 16) * 16 for l in range(64)], "r128", 32),
    ([(l % 16) * 272 + (l // 16) * 16 for l in range(64)], "r128", 8),
    ([(l % 16) * 288 + (l // 16) * 16 for l in range(64)], "r128", 4),
    ([(l % 16) * 528 + (l // 16) * 16 for l in range(64)], "r128", 8),
    ([(l % 16) * 544 + (l // 16) * 16 for l in range(64)], "r128", 4),
    ([16 * l for l in range(64)], "r128", 4),
    (_tr_segments([32 * k for k in range(16)]), "r64", 2),
    (_tr_segments([256 * k for k in range(16)]), "r64", 16),
    (_tr_segments([64 * k if k < 8 else 32 + 64 * (k - 8) for k in range(16)]), "r64", 4),
    (_tr_segments([32 * k if k < 8 else 512 + 32 * (k - 8) for k in range(16)]), "r64", 2),
    (_tr_segments([(k % 4) * 32 + (k // 4) * 512 for k in range(16)]), "r64", 4),
    ([((64 * 0 + l) // 16) * 288 + 16 * (l % 16) for l in range(64)], "r128", 8),
    ([(l % 16) * 544 + 2 * (8 * (l // 16)) for l in range(64)], "w128", 16),
    ([(l % 16) * 288 + 2 * (4 * (l // 16)) for l in range(64)], "w64", 16),
    ([16 * l for l in range(64)], "w128", 8),
]


@pytest.mark.parametrize("case", range(len(MEASURED)))
def test_lds_model_reproduces_measured_costs(case):
    addrs, kind, cycles = MEASURED[case]
    if kind == "r128":
        assert 4 * read_b128_degree(addrs) == cycles
    elif kind == "r64":
        assert 2 * read_b64_degree(addrs) == cycles
    elif kind == "w128":
        assert 8 * write_degree(addrs, 16) == cycles
    else:
        assert 4 * write_degree(addrs, 8) == cycles


def _upd_tau(g, j):
    return 16 * (g >> 1) + 4 * (g & 1) + 8 * (j >> 2) + (j & 3)


def test_tau_and_tile_layout():
    """Token map and padded tile of the update kernel: the forward MFMA rows
    of each lane are the tokens of its backward operand slots; forward row
    reads, transposing reads and staging writes are free of bank conflicts;
    every slot's operand address is the lane's base plus a constant; and the
    transposing read delivers tokens tau(g, 0..7) of column 16 m + i."""
    tau = _upd_tau
    for D in (64, 128):
        pitch = D + 16  # elements

        def off(r, col):  # element offset
            return r * pitch + col

        assert sorted(tau(g, j) for g in range(4) for j in range(8)) == list(range(TOK))
        for g, c in itertools.product(range(4), range(16)):
            row_a = tau(g, c >> 2)
            assert row_a + 8 == tau(g, 4 + (c >> 2))
        for mb, ks in itertools.product(range(2), range(D // 32)):
            addrs = [2 * off(tau((l % 16) >> 2, 4 * mb + (l % 4)), 32 * ks + 8 * (l // 16))
                     for l in range(64)]
            assert read_b128_degree(addrs) == 1
            base = [2 * off(tau((l % 16) >> 2, l % 4), 8 * (l // 16)) for l in range(64)]
            assert len({a - b for a, b in zip(addrs, base)}) == 1      # base + constant
        for h, m in itertools.product(range(2), range(D // 16)):
            addrs = [2 * off(tau(l // 16, 4 * h + (l % 16) // 4), 16 * m + 4 * (l % 4))
                     for l in range(64)]
            assert read_b64_degree(addrs) == 1
            base = [2 * off(tau(l // 16, (l % 16) // 4), 4 * (l % 4)) for l in range(64)]
            assert len({a - b for a, b in zip(addrs, base)}) == 1
        cpt = D // 8
        for w in range(8):
            items = [64 * w + l for l in range(64) if 64 * w + l < TOK * cpt]
            if items:
                addrs = [2 * off(i // cpt, 8 * (i % cpt)) for i in items]
                assert write_degree(addrs, 16) == 1
        # transposing read: lane i gets element i % 4 of source lanes 4 e + i / 4
        for h, m, g in itertools.product(range(2), range(D // 16), range(4)):
            src = [[(tau(g, 4 * h + s // 4), 16 * m + 4 * (s % 4) + x) for x in range(4)]
                   for s in range(16)]
            for i, e in itertools.product(range(16), range(4)):
                assert src[4 * e + i // 4][i % 4] == (tau(g, 4 * h + e), 16 * m + i)
        # forward accumulator row 4 g + i of block mb is the token of slot 4 mb + i
        for g, i, mb in itertools.product(range(4), range(4), range(2)):
            lane_c = 4 * g + i  # the lane whose A-row is MFMA row 4 g + i
            assert tau(lane_c >> 2, 4 * mb + (lane_c & 3)) == tau(g, 4 * mb + i)


def test_unpadded_swizzled_tile_was_conflicted():
    # an unpadded tile with swizzle 2 (r % 8) + (r / 16) % 2 (D = 128) gives
    # 2-way conflicts on the forward row reads, as measured (8 cycles, not 4)
    def off(r, col):
        return r * 128 + (((col >> 3) ^ (2 * (r & 7) + ((r >> 4) & 1))) << 3) + (col & 7)
    addrs = [2 * off(_upd_tau((l % 16) >> 2, l % 4), 8 * (l // 16)) for l in range(64)]
    assert read_b128_degree(addrs) == 2


@pytest.mark.parametrize("D,H", [(128, 256), (64, 128), (128, 128), (64, 256)])
def test_apply_tiles_conflict_free(D, H):
    """Q, U and O tiles of the apply kernel under the fitted bank model."""
    DP, OP = D + 16, D + 4                     # element pitches of the Q and O tiles
    hpw = H // 8                               # phase-1 hidden units per wave
    db_n = D // 16
    wpd = 8 // db_n
    tbw = 2 // wpd

    def u_off(r, col):
        return r * H + (((col >> 3) ^ (r & 15)) << 3) + (col & 7)

    assert sorted(u_off(r, c) for r in range(TOK) for c in range(H)) == list(range(TOK * H))
    for ks, nb in itertools.product(range(D // 32), range(2)):     # phase-1 Q reads
        assert read_b128_degree([2 * ((16 * nb + l % 16) * DP + 32 * ks + 8 * (l // 16))
                                 for l in range(64)]) == 1
    for w in range(8):                                             # Q staging writes
        items = [64 * w + l for l in range(64) if 64 * w + l < TOK * D // 8]
        if items:
            cpt = D // 8
            assert write_degree([2 * ((i // cpt) * DP + 8 * (i % cpt)) for i in items], 16) == 1
    for w, nb in itertools.product(range(8), range(2)):            # U writes
        j0 = w * hpw
        if hpw == 32:
            addrs = [2 * u_off(16 * nb + l % 16, j0 + 8 * (l // 16)) for l in range(64)]
            assert write_degree(addrs, 16) == 1
        else:
            # hidden width 128: 8-byte pieces of 16 rows of 256 bytes; with
            # 16-byte chunks kept whole for the row reads they can only spread
            # over 8 of the 16 write slots, so 2-way is the floor here
            addrs = [2 * u_off(16 * nb + l % 16, j0 + 4 * (l // 16)) for l in range(64)]
            assert write_degree(addrs, 8) == 2
    for w in range(8):                                             # phase-2 U reads
        tb0 = (w // db_n) * tbw
        if tbw == 2:   # slot k: k-step k of both token blocks
            reads = [(16 * (tb0 + y), 32 * k) for k in range(H // 32) for y in range(2)]
        else:          # slot k: k-steps 2 k and 2 k + 1 of the one block
            reads = [(16 * tb0, 64 * k + 32 * y) for k in range(H // 64) for y in range(2)]
        for row0, col0 in reads:
            addrs = [2 * u_off(row0 + l % 16, col0 + 8 * (l // 16)) for l in range(64)]
            assert read_b128_degree(addrs) == 1
    for w in range(8):                                             # O writes (8 bytes)
        db, tb0 = w % db_n, (w // db_n) * tbw
        for tbi in range(tbw):
            addrs = [2 * ((16 * (tb0 + tbi) + l % 16) * OP + 16 * db + 4 * (l // 16))
                     for l in range(64)]
            assert write_degree(addrs, 8) == 1
    cpt = D // 8
    for w in range(TOK * cpt // 64):                               # O reads for the store
        for k in range(2):
            addrs = [2 * (((64 * w + l) // cpt) * OP + 8 * ((64 * w + l) % cpt) + 4 * k)
                     for l in range(64)]
            # head width 64: 136-byte rows put two rows' pieces of one half-wave
            # on 34 slots of 32, so one pair collides (2-way); 128: conflict-free
            assert read_b64_degree(addrs) == (1 if D == 128 else 2)
        # the two halves merged into one 16-byte access per lane (ds_read2_b64)
        # would be 2-way conflicted at the 128 shape: two rows share each bank
        # group of a 16-byte read.  Measured: 1.54e7 conflict cycles per f700
        # launch merged, 0 with the halves as separate reads.
        merged = [2 * (((64 * w + l) // cpt) * OP + 8 * ((64 * w + l) % cpt)) for l in range(64)]
        if D == 128:
            assert read_b128_degree(merged) == 2


# ---------------------------------------------------------------------------
# Newton-Schulz kernel (newton_schulz.hip): a numpy model of its data movement
# with the kernel's offset arithmetic, run in fp64.  It checks that every
# global and LDS offset is in bounds, that each store phase writes distinct
# elements, and that the five steps compute X <- a X + (b A + c A^2) X.
# ---------------------------------------------------------------------------
NS_COEFFS = (3.4445, -4.7750, 2.0315)


def ns_cfg(M, N, pad):
    PW = min(N, 128)
    cfg = dict(PW=PW, NP=N // PW, RB=M // 64, CB1=M // 32, CB3=PW // 32,
               PITCH_X=PW + pad, PITCH_XT=M + pad)
    cfg["PLANE_P"] = max(M * cfg["PITCH_X"], PW * cfg["PITCH_XT"])
    cfg["PLANE_Q"] = M * cfg["PITCH_XT"]
    return cfg


def _lanes():
    for w in range(8):
        for l in range(64):
            yield w, l, l & 15, l >> 4


def ns_model(x0, pad, kb, steps=5, tr=False):
    """Emulates k_newton_schulz on one matrix x0 ([N][M] if tr else [M][N])."""
    M, N = (x0.shape[1], x0.shape[0]) if tr else x0.shape
    C = ns_cfg(M, N, pad)
    PW, NP, RB, CB1, CB3 = C["PW"], C["NP"], C["RB"], C["CB1"], C["CB3"]
    gflat = x0.reshape(-1).astype(float).copy()
    lds_size = C["PLANE_P"] + C["PLANE_Q"]          # one plane of each region
    lds = np.full(lds_size, np.nan)
    QB = C["PLANE_P"]

    def tile(w):
        return (w >> 1) * 16 * RB, (w & 1) * 16 * CB1, (w & 1) * 16 * CB3

    def gofs(i, j):
        o = j * M + i if tr else i * N + j
        assert 0 <= o < M * N
        return o

    # master X per lane: xm[(w, l)][p, rb, cb, ii]
    xm = {}
    seen = set()
    for w, l, c, g in _lanes():
        r0, _, c03 = tile(w)
        a = np.zeros((NP, RB, CB3, 4))
        for p in range(NP):
            for rb in range(RB):
                for cb in range(CB3):
                    for ii in range(4):
                        i, j = r0 + 16 * rb + 4 * g + ii, p * PW + c03 + 16 * cb + c
                        o = gofs(i, j)
                        assert o not in seen
                        seen.add(o)
                        a[p, rb, cb, ii] = gflat[o]
        xm[(w, l)] = a
    assert len(seen) == M * N
    nrm = math.sqrt(sum(float((v * v).sum()) for v in xm.values()))
    for k in xm:
        xm[k] /= max(nrm, 1e-12)

    def store(off, val, region_lo, region_hi, written):
        assert region_lo <= off < region_hi and off not in written
        written.add(off)
        lds[off] = val

    def product(RBc, CBc, K, s1, pitch1, s2, pitch2, c0sel):
        """acc[(w,l)][rb, cb, ii] = sum_k S1[row][k] S2[col][k] per MFMA layout."""
        kof = kb // 4
        kidx = np.array([k0 + kof * gg + e for k0 in range(0, K, kb) for gg in range(4)
                         for e in range(kof)])
        assert sorted(kidx.tolist()) == list(range(K))
        acc = {}
        for w, l, c, g in _lanes():
            r0, c01, c03 = tile(w)
            c0 = c01 if c0sel == 1 else c03
            out = np.zeros((RBc, CBc, 4))
            for rb in range(RBc):
                for cb in range(CBc):
                    for ii in range(4):
                        row = 4 * g + ii       # D row within the block
                        # contraction offsets: fragment steps k0, lane groups gg
                        # (each supplying kof consecutive elements)
                        oa = s1 + (r0 + 16 * rb + row) * pitch1 + kidx
                        ob = s2 + (c0 + 16 * cb + c) * pitch2 + kidx
                        assert oa.min() >= 0 and oa.max() < lds_size
                        assert ob.min() >= 0 and ob.max() < lds_size
                        out[rb, cb, ii] = float(lds[oa] @ lds[ob])
            acc[(w, l)] = out
        return acc

    def store_t(dst, pitch, acc, RBc, CBc, c0sel, lo, hi):
        written = set()
        for w, l, c, g in _lanes():
            r0, c01, c03 = tile(w)
            c0 = c01 if c0sel == 1 else c03
            for rb in range(RBc):
                for cb in range(CBc):
                    for ii in range(4):
                        off = dst + (c0 + 16 * cb + c) * pitch + r0 + 16 * rb + 4 * g + ii
                        store(off, acc[(w, l)][rb, cb, ii], lo, hi, written)
        return written

    a_, b_, c_ = NS_COEFFS
    for _ in range(steps):
        acc_a = None
        for p in range(NP):
            lds[:QB] = np.nan
            written = set()
            for w, l, c, g in _lanes():
                r0, _, c03 = tile(w)
                for rb in range(RB):
                    for cb in range(CB3):
                        for ii in range(4):
                            off = (r0 + 16 * rb + 4 * g + ii) * C["PITCH_X"] + c03 + 16 * cb + c
                            store(off, xm[(w, l)][p, rb, cb, ii], 0, QB, written)
            assert len(written) == M * PW
            part = product(RB, CB1, PW, 0, C["PITCH_X"], 0, C["PITCH_X"], 1)
            acc_a = part if acc_a is None else {k: acc_a[k] + part[k] for k in part}
        lds[QB:] = np.nan
        assert len(store_t(QB, C["PITCH_XT"], acc_a, RB, CB1, 1, QB, lds_size)) == M * M
        acc_c = product(RB, CB1, M, QB, C["PITCH_XT"], QB, C["PITCH_XT"], 1)
        # A read back from its transposed store at the same offsets
        acc_b = {}
        for w, l, c, g in _lanes():
            r0, c01, _ = tile(w)
            back = np.zeros((RB, CB1, 4))
            for rb in range(RB):
                for cb in range(CB1):
                    for ii in range(4):
                        back[rb, cb, ii] = lds[QB + (c01 + 16 * cb + c) * C["PITCH_XT"] + r0
                                               + 16 * rb + 4 * g + ii]
            np.testing.assert_array_equal(back, acc_a[(w, l)])
            acc_b[(w, l)] = b_ * back + c_ * acc_c[(w, l)]
        lds[QB:] = np.nan
        store_t(QB, C["PITCH_XT"], acc_b, RB, CB1, 1, QB, lds_size)
        for p in range(NP):
            lds[:QB] = np.nan
            sub = {k: v[p] for k, v in xm.items()}
            assert len(store_t(0, C["PITCH_XT"], sub, RB, CB3, 3, 0, QB)) == M * PW
            prod = product(RB, CB3, M, QB, C["PITCH_XT"], 0, C["PITCH_XT"], 3)
            for k in xm:
                xm[k][p] = a_ * xm[k][p] + prod[k]
    out = np.zeros(M * N)
    for w, l, c, g in _lanes():
        r0, _, c03 = tile(w)
        for p in range(NP):
            for rb in range(RB):
                for cb in range(CB3):
                    for ii in range(4):
                        out[gofs(r0 + 16 * rb + 4 * g + ii, p * PW + c03 + 16 * cb + c)] = \
                            xm[(w, l)][p, rb, cb, ii]
    return out.reshape(x0.shape), C


def _ns_plain(x, steps=5):
    a, b, c = NS_COEFFS
    x = x / max(np.linalg.norm(x), 1e-12)
    for _ in range(steps):
        A = x @ x.T
        x = a * x + (b * A + c * A @ A) @ x
    return x


@pytest.mark.parametrize("M,N", [(64, 128), (64, 256), (128, 128), (128, 256)])
@pytest.mark.parametrize("pad,kb,elem,lds_limit", [(16, 32, 2, 160 * 1024), (8, 16, 4, 160 * 1024)])
def test_newton_schulz_kernel_data_movement(M, N, pad, kb, elem, lds_limit):
    r = np.random.default_rng(M + N)
    C = ns_cfg(M, N, pad)
    planes = 2 if elem == 2 else 1
    assert planes * (C["PLANE_P"] + C["PLANE_Q"]) * elem + 32 <= lds_limit
    x = r.normal(size=(M, N))
    steps = 2
    got, _ = ns_model(x, pad, kb, steps=steps)
    np.testing.assert_allclose(got, _ns_plain(x, steps), rtol=0, atol=1e-12)
    if N > M:   # the W1 / W3 orientation: [N][M] in memory, X = G^T
        got_t, _ = ns_model(x.T.copy(), pad, kb, steps=1, tr=True)
        np.testing.assert_allclose(got_t, _ns_plain(x, 1).T, rtol=0, atol=1e-12)


def test_newton_schulz_fragment_reads_conflict_free():
    for el, pad in [(2, 16), (4, 8)]:
        for K in (64, 128):
            pitch = (K + pad) * el
            assert read_b128_degree([(l % 16) * pitch + (l // 16) * 16 for l in range(64)]) == 1


@pytest.mark.parametrize("heads,d_hidden", [(1, 128), (1, 256), (3, 256), (8, 256), (16, 256),
                                            (64, 128)])
def test_reserved_slots_cover_every_shorter_update(heads, d_hidden):
    """A multi-chunk call sizes its partial sums for the longest chunk, so the
    reserved slot count must never decrease with n and must cover the realized
    split count of every shorter chunk.  The realized count alone does not:
    it drops and rises again (16 heads of hidden 256: 7 splits at 1058 tokens,
    8 at 949)."""
    realized_drops = False
    best = 0
    prev_slots = 0
    for n in range(1, 70_000, 3):
        splits = plan_update(n, heads, d_hidden)[0]
        slots = update_slots(n, heads, d_hidden)
        assert slots >= prev_slots
        assert slots >= splits
        best = max(best, splits)
        assert slots >= best      # covers every n' <= n
        realized_drops |= splits < best
        prev_slots = slots
    if (heads, d_hidden) == (16, 256):
        assert realized_drops
        assert plan_update(1058, 16, 256)[0] == 7 and plan_update(949, 16, 256)[0] == 8


# ---- the reduce inside the shared read-and-update launch (frame_bf16.hip) ----

RED_PER_XCD = 24


def plan_apply_wgs(n, heads, wgs):
    """plan_apply with a workgroup budget (the compute units the update leaves)."""
    if n <= 0:
        return 0, 0
    if wgs < heads:
        wgs = TARGET_WGS
    target = max(wgs // heads, 1)
    tiles = ceil_div(n, TOK)
    s = min(tiles, target)
    chunk = ceil_div(tiles, s) * TOK
    return ceil_div(n, chunk), chunk


def frame_blocks(n, heads, d, h):
    """The block roles of a fused frame launch: (signalling blocks as
    (block, head), reduce blocks as (block, [(head, first element)]),
    arrivals per head, reduce blocks per XCD)."""
    splits, chunk, tg = plan_update_tg(n, heads, h)
    nsl = h // (128 // tg)
    pairs = heads * splits
    upd_blocks = ceil_div(pairs, 8) * 8 * nsl
    ap_splits, ap_chunk = plan_apply_wgs(n, heads, TARGET_WGS - upd_blocks)
    if ap_chunk > 2 * chunk:
        ap_splits, ap_chunk = plan_apply(n, heads)
    app_blocks = heads * ap_splits
    red_base = ceil_div(upd_blocks + app_blocks, 8) * 8
    p2 = 3 * h * d // 2048
    per_xcd = min(p2, RED_PER_XCD)
    signal = []
    for b in range(upd_blocks):
        pair = ((b >> 3) // nsl) * 8 + (b & 7)
        if pair < pairs:
            signal.append((b, pair % heads))
    for b in range(upd_blocks, red_base):
        ab = b - upd_blocks
        if ab < app_blocks:
            assert (ab // heads) * ap_chunk < n          # a block with tokens
            signal.append((b, ab % heads))
        else:
            assert (ab // heads) * ap_chunk >= n         # padding finds no tokens
    reduce = []
    for b in range(red_base, red_base + 8 * per_xcd):
        rb = b - red_base
        xcd, idx = rb & 7, rb >> 3
        work = []
        for i in range(idx, (heads // 8) * p2, per_xcd):
            hl = i // p2
            hd = xcd + 8 * hl
            work.append((hd, hd * 3 * h * d + (i - hl * p2) * 2048))
        reduce.append((b, work))
    return signal, reduce, splits * nsl + ap_splits, per_xcd


@pytest.mark.parametrize("heads,d,h", [(8, 128, 256), (8, 128, 128), (8, 64, 256), (8, 64, 128),
                                       (16, 128, 256), (24, 64, 256), (64, 64, 128),
                                       (64, 128, 256)])
@pytest.mark.parametrize("n", [1, 33, 500, 1374, 1800, 4000])
def test_fused_reduce_blocks(heads, d, h, n):
    if plan_update_tg(n, heads, h)[2] != 2:
        pytest.skip("one token group: no in-launch reduce")
    signal, reduce, arrivals, per_xcd = frame_blocks(n, heads, d, h)
    assert arrivals <= 255                            # one byte per dispatch offset
    assert per_xcd < 32                                # fewer than an XCD's compute units
    # every signalling block runs on its head's XCD and each head counts
    # exactly the arrivals its reduce blocks wait for
    count = [0] * heads
    for b, hd in signal:
        assert b % 8 == hd % 8
        count[hd] += 1
    assert count == [arrivals] * heads
    # reduce blocks: on their heads' XCD, each weight element exactly once,
    # both halves of an item in one matrix, per_xcd blocks waiting per head
    HD = h * d
    seen = np.zeros(heads * 3 * HD, dtype=np.int32)
    waiters = [0] * heads
    for b, work in reduce:
        heads_here = []
        for hd, e0 in work:
            assert b % 8 == hd % 8
            assert e0 % 2048 == 0 and (e0 % (3 * HD)) // HD == (e0 % (3 * HD) + 2047) // HD
            seen[e0:e0 + 2048] += 1
            if not heads_here or heads_here[-1] != hd:
                heads_here.append(hd)
        assert len(heads_here) == len(set(heads_here))   # one wait per head
        for hd in heads_here:
            waiters[hd] += 1
    assert (seen == 1).all()
    assert waiters == [per_xcd] * heads


# ---- the in-launch reduce's counter protocol (frame_bf16.hip), as a model ----

class SyncModel:
    """One head's sync words: a 64-bit arrival counter with one 8-bit field
    per dispatch offset, the count of reduce blocks past their wait, and the
    sticky error word (shared by the heads; kept here per model)."""

    def __init__(self):
        self.ctr = 0
        self.done = 0
        self.err = 0


def run_launch(sync, arrivals, per_head, rng, offsets=None, err_from_host=False):
    """One launch of one head with a random interleaving of its blocks' steps:
    `arrivals` signalling blocks (offset per block from `offsets`, default 0)
    and `per_head` reduce blocks (offset 0).  A reduce block polls, reads the
    field of its own offset, counts itself past the wait (fetch-add), does
    its items, and if it counted last clears both words.  Returns the list of
    (arrivals seen when passing, trusted) per reduce block."""
    offsets = offsets or [0] * arrivals
    if err_from_host:
        sync.err = 1
    # actor programs as generators yielding after every shared-memory step
    seen = []

    def arriver(off):
        sync.ctr += 1 << (8 * off)          # atomic fetch-add
        yield

    def reducer():
        polls, timeout = 0, False
        while True:                        # poll, bounded like the kernel's wait
            v = sync.ctr
            yield
            if sum((v >> (8 * f)) & 0xff for f in range(8)) >= arrivals:
                break
            polls += 1
            if polls > 20_000:
                timeout = True
                sync.err = 1
                break
        ok = not timeout and ((v >> 0) & 0xff) == arrivals and sync.err == 0
        passed = sync.done                 # atomic fetch-add with return
        sync.done += 1
        yield
        seen.append((sum((v >> (8 * f)) & 0xff for f in range(8)), ok))
        yield                              # the items
        if passed == per_head - 1:         # the last to count clears
            sync.ctr = 0
            sync.done = 0
        yield

    actors = [arriver(o) for o in offsets] + [reducer() for _ in range(per_head)]
    # dispatch order: signalling blocks first, reduce blocks after (a reduce
    # block only starts once started; everything runs to completion)
    started = []
    pending = list(actors)
    while pending or started:   # every actor ends: arrivals at once, reducers within their bound
        if pending and (not started or rng.random() < 0.5):
            started.append(pending.pop(0))
        a = started[rng.integers(len(started))]
        try:
            next(a)
        except StopIteration:
            started.remove(a)
    return seen


@pytest.mark.parametrize("seed", range(40))
def test_reduce_sync_protocol_under_random_interleavings(seed):
    rng = np.random.default_rng(seed)
    sync = SyncModel()
    for launch in range(4):
        arrivals = int(rng.integers(1, 65))
        per_head = int(rng.integers(1, 25))
        seen = run_launch(sync, arrivals, per_head, rng)
        # every reduce block passed only after all arrivals, and trusted them
        assert len(seen) == per_head
        assert all(n == arrivals and ok for n, ok in seen)
        # the launch leaves the words zero for the next one
        assert sync.ctr == 0 and sync.done == 0


@pytest.mark.parametrize("seed", range(10))
def test_reduce_sync_protocol_flags_a_block_off_the_xcd_and_the_error_word(seed):
    rng = np.random.default_rng(100 + seed)
    sync = SyncModel()
    offsets = [0] * 20
    offsets[int(rng.integers(20))] = int(rng.integers(1, 8))   # one block elsewhere
    seen = run_launch(sync, 20, 6, rng, offsets=offsets)
    assert seen and not any(ok for _, ok in seen)
    assert sync.ctr == 0 and sync.done == 0
    seen = run_launch(sync, 20, 6, rng, err_from_host=True)
    assert not any(ok for _, ok in seen)
