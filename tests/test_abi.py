"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/zm_ttt.h declares, and rejects bad arguments on the host with the
documented status codes before any HIP call is made."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import reconstruction_lact_chunk_amd as zm
from reconstruction_lact_chunk_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zm_ttt.h")

pytestmark = pytest.mark.skipif(not os.path.exists(zm.LIB_PATH),
                                reason="libzmttt.so not built (run the build first)")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ZM_API\s+[\w\s\*]+?\b(zm_\w+)\s*\(", text)))


def lib():
    return zm.load_library()


def test_header_declares_what_the_binding_knows():
    assert declared_functions() == sorted(B.EXPORTED)


def test_every_declared_symbol_is_exported():
    L = lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    syms = os.popen(f"nm -D --defined-only {zm.LIB_PATH}").read()
    exported = set(re.findall(r"\b(zm_\w+)\b", syms))
    assert exported == set(declared_functions())


def test_version_and_status_strings():
    assert zm.version() == 10400
    assert zm.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert zm.status_string(s) not in ("ok", "unknown status")
    assert zm.status_string(-99) == "unknown status"


def desc(heads=8, d=128, h=256, io=zm.BF16, renorm=1, ld=None, step_rule=0):
    return zm.Desc(heads, d, h, io, renorm, step_rule, heads * d if ld is None else ld)


def ws_size(de, n_kv, n_q):
    out = ctypes.c_size_t(0)
    st = lib().zm_ttt_workspace_size(ctypes.byref(de), n_kv, n_q, ctypes.byref(out))
    return st, out.value


def test_workspace_size_structure():
    de = desc()
    st0, base = ws_size(de, 0, 0)
    assert st0 == 0
    welems = 8 * 256 * 128
    # two bf16 weight sets and the shared launch's sync words (256 bytes per
    # head and one more block), no partial sums
    assert base == 2 * 4 * welems * 2 + 256 * (8 + 1)
    st, big = ws_size(de, 961_800, 961_800)
    assert st == 0
    # the partial-sum slots (3 h d fp32 per head each), then one fp32 per
    # update workgroup for the virtual loss (heads x h / 64 per slot: the
    # slices of a two-token-group plan), rounded up to 256 bytes
    parts = (big - base) // (3 * welems * 4)
    assert big == base + parts * 3 * welems * 4 + (parts * 8 * 4 * 4 + 255) // 256 * 256
    assert 1 <= parts <= 256
    # more tokens never need fewer partial sums; queries need no workspace
    sizes = [ws_size(de, n, 0)[1] for n in (1, 31, 32, 33, 1000, 10_992, 137_400, 961_800)]
    assert sizes == sorted(sizes)
    assert ws_size(de, 5000, 0)[1] == ws_size(de, 5000, 123_456)[1]


@pytest.mark.parametrize("field,value,expect", [
    ("heads", 0, zm.ERR_INVALID_ARG),
    ("heads", 65, zm.ERR_UNSUPPORTED),
    ("d_head", 96, zm.ERR_UNSUPPORTED),
    ("d_hidden", 512, zm.ERR_UNSUPPORTED),
    ("d_hidden", 0, zm.ERR_INVALID_ARG),
    ("io_dtype", 7, zm.ERR_INVALID_ARG),
    ("renorm", 2, zm.ERR_INVALID_ARG),
    ("step_rule", 2, zm.ERR_INVALID_ARG),
    ("step_rule", -1, zm.ERR_INVALID_ARG),
    ("ld_tok", 8 * 128 - 8, zm.ERR_INVALID_ARG),
    ("ld_tok", 8 * 128 + 4, zm.ERR_INVALID_ARG),
    ("ld_tok", (1 << 24) + 8, zm.ERR_INVALID_ARG),   # 32-bit in-tile token offsets
    ("ld_tok", 1 << 40, zm.ERR_INVALID_ARG),
])
def test_bad_descriptor(field, value, expect):
    de = desc()
    setattr(de, field, value)
    if field == "heads" and value > 0:
        de.ld_tok = value * de.d_head
    assert ws_size(de, 10, 10)[0] == expect


def test_largest_token_stride_accepted():
    assert ws_size(desc(ld=1 << 24), 10, 10)[0] == zm.OK


@pytest.mark.parametrize("heads,d,h", [(16, 64, 256), (8, 128, 256), (3, 64, 128), (1, 1024, 2048)])
def test_workspace_size_never_decreases(heads, d, h):
    # the header promises that a workspace sized for (n_kv, n_q) serves every
    # smaller call; a dense sweep, since the split plan is not monotonic in n
    de = desc(heads=heads, d=d, h=h)
    prev = 0
    for n in list(range(0, 6000)) + [131_071, 131_072, 131_073, 500_000]:
        st, size = ws_size(de, n, 0)
        assert st == zm.OK and size >= prev, (n, size, prev)
        prev = size
    prev = 0
    for n in (0, 1, 100, 131_072, 131_073, 400_000):
        size = ws_size(de, 0, n)[1]
        assert size >= prev
        prev = size


def test_workspace_for_the_longest_chunk_covers_shorter_ones():
    # zm_ttt_chunked sizes its workspace for the longest chunk; a shorter chunk
    # can realize more split slots (16 heads, hidden 256: 1058 tokens -> 7,
    # 949 tokens -> 8), so the size must cover the planned count
    import test_tiling_host as TH
    for heads, d, h in ((16, 64, 256), (8, 128, 256), (1, 128, 128), (3, 64, 256)):
        de = desc(heads=heads, d=d, h=h)
        slot = 3 * heads * h * d * 4
        base = ws_size(de, 0, 0)[1]
        rng = np.random.default_rng(heads * 1000 + d + h)
        for longest in rng.integers(1, 40_000, 40):
            need = max(TH.plan_update(int(m), heads, h)[0]
                       for m in range(1, int(longest) + 1, max(1, int(longest) // 200)))
            need = max(need, TH.plan_update(int(longest), heads, h)[0])
            assert ws_size(de, int(longest), int(longest))[1] - base >= need * slot
    de = desc(heads=16, d=64, h=256)
    assert ws_size(de, 1058, 1058)[1] - ws_size(de, 0, 0)[1] >= 8 * 3 * 16 * 256 * 64 * 4


@pytest.mark.parametrize("rule", [zm.STEP_GRADIENT, zm.STEP_NEWTON_SCHULZ])
def test_step_rules_accepted_without_extra_workspace(rule):
    assert ws_size(desc(step_rule=rule), 10_992, 10_992) == ws_size(desc(), 10_992, 10_992)


def test_full_width_shape_workspace_and_limits():
    de = desc(heads=1, d=1024, h=2048)
    st, base = ws_size(de, 0, 0)
    assert st == 0
    welems = 1024 * 2048
    sets = 2 * 4 * welems * 2
    gemm_ws = 64 << 20
    assert base == sets + gemm_ws
    blk = 131072
    # token-block buffers (3 h bf16 per token, at most one block); 8 fp32
    # partial slots of 3 h d (one for fewer than 8 tokens), and with an update
    # one more 3 h d for the slots' sum in natural layouts
    slot = 3 * welems * 4
    assert ws_size(de, 1000, 0)[1] == base + 1000 * 3 * 2048 * 2 + 8 * slot + slot
    assert ws_size(de, 5, 0)[1] == base + 5 * 3 * 2048 * 2 + slot + slot
    assert ws_size(de, 0, 1000)[1] == base + 1000 * 3 * 2048 * 2
    assert ws_size(de, 200_000, 10)[1] == base + blk * 3 * 2048 * 2 + 8 * slot + slot
    assert ws_size(desc(heads=1, d=1024, h=2048, io=zm.F32), 10, 10)[0] == zm.ERR_UNSUPPORTED
    # the Newton-Schulz rule adds its iteration buffers (fp32 X, B X, A, A^2 and
    # the bf16 planes of X and A for the three matrices, plus norm partials)
    st, ns = ws_size(desc(heads=1, d=1024, h=2048, step_rule=zm.STEP_NEWTON_SCHULZ), 1000, 0)
    assert st == zm.OK
    M, N = 1024, 2048
    ns_bytes = 2 * 3 * M * N * 4 + 2 * 3 * M * M * 4 + 2 * 3 * M * N * 2 + 2 * 3 * M * M * 2 + 768
    assert ns == ws_size(de, 1000, 0)[1] + ns_bytes
    assert ws_size(desc(heads=1, d=1024, h=1024), 10, 10)[0] == zm.ERR_UNSUPPORTED


def test_null_descriptor_and_counts():
    out = ctypes.c_size_t(0)
    assert lib().zm_ttt_workspace_size(None, 1, 1, ctypes.byref(out)) == zm.ERR_INVALID_ARG
    de = desc()
    assert ws_size(de, -1, 0)[0] == zm.ERR_INVALID_ARG
    assert ws_size(de, 0, -5)[0] == zm.ERR_INVALID_ARG
    assert lib().zm_ttt_workspace_size(ctypes.byref(de), 1, 1, None) == zm.ERR_INVALID_ARG


P = ctypes.c_void_p
GOOD = P(1 << 20)       # 1 MiB: aligned to anything; never dereferenced here
ODD = P((1 << 20) + 2)  # misaligned for every check


def call_update(de, n, k=GOOD, v=GOOD, eta=GOOD, w=(GOOD, GOOD, GOOD), wo=(GOOD, GOOD, GOOD),
                ws=GOOD, ws_bytes=0):
    return lib().zm_ttt_update(ctypes.byref(de), n, k, v, eta, *w, *wo, ws, ws_bytes, None)


def call_update_loss(de, n, loss=GOOD, k=GOOD, ws_bytes=0):
    return lib().zm_ttt_update_loss(None if de is None else ctypes.byref(de), n, k, GOOD, GOOD,
                                    GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, loss, GOOD, ws_bytes, None)


def test_update_loss_rejects_before_any_hip_call():
    de = desc()
    need = ws_size(de, 100, 0)[1]
    # only the bf16 narrow-head update carries the loss
    assert call_update_loss(desc(io=zm.F32), 100, ws_bytes=need) == zm.ERR_UNSUPPORTED
    wd = desc(heads=1, d=1024, h=2048)
    assert call_update_loss(wd, 100, ws_bytes=ws_size(wd, 100, 0)[1]) == zm.ERR_UNSUPPORTED
    assert "bf16 narrow-head" in zm.last_error()
    # a null or misaligned loss pointer, then the update's own checks
    assert call_update_loss(de, 100, loss=None, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update_loss(de, 100, loss=P((1 << 20) + 2), ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update_loss(de, 100, k=None, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update_loss(de, 100, ws_bytes=need - 1) == zm.ERR_WORKSPACE
    assert call_update_loss(None, 100, ws_bytes=need) == zm.ERR_INVALID_ARG
    with pytest.raises(zm.ZmError, match="fp32 tensor"):
        w1, w2 = torch.zeros(1, 128, 64), torch.zeros(1, 64, 128)
        zm.update_loss(*[torch.zeros(3, 1, 64, dtype=torch.bfloat16)] * 2, torch.zeros(3, 1),
                       w1, w2, w1.clone(), loss=torch.zeros(2))


def test_update_rejects_bad_pointers_before_any_hip_call():
    de = desc()
    need = ws_size(de, 100, 0)[1]
    assert call_update(de, 100, k=None, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update(de, 100, v=ODD, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update(de, 100, eta=None, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update(de, 100, eta=P((1 << 20) + 1), ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update(de, 100, w=(GOOD, None, GOOD), ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update(de, 100, wo=(GOOD, GOOD, ODD), ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update(de, 100, ws=None, ws_bytes=need) == zm.ERR_WORKSPACE
    assert call_update(de, 100, ws=P((1 << 20) + 128), ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_update(de, 100, ws_bytes=need - 1) == zm.ERR_WORKSPACE
    assert call_update(de, -3, ws_bytes=need) == zm.ERR_INVALID_ARG
    bad = desc(d=48)
    assert call_update(bad, 100, ws_bytes=need) == zm.ERR_UNSUPPORTED


def test_apply_update_apply_stream_reject_bad_arguments():
    L = lib()
    de = desc()
    need = ws_size(de, 100, 100)[1]
    assert L.zm_ttt_apply(ctypes.byref(de), 100, None, GOOD, GOOD, GOOD, GOOD, GOOD, need,
                          None) == zm.ERR_INVALID_ARG
    assert L.zm_ttt_apply(ctypes.byref(de), 100, GOOD, GOOD, GOOD, GOOD, ODD, GOOD, need,
                          None) == zm.ERR_INVALID_ARG
    assert L.zm_ttt_apply(ctypes.byref(de), 100, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 16,
                          None) == zm.ERR_WORKSPACE
    assert L.zm_ttt_update_apply(ctypes.byref(de), 100, GOOD, GOOD, GOOD, 100, None, GOOD, GOOD,
                                 GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, need,
                                 None) == zm.ERR_INVALID_ARG
    assert L.zm_ttt_update_apply(ctypes.byref(de), 100, GOOD, GOOD, GOOD, 100, GOOD, GOOD, GOOD,
                                 GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, need - 256,
                                 None) == zm.ERR_WORKSPACE
    for order in (-1, 2):
        assert L.zm_ttt_stream_step(ctypes.byref(de), order, 100, GOOD, GOOD, GOOD, GOOD, GOOD,
                                    GOOD, GOOD, GOOD, GOOD, need, None) == zm.ERR_INVALID_ARG
    assert L.zm_ttt_stream_step(ctypes.byref(de), 0, 100, GOOD, GOOD, GOOD, None, GOOD, GOOD,
                                GOOD, GOOD, GOOD, need, None) == zm.ERR_INVALID_ARG


def call_chunked(de, offsets, order=0, mask=None, inner=1, q=GOOD, eta=GOOD, ws_bytes=0,
                 n_chunks=None):
    offs = None if offsets is None else (ctypes.c_int64 * len(offsets))(*offsets)
    nc = (len(offsets) - 1 if offsets is not None else 1) if n_chunks is None else n_chunks
    m = None if mask is None else (ctypes.c_uint8 * len(mask))(*mask)
    return lib().zm_ttt_chunked(ctypes.byref(de), order, nc, offs, m, inner, q, GOOD, GOOD, eta,
                                GOOD, GOOD, GOOD, GOOD, GOOD, ws_bytes, None)


def test_chunked_rejects_bad_schedules_before_any_hip_call():
    de = desc()
    need = ws_size(de, 600, 600)[1]        # the longest chunk below has 600 tokens
    good = [0, 400, 1000, 1200]
    assert call_chunked(de, good, order=2, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_chunked(de, good, inner=0, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_chunked(de, good, inner=65, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_chunked(de, [5, 400, 1000], ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_chunked(de, [0, 400, 300], ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_chunked(de, None, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_chunked(de, good, n_chunks=-1, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_chunked(de, good, n_chunks=(1 << 24) + 1, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_chunked(de, good, q=None, ws_bytes=need) == zm.ERR_INVALID_ARG
    assert call_chunked(de, good, eta=P((1 << 20) + 2), ws_bytes=need) == zm.ERR_INVALID_ARG
    # the workspace is sized by the longest chunk, not the whole sequence
    short = ws_size(de, 599, 599)[1]
    if short < need:
        assert call_chunked(de, good, ws_bytes=short) == zm.ERR_WORKSPACE
    assert call_chunked(desc(d=48), good, ws_bytes=need) == zm.ERR_UNSUPPORTED
    # no chunks, or only empty ones: valid and nothing to launch
    assert call_chunked(de, [0], ws_bytes=ws_size(de, 0, 0)[1]) == zm.OK
    assert call_chunked(de, [0, 0, 0], q=None, eta=None, ws_bytes=ws_size(de, 0, 0)[1]) == zm.OK


def lw_struct(d_in=1024, eta_scale=0.01, eps=1e-6, reserved=0, w_in=GOOD, gamma=GOOD):
    return zm.LayerWeights(w_in.value if w_in is not None else None, GOOD.value,
                           gamma.value if gamma is not None else None, d_in, eta_scale, eps,
                           reserved)


def layer_ws(de, lw, n):
    out = ctypes.c_size_t(0)
    st = lib().zm_ttt_layer_workspace_size(ctypes.byref(de), ctypes.byref(lw), n,
                                           ctypes.byref(out))
    return st, out.value


def test_layer_workspace_and_argument_checks():
    de = desc()
    lw = lw_struct()
    st, need = layer_ws(de, lw, 1000)
    assert st == zm.OK
    # projection rows (3 H d + H rounded to 8 bf16), eta, the GEMM workspace, the TTT workspace
    ttt = ws_size(desc(ld=3136), 1000, 1000)[1]
    rows = 1000 * 3136 * 2                        # 3 H d + H = 3080 columns, rows padded to 64
    eta = (1000 * 8 * 4 + 255) // 256 * 256
    assert need == rows + eta + (64 << 20) + ttt
    assert layer_ws(desc(io=zm.F32), lw, 10)[0] == zm.ERR_UNSUPPORTED
    # layer width H d: 8 full-width heads (8192) are accepted, 9 (9216) are not
    assert layer_ws(desc(heads=8, d=1024, h=2048, ld=8192), lw, 10)[0] == zm.OK
    assert layer_ws(desc(heads=9, d=1024, h=2048, ld=9216), lw, 10)[0] == zm.ERR_UNSUPPORTED
    for bad in (lw_struct(d_in=12), lw_struct(d_in=0), lw_struct(eta_scale=-1.0),
                lw_struct(eps=0.0), lw_struct(reserved=1), lw_struct(w_in=None),
                lw_struct(gamma=P((1 << 20) + 4))):
        assert layer_ws(de, bad, 10)[0] == zm.ERR_INVALID_ARG
    L = lib()

    def call(n=1000, x=GOOD, ld_x=1024, o=GOOD, ws_bytes=need, de=de):
        return L.zm_ttt_layer(ctypes.byref(de), ctypes.byref(lw), n, x, ld_x, GOOD, GOOD, GOOD,
                              GOOD, GOOD, GOOD, o, GOOD, ws_bytes, None)
    assert call(x=None) == zm.ERR_INVALID_ARG
    assert call(ld_x=1000) == zm.ERR_INVALID_ARG         # < d_in
    assert call(ld_x=1028) == zm.ERR_INVALID_ARG         # not a multiple of 8
    assert call(o=ODD) == zm.ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == zm.ERR_WORKSPACE
    assert call(de=desc(ld=1016)) == zm.ERR_INVALID_ARG   # o rows narrower than H d


def test_profile_event_argument_checks():
    L = lib()
    assert L.zm_ttt_set_profile_events(None, 3) == zm.ERR_INVALID_ARG
    arr = (ctypes.c_void_p * 10)()
    assert L.zm_ttt_set_profile_events(arr, 4) == zm.ERR_INVALID_ARG
    assert L.zm_ttt_set_profile_events(arr, 9) == zm.ERR_INVALID_ARG
    assert L.zm_ttt_set_profile_events(arr, 8) == zm.OK
    assert L.zm_ttt_set_profile_events(arr, 10) == zm.OK
    arr14 = (ctypes.c_void_p * 14)()
    assert L.zm_ttt_set_profile_events(arr14, 14) == zm.OK
    assert L.zm_ttt_set_profile_events(arr14, 12) == zm.ERR_INVALID_ARG
    assert L.zm_ttt_set_profile_events(None, 0) == zm.OK


def test_binding_rejects_host_tensors_and_bad_shapes():
    w1 = torch.zeros(2, 128, 64)
    w2 = torch.zeros(2, 64, 128)
    w3 = torch.zeros(2, 128, 64)
    q = torch.zeros(10, 2, 64)
    with pytest.raises(zm.ZmError):
        zm.apply(q, w1, w2, w3)             # host tensors
    with pytest.raises(zm.ZmError):
        zm.make_desc(w1, w2.transpose(1, 2), w3, zm.F32, False)
    with pytest.raises(zm.ZmError):
        zm.make_desc(w1.double(), w2, w3, zm.F32, False)


def _host_case(n=10, heads=2, d=64, h=128, dtype=torch.float32):
    w1, w3 = torch.zeros(heads, h, d), torch.zeros(heads, h, d)
    w2 = torch.zeros(heads, d, h)
    tok = lambda m: torch.zeros(m, heads, d, dtype=dtype)  # noqa: E731
    return w1, w2, w3, tok, torch.zeros(n, heads)


def test_binding_checks_every_token_tensor_whatever_its_length():
    # Shape, dtype and stride errors are reported before the device check, so
    # host tensors reach them here; nothing is launched.
    w1, w2, w3, tok, eta = _host_case()
    with pytest.raises(zm.ZmError, match="io dtype"):      # one query row of the wrong dtype
        zm.update_apply(tok(10), tok(10), eta, tok(1).to(torch.bfloat16), w1, w2, w3)
    with pytest.raises(zm.ZmError, match=r"shape \(1, 3, 64\)"):
        zm.update_apply(tok(10), tok(10), eta, torch.zeros(1, 3, 64), w1, w2, w3)
    bad_stride = torch.zeros(1, 64, 2).transpose(1, 2)     # [1, 2, 64], d not unit-stride
    with pytest.raises(zm.ZmError, match="unit stride"):
        zm.apply(bad_stride, w1, w2, w3)
    with pytest.raises(zm.ZmError, match="unit stride"):
        zm.update(bad_stride, tok(1), torch.zeros(1, 2), w1, w2, w3)
    with pytest.raises(zm.ZmError, match="on the GPU"):    # well-formed host tensors
        zm.update_apply(tok(10), tok(10), eta, tok(1), w1, w2, w3)


def test_binding_checks_output_rows_and_weight_shapes():
    w1, w2, w3, tok, eta = _host_case()
    with pytest.raises(zm.ZmError, match="9 rows"):
        zm.apply(tok(10), w1, w2, w3, out=tok(9))
    with pytest.raises(zm.ZmError, match="11 rows"):
        zm.update_apply(tok(10), tok(10), eta, tok(10), w1, w2, w3, out=tok(11))
    with pytest.raises(zm.ZmError, match="1 rows"):        # a one-row output for ten queries
        zm.stream_step(tok(10), tok(10), tok(10), eta, w1, w2, w3, out=tok(1))
    with pytest.raises(zm.ZmError, match="10 rows, the call needs 9"):  # v longer than k
        zm.update(tok(9), tok(10), eta, w1, w2, w3)
    with pytest.raises(zm.ZmError, match="5 rows"):
        zm.chunked(tok(10), tok(10), tok(10), eta, [0, 4, 10], w1, w2, w3, out=tok(5))
    small = (torch.zeros(2, 64, 64), w2.clone(), w3.clone())
    with pytest.raises(zm.ZmError, match="output W1"):
        zm.update(tok(10), tok(10), eta, w1, w2, w3, out=small)
    with pytest.raises(zm.ZmError, match="output W2"):
        zm.update_apply(tok(10), tok(10), eta, tok(10), w1, w2, w3,
                        w_out=(w1.clone(), torch.zeros(2, 64, 64), w3.clone()))


def test_binding_checks_the_layer_output():
    heads, d, h, d_in, n = 2, 64, 128, 64, 6
    w1, w3 = torch.zeros(heads, h, d), torch.zeros(heads, h, d)
    w2 = torch.zeros(heads, d, h)
    x = torch.zeros(n, d_in, dtype=torch.bfloat16)
    w_in = torch.zeros(3 * heads * d + heads, d_in, dtype=torch.bfloat16)
    w_gate = torch.zeros(heads * d, heads * d, dtype=torch.bfloat16)
    gamma = torch.ones(heads * d)
    with pytest.raises(zm.ZmError, match="out must be bf16"):
        zm.layer(x, w_in, w_gate, gamma, w1, w2, w3, out=torch.zeros(n - 1, heads * d,
                                                                      dtype=torch.bfloat16))
    with pytest.raises(zm.ZmError, match="out must be bf16"):
        zm.layer(x, w_in, w_gate, gamma, w1, w2, w3, out=torch.zeros(n, heads * d))
    with pytest.raises(zm.ZmError, match="output W3"):
        zm.layer(x, w_in, w_gate, gamma, w1, w2, w3,
                 w_out=(w1.clone(), w2.clone(), torch.zeros(heads, h, d + 8)))
    with pytest.raises(zm.ZmError, match="on the GPU"):
        zm.layer(x, w_in, w_gate, gamma, w1, w2, w3)


def test_undersized_workspaces_are_rejected_before_any_launch():
    # the sequence that once overran the partial sums: a 1058-token chunk
    # followed by a 949-token one (16 heads, hidden 256: 7 then 8 splits); a
    # workspace with fewer slots than the longest chunk plans is refused
    offs = [0, 1058, 2007]
    for (heads, d, h), longest in (((16, 64, 256), 500), ((16, 64, 256), 700),
                                   ((8, 128, 256), 949), ((8, 128, 256), 1000)):
        de = desc(heads=heads, d=d, h=h)
        assert ws_size(de, longest, longest)[1] < ws_size(de, 1058, 1058)[1]
        assert call_chunked(de, offs, ws_bytes=ws_size(de, longest, longest)[1]) == \
            zm.ERR_WORKSPACE, (heads, longest)
    # the full-width head: token-block buffers hold min(n, 131072) rows of 3 h
    wd = desc(heads=1, d=1024, h=2048)
    L = lib()
    for n_kv, n_q, sized_for in ((131_072, 0, (131_071, 0)), (1000, 200_000, (1000, 1000)),
                                 (200_000, 10, (131_000, 10)), (8, 0, (7, 0))):
        need = ws_size(wd, *sized_for)[1]
        st = L.zm_ttt_update_apply(ctypes.byref(wd), n_kv, GOOD, GOOD, GOOD, n_q, GOOD, GOOD,
                                   GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, need, None)
        assert st == zm.ERR_WORKSPACE, (n_kv, n_q)
    assert L.zm_ttt_apply(ctypes.byref(wd), 131_073, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,
                          ws_size(wd, 0, 100_000)[1], None) == zm.ERR_WORKSPACE


def test_stream_flags_are_validated_with_the_order():
    L = lib()
    de = desc()
    need = ws_size(de, 100, 100)[1]
    args = (GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD)
    # unknown bits around the two flags are rejected before any HIP call
    for order in (0x400, 0x101 | 0x800, 0x1000, 2 | zm.STREAM_EMIT_BF16):
        assert L.zm_ttt_stream_step(ctypes.byref(de), order, 100, *args, need, None) == \
            zm.ERR_INVALID_ARG, hex(order)
    # a valid order with flags still runs the other checks (bad eta pointer here)
    assert L.zm_ttt_stream_step(ctypes.byref(de), 1 | zm.STREAM_EMIT_BF16 | zm.STREAM_REUSE_BF16,
                                100, GOOD, GOOD, GOOD, None, GOOD, GOOD, GOOD, GOOD, GOOD, need,
                                None) == zm.ERR_INVALID_ARG
    with pytest.raises(zm.ZmError, match="reuse_bf16"):
        zm.stream_step(*[torch.zeros(1)] * 7, reuse_bf16=True)


def test_scratch_entry_point_limits_before_any_hip_call():
    L = lib()
    args = (GOOD, GOOD, GOOD)
    # a call needing more workspace than the library's scratch: refused on the
    # host.  The split count is capped by the compute units, so the need stops
    # growing with n (8 heads of 128 / 256: 54.5 MB at any length); 64 heads
    # need 84 MB.
    de = desc()
    many_heads = desc(heads=64)
    assert ws_size(many_heads, 100_000, 0)[1] > zm.SCRATCH_BYTES
    assert L.zm_ttt_update_apply_scratch(ctypes.byref(many_heads), 100_000, *args, 0, GOOD, GOOD,
                                         GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None) == \
        zm.ERR_WORKSPACE
    assert "scratch" in zm.last_error()
    # the full-width head has no scratch variant
    wd = desc(heads=1, d=1024, h=2048)
    assert L.zm_ttt_update_apply_scratch(ctypes.byref(wd), 10, *args, 10, GOOD, GOOD, GOOD, GOOD,
                                         GOOD, GOOD, GOOD, GOOD, None) == zm.ERR_UNSUPPORTED
    # the usual argument checks (null q with queries)
    assert L.zm_ttt_update_apply_scratch(ctypes.byref(de), 100, *args, 100, None, GOOD, GOOD,
                                         GOOD, GOOD, GOOD, GOOD, GOOD, None) == zm.ERR_INVALID_ARG
    assert L.zm_ttt_update_apply_scratch(None, 100, *args, 100, GOOD, GOOD, GOOD, GOOD, GOOD,
                                         GOOD, GOOD, GOOD, None) == zm.ERR_INVALID_ARG
    # the largest 700-frame layer fits
    f700 = ws_size(de, 961_800, 961_800)[1]
    assert f700 <= zm.SCRATCH_BYTES


def test_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define ZM_TTT_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == zm.SCRATCH_BYTES
