"""Workload shapes against the figures the pages print, and generator determinism."""
import json
import math
import os

import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_patch_tokens_match_printed_example():
    g = golden()["patch_tokens_224"]
    extra = golden()["special_tokens"]
    assert W.SPECIAL_TOKENS == extra["camera"] + extra["register"]
    assert W.tokens_per_frame(g["image"], g["image"], g["patch"]) == g["patch_tokens"] + W.SPECIAL_TOKENS


def test_workload_token_counts():
    assert W.WORKLOADS["tiny"].tokens_per_frame == 30
    assert W.WORKLOADS["tiny"].n_kv == 120
    assert W.WORKLOADS["f8"].n_kv == 10_992
    assert W.WORKLOADS["f100"].n_kv == 137_400
    assert W.WORKLOADS["f100"].n_q == 138_774
    assert W.WORKLOADS["f700"].n_kv == 961_800
    assert W.WORKLOADS["stream256"].n_kv == 256 * 1374


def test_state_size_matches_printed_figure():
    g = golden()["state_size"]
    d, h = g["d"], g["hidden"]
    assert 3 * d * h == g["params_per_layer"] == 6 * d * d
    assert abs(g["params_per_layer"] / 1e6 - 6.29) < 0.005
    assert abs(g["layers"] * g["params_per_layer"] / 1e8 - 1.5) < 0.02
    # the 8-head layout keeps the block-diagonal share of that state
    wl = W.WORKLOADS["f700"]
    per_layer = 3 * wl.heads * wl.d_head * wl.d_hidden
    assert per_layer * wl.heads == g["params_per_layer"]


def test_flop_counts():
    wl = W.WORKLOADS["f700"]
    assert wl.flops_per_token_update() == 3_145_728
    assert wl.flops_per_token_apply() == 1_572_864


def test_generators_are_seeded_and_distributed():
    wl = W.WORKLOADS["f8"].with_frames(2)
    a = W.make_inputs(wl, seed=7)
    b = W.make_inputs(wl, seed=7)
    c = W.make_inputs(wl, seed=8)
    for key in a:
        assert torch.equal(a[key], b[key]), key
        assert not torch.equal(a[key], c[key]), key
    assert a["k"].dtype == torch.bfloat16 and a["k"].shape == (2748, 8, 128)
    assert a["eta"].shape == (2748, 8) and a["eta"].dtype == torch.float32
    assert float(a["eta"].min()) > 0 and float(a["eta"].max()) < 0.01
    std_k = a["k"].float().std().item()
    assert abs(std_k - 1 / math.sqrt(128)) < 0.01
    assert abs(a["w2"].std().item() - 1 / math.sqrt(256)) < 0.005
    # independent streams: k and v differ
    assert not torch.equal(a["k"], a["v"])


def test_extra_queries_follow_image_queries():
    wl = W.WORKLOADS["f100"].with_frames(1)
    x = W.make_inputs(wl, seed=3)
    assert x["q"].shape[0] == 1374 + 1374
    assert x["k"].shape[0] == 1374


def test_frame_slices():
    wl = W.WORKLOADS["stream256"].with_frames(3)
    assert W.frame_slices(wl) == [(0, 1374), (1374, 2748), (2748, 4122)]


def test_bad_image_size():
    with pytest.raises(ValueError):
        W.tokens_per_frame(100, 100)


def test_full_width_workloads_match_the_notes_state_size():
    """The full-width head is the notes' fast-weight state: d = 1024, hidden
    2048, 6 d^2 = 6,291,456 parameters per layer."""
    st = golden()["state_size"]
    for name in ("fw8", "fw100", "fw700"):
        wl = W.WORKLOADS[name]
        assert (wl.heads, wl.d_head, wl.d_hidden) == (1, st["d"], st["hidden"])
        assert 3 * wl.d_head * wl.d_hidden * wl.heads == st["params_per_layer"] == 6 * st["d"] ** 2
        assert wl.tokens_per_frame == 1374
    # the 8-head shape splits the same model width
    assert W.WORKLOADS["f700"].heads * W.WORKLOADS["f700"].d_head == st["d"]
