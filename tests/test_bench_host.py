"""Host-side logic of bench.py (no GPU): the one-GPU guard, the counter
record tied to the kernel sources, and the CPU baseline's record."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as WL  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stored_traffic_follows_the_kernel_source_hash_and_workload(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic_update_f700.json")) as f:
        rec = json.load(f)
    assert rec["workload"] == "f700"
    live = bench.source_hash(bench.KERNEL_SOURCES["update"])
    if rec["source_sha256_16"] == live:
        assert bench.stored_traffic("update", "f700") == rec["hbm_bytes_per_launch"]
    # another workload's launch moves other bytes: no record, no figure
    for other in ("f8", "f100", "tiny", "stream256"):
        if not os.path.exists(os.path.join(ROOT, "profiles", f"traffic_update_{other}.json")):
            assert bench.stored_traffic("update", other) is None
    # a source that differs from the one the counters were taken on gives no figure
    monkeypatch.setattr(bench, "source_hash", lambda names: "0" * 16)
    assert bench.stored_traffic("update", "f700") is None
    assert bench.stored_traffic("no_such_kernel", "f700") is None


def test_extra_configs_cover_every_configuration():
    names = [c[0] for c in bench.EXTRA_CONFIGS]
    assert set(names) == {"tiny", "f8", "f100", "stream256", "f700x24", "fw700"}
    for name, steps, warmup in bench.EXTRA_CONFIGS:
        assert name in WL.WORKLOADS and steps >= 1 and warmup >= 1


def test_source_hash_covers_every_listed_file():
    h = bench.source_hash(bench.KERNEL_SOURCES["update"])
    assert len(h) == 16
    assert h != bench.source_hash(bench.KERNEL_SOURCES["update"][:1])


@pytest.mark.parametrize("step_rule", ["gradient", "newton_schulz"])
def test_cpu_baseline_record(step_rule):
    wl = WL.WORKLOADS["f8"]
    n = 64
    x = {key: t[:n] if key in ("q", "k", "v", "eta") else t
         for key, t in WL.make_inputs(wl.with_frames(1), seed=3).items()}
    host = {key: t.float().numpy().astype(np.float64) for key, t in x.items()}
    rec = bench.cpu_baseline(host, n, renorm=True, step_rule=step_rule)
    assert set(rec) == {"value", "unit", "cores", "kind", "sample"}
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert str(n) in rec["sample"] and bench.blas_name() in rec["sample"]


def test_bench_mirrors_the_update_plan_and_the_fused_reduce_rule():
    """bench.py names the update's kernel from its own copies of the planner's
    token-group rule and of the rule that reduces short chunks inside the
    update's launch; both must agree with the host model of the library."""
    import itertools
    import test_tiling_host as TH
    import workloads as WL
    for n, heads, h in itertools.product([1, 33, 1374, 5000, 10_992, 65_536, 137_400],
                                         [8, 16, 64], [128, 256]):
        assert bench.update_token_groups(n, heads, h) == TH.plan_update_tg(n, heads, h)[2]
    fused = {name: bench.update_fuses_reduce(wl) for name, wl in WL.WORKLOADS.items()}
    assert fused["stream256"] and fused["chunked256"]
    assert not fused["f700"] and not fused["f100"] and not fused["f8"] and not fused["tiny"]
    assert not bench.update_fuses_reduce(WL.WORKLOADS["stream256"], rule_gradient=False)
