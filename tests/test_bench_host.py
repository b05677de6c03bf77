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


def test_stored_traffic_follows_the_kernel_source_hash(monkeypatch):
    n = WL.WORKLOADS["f700"].n_kv
    with open(os.path.join(ROOT, "profiles", "traffic_update_f700.json")) as f:
        rec = json.load(f)
    live = bench.source_hash(bench.KERNEL_SOURCES["update"])
    if rec["source_sha256_16"] == live:
        assert bench.stored_traffic("update", n) == rec["hbm_bytes_per_launch"]
    # a source that differs from the one the counters were taken on gives no figure
    monkeypatch.setattr(bench, "source_hash", lambda names: "0" * 16)
    assert bench.stored_traffic("update", n) is None
    assert bench.stored_traffic("no_such_kernel", n) is None


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
