"""Benchmark of the large-chunk TTT layer (update + apply) on one MI355X.

Default workload: 700 frames x 1374 tokens (518x518 frames, patch 14), 8 heads
of d 128, SwiGLU hidden 256, bf16 tokens and fp32 fast weights, one chunk:
update on all 961,800 tokens, then apply to all 961,800 queries, renorm on.
A step is one zm_ttt_update_apply call (weight cast, chunk-gradient partials,
reduce/step/renorm, apply).  Inputs are resident in HBM before timing starts.

Prints one JSON line on stdout.  Besides throughput it reports the roofline
position of the dominant kernel (algorithmic flops per launch / average launch
time from HIP events recorded by the library around that kernel on its own
stream) and the fp64 oracle timed on a bounded sample on this host's cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload f700]
                  [--step-rule gradient|newton_schulz]
                  [--cpu-sample-tokens N | --no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_F32_VALU_TFLOPS = 157.3   # MI355X fp32 vector peak
PEAK_HBM_GBS = 8000.0
# the source files of each roofline kernel (body header, then kernel entry)
STAGE_PASS_STEPS = 5  # steps of the untimed pass that times every stage
KERNEL_SOURCES = {"update": ("update_bf16.h", "update_bf16.hip"),
                  "apply": ("apply_bf16.h", "apply_bf16.hip")}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="f700",
                   choices=["f700", "f100", "f8", "f700x24", "stream256", "chunked256", "fw8",
                            "fw100", "fw700", "layer700"])
    p.add_argument("--seed", type=int, default=4)
    p.add_argument("--cpu-sample-tokens", type=int, default=0,
                   help="tokens for the oracle baseline (default: 262144 at the 8-head shape, "
                        "131072 at the full-width shape; 10-15 s of host time either way)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-renorm", action="store_true")
    p.add_argument("--order", default=None, choices=["apply_then_update", "update_then_apply"],
                   help="read/write order of the streaming and chunked workloads (default: "
                        "apply_then_update per streamed frame, update_then_apply per chunk)")
    p.add_argument("--step-rule", default="gradient", choices=["gradient", "newton_schulz"],
                   help="the update's step: W - g (default) or W - NewtonSchulz(g)")
    p.add_argument("--graph", action="store_true",
                   help="also time the step captured once in a HIP graph and replayed (no host "
                        "launch overhead per call)")
    p.add_argument("--no-configs", action="store_true",
                   help="with the default f700 workload, skip the other configurations (tiny, "
                        "f8, f100 + target view, stream256, f700x24, fw700) timed after it")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="first run one plain device copy of this many MiB (a known-size "
                        "reference dispatch for scaling HBM counters)")
    return p.parse_args()


def source_hash(names):
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "reconstruction_lact_chunk_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter record profiles/traffic_<kernel>_<workload>.json, if one
    exists and was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("workload") != workload:
        return None
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def make_events(torch, n):
    evs = []
    for _ in range(n):
        e = torch.cuda.Event(enable_timing=True)
        e.record()  # creates the underlying hipEvent_t
        evs.append(e)
    return evs


def blas_name():
    """The BLAS library NumPy was built against (name and version)."""
    import numpy as np
    try:
        b = np.__config__.CONFIG["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # pragma: no cover
        return "unknown BLAS"


def cpu_baseline(inputs_host, sample_tokens, renorm, step_rule="gradient"):
    """The fp64 oracle (as it stands) on the first `sample_tokens` tokens."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    x = {k: v.astype(np.float64) if k in ("w1", "w2", "w3") else v for k, v in inputs_host.items()}
    t0 = time.perf_counter()
    oracle.update_apply(x["k"], x["v"], x["eta"], x["q"], x["w1"], x["w2"], x["w3"], renorm=renorm,
                        step=step_rule)
    dt = time.perf_counter() - t0
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of the workload, all heads, update+apply "
                      f"(n_q = n_kv = {sample_tokens}), NumPy fp64 ({blas_name()}), {dt:.2f} s"}


def cpu_baseline_layer(xs, w_in, w_gate, gamma, w, sample_tokens, renorm, step_rule):
    """The fp64 oracle's whole layer on the first `sample_tokens` tokens."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    oracle.layer(xs, w_in, w_gate, gamma, *w, eta_scale=0.01, renorm=renorm, step=step_rule)
    dt = time.perf_counter() - t0
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of the workload through the whole layer "
                      f"(projections, update + apply, output gate), NumPy fp64 ({blas_name()}), "
                      f"{dt:.2f} s"}


# Configurations reported beside the headline, each in its own timed region:
# (name, timed steps, warm-up steps).  A stream256 step is 256 frames, an
# f700x24 step 24 layers; fw700 is the same 961,800 tokens through the one
# full-width head (d 1024, hidden 2048).
EXTRA_CONFIGS = (("tiny", 200, 20), ("f8", 100, 10), ("f100", 30, 5), ("stream256", 3, 1),
                 ("f700x24", 2, 1), ("fw700", 3, 1))


def time_region(torch, stream, fn, steps, warmup):
    """Average ms of fn() over `steps` calls after `warmup` untimed ones, from
    HIP events on `stream` with the device synchronised on both sides."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def update_fuses_reduce(wl, rule_gradient=True):
    """Whether the library reduces the update's partial sums inside the
    update's own launch (its frame_fuses_reduce): heads a multiple of 8, the
    gradient rule, and chunks short enough for the two-token-group update.
    The update stage's events then cover the update and its reduce."""
    n = wl.tokens_per_frame if wl.streaming else wl.n_kv
    return (wl.io_dtype == "bf16" and wl.d_head in (64, 128) and wl.heads % 8 == 0
            and rule_gradient and n > 0 and update_token_groups(n, wl.heads, wl.d_hidden) == 2)


def update_token_groups(n, heads, d_hidden):
    """The update's workgroup shape for n tokens (the library's plan_update):
    2 token groups when chunks of 4 32-token tiles would leave compute units
    idle, else 1."""
    nsl = max(d_hidden // 128, 1)
    target = max(256 // (heads * nsl), 1)
    return 2 if -(-(-(-n // 32)) // 4) < target and d_hidden >= 128 else 1


def stage_ms(torch, zm, fn, steps=5):
    """Average ms of the update partial sums (stage 1) and the apply (stage 3)
    over `steps` calls of fn, from the library's events around each stage."""
    evs = [make_events(torch, 8) for _ in range(steps)]
    for ev in evs:
        zm.set_profile_events(ev)
        fn()
    zm.set_profile_events(None)
    torch.cuda.synchronize()
    out = {}
    for nm, s in (("update", 1), ("apply", 3)):
        out[nm] = round(float(np.mean([ev[2 * s].elapsed_time(ev[2 * s + 1]) for ev in evs])), 4)
    return out


# The plain bf16 GEMM timed beside the headline for context: the layer's input
# projection (961,800 tokens of width 1024 to 3072 columns), through torch's
# vendor BLAS.  It shows what the chip's own dense GEMM sustains on the same
# box in the same process; it is not part of the timed path.
CONTEXT_GEMM = (961800, 1024, 3072)


def plain_gemm_context(dev, torch, reps=5, warmup=2):
    m, k, n = CONTEXT_GEMM
    g = torch.Generator(device=dev).manual_seed(12345)
    a = torch.randn(m, k, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(k, n, device=dev, dtype=torch.bfloat16, generator=g).contiguous()
    for _ in range(warmup):
        c = torch.matmul(a, b)
    torch.cuda.synchronize(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    tflops = 2.0 * m * k * n / (ms / 1e3) / 1e12
    return {"what": f"plain bf16 GEMM {m:,} x {k} by {k} x {n} (the layer's input projection), "
                    "torch.matmul through the vendor BLAS, same process and box as the headline",
            "ms": round(ms, 4), "achieved_tflops": round(tflops, 1),
            "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}


def run_configs(dev, torch, zm, WL, f700_inputs, seed):
    """The other configurations of the benchmark, each timed in its own region
    on the same stream: throughput, fraction of the bf16 matrix peak and, for
    streaming, the per-frame latency."""
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, steps, warmup in EXTRA_CONFIGS:
        wl = WL.WORKLOADS[name]
        log(f"config {name}: {steps} timed steps after {warmup} warm-up")
        if name == "f700x24":
            x = f700_inputs
        else:
            x = WL.make_inputs(wl, seed=seed, device=dev)
        io = zm.BF16 if wl.io_dtype == "bf16" else zm.F32
        desc = zm.make_desc(x["w1"], x["w2"], x["w3"], io, wl.renorm, x["q"], x["k"])
        p = wl.tokens_per_frame
        ws = torch.empty(zm.workspace_size(desc, p, p) if wl.streaming else
                         zm.workspace_size(desc, wl.n_kv, wl.n_q), dtype=torch.uint8, device=dev)
        o = torch.empty_like(x["q"])
        rec = {"workload": wl.description, "n_kv": wl.n_kv, "n_q": wl.n_q, "heads": wl.heads,
               "d_head": wl.d_head, "d_hidden": wl.d_hidden, "io": wl.io_dtype,
               "renorm": wl.renorm, "steps": steps, "warmup": warmup}
        flops = wl.flops_per_token_update() * wl.n_kv + wl.flops_per_token_apply() * wl.n_q
        if wl.streaming:
            state = [t.clone() for t in (x["w1"], x["w2"], x["w3"])]
            frames = WL.frame_slices(wl)

            def frame(s, e, reuse):
                zm.stream_step(x["q"][s:e], x["k"][s:e], x["v"][s:e], x["eta"][s:e], *state,
                               renorm=wl.renorm, order=zm.APPLY_THEN_UPDATE, out=o[s:e],
                               workspace=ws, emit_bf16=True, reuse_bf16=reuse)

            def fn():
                for i, (s, e) in enumerate(frames):
                    frame(s, e, i > 0)
            ms = time_region(torch, stream, fn, steps, warmup)
            lat = []
            for i, (s, e) in enumerate(frames):
                a, b = make_events(torch, 2)
                a.record(stream)
                frame(s, e, i > 0)
                b.record(stream)
                lat.append((a, b))
            torch.cuda.synchronize()
            lat = [a.elapsed_time(b) for a, b in lat]
            med = float(np.median(lat))
            rec.update({"order": "apply_then_update",
                        "bf16_copies": "kept in the workspace from frame to frame (the "
                                       "stream-step EMIT/REUSE flags)",
                        "ms_per_step": round(ms, 4),
                        "per_frame_ms": round(ms / wl.frames, 5),
                        "tokens_per_s": round(wl.n_kv / (ms / 1e3)),
                        "per_frame_latency_ms": {
                            "median": round(med, 4), "p99": round(float(np.percentile(lat, 99)), 4),
                            "tokens_per_s_at_median": round(p / (med / 1e3)),
                            "how": "HIP events around each frame's call, in a pass after the "
                                   "timed region"},
                        "frac_bf16_peak": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
        else:
            if wl.layers > 1:
                wsets = [WL.make_weights(wl.heads, wl.d_head, wl.d_hidden, seed, dev, layer=i)
                         for i in range(wl.layers)]
            else:
                wsets = [(x["w1"], x["w2"], x["w3"])]
            w_out = [tuple(torch.empty_like(w) for w in ws3) for ws3 in wsets]

            def one(li):
                zm.update_apply(x["k"], x["v"], x["eta"], x["q"], *wsets[li], renorm=wl.renorm,
                                w_out=w_out[li], out=o, workspace=ws)

            def fn():
                for li in range(len(wsets)):
                    one(li)
            ms = time_region(torch, stream, fn, steps, warmup)
            per_layer = ms / wl.layers
            rec.update({"ms_per_step": round(ms, 4), "per_layer_ms": round(per_layer, 4),
                        "tokens_per_s": round(wl.n_kv / (per_layer / 1e3)),
                        "frac_bf16_peak": round(flops / (per_layer / 1e3) / 1e12
                                                / PEAK_BF16_TFLOPS, 4),
                        "kernels_ms": stage_ms(torch, zm, lambda: one(0))})
            if update_fuses_reduce(wl):
                rec["kernels_ms"]["update_includes_reduce"] = True
            if name == "f100":
                rec["target_view_queries"] = wl.extra_queries
            del wsets, w_out
        out[name] = rec
        del ws, o
        if name != "f700x24":
            del x
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the layer's "
              "multi-GPU sharding is a design note only, not built.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import reconstruction_lact_chunk_amd as zm
    import workloads as WL

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WL.WORKLOADS[args.workload]
    wide = wl.d_head == 1024
    whole = wl.name.startswith("layer")
    renorm = not args.no_renorm and wl.renorm
    rule = zm.STEP_NEWTON_SCHULZ if args.step_rule == "newton_schulz" else zm.STEP_GRADIENT
    order_name = args.order or ("update_then_apply" if wl.chunked else "apply_then_update")
    order = zm.UPDATE_THEN_APPLY if order_name == "update_then_apply" else zm.APPLY_THEN_UPDATE
    log(f"workload {wl.name}: n_kv={wl.n_kv} n_q={wl.n_q} H={wl.heads} d={wl.d_head} "
        f"h={wl.d_hidden} layers={wl.layers}")
    if args.copy_calibration_mib > 0:
        nb = args.copy_calibration_mib << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {nb} bytes read, {nb} bytes written")
        del src, dst
    x = WL.make_inputs(wl, seed=args.seed, device=dev)
    layers = [x["w1"], x["w2"], x["w3"]]
    if wl.layers > 1:
        ws_layers = [WL.make_weights(wl.heads, wl.d_head, wl.d_hidden, args.seed, dev, layer=i)
                     for i in range(wl.layers)]
    else:
        ws_layers = [tuple(layers)]
    desc = zm.make_desc(x["w1"], x["w2"], x["w3"], zm.BF16, renorm, x["q"], x["k"], step_rule=rule)
    if wl.streaming:
        p = wl.tokens_per_frame
        n_ws = zm.workspace_size(desc, p, p)
    else:
        n_ws = zm.workspace_size(desc, wl.n_kv, wl.n_q)
    ws = torch.empty(n_ws, dtype=torch.uint8, device=dev)
    o = torch.empty_like(x["q"])
    w_out = [tuple(torch.empty_like(w) for w in wl_w) for wl_w in ws_layers]
    stream = torch.cuda.current_stream(dev)
    if whole:
        # the whole layer: tokens of the model width through the projections,
        # the TTT update + apply and the output gate
        lx, lw_in, lw_gate, lgamma = WL.make_layer_tensors(wl.n_kv, wl.heads, wl.d_head,
                                                           args.seed, dev)
        del x
        x = {}
        lo = torch.empty((wl.n_kv, wl.heads * wl.d_head), dtype=torch.bfloat16, device=dev)
        ldesc = zm.Desc(wl.heads, wl.d_head, wl.d_hidden, zm.BF16,
                        zm.RENORM_ROW if renorm else zm.RENORM_NONE, rule, wl.heads * wl.d_head)
        lws = torch.empty(zm.layer_workspace_size(ldesc, zm.make_layer_weights(
            lw_in, lw_gate, lgamma), wl.n_kv), dtype=torch.uint8, device=dev)
        del ws

    def step(prof=None):
        if wl.chunked:
            w = [t.clone() for t in ws_layers[0]]
            offsets = [0] + [e for _, e in WL.frame_slices(wl)]
            zm.chunked(x["q"], x["k"], x["v"], x["eta"], offsets, *w, renorm=renorm, order=order,
                       out=o, workspace=ws, step_rule=rule)
            return
        if wl.streaming:
            w = [t.clone() for t in ws_layers[0]]
            for i, (s, e) in enumerate(WL.frame_slices(wl)):
                zm.stream_step(x["q"][s:e], x["k"][s:e], x["v"][s:e], x["eta"][s:e], *w,
                               renorm=renorm, order=order, out=o[s:e], workspace=ws,
                               step_rule=rule, emit_bf16=True, reuse_bf16=i > 0)
            return
        for li, wl_w in enumerate(ws_layers):
            if prof is not None:
                zm.set_profile_events(prof[li])
            if whole:
                zm.layer(lx, lw_in, lw_gate, lgamma, *wl_w, renorm=renorm, step_rule=rule,
                         w_out=w_out[li], out=lo, workspace=lws)
                continue
            zm.update_apply(x["k"], x["v"], x["eta"], x["q"], *wl_w, renorm=renorm,
                            w_out=w_out[li], out=o, workspace=ws, step_rule=rule)
        if prof is not None:
            zm.set_profile_events(None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    flops_upd = wl.flops_per_token_update() * wl.n_kv
    flops_app = wl.flops_per_token_apply() * wl.n_q
    # Each event record costs the stream a few microseconds, so the timed
    # region records events only around the dominant kernel (the roofline's);
    # the other stages are timed in a separate pass after it.
    n_ev = 14 if whole else 10
    dom = "update" if flops_upd >= flops_app else "apply"
    dom_stage = 1 if dom == "update" else 3

    def dom_events():
        lst = [None] * n_ev
        lst[2 * dom_stage], lst[2 * dom_stage + 1] = make_events(torch, 2)
        return lst

    prof = None
    if not wl.streaming:
        prof = [[dom_events() for _ in ws_layers] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for k in range(K):
        step(prof[k] if prof else None)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end) / K

    graph_ms = None
    if args.graph:
        # one step captured on a side stream of default priority, then replayed
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(K):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / K
        log(f"graph replay: {graph_ms:.4f} ms per step")

    frame_ms = None
    if wl.streaming and not wl.chunked:
        # per-frame latency: events around every frame's call, in a pass after the timed region
        w = [t.clone() for t in ws_layers[0]]
        evs = []
        for i, (s, e) in enumerate(WL.frame_slices(wl)):
            a, b = make_events(torch, 2)
            a.record(stream)
            zm.stream_step(x["q"][s:e], x["k"][s:e], x["v"][s:e], x["eta"][s:e], *w,
                           renorm=renorm, order=order, out=o[s:e], workspace=ws, step_rule=rule,
                           emit_bf16=True, reuse_bf16=i > 0)
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        frame_ms = sorted(a.elapsed_time(b) for a, b in evs)

    stage_prof = None
    if not wl.streaming:  # the stage pass: every stage's events, outside the timed region
        stage_prof = [[make_events(torch, n_ev) for _ in ws_layers]
                      for _ in range(min(K, STAGE_PASS_STEPS))]
        for sp in stage_prof:
            step(sp)
        torch.cuda.synchronize()

    n_tok = wl.n_kv
    result = {
        "metric": "TTT update+apply tokens/sec per layer at 700 frames; % bf16 MFMA peak",
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    if wl.streaming:
        frames = wl.frames
        result["value"] = n_tok / (ms / 1e3)
        result["per_frame_ms"] = ms / frames
        if frame_ms:
            med = float(np.median(frame_ms))
            result["per_frame_latency_ms"] = {
                "median": round(med, 4), "p99": round(float(np.percentile(frame_ms, 99)), 4),
                "tokens_per_s_at_median": round(wl.tokens_per_frame / (med / 1e3)),
                "how": "HIP events on the stream around each frame's call, in a separate pass "
                       "after the timed region"}
    else:
        per_layer_ms = ms / wl.layers
        result["value"] = n_tok / (per_layer_ms / 1e3)
        result["layer_frac_bf16_peak"] = round((flops_upd + flops_app) / (per_layer_ms / 1e3) / 1e12
                                               / PEAK_BF16_TFLOPS, 4)
        # per-kernel durations from the library's event hooks
        names = {1: "update", 2: "reduce", 3: "apply", 0: "cast"}
        if rule == zm.STEP_NEWTON_SCHULZ:
            names[4] = "newton_schulz"
        if whole:
            names[5] = "project"
            names[6] = "output_gate"
        durs = {nm: [] for nm in names.values()}
        for sp in stage_prof:
            for ev in sp:
                for s, nm in names.items():
                    durs[nm].append(ev[2 * s].elapsed_time(ev[2 * s + 1]))
        avg = {nm: float(np.mean(v)) for nm, v in durs.items()}
        # the dominant kernel: its events inside the timed region
        avg[dom] = float(np.mean([ev[2 * dom_stage].elapsed_time(ev[2 * dom_stage + 1])
                                  for pk in prof for ev in pk]))
        units = {"update": (flops_upd, "update"), "apply": (flops_app, "apply")}
        kern = {}
        for nm in ("update", "apply"):
            fl, _ = units[nm]
            ach = fl / (avg[nm] / 1e3) / 1e12
            kern[nm] = {"avg_ms": round(avg[nm], 4), "achieved_tflops": round(ach, 1),
                        "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        if wide:
            kern["update"]["what"] = ("per 131,072-token block: e = W2^T v (hipBLASLt), the W1 / W3 "
                                      "products with the gate backward in their epilogue "
                                      "(k_wide_rows), the reduction products (hipBLASLt)")
            kern["apply"]["what"] = ("per 131,072-token block: the W1 / W3 products with the gate in "
                                     "their epilogue (k_wide_rows), O = U' W2'^T (hipBLASLt)")
        kern["cast"] = {"avg_ms": round(avg["cast"], 4)}
        kern["reduce"] = {"avg_ms": round(avg["reduce"], 4)}
        if whole:
            width = wl.heads * wl.d_head
            fl_proj = 2 * width * (3 * width + wl.heads) * n_tok
            fl_gate = 2 * width * width * n_tok
            kern["project"] = {"avg_ms": round(avg["project"], 4), "achieved_tflops": round(
                fl_proj / (avg["project"] / 1e3) / 1e12, 1), "what": "hipBLASLt GEMM x W_in^T "
                "(q, k, v and rate logits) + k_eta_from_logits"}
            kern["output_gate"] = {"avg_ms": round(avg["output_gate"], 4), "achieved_tflops": round(
                fl_gate / (avg["output_gate"] / 1e3) / 1e12, 1), "what": "hipBLASLt GEMM o' W_g^T "
                "+ k_rmsnorm_gate"}
            per_layer_ms = ms / wl.layers
            result["layer_flops_per_token"] = (fl_proj + fl_gate) // n_tok + \
                wl.flops_per_token_update() + wl.flops_per_token_apply()
            result["layer_frac_bf16_peak"] = round(
                (flops_upd + flops_app + fl_proj + fl_gate) / (per_layer_ms / 1e3) / 1e12
                / PEAK_BF16_TFLOPS, 4)
        if "newton_schulz" in avg:
            # five quintic steps per matrix: 4 M^2 N + 2 M^3 flops each (M = d, N = h)
            m, nn = wl.d_head, wl.d_hidden
            ns_flops = 3 * wl.heads * 5 * (4 * m * m * nn + 2 * m ** 3)
            kern["newton_schulz"] = {
                "avg_ms": round(avg["newton_schulz"], 4),
                "achieved_tflops": round(ns_flops / (avg["newton_schulz"] / 1e3) / 1e12, 2),
                "what": ("batched split-bf16 hipBLASLt GEMMs (3 per product) and elementwise "
                         "kernels" if wide else
                         f"one workgroup per matrix ({3 * wl.heads}), split-bf16 MFMA")}
        fl_dom = units[dom][0]
        ach = fl_dom / (avg[dom] / 1e3) / 1e12
        if wide:
            kname = ("update stage (hipBLASLt E and reduction GEMMs + k_wide_rows update)"
                     if dom == "update" else
                     "apply stage (k_wide_rows read + hipBLASLt output GEMM)")
        elif update_fuses_reduce(wl, rule == zm.STEP_GRADIENT):
            tg = update_token_groups(wl.n_kv, wl.heads, wl.d_hidden)
            kname = (f"k_frame_bf16<128,256,{tg}> (update and its reduce in one launch)"
                     if dom == "update" else "k_apply_bf16<128,256>")
            kern["reduce"]["in_update_launch"] = True
        else:
            kname = "k_update_bf16<128,256,1>" if dom == "update" else "k_apply_bf16<128,256>"
        result["roofline"] = {
            "kernel": kname,
            "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": None if wide else stored_traffic(dom, wl.name),
        }
        result["kernels"] = kern
        result["kernels_timing"] = (f"{dom}: HIP events around it in every timed step; other "
                                    f"stages: a separate pass of {len(stage_prof)} steps with "
                                    "events around every stage")
    result["config"] = {
        "workload": {"f700": "700 frames x 1374 tokens, one chunk: update on 961,800 tokens then "
                             "apply to 961,800 queries",
                     "f100": "100 frames x 1374 tokens + one 1374-token target view",
                     "f8": "8 frames x 1374 tokens",
                     "f700x24": "700-frame layer x 24 layers with fresh weights per layer",
                     "stream256": "256 frames x 1374 tokens, one streaming step per frame",
                     "chunked256": "256 frames x 1374 tokens as the 256 chunks of one "
                                   "zm_ttt_chunked call",
                     "fw8": "8 frames x 1374 tokens, one full-width head (d 1024, hidden 2048)",
                     "fw100": "100 frames x 1374 tokens, one full-width head (d 1024, hidden 2048)",
                     "fw700": "700 frames x 1374 tokens, one full-width head (d 1024, hidden "
                              "2048), one chunk",
                     "layer700": "700 frames x 1374 tokens of width 1024 through the whole layer: "
                                 "projections, update + apply (8 heads 128 / 256), output gate"
                     }[wl.name],
        "n_kv": wl.n_kv, "n_q": wl.n_q, "heads": wl.heads, "d_head": wl.d_head,
        "d_hidden": wl.d_hidden, "layers": wl.layers, "renorm": renorm,
        "io": "bf16 tokens, fp32 fast weights, fp32 accumulation",
        "step_rule": args.step_rule,
    }
    if wl.streaming:
        result["config"]["order"] = order_name
    result["wall_s_timed"] = round(wall, 3)
    if graph_ms is not None:
        result["graph_ms_per_step"] = round(graph_ms, 4)
        result["graph_value"] = (n_tok / (graph_ms / wl.layers / 1e3) if not wl.streaming
                                 else n_tok / (graph_ms / 1e3))

    if wl.name == "f700" and not args.no_configs and rule == zm.STEP_GRADIENT and renorm:
        result["configs"] = run_configs(dev, torch, zm, WL, x, args.seed)
        result["context"] = {"plain_bf16_gemm": plain_gemm_context(dev, torch)}

    if not args.no_cpu_baseline:
        sample = args.cpu_sample_tokens
        if sample <= 0:
            sample = 131072 if wide else 262144
        ns = min(sample, wl.n_kv)
        if whole:
            ns = min(ns, 131072)
            f64 = lambda t: t.to("cpu", torch.float64).numpy()  # noqa: E731
            log(f"cpu baseline: oracle layer on {ns} tokens")
            result["cpu_baseline"] = cpu_baseline_layer(
                f64(lx[:ns]), f64(lw_in), f64(lw_gate), f64(lgamma),
                [f64(t) for t in ws_layers[0]], ns, renorm, args.step_rule)
            print(json.dumps(result), flush=True)
            return
        host = {k: x[k][:ns].to("cpu", torch.float64).numpy() for k in ("q", "k", "v", "eta")}
        for k in ("w1", "w2", "w3"):
            host[k] = x[k].cpu().double().numpy()
        log(f"cpu baseline: oracle on {ns} tokens")
        result["cpu_baseline"] = cpu_baseline(host, ns, renorm, args.step_rule)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
