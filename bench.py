"""Benchmark of Loki decode attention on one MI355X.

Workload: the Llama2-13B-shaped run (B=16, 40 query = 40 KV heads, D=128,
bf16 cache, k_f = d_f = 0.25 -> d = 32) in steady state at S = 3584 cached
tokens (prompt 3072 + 512 generated, the longest cache of the run).  One
step = append the step's new key/value of every sequence at position S-1
(rotate into the PCA basis, split, store) + one Loki decode over all S
tokens (k = 896).  Several copies of the cache ("layers") are cycled so that
a step never finds the previous step's bytes in the 256 MB last-level cache.

Prints one JSON line: head-queries/s of the whole step, per-kernel HBM
roofline of the decode kernel (HIP events on the launch stream), the
same-GPU dense baseline, the pages' 3072 + 512 generation run (decode time
summed with append excluded, as the pages time it) and the CPU oracle on a
bounded sample.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Loki decode attention: head-queries/s + achieved HBM GB/s (13B shape, S=3584)"
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["device.hpp", "select.hpp", "attend.hpp", "score.hpp", "fused_kernels.hip"]


def code_tokens(text: str) -> str:
    """Source text without // comments, with every run of whitespace made one
    space."""
    return " ".join(re.sub(r"//[^\n]*", "", text).split())


def kernel_source_hash() -> str:
    """Hash of the fused kernel's sources with comments and layout removed, so
    that a comment edit does not retire the recorded traffic counters but any
    change of code does."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_attention_decode_loki_amd", "csrc", f)) as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, S, k) -> dict:
    """Bytes Loki must move per decode: the d-wide key slab of every cached
    token once per KV head, plus k full key rows and k value rows per query
    head."""
    e = w.esize
    slab = w.B * w.Hkv * S * w.d * e
    rows = w.B * w.Hq * k * 2 * w.D * e
    dense = w.B * w.Hkv * S * 2 * w.D * e
    return {"slab": slab, "rows": rows, "total": slab + rows, "dense": dense}


def live_traffic(args, log):
    """HBM bytes per launch of the fused step kernel, measured now: two child
    runs of this script's step (20 + 5 launches, no other measurement) under
    rocprofv3, one counter each (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch), each scaled by what the same counter reads for a plain 1 GiB
    device copy in the same child.  Returns (bytes, detail) or (None, reason).
    The children start after every timed measurement of this process."""
    import glob
    import shutil
    import signal
    import subprocess
    import tempfile
    prof = shutil.which("rocprofv3")
    if prof is None:
        return None, "rocprofv3 not found"
    base = [sys.executable, os.path.abspath(__file__), "--config", args.config,
            "--no-per-config", "--no-cpu", "--no-jaccard", "--no-run", "--no-dense",
            "--no-read-probe", "--no-live-traffic", "--steps", "20", "--warmup", "5",
            "--settle", "0", "--copy-probe-mib", "1024"]
    if args.rope_base is not None:
        base += ["--rope-base", str(args.rope_base)]
    env = dict(os.environ, TMPDIR="/tmp")
    per = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        out = tempfile.mkdtemp(prefix="loki_pmc_", dir="/tmp")
        cmd = [prof, "--pmc", counter, "-f", "csv", "-d", out, "-o", "p", "--"] + base
        log(f"counter run: {counter}")
        p = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL, env=env,
                             start_new_session=True)
        try:
            p.wait(timeout=120)
        except subprocess.TimeoutExpired:
            os.killpg(p.pid, signal.SIGKILL)
            p.wait()
            return None, f"{counter} run timed out"
        # (the profiler can exit non-zero after the program ended with its
        # results complete; the files decide)
        vals = {}
        for f in glob.glob(os.path.join(out, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r.get("Counter_Name") == counter:
                        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        shutil.rmtree(out, ignore_errors=True)
        copy = [max(v) for k, v in vals.items() if "copyBuffer" in k]
        step = [v for k, v in vals.items()
                if re.search(r"fused_kernel<[^>]*, (true|false), true, \d+>", k)]
        if not copy or len(step) != 1:
            return None, f"{counter}: no copy or step dispatches in the counter output"
        scale = 1048576.0 / max(copy)
        per[counter] = (float(np.median(step[0])) * 1024.0 * scale, scale, len(step[0]))
    total = per["FETCH_SIZE"][0] + per["WRITE_SIZE"][0]
    detail = {"fetch_bytes": per["FETCH_SIZE"][0], "write_bytes": per["WRITE_SIZE"][0],
              "fetch_scale": per["FETCH_SIZE"][1], "write_scale": per["WRITE_SIZE"][1],
              "dispatches": per["FETCH_SIZE"][2]}
    return total, detail


def measured_traffic(kernel_hash: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_fused_decode_step_{workload}.txt")
    if not os.path.exists(p):
        return None
    t = {}
    with open(p) as fh:
        for line in fh:
            if "=" in line:
                key, val = line.split("=", 1)
                t[key.strip()] = val.strip()
    if t.get("kernel_source_hash") != kernel_hash:
        return None
    return float(t["hbm_bytes_per_launch"])


def timed(torch, fn, n):
    """Launch fn(i) for i < n back to back between two HIP events on the
    launch stream; returns (wall ms per call, event ms per call)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / n, e0.elapsed_time(e1) / n


_QUEUE = {}  # the delay reads' buffer and time, and the host's last submission time


# (bytes, workgroups, threads, loads in flight per lane, which launch it mirrors)
FLOOR_SHAPES = [
    (440_401_920, 640, 512, 4, "13B step: one 512-thread workgroup per row"),
    (440_401_920, 640, 512, 8, "13B step grid, deeper loads"),
    (440_401_920, 2048, 256, 4, "13B step bytes, many workgroups"),
    (33_554_432, 256, 512, 4, "Llama3-8B grouped ranking: one workgroup per CU"),
    (33_554_432, 256, 512, 16, "Llama3-8B grouped ranking, deeper loads"),
    (134_217_728, 1024, 256, 4, "Mistral ranking pass grid"),
    (268_435_456, 2048, 256, 4, "Llama3-8B dense bytes"),
    (536_870_912, 2048, 256, 4, "Mistral dense bytes"),
]


def timed_queued(torch, fn, n):
    """Per-launch GPU time of fn(i), i < n, launched back to back: the
    launches are queued behind a GPU-side delay that outlasts their host-side
    submission, so the two events around them see the kernels run back to
    back and not the host's launch rate.  The delay is a run of the library's
    streaming reads over 1 GiB, which keep every CU and the HBM busy (a spin
    kernel on one CU let the clocks drop before short kernels).  Returns
    (event ms per call, host submission us per call, queue_kept): the last is
    False if the host took longer to submit than the delay and the launches
    lasted (the figure then includes gaps)."""
    import sparse_attention_decode_loki_amd as loki
    state = _QUEUE
    if "buf" not in state:
        state["buf"] = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
        state["sink"] = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
        for _ in range(3):
            loki.stream_read(state["buf"], state["sink"], 2048)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            loki.stream_read(state["buf"], state["sink"], 2048)
        b.record()
        torch.cuda.synchronize()
        state["read_ms"] = max(a.elapsed_time(b) / 10, 1e-3)
        state["host_us"] = 100.0
    # room for the host to submit every launch at its last measured rate, x3
    delay_ms = max(2.0, 3.0 * n * state["host_us"] * 1e-3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for _ in range(int(delay_ms / state["read_ms"]) + 1):
        loki.stream_read(state["buf"], state["sink"], 2048)
    e0.record()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    t1 = time.perf_counter()
    e1.record()
    torch.cuda.synchronize()
    host_ms = (t1 - t0) * 1e3
    state["host_us"] = host_ms * 1e3 / n
    gpu_ms = e0.elapsed_time(e1)
    # the last launch was submitted before the queued work ahead of it ran out
    return gpu_ms / n, host_ms * 1e3 / n, host_ms < delay_ms + gpu_ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=int, default=1000,
                    help="untimed launches of the step before the warmup steps, so that the GPU "
                         "has left its idle clocks when the warmup starts (0: none)")
    ap.add_argument("--config", default="l2_13b_run")
    ap.add_argument("--layers", type=int, default=0,
                    help="cache copies cycled; 0: at least 4 and at least 1 GiB in all, "
                         "4x the last-level cache, so no step finds its bytes cached")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 fused, 2 split, 3 union")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-run", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true")
    ap.add_argument("--no-jaccard", action="store_true")
    ap.add_argument("--kf", type=float, default=None, help="override the budget k_f (k = floor(k_f*S))")
    ap.add_argument("--df", type=float, default=None, help="override d_f (d = d_f*D, d*2 a multiple of 16)")
    ap.add_argument("--rope-base", type=float, default=None,
                    help="RoPE variant: keys embedded at their positions, the query at S-1")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain device copy of this size (counter calibration)")
    ap.add_argument("--no-live-traffic", action="store_true",
                    help="skip the two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE) of the "
                         "step that give roofline.traffic for this run")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the decode measurements of the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle: seconds of work per worker process")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="CPU oracle: worker processes (0: every host core, at most 16)")
    ap.add_argument("--cpu-sequences", type=int, default=4, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_baseline_child:
        # the CPU oracle's timing, in a process that never touches the GPU
        print(json.dumps(cpu_baseline_child(args.config, args.rope_base, args.cpu_seconds,
                                            args.cpu_workers, args.cpu_sequences)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: this implementation runs on a single GPU; --gpus {args.gpus} is not "
              "supported (the decode shards by sequence or head with no communication, but only "
              "the one-GPU slice is built).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_decode_loki_amd as loki
    import synth

    loki.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib:
        # a plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE
        # counters calibrate the byte counts read for the decode kernel
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = synth.WORKLOADS[args.config]
    if args.kf is not None or args.df is not None:
        import dataclasses
        w = dataclasses.replace(w, k_f=w.k_f if args.kf is None else args.kf,
                                d=w.d if args.df is None else int(round(args.df * w.D)))
    S = w.S
    k = w.k
    t_setup = time.time()

    def log(msg):
        print(f"[bench {time.time() - t_setup:6.1f}s] {msg}", file=sys.stderr, flush=True)

    # ---- basis (library calibration, host) and prefill through the GPU append
    Qs = synth.bases(w)
    P = np.stack([loki.calibrate(synth.calib_keys(w, g, Qs[g]).astype(np.float32))[0]
                  for g in range(w.Hkv)])
    Pd = torch.from_numpy(P).to(dev)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    prefill = w.prefill if w.prefill else S - 1
    K_raw, V_raw = synth.raw_cache(w, S - 1)
    log(f"generated raw cache {K_raw.shape}")
    rb = args.rope_base
    base = loki.KVCache(w.B, w.Hkv, S, w.D, w.d, tdt, dev)
    loki.append(base, up(K_raw), up(V_raw), Pd, pos=0, rope_base=rb)
    R = 8
    new_k, new_v, qs = [], [], []
    for r in range(R):
        kn, vn = synth.new_tokens(w, r, Qs)
        new_k.append(up(kn))
        new_v.append(up(vn))
        qs.append(up(synth.queries(w, step=r)))
    loki.append(base, new_k[0], new_v[0], Pd, pos=S - 1, rope_base=rb)
    cache_bytes = sum(t.numel() * t.element_size() for t in (base.k_slab, base.k_rest, base.v)
                      if t is not None)
    if args.layers <= 0:
        args.layers = max(4, -(-(1 << 30) // cache_bytes))
    caches = [base]
    for _ in range(args.layers - 1):
        c = loki.KVCache(w.B, w.Hkv, S, w.D, w.d, tdt, dev)
        c.k_slab.copy_(base.k_slab)
        if c.k_rest is not None:
            c.k_rest.copy_(base.k_rest)
        c.v.copy_(base.v)
        c.length = S
        caches.append(c)
    torch.cuda.synchronize()
    log(f"caches ready: {args.layers} x {cache_bytes / 1e9:.2f} GB")

    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
    idx = torch.empty((w.B, w.Hq, k), dtype=torch.int32, device=dev)
    ws = loki.alloc_workspace(w.B, w.Hq, S, w.D, k, dev)
    # every (layer, token) combination marshalled once, so the timed loop is
    # one C call per step: loki_decode_step appends the step's token at S-1
    # and decodes over S tokens
    L = len(caches)
    n_plans = L * R // np.gcd(L, R)
    new_k2 = [t[:, :, 0].contiguous() for t in new_k]
    new_v2 = [t[:, :, 0].contiguous() for t in new_v]
    step_plans = [loki.StepPlan(qs[i % R], new_k2[i % R], new_v2[i % R], caches[i % L], Pd, k,
                                S - 1, out=out, idx=idx, workspace=ws, path=args.path,
                                rope_base=rb)
                  for i in range(n_plans)]
    dec_plans = [loki.DecodePlan(qs[i % R], caches[i % L], Pd, k, S=S, out=out, idx=idx,
                                 workspace=ws, path=args.path, rope_base=rb)
                 for i in range(n_plans)]

    def step(i):
        step_plans[i % n_plans]()

    def timed_(fn, n):
        return timed(torch, fn, n)

    for i in range(args.settle):
        step(i)
    for i in range(args.warmup):
        step(i)
    ms_per_step, step_avg_ms = timed_(lambda i: step(args.warmup + i), args.steps)
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step, events {step_avg_ms * 1e3:.1f} us/launch")

    # per-launch distribution: each step between its own pair of events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        step(args.warmup + args.steps + i)
        b.record()
    torch.cuda.synchronize()
    lat = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    step_latency = {"median_us": float(np.median(lat)), "p10_us": float(np.percentile(lat, 10)),
                    "p90_us": float(np.percentile(lat, 90)), "launches": len(lat)}
    log(f"per-launch step: median {step_latency['median_us']:.1f} us, "
        f"p10 {step_latency['p10_us']:.1f}, p90 {step_latency['p90_us']:.1f}")

    # decode alone (append excluded, as the pages time it), same caches
    for i in range(args.warmup):
        dec_plans[i % n_plans]()
    _, dec_avg_ms = timed_(lambda i: dec_plans[i % n_plans](), args.steps)
    log(f"decode alone {dec_avg_ms * 1e3:.1f} us/launch")

    hq = w.B * w.Hq
    by = algorithmic_bytes(w, S, k)
    # the step also reads each sequence's new key/value and writes its cache slot
    step_bytes = by["total"] + w.B * w.Hkv * (2 * w.D + 2 * w.D) * w.esize
    achieved = step_bytes / (step_avg_ms * 1e-3) / 1e9
    khash = kernel_source_hash()
    path_name = PATH_NAMES[
        loki.decode_path(w.B, w.Hq, w.Hkv, w.D, w.d, S, k, w.dtype, args.path)]
    overridden = args.kf is not None or args.df is not None
    traffic_recorded = (measured_traffic(khash, args.config)
                        if "fused" in path_name and not overridden else None)
    traffic = traffic_recorded

    result = {
        "metric": METRIC,
        "value": hq / (ms_per_step * 1e-3),
        "unit": "head-queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_launches": args.settle,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 cache, f32 accumulation" if w.dtype == "bf16" else "f32"),
        "data": "synthetic: seeded keys with a decaying PCA spectrum, N(0,1) values and queries",
        "config": {"workload": f"{w.name} steady state at S={S}"
                               + (f" with k_f={w.k_f}, d={w.d}" if overridden else ""),
                   "B": w.B, "Hq": w.Hq,
                   "Hkv": w.Hkv, "D": w.D, "d": w.d, "S": S, "k": k, "cache_dtype": w.dtype,
                   "step": "loki_decode_step: append 1 token/sequence at S-1 + decode over S",
                   "path": path_name,
                   "layers_cycled": args.layers,
                   "rope_base": rb},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "traffic_source": (
                         "recorded, not measured in this run: rocprofv3 --pmc FETCH_SIZE and "
                         f"WRITE_SIZE in profiles/traffic_fused_decode_step_{args.config}.txt, "
                         "taken on this kernel source hash" if traffic is not None else None),
                     "traffic_recorded": traffic_recorded,
                     "kernel": ("fused decode step (append + decode, one launch)" if "fused" in path_name
                                else "decode step (split kernels)"),
                     "algorithmic_bytes_per_launch": step_bytes,
                     "avg_launch_ms": step_avg_ms,
                     "timing": "HIP events around the timed region's back-to-back launches",
                     "kernel_source_hash": khash},
        "step_latency": step_latency,
        "decode_only": {"head_queries_per_s": hq / (dec_avg_ms * 1e-3), "avg_ms": dec_avg_ms,
                        "achieved_GBs": by["total"] / (dec_avg_ms * 1e-3) / 1e9},
    }

    # ---- the practical read ceiling: the library's streaming-read probe over
    # 4 GiB (16x the last-level cache), best of three launch widths
    if not args.no_read_probe:
        buf = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)
        best = 0.0
        for wg in (1024, 2048, 4096):
            sink = torch.empty(wg * 256, dtype=torch.float32, device=dev)
            for _ in range(2):
                loki.stream_read(buf, sink, wg)
            _, rms = timed_(lambda i: loki.stream_read(buf, sink, wg), 10)
            best = max(best, buf.numel() / (rms * 1e-3) / 1e9)
        result["roofline"]["measured_stream_read_GBs"] = best
        result["roofline"]["frac_of_measured_stream_read"] = achieved / best
        log(f"streaming-read probe {best:.0f} GB/s; step at {achieved / best:.3f} of it")
        # floors of the launch shapes the decode kernels use: each workgroup
        # streams its own contiguous share, regions of the 4 GiB buffer cycled
        floors = []
        for nbytes, wg, nt, loads, what in FLOOR_SHAPES:
            nbytes -= nbytes % (16 * wg)
            regions = buf.numel() // nbytes
            views = [buf[r * nbytes:(r + 1) * nbytes] for r in range(regions)]
            sink = torch.empty(wg * nt, dtype=torch.float32, device=dev)
            for i in range(3):
                loki.stream_read_shares(views[i % regions], sink, wg, nt, loads)
            ms, _, _ = timed_queued(
                torch, lambda i: loki.stream_read_shares(views[i % regions], sink, wg, nt, loads), 40)
            floors.append({"bytes": nbytes, "workgroups": wg, "threads": nt, "loads_per_lane": loads,
                           "us": ms * 1e3, "GBs": nbytes / (ms * 1e-3) / 1e9, "shape_of": what})
            log(f"share-read floor: {nbytes / 1e6:.1f} MB, {wg} x {nt} threads, {loads} loads/lane: "
                f"{ms * 1e3:.2f} us ({what})")
        result["streaming_floors"] = floors
        if w.name == "l2_13b_run" and "fused" in path_name and not overridden:
            # the step against a plain stream of its bytes by its own grid
            same = min(f["us"] for f in floors if f["workgroups"] == 640 and f["threads"] == 512)
            result["roofline"]["same_grid_stream_us"] = same
            result["roofline"]["frac_of_same_grid_stream"] = same / (step_avg_ms * 1e3)
            log(f"step at {same / (step_avg_ms * 1e3):.3f} of a plain stream of its bytes by its grid")
        del buf

    # ---- grouped-query shapes: the other gather (union / per-head) on the
    # same caches
    if w.Hq // w.Hkv in (2, 4) and path_name in ("split", "union"):
        other, key = ((loki.PATH_UNION, "union_gather") if path_name == "split"
                      else (loki.PATH_SPLIT, "per_head_gather"))
        alt_plans = [loki.DecodePlan(qs[i % R], caches[i % L], Pd, k, S=S, out=out, idx=idx,
                                     workspace=ws, path=other, rope_base=rb)
                     for i in range(n_plans)]
        for i in range(args.warmup):
            alt_plans[i % n_plans]()
        _, ams = timed_(lambda i: alt_plans[i % n_plans](), args.steps)
        result[key] = {"avg_ms": ams, "head_queries_per_s": hq / (ams * 1e-3),
                       "vs_decode_only": dec_avg_ms / ams}
        log(f"{key.replace('_', ' ')} decode {ams * 1e3:.1f} us/launch")

    # ---- same-GPU dense baseline on the same caches
    if not args.no_dense:
        dws = loki.alloc_workspace(w.B, w.Hq, S, w.D, 1, dev)
        dense_plans = [loki.DensePlan(qs[i % R], caches[i % L], Pd, S=S, out=out, workspace=dws,
                                      rope_base=rb) for i in range(n_plans)]
        for i in range(args.warmup):
            dense_plans[i % n_plans]()
        _, dms = timed_(lambda i: dense_plans[i % n_plans](), args.steps)
        result["dense_baseline"] = {
            "avg_ms": dms, "head_queries_per_s": hq / (dms * 1e-3),
            "achieved_GBs": by["dense"] / (dms * 1e-3) / 1e9,
            "loki_speedup": dms / dec_avg_ms}
        log(f"dense {dms * 1e3:.1f} us, loki speedup {dms / dec_avg_ms:.2f}x")

    # ---- the pages' run: prompt 3072, then 512 x (append 1, decode).  Timed
    # as whole passes between two events: the fused step (append + decode),
    # then the appends alone, the decodes alone (append excluded, as the pages
    # time it) and the dense decodes over the same growing cache lengths.
    if not args.no_run and w.prefill and w.steps:
        run_cache = caches[0]
        toks = []
        for st in range(w.steps):
            kn, vn = synth.new_tokens(w, 1000 + st, Qs)
            toks.append((up(kn[:, :, 0]), up(vn[:, :, 0]), up(kn), up(vn)))
        idx_flat = torch.empty(hq * k, dtype=torch.int32, device=dev)
        Ss = [w.prefill + st + 1 for st in range(w.steps)]
        ks = [w.k_at(x) for x in Ss]
        run_step = [loki.StepPlan(qs[st % R], toks[st][0], toks[st][1], run_cache, Pd, ks[st],
                                  Ss[st] - 1, out=out, idx=idx_flat[:hq * ks[st]].view(w.B, w.Hq, ks[st]),
                                  workspace=ws, path=args.path, rope_base=rb)
                    for st in range(w.steps)]
        run_app = [loki.AppendPlan(run_cache, toks[st][2], toks[st][3], Pd, Ss[st] - 1, rope_base=rb)
                   for st in range(w.steps)]
        run_dec = [loki.DecodePlan(qs[st % R], run_cache, Pd, ks[st], S=Ss[st], out=out,
                                   idx=idx_flat[:hq * ks[st]].view(w.B, w.Hq, ks[st]), workspace=ws,
                                   path=args.path, rope_base=rb) for st in range(w.steps)]
        n = w.steps
        run = {"prompt": w.prefill, "generated": n,
               "step_ms_total": timed_(lambda i: run_step[i](), n)[1] * n,
               "append_ms_total": timed_(lambda i: run_app[i](), n)[1] * n,
               "decode_ms_total": timed_(lambda i: run_dec[i](), n)[1] * n}
        if not args.no_dense:
            run_dense = [loki.DensePlan(qs[st % R], run_cache, Pd, S=Ss[st], out=out, workspace=dws,
                                        rope_base=rb) for st in range(w.steps)]
            run["dense_ms_total"] = timed_(lambda i: run_dense[i](), n)[1] * n
            run["loki_decode_speedup_vs_dense"] = run["dense_ms_total"] / run["decode_ms_total"]
        result["generation_run"] = run
        log(f"run: step {run['step_ms_total']:.2f} ms, decode {run['decode_ms_total']:.2f} ms, "
            f"append {run['append_ms_total']:.2f} ms")

    # ---- Exact-TopK agreement: the same keys cached with d = D give the exact
    # top-k; report the mean Jaccard similarity of Loki's selections at
    # several reduced dimensions (the pages report about 0.9 for Llama2-7B's
    # real keys at their main settings; these keys are synthetic)
    if not args.no_jaccard:
        result["topk_agreement_vs_exact"] = topk_agreement(loki, w, S, k, K_raw, V_raw, new_k[0],
                                                           new_v[0], qs[0], Pd, up, dev, rb)
        log(f"top-k Jaccard vs exact: {result['topk_agreement_vs_exact']}")

    # ---- the other workloads: decode alone on the AUTO path, the dense
    # baseline and (grouped-query shapes) the other gather, same method
    if not args.no_per_config and args.kf is None and args.df is None and rb is None:
        result["per_config"] = {}
        for name in PER_CONFIG:
            if name == args.config:
                continue
            result["per_config"][name] = measure_config(loki, torch, name, dev, args.steps,
                                                        args.warmup, log)
            torch.cuda.empty_cache()

    # ---- CPU oracle on a bounded sample (rank 0, one GPU), in a child process;
    # for the other workloads a shorter sample (every head of one sequence)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args, log)
        for name, res in result.get("per_config", {}).items():
            rec = cpu_baseline(args, log, config=name, seconds=min(args.cpu_seconds, 3.0),
                               sequences=1)
            res["cpu_oracle"] = {k_: rec[k_] for k_ in ("value", "unit", "cores", "sample")}
            res["gpu_over_cpu_oracle"] = res["head_queries_per_s"] / rec["value"]

    # ---- HBM traffic of the step kernel, measured in this run (after every
    # timed measurement): the counters' bytes per launch replace the recorded
    # figure in roofline.traffic
    if not args.no_live_traffic and "fused" in path_name and not overridden:
        tb, det = live_traffic(args, log)
        if tb is not None:
            result["roofline"]["traffic"] = tb
            result["roofline"]["traffic_source"] = (
                "measured in this run: two child runs of the step (20 + 5 launches) under "
                "rocprofv3 --pmc, FETCH_SIZE then WRITE_SIZE (KiB per dispatch, median over the "
                "step kernel's dispatches), each scaled by the same counter's reading for a "
                "plain 1 GiB device copy in that child")
            result["roofline"]["traffic_detail"] = det
            log(f"HBM traffic per step launch: {tb / 1e6:.1f} MB (recorded: "
                f"{(traffic_recorded or 0) / 1e6:.1f} MB)")
        else:
            result["roofline"]["traffic_live_error"] = det
            log(f"live traffic not measured: {det}")

    print(json.dumps(result), flush=True)


def topk_agreement(loki, w, S, k, K_raw, V_raw, kn, vn, q, Pd, up, dev, rb=None):
    """Mean Jaccard similarity |A & B| / |A | B| between Loki's kept set at
    d = D/8, D/4, D/2 and the exact top-k (d = D) over every head-query."""
    import torch
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Kd, Vd = up(K_raw), up(V_raw)

    def kept(d):
        c = loki.KVCache(w.B, w.Hkv, S, w.D, d, tdt, dev)
        loki.append(c, Kd, Vd, Pd, pos=0, rope_base=rb)
        loki.append(c, kn, vn, Pd, pos=S - 1, rope_base=rb)
        _, idx = loki.decode(q, c, Pd, k, S=S, path=loki.PATH_SPLIT, rope_base=rb)
        torch.cuda.synchronize()
        out = idx.cpu().numpy().reshape(-1, k)
        del c
        return out

    exact = kept(w.D)
    res = {"reference": f"exact top-k from all {w.D} rotated dims", "k": k}
    for d in (w.D // 8, w.D // 4, w.D // 2):
        approx = kept(d)
        inter = np.array([np.intersect1d(a, b, assume_unique=True).size
                          for a, b in zip(approx, exact)])
        res[f"d{d}"] = float(np.mean(inter / (2 * k - inter)))
    return res


PATH_NAMES = {1: "fused", 2: "split", 3: "union", 4: "sliced"}
PATH_CODES = {v: c for c, v in PATH_NAMES.items()}
COMPUTE_UNITS = 256


def sliced_slices(rows, kk) -> int:
    """Workgroups per sliced row of the sliced path (the library's plan: for
    fewer rows than compute units, the fewest slices that bring the busiest
    CU's share of rows within 10% of the best any allowed count gives; past
    whole rounds of the CUs, slices of a remainder of at most 64 rows that
    give every CU one more workgroup).  Used only to count the bytes of the
    score exchange."""
    cap = min(16, -(-kk // 64))
    if rows < COMPUTE_UNITS:
        sparse = max(min(-(-1024 // rows), -(-kk // 64)), -(-kk // 2048), 1)
        nmax = max(1, min(cap, sparse))
        load = [(-(-rows * n // COMPUTE_UNITS)) / n for n in range(1, nmax + 1)]
        return next(n for n in range(1, nmax + 1) if load[n - 1] <= 1.1 * min(load))
    rem = rows % COMPUTE_UNITS
    if rows % 8 or rem == 0 or rem > 64:
        return 1
    return max(1, min(COMPUTE_UNITS // rem, cap))


def design_bytes(w, S, k, path, idx) -> int:
    """HBM bytes the chosen path's kernels move by their design, from the
    selections the decode actually made (idx [B, Hq, k] on the host): the
    slab once per KV head (once per query head on the fused and sliced
    paths), the kept tokens' rest and value rows (each query head's own on
    the fused, sliced and split paths, each KV head's union of its query
    heads' on the union path; the slab dims of a kept key are never re-read),
    the ids, on the split and union paths the float32 score rows written and
    read back, and on the sliced path the float32 scores and partials its
    slices exchange (each slice's share written once, read by the row's
    other slices; counted although they may be served by the last-level
    cache)."""
    e = w.esize
    row = (2 * w.D - w.d) * e
    slab_heads = w.Hq if path in ("fused", "sliced") else w.Hkv
    total = w.B * slab_heads * S * w.d * e + w.B * w.Hq * k * 4
    if path == "union":
        G = w.Hq // w.Hkv
        for b in range(w.B):
            for g in range(w.Hkv):
                total += np.unique(idx[b, g * G:(g + 1) * G]).size * row
    else:
        total += w.B * w.Hq * k * row
    if path in ("split", "union"):
        total += 2 * w.B * w.Hq * S * 4
    if path == "sliced":
        rows = w.B * w.Hq
        nsl = sliced_slices(rows, k)
        sliced_rows = 0 if nsl == 1 else (rows if rows < COMPUTE_UNITS else rows % COMPUTE_UNITS)
        total += sliced_rows * (S * 4 * nsl + 2 * (nsl - 1) * (w.D + 2) * 4)
    return int(total)


PER_CONFIG = ["l2_7b", "l3_8b_gqa", "mistral_32k"]


def measure_config(loki, torch, name, dev, steps, warmup, log) -> dict:
    """Decode alone (AUTO path), the dense baseline and every other path the
    shape supports, for one workload at its full size, timed as the
    headline's decode: back-to-back launches between two HIP events after
    untimed warmup launches (and 500 settle launches before the first),
    cache copies cycled so that no launch finds its bytes cached.  At least
    200 launches are timed per path, queued behind a GPU-side delay: a
    Python caller submits a launch in roughly 10-40 us, longer than the
    7B-shape kernel runs, so launches timed as they are submitted would
    measure the host."""
    import synth
    steps = max(steps, 200)
    host = {"ok": True, "us": 0.0}

    def gpu_timed(fn):
        ms, hus, ok = timed_queued(torch, fn, steps)
        host["ok"] &= ok
        host["us"] = max(host["us"], hus)
        return ms
    w = synth.WORKLOADS[name]
    S, k = w.S, w.k
    Qs = synth.bases(w)
    P = np.stack([loki.calibrate(synth.calib_keys(w, g, Qs[g]).astype(np.float32))[0]
                  for g in range(w.Hkv)])
    Pd = torch.from_numpy(P).to(dev)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    K_raw, V_raw = synth.raw_cache(w, S, Qs)
    base = loki.KVCache(w.B, w.Hkv, S, w.D, w.d, tdt, dev)
    loki.append(base, up(K_raw), up(V_raw), Pd, pos=0)
    del K_raw, V_raw
    cache_bytes = sum(t.numel() * t.element_size() for t in (base.k_slab, base.k_rest, base.v)
                      if t is not None)
    L = max(4, -(-(1 << 30) // cache_bytes))
    caches = [base]
    for _ in range(L - 1):
        c = loki.KVCache(w.B, w.Hkv, S, w.D, w.d, tdt, dev)
        c.k_slab.copy_(base.k_slab)
        if c.k_rest is not None:
            c.k_rest.copy_(base.k_rest)
        c.v.copy_(base.v)
        c.length = S
        caches.append(c)
    R = 4
    qs = [up(synth.queries(w, step=r)) for r in range(R)]
    n_plans = L * R // np.gcd(L, R)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
    idx = torch.empty((w.B, w.Hq, k), dtype=torch.int32, device=dev)
    ws = loki.alloc_workspace(w.B, w.Hq, S, w.D, k, dev)
    code = loki.decode_path(w.B, w.Hq, w.Hkv, w.D, w.d, S, k, w.dtype, loki.PATH_AUTO)
    path = PATH_NAMES[code]

    def run(p, settle=0):
        plans = [loki.DecodePlan(qs[i % R], caches[i % L], Pd, k, S=S, out=out, idx=idx,
                                 workspace=ws, path=p) for i in range(n_plans)]
        for i in range(warmup + settle):
            plans[i % n_plans]()
        return gpu_timed(lambda i: plans[i % n_plans]())

    # the first path timed after the host-side set-up would otherwise run
    # while the GPU leaves its idle clocks (about 1.5 us slower per launch)
    dec_ms = run(loki.PATH_AUTO, settle=500)
    loki.DecodePlan(qs[0], caches[0], Pd, k, S=S, out=out, idx=idx, workspace=ws)()
    torch.cuda.synchronize()
    by = algorithmic_bytes(w, S, k)
    moved = design_bytes(w, S, k, path, idx.cpu().numpy())
    res = {"workload": f"{name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} d={w.d} S={S} k={k} "
                       f"{w.dtype} cache",
           "path": path, "decode_us": dec_ms * 1e3,
           "head_queries_per_s": w.B * w.Hq / (dec_ms * 1e-3),
           "algorithmic_bytes": by["total"],
           "achieved_GBs": by["total"] / (dec_ms * 1e-3) / 1e9,
           "frac": by["total"] / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "path_design_bytes": moved,
           "path_design_GBs": moved / (dec_ms * 1e-3) / 1e9,
           "layers_cycled": L, "launches_timed": steps}
    # the other paths this shape supports, on the same caches
    for other in ("fused", "sliced", "split", "union"):
        if other == path:
            continue
        try:
            loki.decode_path(w.B, w.Hq, w.Hkv, w.D, w.d, S, k, w.dtype, PATH_CODES[other])
        except loki.LokiError:
            continue
        res[f"{other}_us"] = run(PATH_CODES[other]) * 1e3
    dws = loki.alloc_workspace(w.B, w.Hq, S, w.D, 1, dev)
    dplans = [loki.DensePlan(qs[i % R], caches[i % L], Pd, S=S, out=out, workspace=dws)
              for i in range(n_plans)]
    for i in range(warmup):
        dplans[i % n_plans]()
    dms = gpu_timed(lambda i: dplans[i % n_plans]())
    res.update({"dense_us": dms * 1e3, "dense_GBs": by["dense"] / (dms * 1e-3) / 1e9,
                "loki_speedup_vs_dense": dms / dec_ms,
                "timing": "HIP events around back-to-back launches queued behind a GPU-side "
                          "delay (the host's submission rate does not enter)",
                "host_submit_us_per_launch": host["us"], "queue_stayed_ahead": host["ok"]})
    log(f"{name}: {path} decode {dec_ms * 1e3:.1f} us ({res['achieved_GBs']:.0f} GB/s "
        f"algorithmic, {res['path_design_GBs']:.0f} GB/s by the path's design), dense "
        f"{dms * 1e3:.1f} us, speedup {dms / dec_ms:.2f}x")
    return res


def cpu_baseline(args, log, config=None, seconds=None, sequences=4):
    """Runs the CPU oracle's timing in a child process (which never touches
    the GPU, so it may fork its workers) and returns its record."""
    import subprocess
    config = config or args.config
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", "--config",
           config, "--cpu-seconds", str(args.cpu_seconds if seconds is None else seconds),
           "--cpu-workers", str(args.cpu_workers), "--cpu-sequences", str(sequences)]
    if args.rope_base is not None and config == args.config:
        cmd += ["--rope-base", str(args.rope_base)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError("CPU oracle timing failed:\n" + r.stderr[-2000:])
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    log(f"cpu oracle ({config}): {rec['value']:.0f} head-queries/s on {rec['cores']} processes")
    return rec


def _cpu_worker(job):
    """One worker of the CPU oracle's timing: decode its share of the sampled
    head-queries again and again for `seconds`, BLAS held to one thread."""
    from threadpoolctl import threadpool_limits

    import oracle
    pairs, seconds = job
    st = _CPU_STATE
    n, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        while n == 0 or elapsed < seconds:
            t = time.perf_counter()
            oracle.decode(st["q"], st["slab"], st["rest"], st["v"], st["P"], st["k"], st["dtype"],
                          S=st["S"], heads=pairs, rope=st["rope"])
            elapsed += time.perf_counter() - t
            n += len(pairs)
    return n, elapsed


_CPU_STATE = {}


def cpu_baseline_child(config, rb, seconds, workers, sequences=4) -> dict:
    """The CPU oracle, as it stands, decoding a bounded sample of the same
    workload (every query head of the first sequences at S tokens) on the
    host's cores: the sampled head-queries are split into one contiguous
    share per worker process, each worker decodes its share repeatedly for
    `seconds`, and the rate is all head-queries decoded over the longest
    worker time.  The oracle gets its own inputs: its own calibration and
    float64 append of the generator's keys."""
    import multiprocessing as mp

    import oracle
    import synth
    w = synth.WORKLOADS[config]
    S, k = w.S, w.k
    nb = max(1, min(sequences, w.B))
    workers = workers if workers > 0 else min(16, os.cpu_count() or 1)
    Qs = synth.bases(w)
    P = np.stack([oracle.calibrate(synth.calib_keys(w, g, Qs[g]))[0]
                  for g in range(w.Hkv)]).astype(np.float32)
    kn, vn = synth.new_tokens(w, 0, Qs)
    st = np.uint16 if w.dtype == "bf16" else np.float32
    slab = np.empty((nb, w.Hkv, S, w.d), st)
    rest = np.empty((nb, w.Hkv, S, w.D - w.d), st)
    vv = np.empty((nb, w.Hkv, S, w.D), st)
    for b in range(nb):
        for g in range(w.Hkv):
            Kg = np.concatenate([synth.to_storage(synth.cache_keys(w, b, g, S - 1, Qs[g]), w.dtype),
                                 kn[b, g]])
            Vg = np.concatenate([synth.to_storage(synth.cache_values(w, b, g, S - 1), w.dtype),
                                 vn[b, g]])
            slab[b, g], rest[b, g], vv[b, g] = oracle.append(
                oracle.to_f64(Kg, w.dtype), oracle.to_f64(Vg, w.dtype),
                P[g].astype(np.float64), w.d, w.dtype, rope_base=rb)
    _CPU_STATE.update(q=synth.queries(w)[:nb], slab=slab, rest=rest, v=vv, P=P, k=k,
                      dtype=w.dtype, S=S, rope=None if rb is None else (rb, S - 1))
    pairs = [(b, h) for b in range(nb) for h in range(w.Hq)]
    shares = [pairs[i * len(pairs) // workers:(i + 1) * len(pairs) // workers]
              for i in range(workers)]
    shares = [sh for sh in shares if sh]
    with mp.get_context("fork").Pool(len(shares)) as pool:
        res = pool.map(_cpu_worker, [(sh, seconds) for sh in shares])
    n = sum(r[0] for r in res)
    wall = max(r[1] for r in res)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": n / wall, "unit": "head-queries/s", "cores": len(shares), "kind": "oracle",
            "sample": f"{len(pairs)} head-queries (all {w.Hq} heads of {nb} sequences) at S={S}, "
                      f"k={k}, split over {len(shares)} worker processes (one BLAS thread each), "
                      f"each decoding its share repeatedly for >= {seconds:g} s; float64 numpy "
                      "oracle; rate = head-queries decoded / longest worker time",
            "host_cpu": cpu, "host_nproc": os.cpu_count()}


if __name__ == "__main__":
    main()
