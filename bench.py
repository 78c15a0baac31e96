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
    args = ap.parse_args()
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
    ws = loki.alloc_workspace(w.B, w.Hq, w.D, S, k, dev)
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

    def timed(fn, n):
        """Launch fn n times back to back between two HIP events on the
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

    for i in range(args.settle):
        step(i)
    for i in range(args.warmup):
        step(i)
    ms_per_step, step_avg_ms = timed(lambda i: step(args.warmup + i), args.steps)
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
    _, dec_avg_ms = timed(lambda i: dec_plans[i % n_plans](), args.steps)
    log(f"decode alone {dec_avg_ms * 1e3:.1f} us/launch")

    hq = w.B * w.Hq
    by = algorithmic_bytes(w, S, k)
    # the step also reads each sequence's new key/value and writes its cache slot
    step_bytes = by["total"] + w.B * w.Hkv * (2 * w.D + 2 * w.D) * w.esize
    achieved = step_bytes / (step_avg_ms * 1e-3) / 1e9
    khash = kernel_source_hash()
    path_name = {1: "fused", 2: "split", 3: "union"}[
        loki.decode_path(w.B, w.Hq, w.Hkv, w.D, w.d, S, k, w.dtype, args.path)]
    overridden = args.kf is not None or args.df is not None
    traffic = (measured_traffic(khash, args.config)
               if "fused" in path_name and not overridden else None)

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
        "dtype": "f32",
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
            _, rms = timed(lambda i: loki.stream_read(buf, sink, wg), 10)
            best = max(best, buf.numel() / (rms * 1e-3) / 1e9)
        del buf
        result["roofline"]["measured_stream_read_GBs"] = best
        result["roofline"]["frac_of_measured_stream_read"] = achieved / best
        log(f"streaming-read probe {best:.0f} GB/s; step at {achieved / best:.3f} of it")

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
        _, ams = timed(lambda i: alt_plans[i % n_plans](), args.steps)
        result[key] = {"avg_ms": ams, "head_queries_per_s": hq / (ams * 1e-3),
                       "vs_decode_only": dec_avg_ms / ams}
        log(f"{key.replace('_', ' ')} decode {ams * 1e3:.1f} us/launch")

    # ---- same-GPU dense baseline on the same caches
    if not args.no_dense:
        dws = loki.alloc_workspace(w.B, w.Hq, w.D, S, 1, dev)
        dense_plans = [loki.DensePlan(qs[i % R], caches[i % L], Pd, S=S, out=out, workspace=dws,
                                      rope_base=rb) for i in range(n_plans)]
        for i in range(args.warmup):
            dense_plans[i % n_plans]()
        _, dms = timed(lambda i: dense_plans[i % n_plans](), args.steps)
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
               "step_ms_total": timed(lambda i: run_step[i](), n)[1] * n,
               "append_ms_total": timed(lambda i: run_app[i](), n)[1] * n,
               "decode_ms_total": timed(lambda i: run_dec[i](), n)[1] * n}
        if not args.no_dense:
            run_dense = [loki.DensePlan(qs[st % R], run_cache, Pd, S=Ss[st], out=out, workspace=dws,
                                        rope_base=rb) for st in range(w.steps)]
            run["dense_ms_total"] = timed(lambda i: run_dense[i](), n)[1] * n
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

    # ---- CPU oracle on a bounded sample (rank 0, one GPU)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, S, k, K_raw, V_raw, log, rb)

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


def cpu_baseline(w, S, k, K_raw, V_raw, log, rb=None):
    """The CPU oracle, as it stands, decoding a bounded sample of the same
    workload: every query head of the first `nb` sequences at S tokens.  The
    oracle gets its own inputs (its own calibration and float64 append of the
    same raw keys); BLAS is held to one thread."""
    import oracle
    import synth
    from threadpoolctl import threadpool_limits

    nb = 4
    Qs = synth.bases(w)
    P = np.stack([oracle.calibrate(synth.calib_keys(w, g, Qs[g]))[0] for g in range(w.Hkv)])
    P32 = P.astype(np.float32)
    kn, vn = synth.new_tokens(w, 0, Qs)
    st = np.uint16 if w.dtype == "bf16" else np.float32
    slab = np.empty((nb, w.Hkv, S, w.d), st)
    rest = np.empty((nb, w.Hkv, S, w.D - w.d), st)
    vv = np.empty((nb, w.Hkv, S, w.D), st)
    for g in range(w.Hkv):
        Kg = np.concatenate([K_raw[:nb, g], kn[:nb, g]], axis=1)
        Vg = np.concatenate([V_raw[:nb, g], vn[:nb, g]], axis=1)
        slab[:, g], rest[:, g], vv[:, g] = oracle.append(oracle.to_f64(Kg, w.dtype),
                                                         oracle.to_f64(Vg, w.dtype),
                                                         P32[g].astype(np.float64), w.d, w.dtype,
                                                         rope_base=rb)
    q = synth.queries(w)[:nb]
    pairs = [(b, h) for b in range(nb) for h in range(w.Hq)]
    reps, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        while reps < 1 or (elapsed < 10.0 and reps < 200):  # about 10 s of CPU work
            t = time.perf_counter()
            oracle.decode(q, slab, rest, vv, P32, k, w.dtype, S=S, heads=pairs,
                          rope=None if rb is None else (rb, S - 1))
            elapsed += time.perf_counter() - t
            reps += 1
    n = reps * len(pairs)
    log(f"cpu oracle: {n} head-queries in {elapsed:.1f}s")
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": n / elapsed, "unit": "head-queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(pairs)} head-queries (all {w.Hq} heads of {nb} sequences) at S={S}, "
                      f"k={k}, x{reps} repetitions, float64 numpy oracle, 1 BLAS thread",
            "host_cpu": cpu, "host_nproc": os.cpu_count()}


if __name__ == "__main__":
    main()
