#!/usr/bin/env python3
"""Benchmark: one decode step of shared-prefix attention on one MI355X.

A step is the whole hot path for one layer: the batch's new tokens go into
the COLD pool and every request attends its context, in one launch of the
step kernel through gkv_decode_step (host dispatch, then prefix splits of the
chosen backend, COLD suffix gather with the new tokens read from their input
rows and written to their slots, log-sum-exp join).  --separate times the
same step as gkv_cold_append followed by gkv_attn_decode (two launches).
Default workload: Llama-3.1-8B attention shape (32 query / 8 KV heads,
head_dim 128, bf16), one 16384-token shared prefix in HOT, 64 requests with
suffixes of 128-1024 tokens scattered token-wise in COLD (seeded N(0,1)
synthetic data standing in for the pages' ShareGPT-V3 workload).

Consecutive steps rotate over R copies of the pools ("layers", >= 1 GiB in
total) so that each step reads its K/V from HBM rather than from the 256 MB
Infinity Cache.  Prints one JSON line (metric, value = query-tokens/s, ...,
roofline of the dominant kernel, cpu_baseline of the float64 oracle).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--separate]
    python bench.py --fit-msat        # dispatcher threshold sweep (JSON lines)
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode query-tokens/s + achieved HBM GB/s, Llama-3.1-8B shape, L_p=16K, B=64"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA
MALL_DEFEAT_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, st):
    """Bytes and flops the method must move / do in one step, whole step and
    per kernel.  K/V of each distinct HOT prefix count once (read once per
    step), every suffix token once; partials and work lists are overhead and
    do not count."""
    s = w.spec
    e = 2 if s.dtype == "bf16" else 4
    d, n_kv, n_q, bsz = s.head_dim, s.n_kv, s.n_q, w.batch
    ids = st.hot_ids
    classes = sorted(set(int(i) for i in ids if i >= 0))
    pre_tokens = sum(st.ctx.hot_prefix_info(c)[1] for c in classes)
    tab = np.diff(st.indptr_h.astype(np.int64))
    suf_tokens = int(tab.sum())
    n_pre_req, n_suf_req = int((ids >= 0).sum()), int((tab > 0).sum())
    q_row = n_q * d * e
    kv_row = n_kv * d * e
    # the step kernel streams every prefix and suffix K/V byte, the slot ids
    # and q, and writes out and lse (partials are overhead)
    k = {"step": 2 * pre_tokens * kv_row + 2 * suf_tokens * kv_row + 4 * suf_tokens + bsz * q_row
         + bsz * q_row + 4 * bsz * n_q}
    append = 2 * 2 * n_suf_req * kv_row + 4 * n_suf_req
    step = (2 * pre_tokens * kv_row + 2 * suf_tokens * kv_row + 4 * suf_tokens + 4 * (bsz + 1)
            + bsz * q_row + bsz * q_row + 4 * bsz * n_q + append)
    group = n_q // n_kv
    flops_prefix = sum(4 * int((ids == c).sum()) * group * st.ctx.hot_prefix_info(c)[1] * d * n_kv
                       for c in classes)
    return {"kernel_bytes": k, "append_bytes": append, "step_bytes": step,
            "prefix_flops": flops_prefix, "suffix_flops": 4 * n_q * d * suf_tokens,
            "prefix_tokens": pre_tokens, "suffix_tokens": suf_tokens}


def estimate_step_bytes(w):
    s = w.spec
    e = 2 if s.dtype == "bf16" else 4
    used = sorted(set(int(p) for p in w.request_prefix if p >= 0))
    tokens = sum(w.prefix_lens[p] for p in used) + int(w.suffix_lens.sum())
    return 2 * tokens * s.n_kv * s.head_dim * e


KERNEL_SOURCES = ("kernels.hip", "kernels.h", "plan_types.h")


def kernel_source_sha() -> str:
    """sha256 over the device-code sources: identifies the kernels a set of
    hardware counters was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "shared_prefix_paged_contiguous_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per step-kernel launch from the committed rocprofv3 summary
    of this workload (calibrated FETCH_SIZE + WRITE_SIZE), or None when the
    summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"step_kernel_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("counters:"):
                kv = dict(x.split("=", 1) for x in line.split()[1:])
                if kv.get("kernel_sha") != kernel_source_sha():
                    return None
                return int(kv["read_bytes"]) + int(kv["write_bytes"])
    return None


def cpu_baseline(w, target_s: float):
    """The float64 oracle, unmodified, on a bounded sample of requests."""
    import torch
    import threadpoolctl

    from oracle.attention import decode_step

    def f64(t):
        return t.to(torch.float64).numpy()

    pk = [f64(x) for x in w.prefix_k]
    pv = [f64(x) for x in w.prefix_v]
    q = f64(w.q)
    # requests of the workload in order, cycling through the batch again
    # until about target_s seconds of oracle work are done
    done, t_used = 0, 0.0
    while t_used < target_s:
        b = done % w.batch
        sk, sv = w.suffix_rows(b)
        sks = [None] * w.batch
        svs = [None] * w.batch
        sks[b], svs[b] = f64(sk), f64(sv)
        t = time.perf_counter()
        decode_step(q, pk, pv, w.request_prefix, sks, svs, requests=[b])
        t_used += time.perf_counter() - t
        done += 1
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    return {"value": done / t_used, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} request decodes ({done / w.batch:.1f} passes over the {w.batch} requests of the "
                      f"same workload, all {w.spec.n_q} query heads each), float64 numpy; BLAS "
                      f"threads={threads}, host cpus={os.cpu_count()}; {t_used:.1f} s of oracle time"}


def build_state(w, replicas, force):
    from shared_prefix_paged_contiguous_amd.harness import DecodeState
    return DecodeState(w, n_layers=replicas, force_backend=force)


def step_inputs(w, st):
    """The batch's current tokens: the last slot-table entry of each request
    (all requests have one in the benchmark workloads) and its K/V row
    (appending them again rewrites identical bytes)."""
    import torch
    tab = np.diff(st.indptr_h.astype(np.int64))
    if not np.all(tab > 0):
        raise ValueError("every request needs a slot table with its current token")
    slots = st.last_slots()
    last = w.suffix_offsets[1:] - 1
    k_new = w.suffix_k[torch.from_numpy(last)].to(st.device).contiguous()
    v_new = w.suffix_v[torch.from_numpy(last)].to(st.device).contiguous()
    return k_new, v_new, torch.from_numpy(slots.astype(np.int32)).to(st.device)


def run_bench(args):
    import torch

    from shared_prefix_paged_contiguous_amd import binding, workloads

    t_setup = time.perf_counter()
    w = workloads.make(args.workload)
    s = w.spec
    force = {"auto": binding.BACKEND_AUTO, "cascade": binding.BACKEND_CASCADE,
             "dense": binding.BACKEND_DENSE}[args.backend]
    replicas = args.replicas or max(2, math.ceil(MALL_DEFEAT_BYTES / estimate_step_bytes(w)))
    st = build_state(w, replicas, force)
    alg = algorithmic(w, st)
    k_new, v_new, slots_new = step_inputs(w, st)
    out, lse = st.new_outputs()
    ctx = st.ctx
    stream = torch.cuda.current_stream()
    log(f"[bench] workload={s.name} B={w.batch} replicas={replicas} step_bytes={alg['step_bytes']/1e6:.1f} MB "
        f"setup={time.perf_counter()-t_setup:.1f}s")

    if args.calibrate_copy_mib:
        # a plain device copy of known size, for scaling HBM byte counters
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: 3 x {args.calibrate_copy_mib} MiB read + written")
        del src, dst

    def step(i, layer=None):
        layer = i % replicas if layer is None else layer
        if args.separate:
            ctx.cold_append(layer, k_new, v_new, slots_new, stream=stream)
            return st.run(out, lse, layer=layer, stream=stream)
        return st.step(out, lse, k_new, v_new, slots_new, layer=layer, stream=stream)

    backend = None
    for i in range(args.warmup):
        backend = step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        backend = step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    plan = ctx.last_plan()
    log(f"[bench] timed {args.steps} steps: {ms_step*1e3:.1f} us/step (wall {wall*1e3/args.steps:.1f} us/step), "
        f"backend={binding.BACKEND_NAMES[backend]}, host plan {plan['host_plan_us']:.2f} us")

    # same-layer ("warm", cache-resident) timing, reported for contrast only
    ms_warm = None
    if not args.no_warm:
        e0.record(stream)
        for i in range(args.steps):
            step(i, layer=0)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_warm = e0.elapsed_time(e1) / args.steps

    # per-kernel durations with HIP events recorded by the library on this stream
    ctx.kernel_timing(args.steps)
    for i in range(args.steps):
        step(i)
    per = ctx.kernel_timing_read(args.steps)
    ctx.kernel_timing(0)
    kern_ms = {"step": float(per.mean())}
    log(f"[bench] kernel avg us: " + ", ".join(f"{k}={v*1e3:.1f}" for k, v in kern_ms.items()))

    dom = max(kern_ms, key=kern_ms.get)
    dom_bytes = alg["kernel_bytes"][dom] + (0 if args.separate else alg["append_bytes"])
    achieved = dom_bytes / (kern_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": counter_traffic(s.name),
                "kernel": dom + "_kernel",
                "kernel_us": round(kern_ms[dom] * 1e3, 2), "kernel_bytes": dom_bytes}
    if alg["prefix_flops"] > 0:
        roofline["step_kernel_mfma_frac"] = round((alg["prefix_flops"] + alg["suffix_flops"]) /
                                                  (kern_ms["step"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    value = w.batch / (ms_step * 1e-3)
    step_gbps = alg["step_bytes"] / (ms_step * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": s.dtype,
        "data": "synthetic (seeded N(0,1), bf16-rounded; stands in for ShareGPT-V3)",
        "config": {"workload": s.name, "description": s.description, "batch": w.batch,
                   "n_q_heads": s.n_q, "n_kv_heads": s.n_kv, "head_dim": s.head_dim,
                   "prefix_tokens": alg["prefix_tokens"], "suffix_tokens": alg["suffix_tokens"],
                   "backend": binding.BACKEND_NAMES[backend], "m_eff": plan["m_eff"],
                   "replicas": replicas},
        "achieved_hbm_gbps": round(step_gbps, 1),
        "step_hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "step_bytes": alg["step_bytes"],
        "warm_ms_per_step": round(ms_warm, 5) if ms_warm is not None else None,
        "kernel_us": {k: round(v * 1e3, 2) for k, v in kern_ms.items()},
        "kernel_note": ("step = the step kernel of gkv_attn_decode (prefix splits, suffix parts, join); "
                        "gkv_cold_append is a launch of its own" if args.separate else
                        "step = the one launch of gkv_decode_step: new tokens appended, prefix splits, "
                        "suffix parts and their join"),
        "step_launches": 2 if args.separate else 1,
        "host_plan_us": round(plan["host_plan_us"], 3),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    return res


def fit_msat(args):
    """Re-fit the dispatcher threshold M_sat on this GPU.

    For each workload and batch size, time the step kernel under both prefix
    backends, once on full decode steps (the workload's suffix mix) and once
    on prefix-only steps (a one-token suffix: the prefix kernels alone).
    The fitted M_sat is the threshold t of the rule "dense iff M_eff >= t"
    (t among the swept M_eff values, or past the largest) with the least
    total relative regret sum(time(rule) / time(best) - 1) over the full-step
    points of all workloads; prefix-only points are reported alongside."""
    import torch

    from shared_prefix_paged_contiguous_amd import binding, workloads
    from shared_prefix_paged_contiguous_amd.harness import DecodeState

    def time_step(w, force, n_layers=2, warm=5, steps=20):
        st = DecodeState(w, n_layers=n_layers, force_backend=force)
        out, lse = st.new_outputs()
        for i in range(warm):
            st.run(out, lse, layer=i % n_layers)
        st.ctx.kernel_timing(steps)
        for i in range(steps):
            st.run(out, lse, layer=i % n_layers)
        us = float(st.ctx.kernel_timing_read(steps).mean()) * 1e3
        del st
        torch.cuda.empty_cache()
        return us

    rows = []
    for name in args.fit_workloads.split(","):
        g = workloads.SPECS[name].n_q // workloads.SPECS[name].n_kv
        for bsz in [int(x) for x in args.fit_batches.split(",")]:
            res = {"workload": name, "batch": bsz, "m_eff": bsz * g}
            for kind, kw in (("full", {}), ("prefix_only", {"suffix_range": (1, 1)})):
                w = workloads.make(name, batch=bsz, **kw)
                for label, force in (("cascade", binding.BACKEND_CASCADE), ("dense", binding.BACKEND_DENSE)):
                    res[f"{kind}_{label}_us"] = round(time_step(w, force), 2)
                flops = 4 * bsz * g * w.prefix_lens[0] * w.spec.head_dim * w.spec.n_kv
                res[f"{kind}_dense_prefix_tflops"] = round(flops / (res[f"{kind}_dense_us"] * 1e-6) / 1e12, 1)
            rows.append(res)
            print(json.dumps(res), flush=True)

    def regret(t, pts, kind):
        tot = 0.0
        for r in pts:
            c, d = r[f"{kind}_cascade_us"], r[f"{kind}_dense_us"]
            tot += (d if r["m_eff"] >= t else c) / min(c, d) - 1.0
        return tot

    cands = sorted({r["m_eff"] for r in rows}) + [math.inf]
    for kind in ("full", "prefix_only"):
        best = min(cands, key=lambda t: (regret(t, rows, kind), t))
        print(json.dumps({"fit": kind, "fitted_m_sat": None if best == math.inf else best,
                          "regret": round(regret(best, rows, kind), 4),
                          "per_workload": {n: round(regret(best, [r for r in rows if r["workload"] == n], kind), 4)
                                           for n in args.fit_workloads.split(",")}}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b_lp16k_b64")
    ap.add_argument("--backend", default="auto", choices=["auto", "cascade", "dense"])
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--separate", action="store_true",
                    help="time gkv_cold_append + gkv_attn_decode (two launches) instead of gkv_decode_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the same-layer pass (profiling: every step kernel then reads from HBM)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run a plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--fit-msat", action="store_true")
    ap.add_argument("--fit-workloads", default="qwen14b_tp2_lp16k_b128,llama8b_lp16k_b64")
    ap.add_argument("--fit-batches", default="8,16,32,64,128,256,384,512,768")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the decode step shards by "
              "KV head with no exchange inside attention; see DESIGN.md). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.fit_msat:
        fit_msat(args)
        return
    res = run_bench(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
