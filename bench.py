#!/usr/bin/env python3
"""Benchmark of the TTR hybrid-attention forward on one MI355X.

One step = one ttr_hybrid_forward over the whole workload (key/value
reduction, then the fused apply + landmark softmax + blend kernel) with the
inputs already resident in HBM. Prints one JSON line:
  metric/value  hybrid-attention tokens/s (B*N / forward time, all heads)
  roofline      the dominant kernel's algorithmic TFLOP/s (per-launch flops /
                its average duration from HIP events recorded inside the timed
                forwards) against the dense bf16 MFMA peak
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded sample

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload flux_1024]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SRC = os.path.join(ROOT, "linear_hybrid_attention_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="flux_1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--distill", action="store_true",
                    help="time one Phase-1 distillation step (teacher, student, loss, backward, Adam) instead")
    ap.add_argument("--lr", type=float, default=1e-4, help="Adam learning rate of the distillation step")
    ap.add_argument("--nq", type=int, default=0,
                    help="with --distill: train on a replay sample of NQ query rows (teacher rows given)")
    ap.add_argument("--cosine", action="store_true",
                    help="time the student/teacher cosine distance of the readiness gate instead")
    ap.add_argument("--replay", action="store_true",
                    help="time the replay buffer's offload (push), fetch and a push overlapped with a distillation "
                         "step instead")
    ap.add_argument("--staged", action="store_true",
                    help="time each staged entry point (feature map, key/value reduction, apply, landmark branch, "
                         "blend) with its own roofline instead")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="untimed forwards for this many milliseconds before the warm-up steps, so that the GPU "
                         "has reached its steady clock (see settle())")
    ap.add_argument("--chunk", type=int, default=0,
                    help="causal workloads: run this chunk (64, 128 or 256) instead of the workload's own")
    ap.add_argument("--cold", action="store_true",
                    help="cold caches: write a 1 GiB scratch buffer before every timed forward (flushes the L2s "
                         "and the 256 MB MALL) and time each forward on its own")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (counter calibration)")
    ap.add_argument("--write-traffic", default=None, metavar="DIR",
                    help="only turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv runs under DIR (fetch/, write/ of "
                         "--workload; copy_fetch/, copy_write/ of --copy-calibration --copy-mib) into "
                         "profiles/traffic_counters.json")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the calibration copy in the counter runs")
    return ap.parse_args()


def settle(step, ms):
    """Untimed calls of step() for about ms milliseconds of wall time. After an
    idle period the GPU runs the forward up to 8% slower until it has been
    under load for a while (the first 200 flux_1024 forwards after a pause run
    at 64 us, the next at 60 us; on a fresh process 200-500 ms of load did not
    always suffice, 1000 ms did in every run), which a handful of warm-up steps
    does not cover. Returns the calls."""
    import torch
    n = 0
    t_end = time.perf_counter() + ms / 1000.0
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    return n


def host_lead(steps):
    """Before the start event of a back-to-back timed region: a spin kernel of
    about 40 us per timed step, so that the host has enqueued the timed calls
    before the GPU reaches the start event. The region then holds the GPU's
    time for the calls and not the host's launch latency (about 14 us of Python
    per call, which otherwise leaves the GPU idle after the start event)."""
    import torch
    torch.cuda._sleep(int(steps) * 80_000)  # cycles; about 40 us each at the measured 2 GHz


def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)


def _pmc_means(run_dir, counter):
    """Mean counter value per dispatch, by kernel name, from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    sums = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                k = sums.setdefault(r["Kernel_Name"], {})
                k[r["Dispatch_Id"]] = k.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {name: sum(d.values()) / len(d) for name, d in sums.items()}


def write_traffic(run_dir, wl, copy_mib):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what they read for a plain copy of known size."""
    import workloads
    fetch, write = _pmc_means(os.path.join(run_dir, "fetch"), "FETCH_SIZE"), \
        _pmc_means(os.path.join(run_dir, "write"), "WRITE_SIZE")
    cf = _pmc_means(os.path.join(run_dir, "copy_fetch"), "FETCH_SIZE")
    cw = _pmc_means(os.path.join(run_dir, "copy_write"), "WRITE_SIZE")
    copy_name = max(cf, key=cf.get)  # the copy kernel is the only large dispatch of that run
    copy_bytes = copy_mib << 20
    f_scale = copy_bytes / (cf[copy_name] * 1024.0)
    w_scale = copy_bytes / (cw[copy_name] * 1024.0)
    layer = wl in workloads.LAYER_WORKLOADS
    w = workloads.LAYER_WORKLOADS[wl] if layer else workloads.WORKLOADS[wl]
    out = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            out = json.load(f)
    ent = {}
    for name, _, _ in (layer_plan(w) if layer else kernel_plan(w)):
        full = [k for k in fetch if trace_name_matches(name, k)]
        if not full or full[0] not in write:
            continue
        kname = full[0]
        srcs = kernel_sources(name)
        ent[name] = {"bytes_per_launch": fetch[kname] * 1024.0 * f_scale + write[kname] * 1024.0 * w_scale,
                     "fetch_bytes": fetch[kname] * 1024.0 * f_scale, "write_bytes": write[kname] * 1024.0 * w_scale,
                     "fetch_scale": f_scale, "write_scale": w_scale, "copy_kernel": copy_name,
                     "sources": srcs, "source_hash": source_hash(srcs)}
    out[w.name] = ent
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out[w.name], indent=1))


def trace_name_matches(plan_name, trace_name):
    """Whether a profiler's kernel name is the dispatch a plan entry names.

    Plan entries name a kernel, a kernel with its template arguments, or a
    projection by role ("proj_gemm_kernel (qkv)": A rows -> Q/K/V heads,
    "(out)": A heads -> rows)."""
    t = trace_name.split("(")[0].replace("void ttr::", "").strip()
    roles = {" (qkv)": ", 0, 1>", " (out)": ", 1, 0>"}
    for suffix, targs in roles.items():
        if plan_name.endswith(suffix):
            return t.startswith(plan_name[:-len(suffix)] + "<") and t.endswith(targs)
    return t in (plan_name, plan_name + "<") or t.split("<")[0] == plan_name


def kernel_sources(name):
    """Source files a kernel is built from (a change to any of them voids stored counters)."""
    common = ["common.hpp", "tiles.hpp", "launch.hpp"]
    if name.startswith("proj_gemm") or name.startswith("wt_transpose"):
        return ["k_proj.hip"] + common
    if name.startswith("kv_stage"):
        return ["k_kv2.hip"] + common
    if name.startswith("fused_"):
        return ["k_fused.hip"] + common
    if name.startswith("causal1_"):
        return ["k_causal2.hip"] + common
    return ["k_hybrid.hip", "k_kv.hip", "k_causal.hip"] + common


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(KERNEL_SRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_plan(w):
    """Kernels of one forward in launch order: (name, algorithmic flops, algorithmic bytes) per launch.

    Both count what the method must compute or move (Q, K, V read once, out
    written once, the products of the method), not what a kernel happens to do:
    workspace traffic of the split reduction is the design's, not the method's.
    """
    BH, N, D, F, L = w.B * w.H, w.N, w.D, w.F, w.L
    io = 2 if w.dtype == "bf16" else 4
    tok = BH * N * D * io  # one [B, H, N, D] tensor
    if w.causal:
        chunk = w.chunk
        nseg, cps = causal_plan(w, chunk)
        # one pass: each segment's state from its K and V (all but the last
        # segment), then the walk; the state pass's reading of K and V again
        # is the design's (its second read comes from cache), so the method's
        # bytes are Q, K, V read once and out written once
        seg_tokens = min(N, (nseg - 1) * cps * chunk)
        state = 2 * D * D + D  # P += phi(k)^T v, z += phi(k) per token
        # per token: its share of the causal score and value tiles (C/2 keys on
        # average, plus the diagonal), the inter-chunk product and the state update
        walk = BH * N * (2 * 2 * D * (chunk // 2 + 16) + 2 * D * D + state)
        return [("causal1_reset_kernel", 0, 0),
                (f"causal1_kernel<{chunk}, 0>", BH * seg_tokens * state + walk, 4 * tok)]
    proj = 2 * N * D * F  # X W_h
    kv = 2 * N * F * D + N * F  # phi(K)^T V and ksum
    apply = 2 * N * F * D + 2 * N * F  # phi(Q) KV and phi(Q) . ksum
    lm = 4 * N * L * D  # Q K_L^T and P V_L
    if w.dtype == "bf16":
        return [("kv_stage_kernel", BH * (proj + kv), 2 * tok),
                ("fused_query_kernel", BH * (proj + apply + lm), 2 * tok)]
    return [("kv_partial_kernel (+ kv_finalize_kernel)", BH * (proj + kv), 2 * tok),
            ("hybrid_kernel", BH * (proj + apply + lm), 2 * tok)]


def roofline(w, flops, nbytes, ms):
    """The binding roofline of one kernel: whichever of MFMA and HBM time is longer at peak."""
    peak_f = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    if flops / (peak_f * 1e12) >= nbytes / (HBM_PEAK_GBS * 1e9):
        a = flops / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
        return {"bound": "mfma", "achieved": a, "peak": peak_f, "unit": "TFLOP/s", "frac": a / peak_f}
    a = nbytes / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
    return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": a / HBM_PEAK_GBS}


def causal_plan(w, chunk):
    """Segments of the single-pass scan: about 1024 tokens each, shorter when that gives fewer than 512 workgroups."""
    nchunks = -(-w.N // chunk)
    want = max(-(-w.N // 1024), -(-512 // (w.B * w.H)))
    want = max(min(want, nchunks), 1)
    cps = -(-nchunks // want)
    return -(-nchunks // cps), cps


def algorithmic_bytes(w):
    io = 2 if w.dtype == "bf16" else 4
    return 4 * w.B * w.H * w.N * w.D * io  # Q, K, V read once, out written once


def host_info():
    """The host's CPU model and physical core count (from /proc/cpuinfo), and the BLAS threads numpy uses."""
    model, cores = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None and core is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = os.cpu_count() or 1
    return {"host_cpu": model, "host_physical_cores": len(cores) or None, "host_logical_cpus": os.cpu_count(),
            "usable_cpus": affinity, "blas_threads": int(threads)}


def cpu_baseline(w, x, target_s):
    """Time the fp64 oracle on a bounded sample; scale to the workload's tokens/s.

    The sample is the first few (batch, head) slices of the same inputs (all of
    them when one pass is quick), repeated until about target_s seconds of CPU
    work have been timed.
    """
    import numpy as np
    import oracle.ttr_oracle as O
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def run(hs):
        sl = slice(0, hs)
        W = None if x["W"] is None else x["W"][sl]
        b = None if x["b"] is None else x["b"][sl]
        t0 = time.perf_counter()
        if w.causal:
            O.causal_forward(x["Q"][:1, sl], x["K"][:1, sl], x["V"][:1, sl], W, b, x["eps"])
        else:
            O.hybrid_forward(x["Q"][:, sl], x["K"][:, sl], x["V"][:, sl], W, b, x["g"][sl], x["eps"], w.L)
        return time.perf_counter() - t0

    t1 = run(1)
    heads = int(max(1, min(w.H, target_s / max(t1, 1e-3))))
    t = run(heads) if heads > 1 else t1
    reps, total = 1, t
    while total < target_s and reps < 64:
        total += run(heads)
        reps += 1
    t = total / reps
    seqs = heads * (1 if w.causal else w.B)  # (batch, head) slices in one pass
    total_seqs = w.B * w.H
    sec_full = t * total_seqs / seqs
    sample = (f"{seqs} of {total_seqs} (batch, head) slices of the {w.name} workload (N={w.N}), fp64 numpy "
              f"oracle, {reps} pass(es) totalling {total:.1f} s, {t:.3f} s per pass, scaled to all slices")
    return {"value": w.B * w.N / sec_full, "unit": "tokens/s", "cores": int(threads), "kind": "oracle", **host_info(),
            "sample": sample, "seconds_full_estimate": sec_full}


def layer_plan(w):
    """Kernels of one NNT layer forward in launch order (name, algorithmic flops, bytes).

    The projections count their matrix products and the activations the method
    must read or write (x in, out back); Q, K, V and the attention output in
    between are the design's staging, as are the transposed weights."""
    import workloads
    io = 2 if w.dtype == "bf16" else 4
    M, E = w.B * w.N, w.E
    core = workloads.Workload(w.name, w.B, w.H, w.N, E // w.H, E // w.H, w.dtype, 0, w.causal, False, 0.0, 0.0, 0)
    plan = [("wt_transpose_kernel", 0, 0),
            ("proj_gemm_kernel (qkv)", 2 * M * E * 3 * E, M * E * io)]
    for name, fl, by in kernel_plan(core):
        if name.startswith("kv_stage_kernel"):  # identity map: the method has no projection flops here
            fl = core.B * core.H * (2 * core.N * core.D * core.D + core.N * core.D)
        if name.startswith("fused_query"):
            fl = core.B * core.H * (2 * core.N * core.D * core.D + 2 * core.N * core.D)
        plan.append((name, fl, by))
    plan.append(("proj_gemm_kernel (out)", 2 * M * E * E, M * E * io))
    return plan


def cpu_baseline_layer(w, x, target_s):
    """The oracle layer on the first sequences of the same inputs, repeated to about target_s seconds."""
    import oracle.ttr_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def run(nb):
        t0 = time.perf_counter()
        O.nnt_layer_forward(x["x"][:nb], x["Wq"], x["bq"], x["Wk"], x["bk"], x["Wv"], x["bv"], x["Wo"], x["bo"],
                            w.H, x["eps"], w.causal, w.fmap)
        return time.perf_counter() - t0

    t1 = run(1)
    nb = int(max(1, min(w.B, target_s / max(t1, 1e-3))))
    t = run(nb) if nb > 1 else t1
    reps, total = 1, t
    while total < target_s and reps < 64:
        total += run(nb)
        reps += 1
    t = total / reps
    sec_full = t * w.B / nb
    sample = (f"{nb} of {w.B} sequences of the {w.name} workload (N={w.N}, E={w.E}), fp64 numpy oracle, "
              f"{reps} pass(es) totalling {total:.1f} s, {t:.3f} s per pass, scaled to all sequences")
    return {"value": w.B * w.N / sec_full, "unit": "tokens/s", "cores": int(threads), "kind": "oracle", **host_info(),
            "sample": sample, "seconds_full_estimate": sec_full}


def main_layer(args):
    import ctypes
    import numpy as np
    import torch
    import linear_hybrid_attention_amd as ttr
    import workloads

    w = workloads.LAYER_WORKLOADS[args.workload]
    x = workloads.make_layer_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def io(name):
        if w.dtype == "bf16":
            return torch.from_numpy(x[name + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x[name]).to(dev)

    X, Wq, Wk, Wv, Wo = (io(k) for k in ("x", "Wq", "Wk", "Wv", "Wo"))
    bq, bk, bv, bo = (torch.from_numpy(x[k]).to(dev) for k in ("bq", "bk", "bv", "bo"))
    out = torch.empty_like(X)
    lib = ttr.load_library()
    nbytes = ttr.nnt_layer_workspace_bytes(w.B, w.N, w.E, w.H, 1 if w.dtype == "bf16" else 0, w.causal, w.fmap)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    plan = layer_plan(w)

    def step(events=None):
        if events is not None:
            lib.ttr_set_stage_events(events, len(plan) + 1)
        ttr.nnt_layer_forward(X, Wq, bq, Wk, bk, Wv, bv, Wo, bo, w.H, float(x["eps"]), w.causal, w.fmap,
                              out=out, ws=ws)

    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nev = len(plan) + 1
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record(stream)
    handles = [(ctypes.c_void_p * nev)(*[e.cuda_event for e in row]) for row in ev]
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    host_lead(args.steps)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    for i in range(args.steps):
        step(handles[i])
    torch.cuda.synchronize()
    kern_ms = {name: float(np.mean([ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(args.steps)]))
               for k, (name, _, _) in enumerate(plan)}
    name, flops, nb = max(plan, key=lambda p: kern_ms[p[0]])
    rl = roofline(w, flops, nb, kern_ms[name])
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            ent = json.load(f).get(w.name, {}).get(name)
        if ent and ent.get("source_hash") == source_hash(ent["sources"]):
            traffic = ent["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None
    kernels = {}
    for kn, kf, kb in plan:
        r = roofline(w, kf, kb, kern_ms[kn]) if (kf or kb) else {"bound": None, "frac": None}
        kernels[kn] = {"ms": kern_ms[kn], "flops": kf, "bytes": kb, "bound": r["bound"], "frac": r["frac"]}
    total_flops = sum(p[1] for p in plan)
    peak_fwd = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    io_b = 2 if w.dtype == "bf16" else 4
    act_bytes = 2 * w.B * w.N * w.E * io_b  # x read, out written
    res = {
        "metric": f"NNT linear-attention layer tokens/sec (B={w.B}, N={w.N}, E={w.E}, {w.H} heads"
                  f"{', causal' if w.causal else ''})",
        "value": w.B * w.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "E": w.E, "H": w.H, "D": w.E // w.H,
                   "feature_map": w.fmap, "causal": w.causal, "global_batch": w.B, "seq_len": w.N,
                   "clock_settle_ms": args.settle_ms, "clock_settle_calls": settled},
        "roofline": {"kernel": name, "bound": rl["bound"], "achieved": rl["achieved"], "peak": rl["peak"],
                     "unit": rl["unit"], "frac": rl["frac"], "traffic": traffic,
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nb,
                     "avg_launch_ms": kern_ms[name]},
        "forward": {"tflops": total_flops / (ms * 1e-3) / 1e12,
                    "frac_mfma_peak": total_flops / (ms * 1e-3) / 1e12 / peak_fwd,
                    "algorithmic_bytes": act_bytes,
                    "frac_hbm_peak": act_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "kernels": kernels, "wall_s": wall},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_layer(w, x, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def distill_plan(w, nq=None):
    """Launches of one distillation step, in order: (name, algorithmic flops,
    algorithmic bytes). nq: a replay sample's query rows (the teacher's rows
    given, so no teacher stage); else every query row and the teacher computed."""
    Z, N, D, F, L = w.B * w.H, w.N, w.D, w.F, w.L
    NQ = N if nq is None else nq
    io = 2 if w.dtype == "bf16" else 4
    gq, gk = 2 * Z * NQ * D * F, 2 * Z * N * D * F  # a product over the query rows / the key rows
    plan = []
    if w.dtype == "bf16":
        plan.append(("to_bf16_kernel (W)", 0, 0))
    if nq is None:
        teacher = ("teacher softmax attention (landmark pack + fused query kernel without its linear branch, every key a landmark)"
                   if w.dtype == "bf16" else "teacher softmax attention (hybrid_kernel, L = N)")
        plan.append((teacher, 4 * Z * N * N * D, 3 * Z * N * D * io + Z * N * D * 4))
    plan += [("bgemm z_q = Q W + b", gq, 0), ("bgemm z_k = K W + b", gk, 0)]
    if w.dtype == "bf16":  # KV and ksum from K and V by the key/value kernel
        plan.append(("KV, ksum = phi(K W + b)^T V, colsum (kv_stage_kernel)", gk, 0))
    else:
        plan += [("ksum (tile sums of the z_k epilogue)", 0, 0), ("bgemm KV = phi_k^T V", gk, 0)]
    plan += [("bgemm lin = phi_q KV / den, den = phi_q . ks + eps (normaliser formed from the staged rows)", gq, 0)]
    if L > 0:
        plan.append(("landmark branch (landmark pack + fused query kernel's landmark loop, fp32 out)"
                     if w.dtype == "bf16" else "landmark branch (hybrid_kernel)", 4 * Z * NQ * L * D, 0))
    plan += [("loss rows and dnum, dden (distill_loss_dlin_kernel)", 0, 0), ("distill_loss_total_kernel", 0, 0),
             ("bgemm dz_q = (dnum KV^T + dden ks^T) phi'(z_q)", gq, 0), ("bgemm dKV = phi_q^T dnum", gq, 0),
             ("dks (tile sums of the dz_q epilogue)", 0, 0), ("bgemm dz_k = (V dKV^T + dks) phi'(z_k)", gk, 0),
             ("bgemm dW += Q^T dz_q", gq, 0), ("bgemm dW += K^T dz_k", gk, 0),
             ("db (tile sums of the dz epilogues), dg", 0, 0), ("adam_kernel", 0, 0)]
    return plan


def cpu_baseline_distill(w, x, target_s, lr, nq=None):
    """The oracle's distillation step on the first heads of the same inputs, scaled to all heads
    (nq: on the replay sample's query rows, with its teacher rows given)."""
    import numpy as np
    import oracle.ttr_oracle as O
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def run(hs):
        sl = slice(0, hs)
        W, b, g = x["W"][sl], x["b"][sl], x["g"][sl]
        st = {k: np.zeros_like(v) for k, v in (("mW", W), ("vW", W), ("mb", b), ("vb", b), ("mg", g), ("vg", g))}
        st["ms"] = np.zeros(2)
        st["vs"] = np.zeros(2)
        Qh = x["Q"][:, sl]
        T = None
        if nq is not None:
            Qh = Qh[:, :, workloads.query_subsample(w.N, nq, w.seed)]
            T = np.random.default_rng(w.seed + 5).standard_normal((w.B, w.H, nq, w.D), dtype=np.float32)[:, sl]
        t0 = time.perf_counter()
        O.distill_step(Qh, x["K"][:, sl], x["V"][:, sl], W, b, g, np.zeros(2), st, 1, lr, x["eps"], w.L, T)
        return time.perf_counter() - t0

    t1 = run(1)
    heads = int(max(1, min(w.H, target_s / max(t1, 1e-3))))
    t = run(heads) if heads > 1 else t1
    reps, total = 1, t
    while total < target_s and reps < 64:
        total += run(heads)
        reps += 1
    t = total / reps
    sec_full = t * w.H / heads
    rows = "" if nq is None else f", {nq} sampled query rows"
    sample = (f"{heads} of {w.H} heads (all {w.B} batch rows) of the {w.name} workload (N={w.N}{rows}), fp64 numpy "
              f"oracle distillation step, {reps} pass(es) totalling {total:.1f} s, {t:.3f} s per pass, scaled to all "
              "heads")
    if nq is not None:
        return {"value": w.B / sec_full, "unit": "samples/s", "cores": int(threads), "kind": "oracle", **host_info(),
                "sample": sample, "seconds_full_estimate": sec_full}
    return {"value": w.B * w.N / sec_full, "unit": "tokens/s", "cores": int(threads), "kind": "oracle", **host_info(),
            "sample": sample, "seconds_full_estimate": sec_full}


def main_distill(args):
    import ctypes
    import numpy as np
    import torch
    import linear_hybrid_attention_amd as ttr
    import workloads

    w = workloads.WORKLOADS[args.workload]
    if w.causal or not w.proj:
        print("--distill needs a non-causal workload with a projection", file=sys.stderr)
        sys.exit(2)
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def io(name):
        if w.dtype == "bf16":
            return torch.from_numpy(x[name + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x[name]).to(dev)

    Q, K, V = io("Q"), io("K"), io("V")
    b = x["b"] if x["b"] is not None else np.zeros((w.H, w.F), np.float32)
    state = ttr.DistillState(torch.from_numpy(x["W"]).to(dev), torch.from_numpy(b).to(dev),
                             torch.from_numpy(x["g"]).to(dev))
    lib = ttr.load_library()
    d = ttr.Dims(w.B, w.H, w.N, w.D, w.F, 1 if w.dtype == "bf16" else 0, 0)
    nq = args.nq if args.nq else None
    teacher = None
    if nq is not None:  # a replay sample: nq query rows over every key, the teacher's rows given
        idx = workloads.query_subsample(w.N, nq, w.seed)
        qsel = x["Q_bits" if w.dtype == "bf16" else "Q"][:, :, idx]
        Q = torch.from_numpy(np.ascontiguousarray(qsel).view(np.int16 if w.dtype == "bf16" else np.float32))
        Q = (Q.view(torch.bfloat16) if w.dtype == "bf16" else Q).to(dev)
        teacher = torch.from_numpy(np.random.default_rng(w.seed + 5).standard_normal(
            (w.B, w.H, nq, w.D), dtype=np.float32)).to(dev)
        ws = torch.empty(lib.ttr_distill_rows_workspace_bytes(d, nq, w.L, 0), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(lib.ttr_distill_workspace_bytes(d, w.L, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    plan = distill_plan(w, nq)
    eps = float(x["eps"])

    def step(events=None):
        if events is not None:
            lib.ttr_set_stage_events(events, len(plan) + 1)
        return ttr.distill_step(state, Q, K, V, w.L, args.lr, eps, teacher=teacher, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nev = len(plan) + 1
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record(stream)
    handles = [(ctypes.c_void_p * nev)(*[e.cuda_event for e in row]) for row in ev]
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        loss = step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    last_loss = loss.cpu().tolist()
    for i in range(args.steps):
        step(handles[i])
    torch.cuda.synchronize()
    kern_ms = {name: float(np.mean([ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(args.steps)]))
               for k, (name, _, _) in enumerate(plan)}
    name, flops, nb = max(plan, key=lambda p: kern_ms[p[0]])
    rl = roofline(w, flops, nb, kern_ms[name])
    kernels = {}
    for kn, kf, kb in plan:
        r = roofline(w, kf, kb, kern_ms[kn]) if (kf or kb) else {"bound": None, "frac": None}
        kernels[kn] = {"ms": kern_ms[kn], "flops": kf, "bytes": kb, "bound": r["bound"], "frac": r["frac"]}
    total_flops = sum(p[1] for p in plan)
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    if nq is None:
        metric = (f"TTR distillation step tokens/sec ({w.name}: B={w.B}, H={w.H}, N={w.N}, L={w.L}; teacher, "
                  "student, loss, backward and Adam)")
        value, unit = w.B * w.N / (ms * 1e-3), "tokens/s"
    else:
        metric = (f"TTR distillation step on a replay sample, samples/sec ({w.name}: B={w.B}, H={w.H}, N={w.N} keys, "
                  f"Nq={nq} query rows, L={w.L}; teacher rows given; student, loss, backward and Adam)")
        value, unit = w.B / (ms * 1e-3), "samples/s"
    res = {
        "metric": metric,
        "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "mode": "distill" if nq is None else "distill_sample", "B": w.B, "H": w.H,
                   "N": w.N, "Nq": w.N if nq is None else nq, "D": w.D, "F": w.F, "L": w.L,
                   "lr": args.lr, "global_batch": w.B, "seq_len": w.N},
        "roofline": {"kernel": name, "bound": rl["bound"], "achieved": rl["achieved"], "peak": rl["peak"],
                     "unit": rl["unit"], "frac": rl["frac"], "traffic": None,
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nb,
                     "avg_launch_ms": kern_ms[name]},
        "forward": {"tflops": total_flops / (ms * 1e-3) / 1e12,
                    "frac_mfma_peak": total_flops / (ms * 1e-3) / 1e12 / peak,
                    "kernels": kernels, "wall_s": wall, "last_loss": last_loss},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_distill(w, x, args.cpu_seconds, args.lr, nq)
    print(json.dumps(res), flush=True)


def main_cosine(args):
    """The gate's cosine distance on [B,H,N,D] tensors of the workload: the
    student is the hybrid forward's output, the teacher the softmax attention
    over every token (both in the IO dtype). HBM-bound: both tensors read once."""
    import ctypes
    import numpy as np
    import torch
    import linear_hybrid_attention_amd as ttr
    import workloads

    w = workloads.WORKLOADS[args.workload]
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    io_t = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def io(name):
        if w.dtype == "bf16":
            return torch.from_numpy(x[name + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x[name]).to(dev)

    Q, K, V = io("Q"), io("K"), io("V")
    W = None if x["W"] is None else io("W")
    b = None if x["b"] is None else torch.from_numpy(x["b"]).to(dev)
    g = torch.from_numpy(x["g"]).to(dev)
    student = ttr.hybrid_forward(Q, K, V, W, b, g, float(x["eps"]), w.L)
    gneg = torch.full_like(g, float("-inf"))
    teacher = ttr.hybrid_forward(Q, K, V, W, b, gneg, float(x["eps"]), w.N)  # alpha = 0, every token a landmark
    lib = ttr.load_library()
    d = ttr.Dims(w.B, w.H, w.N, w.D, w.D, 1 if w.dtype == "bf16" else 0, 0)
    ws = torch.empty(lib.ttr_cosine_workspace_bytes(d), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        out = ttr.cosine_distance(student, teacher, ws=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        out = ttr.cosine_distance(student, teacher, ws=ws)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record(stream)
    handles = [(ctypes.c_void_p * 3)(*[e.cuda_event for e in row]) for row in ev]
    torch.cuda.synchronize()
    for i in range(args.steps):
        lib.ttr_set_stage_events(handles[i], 3)
        ttr.cosine_distance(student, teacher, ws=ws)
    torch.cuda.synchronize()
    part_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]))
    total_ms = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)]))
    io_b = 2 if w.dtype == "bf16" else 4
    nbytes = 2 * w.B * w.H * w.N * w.D * io_b
    rl = roofline(w, 0, nbytes, part_ms)
    res = {"metric": f"readiness-gate cosine distance rows/sec ({w.name}: B={w.B}, H={w.H}, N={w.N}, D={w.D})",
           "value": w.B * w.H * w.N / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
           "config": {"workload": w.name, "mode": "cosine", "B": w.B, "H": w.H, "N": w.N, "D": w.D},
           "roofline": {"kernel": "cos_part_kernel", "bound": rl["bound"],
                        "achieved": rl["achieved"], "peak": rl["peak"], "unit": rl["unit"], "frac": rl["frac"],
                        "traffic": None, "algorithmic_flops_per_launch": 0, "algorithmic_bytes_per_launch": nbytes,
                        "avg_launch_ms": part_ms},
           "kernels": {"cos_part_kernel": {"ms": part_ms}, "cos_total_kernel": {"ms": total_ms}},
           "distance": float(out.cpu()), "cpu_baseline": None}
    if not args.no_cpu_baseline:
        import oracle.ttr_oracle as O
        s_np = student.float().cpu().numpy()
        t_np = teacher.float().cpu().numpy()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) or reps == 0:
            O.cosine_distance(s_np, t_np)
            reps += 1
        sec = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": w.B * w.H * w.N / sec, "unit": "rows/s", "cores": os.cpu_count() or 1,
                               "kind": "oracle", **host_info(), "sample": f"the whole {w.name} pair, {reps} pass(es)"}
    print(json.dumps(res), flush=True)


def main_staged(args):
    """The staged entry points on the workload, one call each: ttr_feature_map (of Q), ttr_kv_reduce,
    ttr_apply, ttr_landmark_attn and ttr_blend, each timed by HIP events around the call while a spin
    kernel keeps the GPU behind the host (so the events see the kernels, not the launch latency), each
    with the roofline of its algorithmic flops and bytes (its fp32 intermediates are part of its
    interface: they are counted)."""
    import numpy as np
    import torch
    import linear_hybrid_attention_amd as ttr
    import workloads

    w = workloads.WORKLOADS[args.workload]
    if w.causal or not w.proj or w.L == 0:
        print("--staged needs a non-causal workload with a projection and landmarks", file=sys.stderr)
        sys.exit(2)
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def io(name):
        if w.dtype == "bf16":
            return torch.from_numpy(x[name + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x[name]).to(dev)

    Q, K, V, W = io("Q"), io("K"), io("V"), io("W")
    b, g = torch.from_numpy(x["b"]).to(dev), torch.from_numpy(x["g"]).to(dev)
    eps = float(x["eps"])
    iot = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    KV, ksum = ttr.kv_reduce(K, V, W, b)
    out_lin = ttr.apply(Q, W, b, KV, ksum, eps)
    out_lm = ttr.landmark_attn(Q, K, V, w.L)
    Z, N, D, F, L = w.B * w.H, w.N, w.D, w.F, w.L
    ib = 2 if w.dtype == "bf16" else 4
    stages = [
        ("ttr_feature_map (phi of Q)", lambda: ttr.feature_map(Q, W, b), 2 * Z * N * D * F, Z * N * (D + F) * ib),
        ("ttr_kv_reduce", lambda: ttr.kv_reduce(K, V, W, b), 4 * Z * N * D * F,
         2 * Z * N * D * ib + Z * F * (D + 1) * 4),
        ("ttr_apply", lambda: ttr.apply(Q, W, b, KV, ksum, eps), 4 * Z * N * D * F,
         Z * N * D * (ib + 4) + Z * F * (D + 1) * 4),
        ("ttr_landmark_attn", lambda: ttr.landmark_attn(Q, K, V, L), 4 * Z * N * L * D,
         Z * N * D * (ib + 4) + 2 * Z * L * D * ib),
        ("ttr_blend", lambda: ttr.blend(out_lin, out_lm, g, iot), 0, Z * N * D * (8 + ib)),
    ]
    stream = torch.cuda.current_stream(dev)
    res_st = {}
    for name, fn, fl, nb in stages:
        for _ in range(max(3, args.warmup // 4)):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda._sleep(50_000_000)  # the GPU spins while the host enqueues every timed call
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
        r = roofline(w, fl, nb, ms)
        res_st[name] = {"ms": ms, "flops": fl, "bytes": nb, "bound": r["bound"], "achieved": r["achieved"],
                        "peak": r["peak"], "unit": r["unit"], "frac": r["frac"]}
    total = sum(v["ms"] for v in res_st.values())
    top = max(res_st, key=lambda k: res_st[k]["ms"])
    t = res_st[top]
    res = {"metric": f"staged TTR hybrid attention tokens/sec ({w.name}: B={w.B}, H={w.H}, N={w.N}, L={w.L}; five "
                     "entry points with fp32 intermediates)",
           "value": w.B * w.N / (total * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": total, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
           "config": {"workload": w.name, "mode": "staged", "B": w.B, "H": w.H, "N": w.N, "D": w.D, "F": w.F,
                      "L": w.L},
           "roofline": {"kernel": top, "bound": t["bound"], "achieved": t["achieved"],
                        "peak": t["peak"],
                        "unit": t["unit"], "frac": t["frac"], "traffic": None,
                        "algorithmic_flops_per_launch": t["flops"], "algorithmic_bytes_per_launch": t["bytes"],
                        "avg_launch_ms": t["ms"]},
           "stages": res_st, "cpu_baseline": None}
    print(json.dumps(res), flush=True)


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def main_replay(args):
    """Replay-buffer offload of one layer call of the workload (K, V whole, a
    quarter of the query rows, fp32 teacher rows there) into the default
    768 MiB pinned ring: push throughput (device -> host), fetch throughput
    (host -> device), and a push issued beside a distillation step."""
    import ctypes
    import numpy as np
    import torch
    import linear_hybrid_attention_amd as ttr
    import workloads

    w = workloads.WORKLOADS[args.workload]
    if w.causal or not w.proj:
        print("--replay needs a non-causal workload with a projection", file=sys.stderr)
        sys.exit(2)
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def io(name):
        if w.dtype == "bf16":
            return torch.from_numpy(x[name + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x[name]).to(dev)

    Q, K, V = io("Q"), io("K"), io("V")
    T = torch.from_numpy(np.random.default_rng(w.seed + 7).standard_normal((w.B, w.H, w.N, w.D),
                                                                           dtype=np.float32)).to(dev)
    Nq = max(1, w.N // 4)
    idx = workloads.query_subsample(w.N, Nq, w.seed)
    io_b = 2 if w.dtype == "bf16" else 4
    slices = w.B * w.H
    payload = 2 * slices * w.N * w.D * io_b + slices * Nq * w.D * (io_b + 4) + Nq * 4
    rb = ttr.ReplayBuffer(768 << 20, 128 << 20)
    for _ in range(args.warmup):
        rb.push(Q, K, V, idx, T)
    rb.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        rb.push(Q, K, V, idx, T)
    rb.synchronize()
    push_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    lib = ttr.load_library()
    stages = ("gather_rows_kernel", "rows D2H", "K D2H", "V D2H")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record(torch.cuda.current_stream(dev))
    handles = [(ctypes.c_void_p * 5)(*[e.cuda_event for e in row]) for row in ev]
    torch.cuda.synchronize()
    for i in range(args.steps):
        lib.ttr_set_stage_events(handles[i], 5)
        rb.push(Q, K, V, idx, T)
    rb.synchronize()
    per = np.array([[ev[i][k].elapsed_time(ev[i][k + 1]) for k in range(4)] for i in range(args.steps)])
    tot = per.sum(axis=1)
    kern_ms = float(tot.mean())
    stage_ms = {n: {"mean": float(per[:, k].mean()), "median": float(np.median(per[:, k]))}
                for k, n in enumerate(stages)}
    held = rb.ids()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rb.fetch(held[0])
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        rb.fetch(held[i % len(held)])
    end.record(stream)
    torch.cuda.synchronize()
    fetch_ms = start.elapsed_time(end) / args.steps

    # a push beside each distillation step (both read Q, K, V only)
    b = x["b"] if x["b"] is not None else np.zeros((w.H, w.F), np.float32)
    state = ttr.DistillState(torch.from_numpy(x["W"]).to(dev), torch.from_numpy(b).to(dev),
                             torch.from_numpy(x["g"]).to(dev))
    d = ttr.Dims(w.B, w.H, w.N, w.D, w.F, 1 if w.dtype == "bf16" else 0, 0)
    ws = torch.empty(lib.ttr_distill_workspace_bytes(d, w.L, 1), dtype=torch.uint8, device=dev)
    eps = float(x["eps"])
    nov = max(5, args.steps // 4)
    for _ in range(3):
        ttr.distill_step(state, Q, K, V, w.L, args.lr, eps, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(nov):
        ttr.distill_step(state, Q, K, V, w.L, args.lr, eps, ws=ws)
    torch.cuda.synchronize()
    alone_ms = (time.perf_counter() - t0) * 1e3 / nov
    t0 = time.perf_counter()
    for _ in range(nov):
        rb.push(Q, K, V, idx, T)
        ttr.distill_step(state, Q, K, V, w.L, args.lr, eps, ws=ws)
    torch.cuda.synchronize()
    rb.synchronize()
    both_ms = (time.perf_counter() - t0) * 1e3 / nov
    st = rb.stats()
    push_gbs = payload / (push_ms * 1e-3) / 1e9
    kern_gbs = payload / (kern_ms * 1e-3) / 1e9
    res = {"metric": f"replay-buffer offload GB/s ({w.name}: B={w.B}, H={w.H}, N={w.N}, D={w.D}, Nq={Nq}, "
                     "K/V whole + query and fp32 teacher rows, 768 MiB pinned ring)",
           "value": push_gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": push_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
           "config": {"workload": w.name, "mode": "replay", "B": w.B, "H": w.H, "N": w.N, "D": w.D, "Nq": Nq,
                      "sample_payload_bytes": payload, "budget_bytes": 768 << 20},
           "roofline": {"kernel": "push copies: gather_rows_kernel to device staging, then DMA of rows, K and V into the pinned ring", "bound": "pcie",
                        "achieved": kern_gbs, "peak": PCIE_PEAK_GBS, "unit": "GB/s", "frac": kern_gbs / PCIE_PEAK_GBS,
                        "traffic": None, "algorithmic_bytes_per_launch": payload, "avg_launch_ms": kern_ms},
           "push_gpu": {"mean_ms": kern_ms, "median_ms": float(np.median(tot)), "stages": stage_ms},
           "fetch": {"ms": fetch_ms, "GB/s": payload / (fetch_ms * 1e-3) / 1e9},
           "overlap": {"distill_step_ms": alone_ms, "push_ms": push_ms, "push_plus_distill_ms": both_ms},
           "held": {"count": st.count, "bytes_used": st.bytes_used, "evicted": st.evicted},
           "cpu_baseline": None}
    rb.close()
    if not args.no_cpu_baseline:
        import oracle.ttr_oracle as O
        hq = x["Q_bits"] if w.dtype == "bf16" else x["Q"]
        hk = x["K_bits"] if w.dtype == "bf16" else x["K"]
        hv = x["V_bits"] if w.dtype == "bf16" else x["V"]
        ht = T.cpu().numpy()
        ref = O.ReplayBuffer(768 << 20)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) or reps == 0:
            ref.push(hq, hk, hv, idx, ht)
            reps += 1
        sec = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": payload / sec / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle", **host_info(),
                               "sample": f"{reps} pushes of the {w.name} sample into the oracle's model (host copies)"}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic, args.workload, args.copy_mib)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (every (batch, head) "
              "slice is independent; see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import linear_hybrid_attention_amd as ttr
    import workloads

    if args.workload in workloads.LAYER_WORKLOADS:
        main_layer(args)
        return
    if args.distill:
        main_distill(args)
        return
    if args.replay:
        main_replay(args)
        return
    if args.staged:
        main_staged(args)
        return
    if args.cosine:
        main_cosine(args)
        return
    w = workloads.WORKLOADS[args.workload]
    if args.chunk and w.causal:
        w = w.with_(chunk=args.chunk)
    x = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def io(name):
        if x[name] is None:
            return None
        if w.dtype == "bf16":
            return torch.from_numpy(x[name + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x[name]).to(dev)

    Q, K, V, W = io("Q"), io("K"), io("V"), io("W")
    b = None if x["b"] is None else torch.from_numpy(x["b"]).to(dev)
    g = torch.from_numpy(x["g"]).to(dev)
    eps = float(x["eps"])
    out = torch.empty_like(Q)
    lib = ttr.load_library()
    F = w.F
    nbytes = ttr.workspace_bytes(w.B, w.H, w.N, w.D, F, 1 if w.dtype == "bf16" else 0, w.L, w.causal,
                                 w.chunk if w.causal else 0)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        if events is not None:
            lib.ttr_set_stage_events(events, len(plan) + 1)
        ttr.hybrid_forward(Q, K, V, W, b, g, eps, w.L, causal=w.causal, out=out, ws=ws,
                           chunk=w.chunk if w.causal else 0)

    plan = kernel_plan(w)
    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel events: len(plan) + 1 per step, created (recorded once) before the timed region
    import ctypes
    nev = len(plan) + 1
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for row in ev:
        for e in row:
            e.record(stream)
    handles = [(ctypes.c_void_p * nev)(*[e.cuda_event for e in row]) for row in ev]
    torch.cuda.synchronize()

    # Headline: K forwards back to back, nothing recorded between kernels.
    # Cold: before each forward a 1 GiB buffer is written (every L2 line and
    # the MALL now hold other data) and each forward is timed on its own.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.cold else None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if flush is None:
        host_lead(args.steps)
        start.record(stream)
        for i in range(args.steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)
    else:
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            pairs[i][0].record(stream)
            step()
            pairs[i][1].record(stream)
        torch.cuda.synchronize()
        total_ms = sum(a.elapsed_time(b) for a, b in pairs)
    wall = time.perf_counter() - t0
    ms = total_ms / args.steps
    # Per-kernel durations: another K forwards with an event between kernels.
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        step(handles[i])
    torch.cuda.synchronize()
    kern_ms = {}
    for k, (name, _, _) in enumerate(plan):
        kern_ms[name] = float(np.mean([ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(args.steps)]))
    name, flops, nbytes = max(plan, key=lambda p: kern_ms[p[0]])
    rl = roofline(w, flops, nbytes, kern_ms[name])
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        ent = tr.get(w.name, {}).get(name)
        if ent and ent.get("source_hash") == source_hash(ent["sources"]):
            traffic = ent["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None
    kernels = {}
    for kn, kf, kb in plan:
        r = roofline(w, kf, kb, kern_ms[kn]) if (kf or kb) else {"bound": None, "frac": None}
        kernels[kn] = {"ms": kern_ms[kn], "flops": kf, "bytes": kb, "bound": r["bound"], "frac": r["frac"]}
    total_flops = sum(p[1] for p in plan)
    peak_fwd = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    if w.causal:
        metric = f"causal linear-attention tokens/sec (B={w.B}, H={w.H}, N={w.N}, D={w.D})"
    elif w.name == "flux_1024":
        metric = "hybrid-attention tokens/sec at Flux 1024^2 (24 heads) + % bf16 MFMA peak"
    else:
        metric = f"hybrid-attention tokens/sec ({w.name}: B={w.B}, H={w.H}, N={w.N}, D={w.D}, L={w.L})"
    res = {
        "metric": metric,
        "value": w.B * w.N / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "F": w.F, "L": w.L,
                   "causal": w.causal, **({"chunk": w.chunk} if w.causal else {}),
                   "caches": "cold" if args.cold else "hot", "global_batch": w.B, "seq_len": w.N,
                   "clock_settle_ms": args.settle_ms, "clock_settle_calls": settled},
        "roofline": {"kernel": name, "bound": rl["bound"], "achieved": rl["achieved"], "peak": rl["peak"],
                     "unit": rl["unit"], "frac": rl["frac"], "traffic": traffic,
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_ms": kern_ms[name]},
        "forward": {"tflops": total_flops / (ms * 1e-3) / 1e12,
                    "frac_mfma_peak": total_flops / (ms * 1e-3) / 1e12 / peak_fwd,
                    "algorithmic_bytes": algorithmic_bytes(w),
                    "frac_hbm_peak": algorithmic_bytes(w) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "kernels": kernels, "wall_s": wall},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
