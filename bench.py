#!/usr/bin/env python3
"""Benchmark of the fused AllGather-GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-extras]

A step is one fused AG-GEMM call (copy tasks + flag waits + MFMA tiles, one
persistent kernel) on the 70B-class TP=8 share: R = 8 ranks x [1024, 8192]
bf16 shards gathered to [8192, 8192], times B [8192, 3584], bf16 output. All
inputs are seeded synthetic data (N(0, 0.02), seed 3) already resident in HBM
when the timed region starts. The same JSON line also reports:
  * overlap: T_fused, T_gemm (GEMM tiles only, flags treated as published),
    T_copy (copy tasks only), T_serial (copy kernel, event, GEMM kernel on a
    second stream), E_max = max(T_copy, T_gemm) / T_fused, E_serial;
  * the other hot-path operations at their workloads (8B-class AG-GEMM,
    GEMM-ReduceScatter, AllGather + MoE grouped GEMM);
  * roofline of the dominant kernel and the CPU oracle timed on a sample.
--skip-extras drops those extra measurements (profiler runs); the timed step
is unchanged.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
WORKLOAD = "ag_gemm_70b"
METRIC = "fused AG-GEMM TFLOP/s + % bf16 MFMA peak; overlap eff. vs serial copy+GEMM"


# Sources the AG-GEMM kernel is built from (the other kernels' files do not
# change it, so they do not invalidate its counter record).
AG_KERNEL_SOURCES = ["kernels.hip", "gemm_core.h", "sync.h", "sched.h", "ocg_internal.h", "api.cpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "communication_overlapped_gemm_amd", "csrc")
    for name in AG_KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_record(kernel_hash: str, launches_per_step: int = 1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", "ag_gemm_70b_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def make_events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def timed_launches(torch, fn, n, stream, ev=None):
    """Per-launch durations (ms) from HIP events on the launch stream (events
    created beforehand when `ev` is given, so their creation is not timed)."""
    ev = ev or make_events(torch, n)
    for s, e in ev:
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def cold_launch_ms(torch, fn, n, stream, flush_bytes=512 << 20):
    """Median launch time with the caches cold: a 512 MiB buffer is written
    before each launch, more than the XCD L2s and the Infinity Cache hold."""
    buf = torch.empty(flush_bytes // 4, dtype=torch.int32, device="cuda")
    ev = make_events(torch, n)
    for i, (s, e) in enumerate(ev):
        buf.fill_(i)
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    del buf
    return statistics.median(s.elapsed_time(e) for s, e in ev)


def median_ms(torch, fn, n, stream, warm=2):
    for _ in range(warm):
        fn()
    return statistics.median(timed_launches(torch, fn, n, stream))


def cpu_baseline(x, target_s=10.0, max_runs=40):
    """The float64 oracle as it stands, timed on the host cores: the whole
    AG-GEMM of the workload (gather + matmul of all R chunks), repeated until
    about `target_s` seconds of CPU work have run (a bounded sample)."""
    import numpy as np
    from oracle import reference as ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    flops = 2.0 * x.R * x.m * x.K * x.N
    ts = []
    t_all = time.perf_counter()
    while len(ts) < max_runs and (time.perf_counter() - t_all) < target_s:
        t0 = time.perf_counter()
        ref.ag_gemm(x.a_chunks, x.b)
        ts.append(time.perf_counter() - t0)
    total = sum(ts)
    return {"value": round(flops * len(ts) / total / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"numpy float64 oracle (gather + matmul) on the whole {WORKLOAD} workload "
                      f"([{x.R * x.m},{x.K}] x [{x.K},{x.N}], {flops / 1e9:.1f} GFLOP per run), "
                      f"{len(ts)} runs in {total:.1f} s (median run {statistics.median(ts):.2f} s)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--skip-extras", action="store_true")
    ap.add_argument("--op", default=WORKLOAD, choices=[WORKLOAD, "ag_gemm_8b", "gemm_rs_8b", "ag_moe", "moe_combine_rs",
                                                     "ag_attention"],
                    help="profiling aid: launch only this operation (no benchmark record)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("this build runs on one GPU: the R peer ranks are stand-in buffers in that GPU's HBM; "
              "use --gpus 1", file=sys.stderr)
        return 2
    if args.op != WORKLOAD:
        return profile_op(args.op, args.steps, args.warmup)

    import numpy as np
    import torch
    import communication_overlapped_gemm_amd as ocg
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    w = workloads.workload(WORKLOAD)
    x = w.make()
    flops = w.flops()

    def upload(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    chunks = [upload(c) for c in x.a_chunks]
    b = upload(x.b)
    M = x.R * x.m
    ag = torch.empty((M, x.K), dtype=torch.bfloat16, device=dev)
    c = torch.empty((M, x.N), dtype=torch.bfloat16, device=dev)
    ws = ocg.Workspace(ocg.OP_AG_GEMM, x.R, x.m, x.K, x.N)
    fused = ocg.default_config()

    def step():
        ocg.ag_gemm(chunks, b, 0, a_gathered=ag, c=c, workspace=ws, config=fused)

    for _ in range(args.warmup):
        step()
    ev = make_events(torch, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    per_launch = timed_launches(torch, step, args.steps, stream, ev)   # ends with synchronize
    wall = time.perf_counter() - t0
    ws.check()
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    avg_launch_ms = sum(per_launch) / len(per_launch)
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    khash = kernel_source_hash()
    info = ocg.plan_info(ocg.OP_AG_GEMM, x.R, 0, x.m, x.K, x.N)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: fused AllGather-GEMM, R=8 simulated ranks x A_r bf16 [1024,8192] "
                               f"(M=8192), B bf16 [8192,3584], N(0,0.02) seed 3, C bf16 [8192,3584]",
                   "tile": f"{info['BM']}x{info['BN']}", "slab_rows": info["slab_rows"],
                   "copy_rows": info["copy_rows"], "local_rank": 0},
        "pct_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_record(khash),
                     "kernel": f"ag_gemm_kernel<{info['BM']},{info['BN']}>",
                     "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                     "algorithmic_flops_per_launch": flops, "kernel_hash": khash},
    }

    if not args.skip_extras:
        n = max(10, args.steps)
        gemm_only = ocg.default_config(mode=ocg.MODE_GEMM_ONLY)
        copy_only = ocg.default_config(mode=ocg.MODE_COPY_ONLY)
        t_fused = statistics.median(per_launch)
        t_gemm = median_ms(torch, lambda: ocg.ag_gemm(chunks, b, 0, a_gathered=ag, c=c, workspace=ws,
                                                       config=gemm_only), n, stream)
        t_copy = median_ms(torch, lambda: ocg.ag_gemm(chunks, b, 0, a_gathered=ag, c=c, workspace=ws,
                                                       config=copy_only), n, stream)
        s2 = torch.cuda.Stream()
        ev = torch.cuda.Event()

        def serial():
            ocg.ag_gemm(chunks, b, 0, a_gathered=ag, c=c, workspace=ws, config=copy_only, stream=stream)
            ev.record(stream)
            s2.wait_event(ev)
            ocg.ag_gemm(chunks, b, 0, a_gathered=ag, c=c, workspace=ws, config=gemm_only, stream=s2)
            stream.wait_stream(s2)
        t_serial = median_ms(torch, serial, n, stream)
        full = torch.cat(chunks)
        t_d2d = median_ms(torch, lambda: ag.copy_(full), n, stream)
        t_mm = median_ms(torch, lambda: torch.matmul(full, b), n, stream)
        ws.check()
        copy_bytes = 2.0 * M * x.K * 2
        rec["overlap"] = {
            "t_fused_us": round(t_fused * 1e3, 2), "t_gemm_us": round(t_gemm * 1e3, 2),
            "t_copy_us": round(t_copy * 1e3, 2), "t_serial_us": round(t_serial * 1e3, 2),
            "e_max": round(max(t_copy, t_gemm) / t_fused, 4), "e_serial": round(t_serial / t_fused, 4),
            "gemm_only_tflops": round(flops / (t_gemm * 1e-3) / 1e12, 2),
            "copy_only_gbs": round(copy_bytes / (t_copy * 1e-3) / 1e9, 1),
            "d2d_copy_gbs_yardstick": round(copy_bytes / (t_d2d * 1e-3) / 1e9, 1),
            "torch_matmul_tflops_yardstick": round(flops / (t_mm * 1e-3) / 1e12, 2),
        }
        del full
        q = sorted(per_launch)
        pct = lambda f: q[min(len(q) - 1, int(round(f * (len(q) - 1))))] * 1e3
        rec["launch_stats"] = {"p10_us": round(pct(0.1), 2), "p50_us": round(pct(0.5), 2),
                               "p90_us": round(pct(0.9), 2),
                               "cold_us": round(cold_launch_ms(torch, step, 10, stream) * 1e3, 2)}
        rec["ops"] = other_ops(torch, np, ocg, workloads, upload, stream, n)
        rec["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(rec), flush=True)
    return 0


def op_setups(torch, ocg, workloads, upload):
    """name -> (workload, setup()) where setup() returns (launch_fused(), extras)
    for the other operations (fused launches with caller-owned buffers)."""
    import numpy as np

    def ag8():
        w = workloads.workload("ag_gemm_8b")
        x = w.make()
        chunks = [upload(a) for a in x.a_chunks]
        b = upload(x.b)
        ag = torch.empty((x.R * x.m, x.K), dtype=torch.bfloat16, device="cuda")
        c = torch.empty((x.R * x.m, x.N), dtype=torch.bfloat16, device="cuda")
        ws = ocg.Workspace(ocg.OP_AG_GEMM, x.R, x.m, x.K, x.N)

        def launch(mode=0):
            ocg.ag_gemm(chunks, b, 0, a_gathered=ag, c=c, workspace=ws, config=ocg.default_config(mode=mode))
        return w, x, ws, launch

    def rs8():
        w = workloads.workload("gemm_rs_8b")
        x = w.make()
        a, b = upload(x.a), upload(x.b)
        peers = [None] + [upload(x.peers[s]) for s in range(1, x.R)]
        part = torch.empty((x.M, x.N), dtype=torch.bfloat16, device="cuda")
        o = torch.empty((x.M // x.R, x.N), dtype=torch.bfloat16, device="cuda")
        ws = ocg.Workspace(ocg.OP_GEMM_RS, x.R, x.M, x.K, x.N)

        def launch(mode=0):
            ocg.gemm_rs(a, b, peers, 0, partial=part, out=o, workspace=ws)
        return w, x, ws, launch

    def moe():
        w = workloads.workload("ag_moe")
        x = w.make()
        chunks = [upload(a) for a in x.a_chunks]
        lg = torch.from_numpy(x.logits).to("cuda")
        wt = upload(x.w)
        ws = ocg.Workspace(ocg.OP_AG_GROUPED_GEMM, x.R, x.m, x.K, x.N, x.E, x.topk)
        outs = ocg.ag_grouped_gemm(chunks, lg, wt, x.topk, 0, workspace=ws)

        def launch(mode=0):
            ocg.ag_grouped_gemm(chunks, lg, wt, x.topk, 0, workspace=ws, outputs=outs)
        return w, x, ws, launch

    def comb():
        w = workloads.workload("moe_combine_rs")
        x = w.make()
        y = upload(x.y)
        wt = torch.from_numpy(np.ascontiguousarray(x.w)).to("cuda")
        T = x.R * x.m
        peers = [None if s == x.local_rank else upload(x.peers[s]) for s in range(x.R)]
        part = torch.empty((T, x.N), dtype=torch.bfloat16, device="cuda")
        o = torch.empty((x.m, x.N), dtype=torch.bfloat16, device="cuda")
        ws = ocg.Workspace(ocg.OP_MOE_COMBINE_RS, x.R, x.m, 0, x.N, 0, x.topk)

        def launch(mode=0):
            ocg.moe_combine_rs(y, wt, peers, x.local_rank, partial=part, out=o, workspace=ws)
        return w, x, ws, launch

    def attn():
        w = workloads.workload("ag_attention")
        x = w.make()
        q = upload(x.q)
        ks = [upload(c) for c in x.k_chunks]
        vs = [upload(c) for c in x.v_chunks]
        S = x.R * x.m
        kg = torch.empty((S, x.Hkv, x.d), dtype=torch.bfloat16, device="cuda")
        vg = torch.empty((S, x.Hkv, x.d), dtype=torch.bfloat16, device="cuda")
        o = torch.empty((x.m, x.Hq, x.d), dtype=torch.bfloat16, device="cuda")
        ws = ocg.Workspace(ocg.OP_AG_ATTENTION, x.R, x.m, x.Hq, x.Hkv)

        def launch(mode=0):
            ocg.ag_attention(q, ks, vs, x.local_rank, k_gathered=kg, v_gathered=vg, out=o, workspace=ws,
                             config=ocg.default_config(mode=mode))
        return w, x, ws, launch

    return {"ag_gemm_8b": ag8, "gemm_rs_8b": rs8, "ag_moe": moe, "moe_combine_rs": comb, "ag_attention": attn}


def other_ops(torch, np, ocg, workloads, upload, stream, n):
    out = {}
    setups = op_setups(torch, ocg, workloads, upload)
    # 8B-class AG-GEMM share
    w, x, ws, launch = setups["ag_gemm_8b"]()
    times = {label: median_ms(torch, lambda: launch(mode), n, stream)
             for label, mode in (("fused", 0), ("gemm", 1), ("copy", 2))}
    ws.check()
    out["ag_gemm_8b"] = {"t_fused_us": round(times["fused"] * 1e3, 2), "t_gemm_us": round(times["gemm"] * 1e3, 2),
                         "t_copy_us": round(times["copy"] * 1e3, 2),
                         "tflops": round(w.flops() / (times["fused"] * 1e-3) / 1e12, 2),
                         "e_max": round(max(times["gemm"], times["copy"]) / times["fused"], 4)}
    del launch
    # GEMM-ReduceScatter share
    w, x, ws, launch = setups["gemm_rs_8b"]()
    t = median_ms(torch, launch, n, stream)
    ws.check()
    blk_bytes = (x.M // x.R) * x.N * 2
    out["gemm_rs_8b"] = {"t_us": round(t * 1e3, 2), "tflops": round(w.flops() / (t * 1e-3) / 1e12, 2),
                         "reduce_bytes": 9 * blk_bytes}
    del launch
    # AllGather + MoE grouped GEMM
    w, x, ws, launch = setups["ag_moe"]()
    t = median_ms(torch, launch, n, stream)
    ws.check()
    T = x.R * x.m
    hbm = x.E * x.K * x.N * 2 + 2 * 7 * x.m * x.K * 2 + T * x.K * 2 + T * x.topk * x.N * 2 + T * x.E * 4
    out["ag_moe"] = {"t_us": round(t * 1e3, 2), "tflops": round(w.flops() / (t * 1e-3) / 1e12, 2),
                     "hbm_gbs_algorithmic": round(hbm / (t * 1e-3) / 1e9, 1),
                     "hbm_frac": round(hbm / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del launch
    # MoE TopK-Reduce + ReduceScatter (HBM-bound)
    w, x, ws, launch = setups["moe_combine_rs"]()
    t = median_ms(torch, launch, n, stream)
    ws.check()
    T = x.R * x.m
    hbm = T * x.topk * x.N * 2 + T * x.topk * 4 + T * x.N * 2 + x.R * x.m * x.N * 2 + x.m * x.N * 2
    out["moe_combine_rs"] = {"t_us": round(t * 1e3, 2), "hbm_bytes": hbm,
                             "hbm_gbs_algorithmic": round(hbm / (t * 1e-3) / 1e9, 1),
                             "hbm_frac": round(hbm / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del launch
    # AllGather-KV attention (MFMA-bound): fused, attention only, copies only
    w, x, ws, launch = setups["ag_attention"]()
    # the modes alternate in three rounds (the clock drifts while the chip
    # warms, and one block of launches per mode would fold that drift into
    # the comparison); median over all of a mode's launches
    samples = {"fused": [], "attn": [], "copy": []}
    for _ in range(3):
        for label, mode in (("fused", 0), ("attn", 1), ("copy", 2)):
            launch(mode)
            samples[label] += timed_launches(torch, lambda: launch(mode), max(n // 3, 5), stream)
    times = {label: statistics.median(v) for label, v in samples.items()}
    ws.check()
    tf = w.flops() / (times["fused"] * 1e-3) / 1e12
    out["ag_attention"] = {"t_fused_us": round(times["fused"] * 1e3, 2), "t_attn_us": round(times["attn"] * 1e3, 2),
                           "t_copy_us": round(times["copy"] * 1e3, 2), "tflops": round(tf, 2),
                           "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                           "e_max": round(max(times["attn"], times["copy"]) / times["fused"], 4)}
    return out


def profile_op(op, steps, warmup):
    """Launch one of the other operations `warmup + steps` times (fused), for
    kernel profiles; prints one summary line."""
    import numpy as np
    import torch
    import communication_overlapped_gemm_amd as ocg
    import workloads

    def upload(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")
    w, x, ws, launch = op_setups(torch, ocg, workloads, upload)[op]()
    for _ in range(warmup + steps):
        launch()
    torch.cuda.synchronize()
    ws.check()
    print(json.dumps({"profile_op": op, "launches": warmup + steps}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
