#!/usr/bin/env python3
"""Benchmark of the fused AllGather-GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-extras]

A step is one fused AG-GEMM call on the 70B-class TP=8 share: R = 8 ranks x
[1024, 8192] bf16 shards gathered to [8192, 8192], times B [8192, 3584], bf16
output: one persistent kernel whose workgroups copy the peers' rows slab by
slab and publish the flags the GEMM tiles then wait on (the default, inline
transfer). The overlap legs also time the side transfer, in which a
producer kernel on a second stream copies K-slab by K-slab beside the GEMM
kernel. All inputs are seeded synthetic data (N(0, 0.02), seed 3) already
resident in HBM when the timed region starts.

Order of work: (1) the overlap legs -- fused (inline copies), fused with the
side producer, GEMM tiles only, copies only (both forms) and copy-then-GEMM
on two streams -- timed in alternating rounds, so clock drift is shared by
all legs; they also carry the chip through the power-management transient
of its first ~35 ms under load (launches of a fresh process first run fast,
then ~30 % slow, then settle), whose first launches are reported as
`transient`; (2) W warm-up steps, then exactly K timed steps between
synchronisations -- the headline; (3) the shader clock, read from traced
launches (s_memtime cycles against the 100 MHz clock), the other operations
and the CPU oracle. --skip-extras keeps (1)'s settling launches of the fused
step only and drops (3) (profiler runs).
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


def git_sha() -> str:
    try:
        import subprocess
        return subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"], capture_output=True,
                              text=True, timeout=10).stdout.strip() or "unknown"
    except Exception:
        return "unknown"


def gpu_temperature():
    """Edge/junction temperature from rocm-smi, or None if it cannot be read."""
    try:
        import subprocess
        out = subprocess.run(["rocm-smi", "--showtemp", "--json"], capture_output=True, text=True, timeout=20).stdout
        card = next(iter(json.loads(out).values()))
        return {k: v for k, v in card.items() if "emperature" in k}
    except Exception:
        return None


def trace_dtype():
    """One ocg_trace_rec (80 bytes) as a numpy record."""
    import numpy as np
    return np.dtype([("ticket", "<u4"), ("kind", "<u4"), ("a", "<u4"), ("b", "<u4"), ("c", "<u4"),
                     ("d", "<u4"), ("hw", "<u4"), ("epoch", "<u4"), ("t_start", "<u8"), ("t_ready", "<u8"),
                     ("t_end", "<u8"), ("flag_seen", "<u4"), ("queue", "<u4"), ("cycles", "<u8"),
                     ("wait_ticks", "<u4"), ("pad", "<u4")])


def traced_clock_ghz(torch, ocg, launch_cfg, n_rec, runs=5, with_cycles=False):
    """Compute-unit clock while the tiles run: per tile, shader-clock cycles
    (s_memtime) over its 100 MHz duration, median over the tiles of `runs`
    traced launches; with_cycles: also the median shader cycles per tile."""
    import numpy as np
    buf = torch.zeros(n_rec * 80, dtype=torch.uint8, device="cuda")
    cfg = launch_cfg[1]
    cfg.trace = buf.data_ptr()
    cfg.trace_capacity = n_rec
    ghz, cyc = [], []
    for _ in range(runs):
        launch_cfg[0](cfg)
        torch.cuda.synchronize()
        rec = buf.cpu().numpy().view(trace_dtype())
        t = rec[(rec["kind"] == 2) & (rec["t_end"] > rec["t_start"])]
        ghz += list(t["cycles"] / (t["t_end"] - t["t_start"]) * 0.1)   # 100 MHz ticks -> GHz
        cyc += list(t["cycles"])
    cfg.trace = None
    cfg.trace_capacity = 0
    clk = float(np.median(ghz)) if ghz else None
    if with_cycles:
        return clk, (int(np.median(cyc)) if cyc else None)
    return clk


def side_trace_summary(torch, ocg, launch, n_rec):
    """One traced fused call with the side transfer: when the producer's
    copies ran, relative to the GEMM tiles (device clock, 100 MHz)."""
    import numpy as np
    buf = torch.zeros(n_rec * 80, dtype=torch.uint8, device="cuda")
    cfg = ocg.default_config(transfer=ocg.TRANSFER_SIDE)
    cfg.trace = buf.data_ptr()
    cfg.trace_capacity = n_rec
    launch(cfg)
    torch.cuda.synchronize()
    rec = buf.cpu().numpy().view(trace_dtype())
    cp, tl = rec[rec["kind"] == 1], rec[rec["kind"] == 2]
    if not len(cp) or not len(tl):
        return None
    t0 = int(min(cp["t_start"].min(), tl["t_start"].min()))
    us = lambda v: round((float(v) - t0) / 100.0, 1)
    prod = cp[(cp["d"] & 2) != 0]
    last_copy = int(cp["t_end"].max())
    return {"copies": int(len(cp)), "producer_copies": int(len(prod)),
            "copies_us": [us(cp["t_start"].min()), us(last_copy)],
            "tiles_started_us": [us(tl["t_start"].min()), us(tl["t_start"].max())],
            "tiles_computing_while_copies_in_flight": int((tl["t_ready"] < last_copy).sum()),
            "tile_start_wait_us_median": round(float(np.median(tl["t_ready"] - tl["t_start"])) / 100.0, 2),
            "tile_kloop_wait_us_total": round(float(tl["wait_ticks"].sum()) / 100.0, 1),
            "last_tile_end_us": us(tl["t_end"].max())}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--skip-extras", action="store_true")
    ap.add_argument("--op", default=WORKLOAD, choices=[WORKLOAD, "ag_gemm_8b", "gemm_rs_8b", "ag_moe", "moe_combine_rs",
                                                     "ag_attention", "ag_moe_layer"],
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
    h = ocg.handle()
    plan = ocg.plan_ag(x.R, 0, x.m, x.K, x.N, fused, handle=h)
    transfer = {ocg.TRANSFER_INLINE: "inline", ocg.TRANSFER_SIDE: "side"}[plan["transfer"]]

    def launch(cfg, s=None):
        ocg.ag_gemm(chunks, b, 0, a_gathered=ag, c=c, workspace=ws, config=cfg, stream=s)

    def step():
        launch(fused)

    # (1) overlap legs in alternation (also the settling launches)
    first = timed_launches(torch, step, 20, stream)
    legs = {}
    if not args.skip_extras:
        gemm_only = ocg.default_config(mode=ocg.MODE_GEMM_ONLY)
        copy_only = ocg.default_config(mode=ocg.MODE_COPY_ONLY)
        copy_side = ocg.default_config(mode=ocg.MODE_COPY_ONLY, transfer=ocg.TRANSFER_SIDE)
        fused_side = ocg.default_config(transfer=ocg.TRANSFER_SIDE)
        s2 = torch.cuda.Stream()
        ev = torch.cuda.Event()

        def serial():
            launch(copy_only, stream)
            ev.record(stream)
            s2.wait_event(ev)
            launch(gemm_only, s2)
            stream.wait_stream(s2)
        full = torch.cat(chunks)
        legs = {"fused": step, "fused_side": lambda: launch(fused_side), "gemm": lambda: launch(gemm_only),
                "copy": lambda: launch(copy_only), "copy_side": lambda: launch(copy_side), "serial": serial,
                "d2d": lambda: ag.copy_(full), "matmul": lambda: torch.matmul(full, b)}
        samples = {k: [] for k in legs}
        for _ in range(6):
            for k, fn in legs.items():
                fn()
                samples[k] += timed_launches(torch, fn, 8, stream)
        ws.check()
        med = {k: statistics.median(v) for k, v in samples.items()}
        del full
    else:
        t_end = time.perf_counter() + 0.15      # settle: ~150 ms of fused launches
        while time.perf_counter() < t_end:
            timed_launches(torch, step, 20, stream)

    # (2) the headline: W warm-up steps, K timed steps
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
    info = ocg.plan_info(ocg.OP_AG_GEMM, x.R, 0, x.m, x.K, x.N, handle=h)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: fused AllGather-GEMM, R=8 simulated ranks x A_r bf16 [1024,8192] "
                               f"(M=8192), B bf16 [8192,3584], N(0,0.02) seed 3, C bf16 [8192,3584]",
                   "tile": f"{info['BM']}x{info['BN']}", "slab_rows": info["slab_rows"],
                   "copy_rows": info["copy_rows"], "kslab_cols": plan["kslab_cols"], "transfer": transfer,
                   "split_k": plan["split_k"], "local_rank": 0},
        "pct_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_record(khash),
                     # as the profiler names it: the template flag marks split-K units
                     "kernel": f"ag_gemm_kernel<{info['BM']}, {info['BN']}, {'true' if plan['split_k'] > 1 else 'false'}>",
                     "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                     "algorithmic_flops_per_launch": flops, "kernel_hash": khash},
        "git_sha": git_sha(),
    }
    q = sorted(per_launch)
    pct = lambda f: q[min(len(q) - 1, int(round(f * (len(q) - 1))))] * 1e3
    rec["launch_stats"] = {"p10_us": round(pct(0.1), 2), "p50_us": round(pct(0.5), 2), "p90_us": round(pct(0.9), 2)}
    rec["transient"] = {"first_launches_us": [round(v * 1e3, 1) for v in first],
                        "note": "the process's first 20 fused launches, before the overlap legs"}

    if not args.skip_extras:
        rec["launch_stats"]["cold_us"] = round(cold_launch_ms(torch, step, 10, stream) * 1e3, 2)
        # (3) clock while the tiles run
        n_rec = info["n_copy_or_strips"] + info["n_tiles"]
        clk = traced_clock_ghz(torch, ocg, (lambda cfg: launch(cfg), ocg.default_config()), n_rec)
        if clk:
            peak_clk = PEAK_BF16_TFLOPS * clk / 2.4
            rec["roofline"]["clock_ghz"] = round(clk, 3)
            rec["roofline"]["peak_at_clock"] = round(peak_clk, 1)
            rec["roofline"]["frac_at_clock"] = round(achieved / peak_clk, 4)
        rec["temperature"] = gpu_temperature()
        side_plan = ocg.plan_info(ocg.OP_AG_GEMM, x.R, 0, x.m, x.K, x.N,
                                  ocg.default_config(transfer=ocg.TRANSFER_SIDE), handle=h)
        rec["side_trace"] = side_trace_summary(torch, ocg, lambda cfg: launch(cfg),
                                               side_plan["n_copy_or_strips"] + side_plan["n_tiles"])
        legs_clock = {}
        for name, lcfg in (("gemm", ocg.default_config(mode=ocg.MODE_GEMM_ONLY)), ("fused", ocg.default_config()),
                           ("fused_side", ocg.default_config(transfer=ocg.TRANSFER_SIDE))):
            clk_l, cyc_l = traced_clock_ghz(torch, ocg, (lambda cfg: launch(cfg), lcfg),
                                            side_plan["n_copy_or_strips"] + side_plan["n_tiles"] + n_rec, runs=3,
                                            with_cycles=True)
            legs_clock[name] = {"clock_ghz": round(clk_l, 3) if clk_l else None, "tile_cycles_median": cyc_l}
        t_f = med["fused"]
        copy_bytes = 2.0 * M * x.K * 2
        rec["overlap"] = {
            "timing": "medians of 6 alternating rounds x 8 launches per leg",
            "transfer": transfer,
            "t_fused_us": round(t_f * 1e3, 2), "t_fused_side_us": round(med["fused_side"] * 1e3, 2),
            "t_gemm_us": round(med["gemm"] * 1e3, 2), "t_copy_us": round(med["copy"] * 1e3, 2),
            "t_copy_side_us": round(med["copy_side"] * 1e3, 2), "t_serial_us": round(med["serial"] * 1e3, 2),
            "e_max": round(max(med["copy"], med["gemm"]) / t_f, 4),
            "legs_clock": legs_clock,
            "e_serial": round(med["serial"] / t_f, 4),
            "e_max_side": round(max(med["copy"], med["gemm"]) / med["fused_side"], 4),
            "hidden_copy_frac": round((med["gemm"] + med["copy"] - t_f) / med["copy"], 4),
            "gemm_only_tflops": round(flops / (med["gemm"] * 1e-3) / 1e12, 2),
            "fused_side_tflops": round(flops / (med["fused_side"] * 1e-3) / 1e12, 2),
            "copy_only_gbs": round(copy_bytes / (med["copy"] * 1e-3) / 1e9, 1),
            "copy_side_gbs": round(copy_bytes / (med["copy_side"] * 1e-3) / 1e9, 1),
            "d2d_copy_gbs_yardstick": round(copy_bytes / (med["d2d"] * 1e-3) / 1e9, 1),
            "torch_matmul_tflops_yardstick": round(flops / (med["matmul"] * 1e-3) / 1e12, 2),
        }
        rec["ops"] = other_ops(torch, np, ocg, workloads, upload, stream, max(10, args.steps))
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
        # push transfers: stand-in receive buffers / flags of every rank; the
        # peers' pushes into ours are in place and flagged before each call
        blk = x.M // x.R
        info = ocg.plan_info(ocg.OP_GEMM_RS, x.R, 0, x.M, x.K, x.N, handle=ocg.handle())
        T = (blk // info["BM"]) * (-(-x.N // info["BN"]))
        recv = [torch.empty((x.R, blk, x.N), dtype=torch.bfloat16, device="cuda") for _ in range(x.R)]
        flags = [torch.zeros(x.R * T, dtype=torch.int32, device="cuda") for _ in range(x.R)]
        for s in range(1, x.R):
            recv[0][s].copy_(peers[s][:blk])
        step = [0]

        def launch(mode=0):
            if mode == 3:      # push
                step[0] += 1
                ocg.signal(flags[0][T:], step[0])
                ocg.gemm_rs_push(a, b, recv, flags, step[0], 0, out=o, workspace=ws)
            else:
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

    def layer():
        w = workloads.workload("ag_moe_layer")
        x = w.make()
        pr = w.params
        peers = workloads.make_moe_peers(pr["R"], pr["m"], pr["N"], pr["peer_seed"], pr["local_rank"])
        chunks = [upload(a) for a in x.a_chunks]
        lg = torch.from_numpy(x.logits).to("cuda")
        wt = upload(x.w)
        pp = [None if s_ == pr["local_rank"] else upload(peers[s_]) for s_ in range(x.R)]
        ws = ocg.Workspace(ocg.OP_AG_GROUPED_GEMM, x.R, x.m, x.K, x.N, x.E, x.topk)
        ws2 = ocg.Workspace(ocg.OP_MOE_COMBINE_RS, x.R, x.m, 0, x.N, 0, x.topk)
        outs = ocg.ag_moe_layer(chunks, lg, wt, pp, x.topk, 0, workspace=ws)
        g = ocg.ag_grouped_gemm(chunks, lg, wt, x.topk, 0, workspace=ws)

        def launch(mode=0):
            if mode == 0:      # the chain in one call
                ocg.ag_moe_layer(chunks, lg, wt, pp, x.topk, 0, workspace=ws, outputs=outs)
            else:              # the two calls one after the other
                ocg.ag_grouped_gemm(chunks, lg, wt, x.topk, 0, workspace=ws, outputs=g)
                ocg.moe_combine_rs(g["out"], g["topk_w"], pp, 0, workspace=ws2)
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

    return {"ag_gemm_8b": ag8, "gemm_rs_8b": rs8, "ag_moe": moe, "moe_combine_rs": comb, "ag_attention": attn,
            "ag_moe_layer": layer}


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
    # GEMM-ReduceScatter share: pull (the default) and push transfers, in
    # alternation (push includes the peer-notify stand-in launch)
    w, x, ws, launch = setups["gemm_rs_8b"]()
    samples = {"pull": [], "push": []}
    for _ in range(3):
        for label, mode in (("pull", 0), ("push", 3)):
            launch(mode)
            samples[label] += timed_launches(torch, lambda: launch(mode), max(n // 3, 5), stream)
    t, t_push = statistics.median(samples["pull"]), statistics.median(samples["push"])
    ws.check()
    blk_bytes = (x.M // x.R) * x.N * 2
    out["gemm_rs_8b"] = {"t_us": round(t * 1e3, 2), "tflops": round(w.flops() / (t * 1e-3) / 1e12, 2),
                         "t_push_us": round(t_push * 1e3, 2),
                         "push_tflops": round(w.flops() / (t_push * 1e-3) / 1e12, 2),
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
    # the MoE layer chain in one call against the two calls in sequence
    w, x, ws, launch = setups["ag_moe_layer"]()
    samples = {"chain": [], "separate": []}
    for _ in range(3):
        for label, mode in (("chain", 0), ("separate", 1)):
            launch(mode)
            samples[label] += timed_launches(torch, lambda: launch(mode), max(n // 3, 5), stream)
    ws.check()
    tc, tsep = statistics.median(samples["chain"]), statistics.median(samples["separate"])
    T = x.R * x.m
    hbm = (x.E * x.K * x.N * 2 + 2 * 7 * x.m * x.K * 2 + T * x.K * 2 + T * x.topk * x.N * 2 + T * x.E * 4
           + T * x.topk * x.N * 2 + T * x.topk * 4 + T * x.N * 2 + x.R * x.m * x.N * 2 + x.m * x.N * 2)
    out["ag_moe_layer"] = {"t_chain_us": round(tc * 1e3, 2), "t_separate_us": round(tsep * 1e3, 2),
                           "hbm_bytes_algorithmic": hbm,
                           "hbm_frac": round(hbm / (tc * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
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
