#!/usr/bin/env python3
"""Benchmark of the SS2D forward operator on one MI355X.

A step is one full forward call (transpose, scan, merge: every kernel of the operator) on
one batch of seeded synthetic input already resident in HBM.  W untimed warm-up steps, then
K timed steps between device synchronisations, timed with HIP events on the stream the
library launches on.  Prints ONE JSON line on stdout (details go to stderr):

  value        state updates per second (B*K*D*L*N per step / seconds per step)
  roofline     the dominant kernel (the scan) against the fp32 VALU peak
  cpu_baseline the float64 CPU oracle timed on a bounded sample of the same workload

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = ("SS2D fwd state-updates/s (B·K·D·L·N) + achieved HBM GB/s, "
          "VMamba-T stage1")
# ALU roofline of the state update on MI355X.  The VALU issues one wave64 instruction per
# 4 cycles on each of 256 CUs x 4 SIMDs at 2.4 GHz: 256 * 4 * 16 * 2.4e9 = 3.93e13 lane-ops/s
# (78.6 TFLOP/s counting an FMA as 2 flops; the published 157.3 assumes packed fp32, which
# this build does not emit).  One state update must issue 2 multiplies and 2 FMAs (6 flops)
# plus one v_exp_f32, which occupies the VALU for two issue slots (8 cycles): 6 slots per 6
# flops, so the update's arithmetic peaks at 3.93e13 * 6 / 6 = 39.3 TFLOP/s.
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
FMA_PEAK_TFLOPS = VALU_LANE_OPS * 2 / 1e12
FLOPS_PER_UPDATE = 6
ISSUE_SLOTS_PER_UPDATE = 4 + 2
UPDATE_PEAK_TFLOPS = VALU_LANE_OPS / ISSUE_SLOTS_PER_UPDATE * FLOPS_PER_UPDATE / 1e12
# With zero-order hold the update is delta*A (1 flop), (a - 1) / A as one FMA (2), times B
# and u (2), the h update (2) and C*h (2): 9 flops in at least 6 VALU slots plus the exp.
ZOH_FLOPS_PER_UPDATE = 9
ZOH_ISSUE_SLOTS_PER_UPDATE = 6 + 2
ZOH_UPDATE_PEAK_TFLOPS = (VALU_LANE_OPS / ZOH_ISSUE_SLOTS_PER_UPDATE * ZOH_FLOPS_PER_UPDATE
                          / 1e12)
# Backward, per state update: the forward recompute (delta*A, (delta*u)*B, the h update: 4
# flops, one exp) and the adjoint (g*C and the lambda update: 3; dC, dB: 2; lambda*h_prev*a:
# 2; the sums over n for ddelta and du: 4; dA: 2): 17 flops in at least 12 VALU slots plus
# the exp.
BWD_FLOPS_PER_UPDATE = 17
BWD_ISSUE_SLOTS_PER_UPDATE = 12 + 2
BWD_UPDATE_PEAK_TFLOPS = (VALU_LANE_OPS / BWD_ISSUE_SLOTS_PER_UPDATE * BWD_FLOPS_PER_UPDATE
                          / 1e12)
# Backward with zero-order hold, per state update: the recompute (delta*A, (a - 1) / A as one
# FMA, times u and B, the h update: 7 flops, one exp) and the adjoint (g*C and the lambda
# update: 3; dC: 1; dB = lambda*(bb*u): 2; lambda*h_prev*a: 2; the sums over n for ddelta
# (lambda h_prev a A and lambda a B) and du (lambda bb B): 8; dA with d bb / dA from a and
# bb: 8): 31 flops in at least 22 VALU slots plus the exp.
ZOH_BWD_FLOPS_PER_UPDATE = 31
ZOH_BWD_ISSUE_SLOTS_PER_UPDATE = 22 + 2
ZOH_BWD_UPDATE_PEAK_TFLOPS = (VALU_LANE_OPS / ZOH_BWD_ISSUE_SLOTS_PER_UPDATE
                              * ZOH_BWD_FLOPS_PER_UPDATE / 1e12)
HBM_PEAK_GBPS = 8000.0
ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


SCAN_SOURCES = ("ss2d_scan.inc", "ss2d_scan_bf16.hip", "ss2d_scan_f32.hip", "ss2d_device.h")


def kernel_source_hash() -> str:
    """Hash of the sources of the scan kernel (the kernel the roofline line describes)."""
    h = hashlib.sha256()
    for name in SCAN_SOURCES:
        f = ROOT / "selective_scan_ss2d_amd" / "csrc" / name
        h.update(name.encode())
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


FRONT_SOURCES = ("ss2d_proj.hip", "ss2d_device.h")


def source_hash(names) -> str:
    h = hashlib.sha256()
    for name in names:
        f = ROOT / "selective_scan_ss2d_amd" / "csrc" / name
        h.update(name.encode())
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, front: bool = False, R: int = 1, KW: int = 4,
                     lowrank: bool = False):
    """HBM bytes per launch of the scan kernel (or, with front, of k_project for the given
    R and KW, with lowrank in its variant that stores the R dt rows) from the committed
    counter summary, if it was taken on the current kernel sources; else None."""
    name = (f"traffic_front_lr_{workload}.json" if front and lowrank else
            f"traffic_front_{workload}.json" if front else f"traffic_{workload}.json")
    f = ROOT / "profiles" / name
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
    except ValueError:
        return None
    want = source_hash(FRONT_SOURCES) if front else kernel_source_hash()
    if d.get("source_hash") != want:
        return None
    if front and (d.get("R") != R or d.get("KW") != KW):
        return None
    return d.get("traffic_bytes_per_launch")


def cpu_baseline_backward(wl, inp, dy, target_s: float, z=None, zoh=False, u=None) -> dict:
    """The float64 oracle's backward (gated with z), as it is, on all host cores, over a
    bounded sample of whole images (its unit of work: dBs and dCs sum over every channel of
    an image)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    orc = oracle.Oracle()

    def run(n):
        sl = [inp[k][:n] if k in ("x", "dt_raw", "Bs", "Cs") else inp[k] for k in ARGS]
        zs = None if z is None else z[:n]
        t0 = time.perf_counter()
        if u is None:
            orc.backward(wl.K, *sl, dy[:n], threads=cores, z=zs, zoh=zoh)
        else:  # the operator over per-route inputs u (B, K, D, L)
            orc.backward_routes(wl.K, u[:n], *sl[1:], dy[:n], wl.H, wl.W, threads=cores, z=zs,
                                zoh=zoh)
        return time.perf_counter() - t0

    n = min(wl.B, max(1, cores))
    dt = run(n)
    if n < wl.B and dt < target_s:
        n = int(min(wl.B, max(n, n * target_s / max(dt, 1e-3))))
        dt = run(n)
    upd = n * wl.K * wl.D * wl.L * wl.N
    return {"value": upd / dt, "unit": "state-updates/s", "cores": orc.last_threads,
            "kind": "oracle",
            "sample": f"{'gated ' if z is not None else ''}{'zero-order-hold ' if zoh else ''}"
                      f"{'per-route-input ' if u is not None else ''}backward of {n} of {wl.B} "
                      f"images "
                      f"of {wl.name} (all {wl.K} routes and {wl.D} channels), {upd:.3e} state "
                      f"updates in {dt:.2f} s"}


def cpu_baseline_front(wl, inp, w, target_s: float, z=None, zoh=False,
                       lowrank=False) -> dict:
    """The float64 oracle's per-route front end followed by its operator over per-route
    inputs (with lowrank, its variants with dt_proj folded into the operator), as they are,
    on all host cores, over a bounded sample of whole images."""
    import numpy as np

    import oracle
    orc = oracle.Oracle()
    cores = len(os.sched_getaffinity(0))
    front = [w[k] for k in ("conv_w", "conv_b", "x_proj_w", "dt_proj_w")]
    R = w["dt_proj_w"].shape[-1]

    def run(n):
        t0 = time.perf_counter()
        zn = None if z is None else z[:n]
        if lowrank:
            pr = orc.project_lr(wl.K, inp["x"][:n], *front[:3], R, threads=cores)
            f32 = {k: v.astype(np.float32) for k, v in pr.items()}
            orc.forward_routes_lr(wl.K, f32["u"], f32["dt_lr"], front[3], inp["A_log"],
                                  f32["Bs"], f32["Cs"], inp["Ds"], inp["dt_bias"], wl.H, wl.W,
                                  threads=cores, z=zn, zoh=zoh)
        else:
            pr = orc.project(wl.K, inp["x"][:n], *front, threads=cores)
            f32 = {k: v.astype(np.float32) for k, v in pr.items()}
            orc.forward_routes(wl.K, f32["u"], f32["dt_raw"], inp["A_log"], f32["Bs"],
                               f32["Cs"], inp["Ds"], inp["dt_bias"], wl.H, wl.W,
                               threads=cores, z=zn, zoh=zoh)
        return time.perf_counter() - t0

    n = min(wl.B, max(1, cores // 4))
    dt = run(n)
    if n < wl.B and dt < target_s:
        n = int(min(wl.B, max(n, n * target_s / max(dt, 1e-3))))
        dt = run(n)
    upd = n * wl.K * wl.D * wl.L * wl.N
    return {"value": upd / dt, "unit": "state-updates/s", "cores": orc.last_threads,
            "kind": "oracle",
            "sample": f"front end + scan of {n} of {wl.B} images of {wl.name} (all {wl.K} "
                      f"routes and {wl.D} channels), {upd:.3e} state updates in {dt:.2f} s"}


def cpu_baseline(wl, inp, target_s: float, z=None, zoh=False) -> dict:
    """The float64 oracle, as it is, on all host cores, over a bounded sample of channels."""
    import numpy as np

    import oracle
    cores = len(os.sched_getaffinity(0))
    orc = oracle.Oracle()
    args = [inp[k] for k in ARGS]
    opts = dict(z=z, zoh=zoh)
    total = wl.B * wl.D
    rng = np.random.default_rng(0)
    n = min(total, max(cores, 64))
    order = rng.permutation(total)
    t0 = time.perf_counter()
    sel = order[:n]
    orc.forward_channels(wl.K, *args, sel // wl.D, sel % wl.D, threads=cores, **opts)
    dt = time.perf_counter() - t0
    if n < total and dt < target_s:
        n = int(min(total, max(n, n * target_s / max(dt, 1e-3))))
        sel = order[:n]
        t0 = time.perf_counter()
        orc.forward_channels(wl.K, *args, sel // wl.D, sel % wl.D, threads=cores, **opts)
        dt = time.perf_counter() - t0
    upd = n * wl.K * wl.L * wl.N
    return {"value": upd / dt, "unit": "state-updates/s", "cores": orc.last_threads,
            "kind": "oracle",
            "sample": f"{n} of {total} (b,d) channels of {wl.name} (all {wl.K} routes, full "
                      f"L={wl.L}, N={wl.N}), {upd:.3e} state updates in {dt:.2f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="vmamba_t_stage1_bf16")
    ap.add_argument("--a-log", default="init", choices=["init", "random"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gate", action="store_true",
                    help="gated entry point: y * SiLU(z), z of the shape of x")
    ap.add_argument("--zoh", action="store_true",
                    help="zero-order-hold discretisation of B")
    ap.add_argument("--kernel-sample", type=int, default=4,
                    help="time the kernels of every n-th timed step with HIP events (1: all)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward entry point (gradients of sum(dy * y); with "
                         "--gate and/or --zoh, of that operator's output, z included)")
    ap.add_argument("--front", action="store_true",
                    help="per-route front end: time ss2d_project (causal conv + SiLU, x_proj, "
                         "dt_proj) followed by ss2d_forward_routes on its outputs; with "
                         "--backward, time ss2d_backward_routes on those outputs")
    ap.add_argument("--front-r", type=int, default=1, metavar="R",
                    help="dt rank R of the front end (x_proj rows R + 2N)")
    ap.add_argument("--front-kw", type=int, default=4, metavar="KW",
                    help="conv length of the front end")
    ap.add_argument("--front-lowrank", action="store_true",
                    help="with --front: dt_proj folded into the scan (ss2d_project_lr, then "
                         "ss2d_forward_routes_lr on its R dt rows)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 5 device-to-device copies of MIB "
                         "MiB (a plain copy kernel of known size, for scaling the HBM byte "
                         "counters of a profiler run)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.kernel_sample < 1:
        log("--kernel-sample must be at least 1")
        return 2
    if args.gpus != 1 or world != 1:
        print("bench.py measures the operator on one GPU only: it has no multi-GPU path "
              "(sharding across GPUs is a design note, not implemented). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import selective_scan_ss2d_amd as ss
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written":
                          n * 4, "copies": 5}), flush=True)
        return 0
    ss.load_library()  # raises when the HIP library is not built: there is no fallback
    wl = workloads.workload(args.workload)
    log(f"workload {wl.name}: {wl.as_dict()}; generating seeded inputs")
    inp = workloads.make_inputs(wl, seed=0, a_log=args.a_log)
    dev = {}
    for k in ("x", "dt_raw", "Bs", "Cs"):
        if wl.dtype == "bf16":
            dev[k] = torch.from_numpy(inp[k + "_bf16"].view(np.int16)).view(torch.bfloat16)
        else:
            dev[k] = torch.from_numpy(inp[k])
        dev[k] = dev[k].to("cuda:0")
    for k in ("A_log", "Ds", "dt_bias"):
        dev[k] = torch.from_numpy(inp[k]).to("cuda:0")
    y = torch.empty(tuple(dev["x"].shape), dtype=dev["x"].dtype, device="cuda:0")
    gate = workloads.make_gate(wl, 0) if args.gate else None
    if args.backward and args.front_lowrank:
        log("no backward for the operator with dt_proj folded in")
        return 2
    # --backward --front: the backward of the operator over the front end's per-route
    # outputs (computed once, outside the timed region; the front end's own layers have no
    # backward here)
    routes_bwd = args.backward and args.front
    z = None
    if gate is not None:
        z = (torch.from_numpy(gate["z_bf16"].view(np.int16)).view(torch.bfloat16)
             if wl.dtype == "bf16" else torch.from_numpy(gate["z"])).to("cuda:0")
    front_w = None
    if args.front_lowrank and not args.front:
        log("--front-lowrank needs --front")
        return 2
    if args.front:
        front_w = workloads.make_front_weights(wl, 0, R=args.front_r, KW=args.front_kw)
        fw = [torch.from_numpy(front_w[k]).to("cuda:0")
              for k in ("conv_w", "conv_b", "x_proj_w", "dt_proj_w")]
        hw = (wl.H, wl.W) if wl.K == 4 else ()
        if args.front_lowrank:
            proj = ss.ss2d_project_lr if wl.K == 4 else ss.ss1d_bidir_project_lr
            fwd = ss.ss2d_forward_routes_lr if wl.K == 4 else ss.ss1d_bidir_forward_routes_lr

            def call():
                o = proj(dev["x"], *fw[:3], args.front_r)
                return fwd(o["u"], o["dt_lr"], fw[3], dev["A_log"], o["Bs"], o["Cs"],
                           dev["Ds"], dev["dt_bias"], *hw, z=z, zoh=args.zoh, y=y)
        elif routes_bwd:
            proj = ss.ss2d_project if wl.K == 4 else ss.ss1d_bidir_project
            bwd = ss.ss2d_backward_routes if wl.K == 4 else ss.ss1d_bidir_backward_routes
            po = proj(dev["x"], *fw)
            g = workloads.make_output_grad(wl, 0)
            dy = (torch.from_numpy(g["dy_bf16"].view(np.int16)).view(torch.bfloat16)
                  if wl.dtype == "bf16" else torch.from_numpy(g["dy"])).to("cuda:0")

            def call():
                return bwd(po["u"], po["dt_raw"], dev["A_log"], po["Bs"], po["Cs"], dev["Ds"],
                           dev["dt_bias"], dy, *hw, z=z, zoh=args.zoh)
        else:
            proj = ss.ss2d_project if wl.K == 4 else ss.ss1d_bidir_project
            fwd = ss.ss2d_forward_routes if wl.K == 4 else ss.ss1d_bidir_forward_routes

            def call():
                o = proj(dev["x"], *fw)
                return fwd(o["u"], o["dt_raw"], dev["A_log"], o["Bs"], o["Cs"], dev["Ds"],
                           dev["dt_bias"], *hw, z=z, zoh=args.zoh, y=y)
    elif args.backward:
        g = workloads.make_output_grad(wl, 0)
        dy = (torch.from_numpy(g["dy_bf16"].view(np.int16)).view(torch.bfloat16)
              if wl.dtype == "bf16" else torch.from_numpy(g["dy"])).to("cuda:0")
        if z is None and not args.zoh:
            fn = ss.ss2d_backward if wl.K == 4 else ss.ss1d_bidir_backward
            call = lambda: fn(*[dev[k] for k in ARGS], dy)  # noqa: E731
        else:
            fn = ss.ss2d_backward_ex if wl.K == 4 else ss.ss1d_bidir_backward_ex
            call = lambda: fn(*[dev[k] for k in ARGS], dy, z=z, zoh=args.zoh)  # noqa: E731
    elif args.gate or args.zoh:
        fn = ss.ss2d_forward_ex if wl.K == 4 else ss.ss1d_bidir_forward_ex
        call = lambda: fn(*[dev[k] for k in ARGS], z=z, zoh=args.zoh, y=y)  # noqa: E731
    else:
        fn = ss.ss2d_forward if wl.K == 4 else ss.ss1d_bidir_forward
        call = lambda: fn(*[dev[k] for k in ARGS], y=y)  # noqa: E731

    log(f"warm-up {args.warmup} steps")
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    # Every kernel of every KERNEL_SAMPLE-th step is bracketed by HIP events (on the stream
    # it runs on) for the per-kernel durations; an event pair around each kernel of every
    # step would add ~22 us to a 0.66 ms step, a perturbation of the throughput it measures.
    ss.timing_enable(False)
    ss.timing_read()  # clear
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        ss.timing_enable(i % args.kernel_sample == 0)
        call()
    ss.timing_enable(False)
    ev1.record(stream)
    torch.cuda.synchronize()
    kernels = ss.timing_read()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    upd_per_s = wl.updates / (ms_step / 1e3)
    alg_bytes = wl.algorithmic_bytes() + (wl.elem_bytes * wl.B * wl.D * wl.L if args.gate else 0)
    e, M, R = wl.elem_bytes, args.front_r + 2 * wl.N, args.front_r
    # front end, per launch: x read once; u and dt_raw (B, K, D, L) and Bs, Cs (B, K, N, L)
    # written once; the fp32 weights read once.  With dt_proj folded into the scan, the
    # front end writes the R dt rows (B, K, R, L) in place of dt_raw and reads no dt_proj_w.
    BKL = wl.B * wl.K * wl.L
    proj_bytes = (e * (wl.B * wl.D * wl.L + BKL * wl.D + 2 * BKL * wl.N)
                  + 4 * wl.K * wl.D * (args.front_kw + 1 + M))
    proj_bytes += e * BKL * R if args.front_lowrank else e * BKL * wl.D + 4 * wl.K * wl.D * R
    if args.front and not routes_bwd:  # the scan then reads u (B, K, D, L), not x (B, D, L)
        alg_bytes += proj_bytes + e * (wl.K - 1) * wl.B * wl.D * wl.L
    if args.front_lowrank:  # ... and dt_lr (B, K, R, L) and dt_w (K, D, R) for dt_raw
        alg_bytes += e * BKL * R + 4 * wl.K * wl.D * R - e * BKL * wl.D
    gbps = alg_bytes / (ms_step / 1e3) / 1e9
    for name, (ms, n) in kernels.items():
        if n:
            log(f"  kernel {name:10s}: {n} launches, {ms / n * 1e3:9.1f} us avg")
    log(f"step {ms_step * 1e3:.1f} us, {upd_per_s:.4e} updates/s, algorithmic {gbps:.1f} GB/s")

    # Dominant kernel: the scan (with the chunked plan, both scan passes are counted).
    if args.backward:
        scan_ms, scan_n = kernels["scan_bwd"]
        agg_ms = 0.0
    else:
        scan_ms, scan_n = kernels["scan"]
        agg_ms, _ = kernels["chunk_agg"]
    scan_avg_s = (scan_ms + agg_ms) / max(scan_n, 1) / 1e3
    flops, peak = ((ZOH_BWD_FLOPS_PER_UPDATE, ZOH_BWD_UPDATE_PEAK_TFLOPS)
                   if args.backward and args.zoh
                   else (BWD_FLOPS_PER_UPDATE, BWD_UPDATE_PEAK_TFLOPS) if args.backward
                   else (ZOH_FLOPS_PER_UPDATE, ZOH_UPDATE_PEAK_TFLOPS) if args.zoh
                   else (FLOPS_PER_UPDATE, UPDATE_PEAK_TFLOPS))
    achieved = wl.updates * flops / scan_avg_s / 1e12
    traffic = measured_traffic(wl.name)
    roofline = {"bound": "alu", "achieved": round(achieved, 3),
                "peak": round(peak, 1), "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                "traffic": (traffic if not (args.gate or args.zoh or args.backward
                                            or args.front) else None),
                "kernel": "k_scan_bwd" if args.backward else "k_scan",
                "kernel_avg_us": round(scan_avg_s * 1e6, 1),
                "kernel_launches_timed": int(scan_n),
                "frac_of_fma_peak": round(achieved / FMA_PEAK_TFLOPS, 4),
                "hbm_gbps_algorithmic_in_kernel": round(alg_bytes / scan_avg_s / 1e9, 1)}

    roofline_front = None
    if args.front and not routes_bwd:
        p_ms, p_n = kernels["project"]
        p_avg_s = p_ms / max(p_n, 1) / 1e3
        p_gbps = proj_bytes / p_avg_s / 1e9
        roofline_front = {"bound": "hbm", "achieved": round(p_gbps, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(p_gbps / HBM_PEAK_GBPS, 4),
                          "traffic": measured_traffic(wl.name, front=True, R=args.front_r,
                                                      KW=args.front_kw,
                                                      lowrank=args.front_lowrank),
                          "kernel": "k_project",
                          "kernel_avg_us": round(p_avg_s * 1e6, 1),
                          "algorithmic_bytes_per_launch": proj_bytes,
                          "R": args.front_r, "KW": args.front_kw,
                          "dt_proj_in_scan": bool(args.front_lowrank)}

    cpu = None
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        if routes_bwd:  # seeded per-route inputs of the same shape (not the GPU's outputs)
            cpu = cpu_baseline_backward(wl, inp, g["dy"], args.cpu_seconds,
                                        z=gate["z"] if gate else None, zoh=args.zoh,
                                        u=workloads.make_route_inputs(wl, 0)["u"])
        elif args.front:
            cpu = cpu_baseline_front(wl, inp, front_w, args.cpu_seconds,
                                     z=gate["z"] if gate else None, zoh=args.zoh,
                                     lowrank=args.front_lowrank)
        elif args.backward:
            cpu = cpu_baseline_backward(wl, inp, g["dy"], args.cpu_seconds,
                                        z=gate["z"] if gate else None, zoh=args.zoh)
        else:
            cpu = cpu_baseline(wl, inp, args.cpu_seconds, z=gate["z"] if gate else None,
                               zoh=args.zoh)
        log(f"  {cpu['sample']} on {cpu['cores']} threads: {cpu['value']:.3e} updates/s")

    out = {
        "metric": METRIC,
        "value": upd_per_s,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "D": wl.D, "H": wl.H, "W": wl.W,
                   "L": wl.L, "N": wl.N, "K": wl.K, "io_dtype": wl.dtype,
                   "state_dtype": "f32", "A_log": args.a_log, "gate": bool(args.gate),
                   "zoh": bool(args.zoh),
                   "pass": ("backward (per-route inputs from the front end)" if routes_bwd
                            else "backward" if args.backward else
                            "front(dt_proj in scan)+forward" if args.front_lowrank else
                            "front+forward" if args.front else "forward")},
        "hbm_gbps_algorithmic": round(gbps, 1),
        "hbm_frac_algorithmic": round(gbps / HBM_PEAK_GBPS, 4),
        "kernels_us": {k: round(ms / n * 1e3, 1) for k, (ms, n) in kernels.items() if n},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if roofline_front is not None:
        out["roofline_front"] = roofline_front
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
