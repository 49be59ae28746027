#!/usr/bin/env python3
"""Benchmark of the SS2D forward operator on one MI355X.

A step is one full forward call (transpose, scan, merge: every kernel of the operator) on
one batch of seeded synthetic input already resident in HBM (with --backward, one backward
call; with --train, a training step: the forward that keeps the scan's tile states, then the
backward from them).  W untimed warm-up steps (then,
if the GPU has been under load for less than --settle-ms, more untimed steps until it has:
the clock ramps up over the first ~20 ms of load), then K timed steps between device
synchronisations, timed with HIP events on the stream the library launches on.  Prints ONE
JSON line on stdout (details go to stderr):

  value        state updates per second (B*K*D*L*N per step / seconds per step)
  roofline     the dominant kernel (the scan) against MI355X's 8 TB/s HBM peak, with the
               fp32 and issue-slot fractions as diagnostics beside it, the latter also
               priced at the instruction rates the library's probe measures on the chip
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
# Diagnostics beside the HBM roofline.  fp32: MI355X's published vector fp32 peak,
# 157.3 TFLOP/s, against the algorithmic 4 flops of one state update (delta*A, the decay
# times h, (delta*u)*B, C*h) plus its exponential.  Issue slots: the VALU issues one wave64
# instruction per 4 cycles on each of 256 CUs x 4 SIMDs at 2.4 GHz, 3.93e13 lane-slots/s
# without packed fp32 (which the library's compile flags exclude); one update needs at least 2
# multiplies, 2 FMAs and one v_exp_f32, which takes two issue slots: 6 slots.  The
# issue-floor fraction is that floor's time over the measured time.
FP32_PEAK_TFLOPS = 157.3
ALG_FLOPS_PER_UPDATE = 4
VALU_LANE_SLOTS = 256 * 4 * 16 * 2.4e9
ISSUE_SLOTS_PER_UPDATE = 4 + 2
# With zero-order hold: at least 6 VALU slots (delta*A, (a - 1) / A as one FMA, times B and
# u, the h update, C*h) plus the exponential.
ZOH_ISSUE_SLOTS_PER_UPDATE = 6 + 2
# Backward, per state update: the forward recompute (3 VALU and the exp) and the adjoint
# (g*C and the lambda update, dC, dB, lambda*h_prev*a, the sums over n for ddelta and du,
# dA): at least 12 VALU slots plus the exp.
BWD_ISSUE_SLOTS_PER_UPDATE = 12 + 2
# Backward with zero-order hold: the recompute's 6 and the adjoint's 16: 22 VALU slots
# plus the exp.
ZOH_BWD_ISSUE_SLOTS_PER_UPDATE = 22 + 2
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


def cpu_model() -> str:
    try:
        for line in pathlib.Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, target_s: float, z=None, zoh=False) -> dict:
    """The float64 oracle, as it is, on all host cores, over a bounded sample of channels,
    and on one core over a smaller sample (extrapolated to the whole workload).  Returns
    the record and the sample (its (b, d) channels and the oracle's outputs there), which
    the caller compares with the GPU's output."""
    import numpy as np

    import oracle
    cores = len(os.sched_getaffinity(0))
    orc = oracle.Oracle()
    args = [inp[k] for k in ARGS]
    opts = dict(z=z, zoh=zoh)
    total = wl.B * wl.D
    rng = np.random.default_rng(0)
    order = rng.permutation(total)

    def run(n, threads):
        sel = order[:n]
        t0 = time.perf_counter()
        ref = orc.forward_channels(wl.K, *args, sel // wl.D, sel % wl.D, threads=threads,
                                   **opts)
        return time.perf_counter() - t0, sel, ref

    n = min(total, max(cores, 64))
    dt, sel, ref = run(n, cores)
    if n < total and dt < target_s:
        n = int(min(total, max(n, n * target_s / max(dt, 1e-3))))
        dt, sel, ref = run(n, cores)
    threads = orc.last_threads
    upd = n * wl.K * wl.L * wl.N
    # one core: a sample of about a tenth of the wall-time budget
    n1 = max(1, min(total, int(n * min(1.0, 0.1 * target_s / max(dt * threads, 1e-3)))))
    dt1, _, _ = run(n1, 1)
    upd1 = n1 * wl.K * wl.L * wl.N
    rec = {"value": upd / dt, "unit": "state-updates/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{n} of {total} (b,d) channels of {wl.name} (all {wl.K} routes, full "
                     f"L={wl.L}, N={wl.N}), {upd:.3e} state updates in {dt:.2f} s",
           "one_core_value": upd1 / dt1,
           "one_core_sample": f"{n1} channels in {dt1:.2f} s on 1 thread",
           "one_core_whole_workload_s_extrapolated": wl.updates / (upd1 / dt1)}
    return rec, (sel // wl.D, sel % wl.D, ref)


def sample_error(y, sample, dtype: str) -> dict:
    """Parity of the GPU's output y (B, D, ...) on the oracle's sampled channels: the gate
    metric max |y - y*| / max(|y*|, 0.01 RMS(y*)), the same unfloored, and the limit."""
    import numpy as np
    import torch
    b_idx, d_idx, ref = sample
    got = y.detach().to(torch.float32).cpu().numpy().astype(np.float64)[b_idx, d_idx]
    ref = ref.reshape(got.shape)
    floor = 0.01 * float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    return {"max_rel_err": float(np.max(err / np.maximum(np.abs(ref), max(floor, 1e-30)))),
            "max_rel_err_unfloored": float(np.max(err / np.maximum(np.abs(ref), 1e-30))),
            "tolerance": 1e-4 if dtype == "f32" else 2e-2,
            "metric": "max |y - y*| / max(|y*|, 0.01 RMS(y*)) over the CPU sample's channels"}


def copy_bandwidth_gbps(torch, mib: int = 1024) -> float:
    """Best of 5 device-to-device copies of `mib` MiB (read + write bytes over the time),
    timed with HIP events: the HBM rate a plain copy reaches on this GPU."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    del src, dst
    return 2 * n * 4 / best / 1e9


def backward_bytes(wl, gate: bool, routes: bool) -> int:
    """Algorithmic bytes of one backward call: every input (x, or each route's u
    (B, K, D, L) with routes, dt_raw, Bs, Cs, dy, z with the gate, the fp32 parameters) read
    once and every gradient (of the same shapes; dz with the gate) written once."""
    e, B, K, D, L, N = wl.elem_bytes, wl.B, wl.K, wl.D, wl.L, wl.N
    xs = B * D * L * (K if routes else 1)
    data = xs + B * K * D * L + 2 * B * K * N * L  # x (u), dt_raw, Bs, Cs
    params = K * D * N + 2 * K * D
    img = B * D * L * (2 if gate else 1)  # dy (and z)
    return e * (2 * data + img + (B * D * L if gate else 0)) + 4 * 2 * params


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="keep warming up (untimed) until the GPU has run the step for this "
                         "long: the clock reaches its sustained rate after ~20 ms of load")
    ap.add_argument("--workload", default="vmamba_t_stage1_bf16")
    ap.add_argument("--a-log", default="init", choices=["init", "random"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets used in turn (0: 3 when the working set is under 512 MB, "
                         "twice the 256 MB Infinity Cache, else 1)")
    ap.add_argument("--gate", action="store_true",
                    help="gated entry point: y * SiLU(z), z of the shape of x")
    ap.add_argument("--zoh", action="store_true",
                    help="zero-order-hold discretisation of B")
    ap.add_argument("--kernel-sample", type=int, default=4,
                    help="time the kernels of every n-th timed step with HIP events (1: all)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward entry point (gradients of sum(dy * y); with "
                         "--gate and/or --zoh, of that operator's output, z included)")
    ap.add_argument("--train", action="store_true",
                    help="time a training step of the operator: ss2d_forward_save (y, and the "
                         "scan's tile states kept) then ss2d_backward_saved from those states "
                         "(with --gate and/or --zoh, of that operator)")
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
    ap.add_argument("--plan", default="", metavar="SPLIT,CHUNK",
                    help="launch-plan override of the forward scan for this run (lanes per "
                         "channel, chunk length; 0,-1 is automatic), for comparing plans; "
                         "the line then names the plan in its config")
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
    plan = None
    if args.plan:
        plan = [int(v) for v in args.plan.split(",")]
        if len(plan) != 2:
            log("--plan takes SPLIT,CHUNK")
            return 2
        ss.launch_plan(*plan).__enter__()  # this thread, for the rest of the run
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
    if args.backward and args.front_lowrank:
        log("no backward for the operator with dt_proj folded in")
        return 2
    if args.train and (args.backward or args.front):
        log("--train times the forward and the backward together: without --backward "
            "or --front")
        return 2
    if args.front_lowrank and not args.front:
        log("--front-lowrank needs --front")
        return 2
    # --backward --front: the backward of the operator over the front end's per-route
    # outputs (computed once per input set, outside the timed region; the front end's own
    # layers have no backward here)
    routes_bwd = args.backward and args.front
    e, M, R = wl.elem_bytes, args.front_r + 2 * wl.N, args.front_r
    # front end, per launch: x read once; u and dt_raw (B, K, D, L) and Bs, Cs (B, K, N, L)
    # written once; the fp32 weights read once.  With dt_proj folded into the scan, the
    # front end writes the R dt rows (B, K, R, L) in place of dt_raw and reads no dt_proj_w.
    BKL = wl.B * wl.K * wl.L
    proj_bytes = (e * (wl.B * wl.D * wl.L + BKL * wl.D + 2 * BKL * wl.N)
                  + 4 * wl.K * wl.D * (args.front_kw + 1 + M))
    proj_bytes += e * BKL * R if args.front_lowrank else e * BKL * wl.D + 4 * wl.K * wl.D * R
    if args.backward:
        alg_bytes = backward_bytes(wl, args.gate, routes_bwd)
    elif args.train:  # the forward's bytes and the backward's (the kept state is scratch)
        alg_bytes = (wl.algorithmic_bytes() + (e * wl.B * wl.D * wl.L if args.gate else 0)
                     + backward_bytes(wl, args.gate, False))
    else:
        alg_bytes = wl.algorithmic_bytes() + (e * wl.B * wl.D * wl.L if args.gate else 0)
        if args.front:  # the scan then reads u (B, K, D, L), not x (B, D, L)
            alg_bytes += proj_bytes + e * (wl.K - 1) * wl.B * wl.D * wl.L
        if args.front_lowrank:  # ... and dt_lr (B, K, R, L) and dt_w (K, D, R) for dt_raw
            alg_bytes += e * BKL * R + 4 * wl.K * wl.D * R - e * BKL * wl.D
    # the kernel the roofline line describes moves the step's algorithmic bytes: its own
    # share when the front end runs before it (its inputs u, dt_raw, Bs, Cs; y)
    kernel_bytes = (alg_bytes - proj_bytes if (args.front and not routes_bwd)
                    else backward_bytes(wl, args.gate, False) if args.train else alg_bytes)
    bwd_kernel = args.backward or args.train  # the adjoint scan is the dominant kernel
    rotate = args.rotate or (3 if alg_bytes < 512e6 else 1)

    def upload(arrays):
        d = {}
        for k in ("x", "dt_raw", "Bs", "Cs"):
            if wl.dtype == "bf16":
                d[k] = torch.from_numpy(arrays[k + "_bf16"].view(np.int16)).view(torch.bfloat16)
            else:
                d[k] = torch.from_numpy(arrays[k])
            d[k] = d[k].to("cuda:0")
        for k in ("A_log", "Ds", "dt_bias"):
            d[k] = torch.from_numpy(arrays[k]).to("cuda:0")
        return d

    def image(arrays, key):
        """An image-shaped input (B, D, ...) on the device: its bf16 bit patterns for bf16
        workloads, else the fp32 array."""
        return (torch.from_numpy(arrays[key + "_bf16"].view(np.int16)).view(torch.bfloat16)
                if wl.dtype == "bf16" else torch.from_numpy(arrays[key])).to("cuda:0")

    gate = workloads.make_gate(wl, 0) if args.gate else None
    z0 = image(gate, "z") if gate is not None else None
    g = workloads.make_output_grad(wl, 0) if (args.backward or args.train) else None
    dy0 = image(g, "dy") if g is not None else None
    front_w = workloads.make_front_weights(wl, 0, R=args.front_r, KW=args.front_kw) \
        if args.front else None
    fw = [torch.from_numpy(front_w[k]).to("cuda:0")
          for k in ("conv_w", "conv_b", "x_proj_w", "dt_proj_w")] if args.front else None
    hw = (wl.H, wl.W) if wl.K == 4 else ()

    def make_call(dev, z, dy, y):
        if args.train:
            fs = ss.ss2d_forward_save if wl.K == 4 else ss.ss1d_bidir_forward_save
            bs = ss.ss2d_backward_saved if wl.K == 4 else ss.ss1d_bidir_backward_saved
            saved = torch.empty(ss.saved_state_bytes(wl.K, wl.B, wl.D, wl.L, wl.N,
                                                     z is not None) // 4,
                                dtype=torch.float32, device="cuda:0")
            a = [dev[k] for k in ARGS]

            def call():
                fs(*a, z=z, zoh=args.zoh, y=y, saved=saved)
                return bs(*a, dy, saved, z=z, zoh=args.zoh)
            return call
        if args.front and args.front_lowrank:
            proj = ss.ss2d_project_lr if wl.K == 4 else ss.ss1d_bidir_project_lr
            fwd = ss.ss2d_forward_routes_lr if wl.K == 4 else ss.ss1d_bidir_forward_routes_lr

            def call():
                o = proj(dev["x"], *fw[:3], args.front_r)
                return fwd(o["u"], o["dt_lr"], fw[3], dev["A_log"], o["Bs"], o["Cs"],
                           dev["Ds"], dev["dt_bias"], *hw, z=z, zoh=args.zoh, y=y)
            return call
        if routes_bwd:
            proj = ss.ss2d_project if wl.K == 4 else ss.ss1d_bidir_project
            bwd = ss.ss2d_backward_routes if wl.K == 4 else ss.ss1d_bidir_backward_routes
            po = proj(dev["x"], *fw)
            return lambda: bwd(po["u"], po["dt_raw"], dev["A_log"], po["Bs"], po["Cs"],
                               dev["Ds"], dev["dt_bias"], dy, *hw, z=z, zoh=args.zoh)
        if args.front:
            proj = ss.ss2d_project if wl.K == 4 else ss.ss1d_bidir_project
            fwd = ss.ss2d_forward_routes if wl.K == 4 else ss.ss1d_bidir_forward_routes

            def call():
                o = proj(dev["x"], *fw)
                return fwd(o["u"], o["dt_raw"], dev["A_log"], o["Bs"], o["Cs"], dev["Ds"],
                           dev["dt_bias"], *hw, z=z, zoh=args.zoh, y=y)
            return call
        if args.backward:
            if z is None and not args.zoh:
                fn = ss.ss2d_backward if wl.K == 4 else ss.ss1d_bidir_backward
                return lambda: fn(*[dev[k] for k in ARGS], dy)
            fn = ss.ss2d_backward_ex if wl.K == 4 else ss.ss1d_bidir_backward_ex
            return lambda: fn(*[dev[k] for k in ARGS], dy, z=z, zoh=args.zoh)
        if args.gate or args.zoh:
            fn = ss.ss2d_forward_ex if wl.K == 4 else ss.ss1d_bidir_forward_ex
            return lambda: fn(*[dev[k] for k in ARGS], z=z, zoh=args.zoh, y=y)
        fn = ss.ss2d_forward if wl.K == 4 else ss.ss1d_bidir_forward
        return lambda: fn(*[dev[k] for k in ARGS], y=y)

    # Input sets used in turn: each its own copy of every input and output, so that a step
    # whose working set fits in the Infinity Cache does not find it there from the step
    # before.
    dev0 = upload(inp)
    sets = []
    for i in range(rotate):
        dev = dev0 if i == 0 else {k: v.clone() for k, v in dev0.items()}
        z = z0 if (i == 0 or z0 is None) else z0.clone()
        dy = dy0 if (i == 0 or dy0 is None) else dy0.clone()
        y = torch.empty(tuple(dev["x"].shape), dtype=dev["x"].dtype, device="cuda:0")
        sets.append((make_call(dev, z, dy, y), y))
    calls = [c for c, _ in sets]
    log(f"{rotate} input set(s) in turn")

    log(f"warm-up {args.warmup} steps, then until {args.settle_ms:.0f} ms of load")
    t_start = time.perf_counter()
    done = 0
    for _ in range(args.warmup):
        calls[done % rotate]()
        done += 1
    torch.cuda.synchronize()
    settle = 0
    while (time.perf_counter() - t_start) * 1e3 < args.settle_ms:
        for _ in range(10):
            calls[done % rotate]()
            done += 1
            settle += 1
        torch.cuda.synchronize()
    log(f"  {done} untimed steps ({settle} to settle the clock) in "
        f"{(time.perf_counter() - t_start) * 1e3:.0f} ms")

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
        calls[(done + i) % rotate]()
    ss.timing_enable(False)
    ev1.record(stream)
    torch.cuda.synchronize()
    done += args.steps
    kernels = ss.timing_read()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    upd_per_s = wl.updates / (ms_step / 1e3)
    # The distribution of single steps, in a second timed run of K steps with an event
    # between consecutive steps (not part of the line's value).
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        calls[(done + i) % rotate]()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    ms_min = per_step[0]
    gbps = alg_bytes / (ms_step / 1e3) / 1e9
    for name, (ms, n) in kernels.items():
        if n:
            log(f"  kernel {name:10s}: {n} launches, {ms / n * 1e3:9.1f} us avg")
    log(f"step {ms_step * 1e3:.1f} us (median {ms_median * 1e3:.1f}, min {ms_min * 1e3:.1f}), "
        f"{upd_per_s:.4e} updates/s, algorithmic {gbps:.1f} GB/s")
    copy_gbps = copy_bandwidth_gbps(torch)
    # The rates the issue-slot model assumes, measured on this chip: fused multiply-adds and
    # v_exp_f32 alone, and one update's mix (4 multiply-adds + 1 exponential) at full occupancy.
    rates = ss.probe_issue_rates()
    exp_slots = rates["fma_per_s"] / rates["exp_per_s"]
    mix_slots = rates["fma_per_s"] / rates["update_mix_per_s"]
    log(f"issue rates: {rates['fma_per_s']:.4g} FMA/s, {rates['exp_per_s']:.4g} exp/s "
        f"({exp_slots:.2f} FMA slots each), update mix {rates['update_mix_per_s']:.4g}/s "
        f"({mix_slots:.2f} slots), clock {rates['clock_hz'] / 1e9:.2f} GHz")
    log(f"device-to-device copy: {copy_gbps:.0f} GB/s")

    # Dominant kernel: the scan (with the chunked plan, both scan passes are counted).
    if bwd_kernel:
        scan_ms, scan_n = kernels["scan_bwd"]
        agg_ms = 0.0
    else:
        scan_ms, scan_n = kernels["scan"]
        agg_ms, _ = kernels["chunk_agg"]
    scan_avg_s = (scan_ms + agg_ms) / max(scan_n, 1) / 1e3
    slots = (ZOH_BWD_ISSUE_SLOTS_PER_UPDATE if bwd_kernel and args.zoh
             else BWD_ISSUE_SLOTS_PER_UPDATE if bwd_kernel
             else ZOH_ISSUE_SLOTS_PER_UPDATE if args.zoh else ISSUE_SLOTS_PER_UPDATE)
    achieved = kernel_bytes / scan_avg_s / 1e9
    traffic = measured_traffic(wl.name)
    traffic = traffic if not (args.gate or args.zoh or bwd_kernel or args.front) else None
    fp32_tflops = wl.updates * ALG_FLOPS_PER_UPDATE / scan_avg_s / 1e12
    issue_floor_s = wl.updates * slots / VALU_LANE_SLOTS
    # the same floor priced at the measured multiply-add rate (the sustained clock's)
    issue_floor_meas_s = wl.updates * slots / rates["fma_per_s"]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "kernel": "k_scan_bwd" if bwd_kernel else "k_scan",
                "kernel_avg_us": round(scan_avg_s * 1e6, 1),
                "kernel_launches_timed": int(scan_n),
                "algorithmic_bytes_per_launch": int(kernel_bytes),
                "traffic_ratio": (round(traffic / kernel_bytes, 3) if traffic else None),
                "copy_gbps_measured": round(copy_gbps, 1),
                "frac_of_copy": round(achieved / copy_gbps, 4),
                "fp32_tflops": round(fp32_tflops, 2),
                "fp32_frac": round(fp32_tflops / FP32_PEAK_TFLOPS, 4),
                "issue_slots_per_update": slots,
                "issue_floor_us": round(issue_floor_s * 1e6, 1),
                "issue_floor_frac": round(issue_floor_s / scan_avg_s, 4),
                "issue_rates_measured": {
                    "fma_per_s": float(f"{rates['fma_per_s']:.4g}"),
                    "exp_per_s": float(f"{rates['exp_per_s']:.4g}"),
                    "update_mix_per_s": float(f"{rates['update_mix_per_s']:.4g}"),
                    "exp_fma_slots": round(exp_slots, 3),
                    "update_mix_slots": round(mix_slots, 3),
                    "clock_ghz": round(rates["clock_hz"] / 1e9, 3),
                    "compute_units": rates["compute_units"]},
                "issue_floor_us_measured": round(issue_floor_meas_s * 1e6, 1),
                "issue_floor_frac_measured": round(issue_floor_meas_s / scan_avg_s, 4)}
    if not (bwd_kernel or args.zoh):
        # the plain update is exactly the probe's mix: its measured rate is the scan's ceiling
        mix_s = wl.updates / rates["update_mix_per_s"]
        roofline["update_mix_floor_us_measured"] = round(mix_s * 1e6, 1)
        roofline["update_mix_floor_frac_measured"] = round(mix_s / scan_avg_s, 4)

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
    parity = None
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
        elif bwd_kernel:  # the oracle's backward runs its own forward recurrence first
            cpu = cpu_baseline_backward(wl, inp, g["dy"], args.cpu_seconds,
                                        z=gate["z"] if gate else None, zoh=args.zoh)
        else:
            cpu, sample = cpu_baseline(wl, inp, args.cpu_seconds,
                                       z=gate["z"] if gate else None, zoh=args.zoh)
            parity = sample_error(sets[0][1], sample, wl.dtype)
            log(f"  GPU output against the oracle on the sample: max_rel_err "
                f"{parity['max_rel_err']:.3e} (limit {parity['tolerance']:.0e})")
        cpu.setdefault("cpu_model", cpu_model())
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
                            "training step (forward keeping the tile states, backward "
                            "from them)" if args.train else
                            "front(dt_proj in scan)+forward" if args.front_lowrank else
                            "front+forward" if args.front else "forward"),
                   **({"plan": {"split": plan[0], "chunk_len": plan[1]}} if plan else {})},
        "ms_per_step_median": round(ms_median, 5),
        "ms_per_step_min": round(ms_min, 5),
        "clock_settle_steps": settle,
        "input_sets_rotated": rotate,
        "hbm_gbps_algorithmic": round(gbps, 1),
        "hbm_frac_algorithmic": round(gbps / HBM_PEAK_GBPS, 4),
        "kernels_us": {k: round(ms / n * 1e3, 1) for k, (ms, n) in kernels.items() if n},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        # The only speed figure the pages give for SS2D on named hardware: a module-level
        # comparison with attention, not this operator's metric, so never a baseline.
        "published_context": {
            "claim": "SS2D module against conventional attention: memory use down 63%, "
                     "throughput up 2.4x",
            "hardware": "A100",
            "source": "mhpn.cn, VMamba架构解析, section 2",
            "comparable": False,
        },
    }
    if roofline_front is not None:
        out["roofline_front"] = roofline_front
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
