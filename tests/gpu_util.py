"""Helpers shared by the GPU tests: moving seeded inputs to the device, calling the GPU path
through the binding, and the parity metric."""
from __future__ import annotations

import os
import sys

import numpy as np

import workloads

# Parity gate: max_i |y_i - y*_i| / max(|y*_i|, 0.01 * RMS(y*)).  The floor keeps outputs
# that cancel to near zero from dominating a relative measure.  Limits: 1e-4 for fp32 data,
# 2e-2 for bfloat16 data with fp32 state (bf16 output rounding alone is up to 2^-9 = 2e-3).
TOL = {"f32": 1e-4, "bf16": 2e-2}
# Gradients chain two fp32 recurrences (the recomputed forward and the adjoint) and sum up
# to B * L terms of both signs for the parameters: twice the forward bar for fp32 data.
TOL_BWD = {"f32": 2e-4, "bf16": 2e-2}
# The front end's outputs (u, x_proj's B, C and dt rows) and the chained forward meet the
# forward bar.  dt_raw = dt_proj(x_proj's R dt rows) combines R fp32 D-term sums with either
# sign: its entries that cancel to below the 1% floor carry those sums' rounding against
# the floor, and a plain fp32 implementation already reaches 1e-4 there for some summation
# orders (tests/test_front_fp32_floor.py): twice the forward bar for fp32 dt_raw.
TOL_FRONT = {"f32": 1e-4, "bf16": 2e-2}
TOL_DT_RAW = {"f32": 2e-4, "bf16": 2e-2}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: dict, wl: workloads.Workload, device="cuda:0") -> dict:
    import torch
    out = {}
    for k in ("x", "dt_raw", "Bs", "Cs"):
        if wl.dtype == "bf16":
            bits = inp[k + "_bf16"]
            t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32))
        out[k] = t.to(device)
    for k in ("A_log", "Ds", "dt_bias"):
        out[k] = torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).to(device)
    return out


def run_gpu(dev: dict, wl: workloads.Workload, y=None):
    import selective_scan_ss2d_amd as ss
    fn = ss.ss2d_forward if wl.K == 4 else ss.ss1d_bidir_forward
    return fn(dev["x"], dev["dt_raw"], dev["A_log"], dev["Bs"], dev["Cs"], dev["Ds"],
              dev["dt_bias"], y=y)


def to_numpy_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def parity_error(y: np.ndarray, ref: np.ndarray) -> dict:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    floor = max(0.01 * rms, 1e-30)
    err = np.abs(y - ref)
    gate = float(np.max(err / np.maximum(np.abs(ref), floor))) if ref.size else 0.0
    unfloored = float(np.max(err / np.maximum(np.abs(ref), 1e-30))) if ref.size else 0.0
    normwise = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-30))
    return dict(gate=gate, unfloored=unfloored, normwise=normwise, rms=rms,
                finite=bool(np.isfinite(y).all()))


def assert_parity(y, ref, dtype: str, what: str, tol: dict = TOL) -> dict:
    e = parity_error(y, ref)
    record = os.environ.get("SS2D_PARITY_LOG")
    if record:  # one JSON line per checked case, for the parity summary
        import json
        with open(record, "a") as f:
            f.write(json.dumps(dict(case=what, dtype=dtype, limit=tol[dtype], **e)) + "\n")
    log(f"  parity {what}: gate={e['gate']:.3e} (limit {tol[dtype]:.0e}) "
        f"normwise={e['normwise']:.3e} unfloored={e['unfloored']:.3e}")
    assert e["finite"], f"{what}: non-finite output"
    assert e["gate"] <= tol[dtype], f"{what}: parity error {e['gate']:.3e} > {tol[dtype]}"
    return e


class plan_override:
    """Force the library's launch plan for calls from this thread inside the block: split
    (lanes per channel; 0 automatic) and chunk_len (0: one pass; -1 automatic), set through
    ss2d_set_launch_plan."""

    def __init__(self, split=0, chunk_len=-1):
        import selective_scan_ss2d_amd as ss
        self.ctx = ss.launch_plan(int(split), int(chunk_len))

    def __enter__(self):
        return self.ctx.__enter__()

    def __exit__(self, *exc):
        return self.ctx.__exit__(*exc)
