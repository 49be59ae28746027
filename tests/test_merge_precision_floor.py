"""CPU evidence for the precision of the per-route outputs the merge sums (no GPU, no library).

The scan writes each route's output in fp32 and the merge rounds the fixed-order sum once to
the data type.  Writing the route outputs in 16 bits would halve the merge's reads (and the
scan's writes), but every route output carries the skip term D u of the same input, so the
four outputs are each about a quarter of y and a 16-bit rounding of each is not small
against y where the routes' scan terms cancel.  On stage-1 shaped bf16 inputs (8 images,
48 channels, 56 x 56, N = 16) the float64 oracle's route outputs, rounded per route to
bf16 or fp16 and summed in fp32, miss the bf16 forward bar 2e-2; rounded to fp32 and summed
the kernel's way, they stay at the bf16 output rounding (~4e-3).
"""
import numpy as np

import oracle
import workloads
from tests.gpu_util import TOL, parity_error

ARGS = ("dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")


def route_outputs(inp):
    """The four routes' outputs (image layout, float64), each from the operator over per-route
    inputs with every other route's input zero, and the full forward."""
    x = inp["x"]
    B, D, H, W = x.shape
    L = H * W
    flat = x.reshape(B, D, L)
    cols = x.transpose(0, 1, 3, 2).reshape(B, D, L)
    seqs = (flat, flat[..., ::-1], cols, cols[..., ::-1])
    o = oracle.Oracle()
    args = [inp[k] for k in ARGS]
    ys = []
    for k in range(4):
        u = np.zeros((B, 4, D, L), np.float32)
        u[:, k] = seqs[k]
        ys.append(o.forward_routes(4, u, *args, H, W))
    return ys, o.forward(4, x, *args)


def merged(ys, rnd):
    r = [rnd(y) for y in ys]
    return workloads.round_bf16((((r[0] + r[1]) + r[2]) + r[3]).astype(np.float32))


def test_route_outputs_need_fp32():
    wl = workloads.custom(B=8, D=48, H=56, W=56, N=16, K=4, dtype="bf16")
    ys, full = route_outputs(workloads.make_inputs(wl, seed=3))
    # the routes, each with its own zero-input complement, add up to the forward
    assert np.abs(sum(ys) - full).max() <= 1e-12 * np.abs(full).max()
    schemes = {
        "fp32": lambda y: y.astype(np.float32),
        "bf16": lambda y: workloads.round_bf16(y.astype(np.float32)),
        "fp16": lambda y: y.astype(np.float16).astype(np.float32),
    }
    err = {k: parity_error(merged(ys, f), full)["gate"] for k, f in schemes.items()}
    print("route outputs rounded to", {k: f"{v:.3e}" for k, v in err.items()})
    assert err["fp32"] <= TOL["bf16"], err
    assert err["bf16"] > TOL["bf16"] and err["fp16"] > TOL["bf16"], err
