"""GPU parity of the backward entry points (gradients of sum(dy * y) for every input) against
the float64 oracle's reverse-mode gradients, through the C ABI: small shapes with ragged
tiles and channel blocks, every supported state size, both element types and route sets,
and the benchmark sizes; plus bitwise determinism."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL_BWD, assert_parity, log, to_device, to_numpy_f64

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
IO_GRADS = ("x", "dt_raw", "Bs", "Cs")          # in the data type of x
PARAM_GRADS = ("A_log", "Ds", "dt_bias")         # fp32


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def dy_to_device(g, wl):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(g["dy_bf16"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(g["dy"]).to("cuda:0")


def run_bwd(dev, wl, dy):
    import selective_scan_ss2d_amd as ss
    fn = ss.ss2d_backward if wl.K == 4 else ss.ss1d_bidir_backward
    return fn(*[dev[k] for k in ARGS], dy)


def check(orc, wl, a_log="random", seed=0, what=None):
    import torch
    what = what or f"B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} {wl.dtype}"
    log(f"case backward {what}")
    inp = workloads.make_inputs(wl, seed=seed, a_log=a_log)
    g = workloads.make_output_grad(wl, seed)
    ref = orc.backward(wl.K, *[inp[k] for k in ARGS], g["dy"])
    dev = to_device(inp, wl)
    grads = run_bwd(dev, wl, dy_to_device(g, wl))
    torch.cuda.synchronize()
    for name in ARGS:
        tol_dtype = wl.dtype if name in IO_GRADS else "f32"
        got = to_numpy_f64(grads[name]).reshape(ref[name].shape)
        assert_parity(got, ref[name], tol_dtype, f"backward d{name} {what}", tol=TOL_BWD)


SHAPES = [  # B, D, H, W, N, K, dtype
    (2, 70, 5, 7, 16, 4, "f32"),
    (2, 70, 5, 7, 16, 4, "bf16"),
    (2, 130, 24, 24, 16, 4, "bf16"),
    (2, 130, 24, 24, 16, 4, "f32"),
    (1, 33, 3, 5, 4, 4, "f32"),
    (1, 20, 4, 6, 8, 4, "bf16"),
    (3, 64, 9, 13, 8, 4, "f32"),
    (1, 1, 2, 2, 16, 4, "f32"),
    (3, 100, 1, 197, 16, 2, "bf16"),
    (2, 64, 1, 320, 16, 2, "f32"),
    (1, 65, 1, 37, 4, 2, "f32"),
    (1, 33, 1, 40, 8, 4, "f32"),      # degenerate maps: the column routes need no transpose
    (2, 24, 17, 1, 16, 4, "bf16"),
    # N = 1 and 2 (run as four states with zero-padded B and C), N = 32 (two waves per SIMD)
    (2, 70, 5, 7, 1, 4, "f32"),
    (2, 70, 5, 7, 2, 4, "bf16"),
    (1, 33, 1, 150, 2, 2, "f32"),
    (2, 70, 5, 7, 32, 4, "f32"),
    (2, 130, 12, 20, 32, 4, "bf16"),
    (2, 64, 1, 197, 32, 2, "bf16"),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}".format(*c))
def test_backward_small(orc, case):
    B, D, H, W, N, K, dt = case
    check(orc, workloads.custom(B, D, H, W, N, K, dt), seed=31)


@pytest.mark.parametrize("name", ["vmamba_t_stage1_bf16", "vim_bidir_bf16"])
def test_backward_full_size(orc, name):
    check(orc, workloads.workload(name), a_log="init", seed=0, what=name)


def test_backward_deterministic():
    import torch
    wl = workloads.custom(2, 130, 24, 24, 16, 4, "bf16")
    inp = workloads.make_inputs(wl, seed=32)
    dev = to_device(inp, wl)
    dy = dy_to_device(workloads.make_output_grad(wl, 32), wl)
    g1 = {k: v.clone() for k, v in run_bwd(dev, wl, dy).items()}
    g2 = run_bwd(dev, wl, dy)
    torch.cuda.synchronize()
    for k in ARGS:
        a, b = g1[k], g2[k]
        view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(view), b.view(view)), k
