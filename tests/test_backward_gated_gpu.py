"""GPU parity of the gated backward entry points (gradients of sum(dy * y * SiLU(z)) for every
input and for z) against the float64 oracle, through the C ABI: small shapes with ragged
tiles, channel blocks and maps whose sides are not multiples of 4 (the merge's element
path), both element types and route sets, and the benchmark sizes; the closed form at
z = 0; bitwise determinism."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL_BWD, assert_parity, log, to_device, to_numpy_f64

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
IO_GRADS = ("x", "dt_raw", "Bs", "Cs", "z")      # in the data type of x
PARAM_GRADS = ("A_log", "Ds", "dt_bias")         # fp32


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def image_to_device(g, key, wl):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(g[key + "_bf16"].view(np.int16)).view(torch.bfloat16).to(
            "cuda:0")
    return torch.from_numpy(g[key]).to("cuda:0")


def run_bwd_gated(dev, wl, z, dy):
    import selective_scan_ss2d_amd as ss
    fn = ss.ss2d_backward_gated if wl.K == 4 else ss.ss1d_bidir_backward_gated
    return fn(*[dev[k] for k in ARGS], z, dy)


def check(orc, wl, a_log="random", seed=0, what=None):
    import torch
    what = what or f"B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} {wl.dtype}"
    log(f"case gated backward {what}")
    inp = workloads.make_inputs(wl, seed=seed, a_log=a_log)
    g = workloads.make_output_grad(wl, seed)
    zg = workloads.make_gate(wl, seed)
    ref = orc.backward(wl.K, *[inp[k] for k in ARGS], g["dy"], z=zg["z"])
    dev = to_device(inp, wl)
    grads = run_bwd_gated(dev, wl, image_to_device(zg, "z", wl),
                          image_to_device(g, "dy", wl))
    torch.cuda.synchronize()
    for name in ARGS + ("z",):
        tol_dtype = wl.dtype if name in IO_GRADS else "f32"
        got = to_numpy_f64(grads[name]).reshape(ref[name].shape)
        assert_parity(got, ref[name], tol_dtype, f"gated backward d{name} {what}", tol=TOL_BWD)


SHAPES = [  # B, D, H, W, N, K, dtype
    (2, 70, 5, 7, 16, 4, "f32"),
    (2, 70, 5, 7, 16, 4, "bf16"),
    (2, 130, 24, 24, 16, 4, "bf16"),
    (2, 130, 24, 24, 16, 4, "f32"),
    (1, 33, 3, 5, 4, 4, "f32"),
    (1, 20, 4, 6, 8, 4, "bf16"),
    (3, 64, 8, 12, 8, 4, "f32"),
    (1, 1, 2, 2, 16, 4, "f32"),
    (3, 100, 1, 197, 16, 2, "bf16"),
    (2, 64, 1, 320, 16, 2, "f32"),
    (1, 65, 1, 37, 4, 2, "f32"),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}".format(*c))
def test_backward_gated_small(orc, case):
    B, D, H, W, N, K, dt = case
    check(orc, workloads.custom(B, D, H, W, N, K, dt), seed=41)


@pytest.mark.parametrize("name", ["vmamba_t_stage1_bf16", "vim_bidir_bf16"])
def test_backward_gated_full_size(orc, name):
    check(orc, workloads.workload(name), a_log="init", seed=0, what=name)


@pytest.mark.parametrize("K", [4, 2])
def test_backward_gated_at_zero(monkeypatch, K):
    """At z = 0 the gate passes nothing on (SiLU(0) = 0): every input's gradient is exactly
    zero, and dz = dy * y * SiLU'(0) = dy * y / 2, bit for bit the forward entry point's y
    (fp32, the same one-pass scan) times dy, halved."""
    import torch
    import selective_scan_ss2d_amd as ss
    monkeypatch.setenv("SS2D_CHUNK_LEN", "0")  # the forward in one pass, as the checkpoints
    wl = workloads.custom(2, 96, 8, 12, 16, 4, "f32") if K == 4 else \
        workloads.custom(2, 96, 1, 100, 16, 2, "f32")
    log(f"case gated backward at z = 0, K={K}")
    dev = to_device(workloads.make_inputs(wl, seed=42), wl)
    dy = image_to_device(workloads.make_output_grad(wl, 42), "dy", wl)
    z = torch.zeros_like(dy)
    grads = run_bwd_gated(dev, wl, z, dy)
    fwd = ss.ss2d_forward if K == 4 else ss.ss1d_bidir_forward
    y = fwd(*[dev[k] for k in ARGS])
    torch.cuda.synchronize()
    for name in ARGS:
        assert torch.count_nonzero(grads[name]).item() == 0, name
    want = (dy * y) * 0.5
    assert torch.equal(grads["z"].view(torch.int32), want.view(torch.int32))


def test_backward_gated_deterministic_and_errors():
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 130, 24, 24, 16, 4, "bf16")
    inp = workloads.make_inputs(wl, seed=43)
    dev = to_device(inp, wl)
    dy = image_to_device(workloads.make_output_grad(wl, 43), "dy", wl)
    z = image_to_device(workloads.make_gate(wl, 43), "z", wl)
    g1 = {k: v.clone() for k, v in run_bwd_gated(dev, wl, z, dy).items()}
    g2 = run_bwd_gated(dev, wl, z, dy)
    torch.cuda.synchronize()
    for k in ARGS + ("z",):
        a, b = g1[k], g2[k]
        view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(view), b.view(view)), k
    with pytest.raises(ValueError):
        run_bwd_gated(dev, wl, z[:1], dy)
