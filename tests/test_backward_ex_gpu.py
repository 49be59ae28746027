"""GPU parity of the extended backward entry points (gradients of sum(dy * y) for the gated
output y * SiLU(z), for the zero-order-hold operator, and for both together; every input's
gradient and z's) against the float64 oracle, through the C ABI: small shapes with ragged
tiles, channel blocks and maps whose sides are not multiples of 4 (the merge's element
path), both element types and route sets, decay rates over the whole fp32 range, and the
benchmark sizes; the closed form at z = 0; bitwise determinism."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL_BWD, assert_parity, log, to_device, to_numpy_f64

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
IO_GRADS = ("x", "dt_raw", "Bs", "Cs", "z")      # in the data type of x
PARAM_GRADS = ("A_log", "Ds", "dt_bias")         # fp32
OPTIONS = [(True, False), (False, True), (True, True)]
OPTION_IDS = ["gate", "zoh", "gate_zoh"]


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def image_to_device(g, key, wl):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(g[key + "_bf16"].view(np.int16)).view(torch.bfloat16).to(
            "cuda:0")
    return torch.from_numpy(g[key]).to("cuda:0")


def run_bwd_ex(dev, wl, dy, z, zoh):
    import selective_scan_ss2d_amd as ss
    fn = ss.ss2d_backward_ex if wl.K == 4 else ss.ss1d_bidir_backward_ex
    return fn(*[dev[k] for k in ARGS], dy, z=z, zoh=zoh)


def check(orc, wl, gate, zoh, a_log="random", seed=0, inp=None, what=None):
    import torch
    what = (what or f"B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} {wl.dtype}") + \
        f" gate={gate} zoh={zoh}"
    log(f"case backward {what}")
    if inp is None:
        inp = workloads.make_inputs(wl, seed=seed, a_log=a_log)
    g = workloads.make_output_grad(wl, seed)
    zg = workloads.make_gate(wl, seed) if gate else None
    ref = orc.backward(wl.K, *[inp[k] for k in ARGS], g["dy"], z=zg["z"] if gate else None,
                       zoh=zoh)
    dev = to_device(inp, wl)
    grads = run_bwd_ex(dev, wl, image_to_device(g, "dy", wl),
                       image_to_device(zg, "z", wl) if gate else None, zoh)
    torch.cuda.synchronize()
    for name in ARGS + (("z",) if gate else ()):
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
    (3, 64, 8, 12, 8, 4, "f32"),
    (1, 1, 2, 2, 16, 4, "f32"),
    (3, 100, 1, 197, 16, 2, "bf16"),
    (2, 64, 1, 320, 16, 2, "f32"),
    (1, 65, 1, 37, 4, 2, "f32"),
    (1, 33, 1, 40, 8, 4, "f32"),      # degenerate maps: the column routes need no transpose
    (2, 24, 17, 1, 16, 4, "bf16"),
    (2, 70, 5, 7, 1, 4, "f32"),       # N = 1, 2: four states with zero-padded B and C
    (1, 40, 1, 100, 2, 2, "bf16"),
    (2, 70, 5, 7, 32, 4, "f32"),      # N = 32: two waves per SIMD
    (2, 64, 1, 197, 32, 2, "bf16"),
]


@pytest.mark.parametrize("gate,zoh", OPTIONS, ids=OPTION_IDS)
@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}".format(*c))
def test_backward_ex_small(orc, case, gate, zoh):
    B, D, H, W, N, K, dt = case
    check(orc, workloads.custom(B, D, H, W, N, K, dt), gate, zoh, seed=41)


@pytest.mark.parametrize("K,dt", [(4, "f32"), (2, "bf16")])
def test_backward_zoh_extreme_decay_rates(orc, K, dt):
    """A_log from -120 (A underflows to -0 in fp32: the hold's factor takes its limit delta,
    and 1 / A is infinite) through 8 (|A| ~ 3000), deltas over decades: both sides of the
    power-series switches of the factor and of its derivative in A are crossed."""
    wl = workloads.custom(2, 40, 6, 9, 16, 4, dt) if K == 4 else \
        workloads.custom(2, 40, 1, 61, 16, 2, dt)
    inp = workloads.make_inputs(wl, seed=44)
    levels = np.array([-120.0, -30.0, -12.0, -6.0, -3.0, -1.0, -0.2, 0.0, 0.3, 0.7, 1.2, 2.0,
                       3.0, 4.5, 6.0, 8.0], np.float32)
    inp["A_log"] = np.ascontiguousarray(np.broadcast_to(levels, inp["A_log"].shape))
    dt_raw = (inp["dt_raw"] * np.float32(6.0)).astype(np.float32)  # delta over decades
    if dt == "bf16":
        bits = workloads.f32_to_bf16_bits(dt_raw)
        inp["dt_raw_bf16"] = bits
        dt_raw = workloads.bf16_bits_to_f32(bits)
    inp["dt_raw"] = dt_raw
    check(orc, wl, False, True, inp=inp, what=f"zoh extreme A_log {dt}")
    check(orc, wl, True, True, inp=inp, what=f"zoh extreme A_log {dt}")


@pytest.mark.parametrize("name,gate,zoh", [("vmamba_t_stage1_bf16", True, False),
                                           ("vmamba_t_stage1_bf16", False, True),
                                           ("vim_bidir_bf16", True, False),
                                           ("vim_bidir_bf16", True, True)])
def test_backward_ex_full_size(orc, name, gate, zoh):
    check(orc, workloads.workload(name), gate, zoh, a_log="init", seed=0, what=name)


@pytest.mark.parametrize("zoh", [False, True], ids=["plain", "zoh"])
@pytest.mark.parametrize("K", [4, 2])
def test_backward_gated_at_zero(K, zoh):
    """At z = 0 the gate passes nothing on (SiLU(0) = 0): every input's gradient is exactly
    zero, and dz = dy * y * SiLU'(0) = dy * y / 2, bit for bit the forward entry point's y
    (fp32, the same one-pass scan) times dy, halved."""
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 96, 8, 12, 16, 4, "f32") if K == 4 else \
        workloads.custom(2, 96, 1, 100, 16, 2, "f32")
    log(f"case gated backward at z = 0, K={K} zoh={zoh}")
    dev = to_device(workloads.make_inputs(wl, seed=42), wl)
    dy = image_to_device(workloads.make_output_grad(wl, 42), "dy", wl)
    z = torch.zeros_like(dy)
    grads = run_bwd_ex(dev, wl, dy, z, zoh)
    fwd = ss.ss2d_forward_ex if K == 4 else ss.ss1d_bidir_forward_ex
    with ss.launch_plan(0, 0):  # the forward in one pass, as the checkpoints
        y = fwd(*[dev[k] for k in ARGS], zoh=zoh)
    torch.cuda.synchronize()
    for name in ARGS:
        assert torch.count_nonzero(grads[name]).item() == 0, name
    want = (dy * y) * 0.5
    assert torch.equal(grads["z"].view(torch.int32), want.view(torch.int32))


def test_backward_ex_plain_is_the_plain_entry_point():
    """Without gate and flag the extended entry point is the plain one, bit for bit."""
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 130, 24, 24, 16, 4, "bf16")
    dev = to_device(workloads.make_inputs(wl, seed=45), wl)
    dy = image_to_device(workloads.make_output_grad(wl, 45), "dy", wl)
    g0 = {k: v.clone() for k, v in ss.ss2d_backward(*[dev[k] for k in ARGS], dy).items()}
    g1 = run_bwd_ex(dev, wl, dy, None, False)
    torch.cuda.synchronize()
    assert set(g1) == set(ARGS)
    for k in ARGS:
        view = torch.int16 if g0[k].dtype == torch.bfloat16 else torch.int32
        assert torch.equal(g0[k].view(view), g1[k].view(view)), k


@pytest.mark.parametrize("zoh", [False, True], ids=["gate", "gate_zoh"])
def test_backward_ex_deterministic_and_errors(zoh):
    import torch
    wl = workloads.custom(2, 130, 24, 24, 16, 4, "bf16")
    inp = workloads.make_inputs(wl, seed=43)
    dev = to_device(inp, wl)
    dy = image_to_device(workloads.make_output_grad(wl, 43), "dy", wl)
    z = image_to_device(workloads.make_gate(wl, 43), "z", wl)
    g1 = {k: v.clone() for k, v in run_bwd_ex(dev, wl, dy, z, zoh).items()}
    g2 = run_bwd_ex(dev, wl, dy, z, zoh)
    torch.cuda.synchronize()
    for k in ARGS + ("z",):
        a, b = g1[k], g2[k]
        view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(view), b.view(view)), k
    with pytest.raises(ValueError):
        run_bwd_ex(dev, wl, dy, z[:1], zoh)
