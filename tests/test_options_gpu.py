"""GPU parity of the gated (y * SiLU(z)) and zero-order-hold entry points against the float64
oracle, through the C ABI: small shapes element by element (every launch variant of the
scan, both element types, both route sets), every output at the benchmark sizes, and
extreme decay rates for the zero-order hold."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import assert_parity, plan_override, log, to_device, to_numpy_f64

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def gate_to_device(g, wl):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(g["z_bf16"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(g["z"]).to("cuda:0")


def run_ex(dev, wl, z, zoh):
    import selective_scan_ss2d_amd as ss
    fn = ss.ss2d_forward_ex if wl.K == 4 else ss.ss1d_bidir_forward_ex
    return fn(*[dev[k] for k in ARGS], z=z, zoh=zoh)


def check(orc, wl, gate, zoh, a_log="random", seed=0, inp=None, what=None, **overrides):
    import torch
    what = what or (f"{wl.name} B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} {wl.dtype} "
                    f"gate={gate} zoh={zoh} {overrides}")
    log(f"case {what}")
    inp = inp if inp is not None else workloads.make_inputs(wl, seed=seed, a_log=a_log)
    g = workloads.make_gate(wl, seed) if gate else None
    ref = orc.forward(wl.K, *[inp[k] for k in ARGS], z=g["z"] if gate else None, zoh=zoh)
    dev = to_device(inp, wl)
    z = gate_to_device(g, wl) if gate else None
    with plan_override(**overrides):
        y = run_ex(dev, wl, z, zoh)
    torch.cuda.synchronize()
    return assert_parity(to_numpy_f64(y), ref, wl.dtype, what)


SHAPES = [  # B, D, H, W, N, K, dtype
    (2, 70, 5, 7, 16, 4, "f32"),
    (2, 70, 5, 7, 16, 4, "bf16"),
    (2, 130, 24, 24, 16, 4, "bf16"),
    (2, 130, 24, 24, 16, 4, "f32"),
    (1, 33, 3, 5, 4, 4, "f32"),
    (3, 100, 1, 197, 16, 2, "bf16"),
    (2, 64, 1, 320, 16, 2, "f32"),
]


@pytest.mark.parametrize("gate,zoh", [(True, False), (False, True), (True, True)],
                         ids=["gate", "zoh", "gate_zoh"])
@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}".format(*c))
def test_options_small(orc, case, gate, zoh):
    B, D, H, W, N, K, dt = case
    check(orc, workloads.custom(B, D, H, W, N, K, dt), gate, zoh, seed=21)


VARIANTS = [dict(split=s, chunk_len=0) for s in (1, 2, 4)] + [
    dict(split=sp, chunk_len=c) for sp in (1, 4) for c in (64, 96)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: "S{}_C{}".format(
    v["split"], v["chunk_len"]))
def test_zoh_launch_variants(orc, dt, var):
    check(orc, workloads.custom(2, 72, 13, 11, 16, 4, dt), True, True, seed=22, **var)


def test_zoh_extreme_decay_rates(orc):
    """A_log from -120 (A underflows to -0 in fp32: the limit delta * B) through 8 (|A| ~ 3000,
    the state forgets at once), and the series / direct switch of the kernel crossed by
    random deltas."""
    wl = workloads.custom(2, 40, 6, 9, 16, 4, "f32")
    inp = workloads.make_inputs(wl, seed=23)
    levels = np.array([-120.0, -30.0, -12.0, -6.0, -3.0, -1.0, -0.2, 0.0, 0.3, 0.7, 1.2, 2.0,
                       3.0, 4.5, 6.0, 8.0], np.float32)
    inp["A_log"] = np.ascontiguousarray(np.broadcast_to(levels, inp["A_log"].shape))
    inp["dt_raw"] = (inp["dt_raw"] * np.float32(6.0)).astype(np.float32)  # delta over decades
    check(orc, wl, False, True, inp=inp, what="zoh extreme A_log")
    check(orc, wl, True, True, inp=inp, what="zoh extreme A_log, gated")


@pytest.mark.parametrize("name,gate,zoh", [("vmamba_t_stage1_bf16", True, False),
                                           ("vmamba_t_stage1_bf16", True, True),
                                           ("vmamba_t_stage1_f32", True, True),
                                           ("highres_1024px_bf16", False, True),
                                           ("vim_bidir_bf16", True, True)])
def test_options_full_size(orc, name, gate, zoh):
    """Every output element of the gated and zero-order-hold operator at the benchmark
    sizes against the oracle's whole output."""
    import torch
    wl = workloads.workload(name)
    log(f"case full-size {name} gate={gate} zoh={zoh}: generating inputs")
    inp = workloads.make_inputs(wl, seed=0)
    g = workloads.make_gate(wl, 0) if gate else None
    dev = to_device(inp, wl)
    z = gate_to_device(g, wl) if gate else None
    log(f"case full-size {name}: GPU run")
    y = to_numpy_f64(run_ex(dev, wl, z, zoh))
    torch.cuda.synchronize()
    del dev, z
    log(f"case full-size {name}: oracle")
    ref = orc.forward(wl.K, *[inp[k] for k in ARGS], z=g["z"] if gate else None, zoh=zoh)
    assert_parity(y, ref, wl.dtype, f"{name} gate={gate} zoh={zoh} (all {y.size} outputs)")


def test_plain_and_ex_agree_bitwise():
    """Without gate and flag the extended entry point is the plain one."""
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 96, 12, 20, 16, 4, "bf16")
    dev = to_device(workloads.make_inputs(wl, seed=24), wl)
    y0 = ss.ss2d_forward(*[dev[k] for k in ARGS])
    y1 = ss.ss2d_forward_ex(*[dev[k] for k in ARGS])
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


def test_gate_at_zero_gives_zero_and_ex_errors():
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(1, 16, 4, 8, 8, 4, "f32")
    dev = to_device(workloads.make_inputs(wl, seed=25), wl)
    z = torch.zeros_like(dev["x"])
    y = ss.ss2d_forward_ex(*[dev[k] for k in ARGS], z=z, zoh=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    with pytest.raises(ss.SS2DError) as ei:
        ss.ss2d_forward_ex(*[dev[k] for k in ARGS], z=z, y=z)
    assert ei.value.status == ss.SS2D_ERR_ALIAS
