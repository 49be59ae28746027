"""GPU parity of the backward of the operator over per-route inputs (ss2d_backward_routes,
ss1d_bidir_backward_routes: each route's du per step, and every other input's gradient)
against the float64 oracle, through the C ABI: small shapes with ragged tiles, both element
types and route sets, with and without the gate and the zero-order hold, and the benchmark
size; plus bitwise determinism."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL_BWD, assert_parity, log, to_device, to_numpy_f64

pytestmark = pytest.mark.gpu

ARGS = ("dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
IO_GRADS = ("u", "dt_raw", "Bs", "Cs", "z")      # in the data type
OPTIONS = [(False, False), (True, False), (False, True), (True, True)]
OPTION_IDS = ["plain", "gate", "zoh", "gate_zoh"]


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _dev(g, key, wl):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(g[key + "_bf16"].view(np.int16)).view(torch.bfloat16).to(
            "cuda:0")
    return torch.from_numpy(g[key]).to("cuda:0")


def run(wl, u, dev, dy, z, zoh):
    import selective_scan_ss2d_amd as ss
    args = [dev[k] for k in ARGS]
    if wl.K == 4:
        return ss.ss2d_backward_routes(u, *args, dy, wl.H, wl.W, z=z, zoh=zoh)
    return ss.ss1d_bidir_backward_routes(u, *args, dy, z=z, zoh=zoh)


def check(orc, wl, gate, zoh, seed=0, a_log="random", what=None):
    import torch
    what = (what or f"B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} {wl.dtype}") + \
        f" gate={gate} zoh={zoh}"
    log(f"case routes backward {what}")
    inp = workloads.make_inputs(wl, seed=seed, a_log=a_log)
    ri = workloads.make_route_inputs(wl, seed)
    g = workloads.make_output_grad(wl, seed)
    zg = workloads.make_gate(wl, seed) if gate else None
    ref = orc.backward_routes(wl.K, ri["u"], *[inp[k] for k in ARGS], g["dy"], wl.H, wl.W,
                              z=zg["z"] if gate else None, zoh=zoh)
    dev = to_device(inp, wl)
    grads = run(wl, _dev(ri, "u", wl), dev, _dev(g, "dy", wl),
                _dev(zg, "z", wl) if gate else None, zoh)
    torch.cuda.synchronize()
    for name in ("u",) + ARGS + (("z",) if gate else ()):
        tol_dtype = wl.dtype if name in IO_GRADS else "f32"
        got = to_numpy_f64(grads[name]).reshape(ref[name].shape)
        assert_parity(got, ref[name], tol_dtype, f"routes backward d{name} {what}",
                      tol=TOL_BWD)


SHAPES = [  # B, D, H, W, N, K, dtype
    (2, 70, 5, 7, 16, 4, "f32"),
    (2, 70, 5, 7, 16, 4, "bf16"),
    (2, 130, 24, 24, 16, 4, "bf16"),
    (1, 33, 3, 5, 4, 4, "f32"),
    (1, 33, 1, 40, 8, 4, "f32"),
    (3, 100, 1, 197, 16, 2, "bf16"),
    (2, 64, 1, 320, 16, 2, "f32"),
    (2, 70, 5, 7, 2, 4, "f32"),       # N = 2: four states with zero-padded B and C
    (2, 70, 5, 7, 32, 4, "bf16"),     # N = 32
]


@pytest.mark.parametrize("gate,zoh", OPTIONS, ids=OPTION_IDS)
@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}".format(*c))
def test_backward_routes_small(orc, case, gate, zoh):
    B, D, H, W, N, K, dt = case
    check(orc, workloads.custom(B, D, H, W, N, K, dt), gate, zoh, seed=71)


@pytest.mark.parametrize("name,gate", [("vmamba_t_stage1_bf16", True),
                                       ("vim_bidir_bf16", False)])
def test_backward_routes_full_size(orc, name, gate):
    check(orc, workloads.workload(name), gate, False, seed=0, a_log="init", what=name)


def test_backward_routes_deterministic():
    import torch
    wl = workloads.custom(2, 130, 24, 24, 16, 4, "bf16")
    inp = workloads.make_inputs(wl, seed=72)
    dev = to_device(inp, wl)
    u = _dev(workloads.make_route_inputs(wl, 72), "u", wl)
    dy = _dev(workloads.make_output_grad(wl, 72), "dy", wl)
    z = _dev(workloads.make_gate(wl, 72), "z", wl)
    g1 = {k: v.clone() for k, v in run(wl, u, dev, dy, z, True).items()}
    g2 = run(wl, u, dev, dy, z, True)
    torch.cuda.synchronize()
    for k, a in g1.items():
        view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(view), g2[k].view(view)), k
