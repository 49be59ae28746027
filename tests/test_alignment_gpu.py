"""Element-aligned but otherwise misaligned buffers (every data tensor a view one element into
its allocation: 2-byte aligned for bfloat16, 4-byte for fp32) give bit for bit the results
of the same call on 256-byte aligned buffers: the 16-byte loads and stores of whole tiles
take any alignment, and the kernels that need more fall back to element access with the
same arithmetic.  Covers the forward (plain and gated), the backward and the front end with
the routes operator, for both route sets and both data types."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
DATA = ("x", "dt_raw", "Bs", "Cs")


def _shifted(t):
    """A contiguous copy of t that starts one element into its allocation."""
    import torch
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    return v


def _inputs(wl, seed):
    import torch
    inp = workloads.make_inputs(wl, seed=seed, a_log="random")
    dev = {}
    for k in DATA:
        if wl.dtype == "bf16":
            dev[k] = torch.from_numpy(inp[k + "_bf16"].view(np.int16)).view(torch.bfloat16)
        else:
            dev[k] = torch.from_numpy(np.ascontiguousarray(inp[k], np.float32))
        dev[k] = dev[k].cuda()
    for k in ("A_log", "Ds", "dt_bias"):
        dev[k] = torch.from_numpy(inp[k]).cuda()
    return dev


def _same(a, b, what):
    import torch
    ok = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                     b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    log(f"  {what}: {'identical' if ok else 'DIFFERENT'}")
    assert ok, f"{what}: misaligned buffers changed the result"


CASES = [  # B, D, H, W, N, K, dtype
    (2, 70, 8, 12, 16, 4, "bf16"),
    (2, 70, 5, 7, 16, 4, "f32"),
    (2, 48, 1, 197, 16, 2, "bf16"),
    (2, 40, 1, 64, 8, 2, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}".format(*c))
def test_forward_misaligned(case):
    import torch
    import selective_scan_ss2d_amd as ss
    B, D, H, W, N, K, dt = case
    wl = workloads.custom(B, D, H, W, N, K, dt)
    log(f"case forward misaligned {case}")
    dev = _inputs(wl, 61)
    sh = dict(dev, **{k: _shifted(dev[k]) for k in DATA})
    g = workloads.make_gate(wl, 61)
    z = (torch.from_numpy(g["z_bf16"].view(np.int16)).view(torch.bfloat16) if dt == "bf16"
         else torch.from_numpy(g["z"])).cuda()
    fn = ss.ss2d_forward_ex if K == 4 else ss.ss1d_bidir_forward_ex
    for gate in (None, z):
        y = fn(*[dev[k] for k in ARGS], z=gate)
        y_sh = _shifted(torch.zeros_like(y))
        fn(*[sh[k] for k in ARGS], z=None if gate is None else _shifted(gate), y=y_sh)
        torch.cuda.synchronize()
        _same(y_sh, y, f"y gate={gate is not None}")


@pytest.mark.parametrize("case", [CASES[0], CASES[2]],
                         ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}".format(*c))
def test_backward_misaligned(case):
    import torch
    import selective_scan_ss2d_amd as ss
    B, D, H, W, N, K, dt = case
    wl = workloads.custom(B, D, H, W, N, K, dt)
    log(f"case backward misaligned {case}")
    dev = _inputs(wl, 62)
    sh = dict(dev, **{k: _shifted(dev[k]) for k in DATA})
    gr = workloads.make_output_grad(wl, 62)
    dy = torch.from_numpy(gr["dy_bf16"].view(np.int16)).view(torch.bfloat16).cuda()
    fn = ss.ss2d_backward if K == 4 else ss.ss1d_bidir_backward
    g0 = fn(*[dev[k] for k in ARGS], dy)
    g1 = fn(*[sh[k] for k in ARGS], _shifted(dy))
    torch.cuda.synchronize()
    for k in ARGS:
        _same(g1[k], g0[k], f"d{k}")


@pytest.mark.parametrize("K,H,W", [(4, 8, 12), (2, 1, 197)])
def test_front_end_misaligned(K, H, W):
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 70, H, W, 16, K, "bf16")
    log(f"case front end misaligned K={K} {H}x{W}")
    dev = _inputs(wl, 63)
    w = workloads.make_front_weights(wl, 63, R=2, KW=4)
    fw = [torch.from_numpy(w[k]).cuda() for k in ("conv_w", "conv_b", "x_proj_w", "dt_proj_w")]
    proj = ss.ss2d_project if K == 4 else ss.ss1d_bidir_project
    routes = ss.ss2d_forward_routes if K == 4 else ss.ss1d_bidir_forward_routes
    hw = (H, W) if K == 4 else ()
    o0 = proj(dev["x"], *fw)
    o1 = proj(_shifted(dev["x"]), *fw)
    y0 = routes(o0["u"], o0["dt_raw"], dev["A_log"], o0["Bs"], o0["Cs"], dev["Ds"],
                dev["dt_bias"], *hw)
    y1 = routes(*[_shifted(o1[k]) for k in ("u", "dt_raw")], dev["A_log"],
                *[_shifted(o1[k]) for k in ("Bs", "Cs")], dev["Ds"], dev["dt_bias"], *hw)
    torch.cuda.synchronize()
    for k in ("u", "dt_raw", "Bs", "Cs"):
        _same(o1[k], o0[k], f"project {k}")
    _same(y1, y0, "routes y")
