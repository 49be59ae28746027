"""The training entry points through the C ABI: ss2d_forward_save's y is ss2d_forward_ex's
(one pass) bit for bit, and ss2d_backward_saved, starting from the state it kept, gives
ss2d_backward_ex's gradients bit for bit; for both route sets and element types, with and
without the gate and the zero-order hold, on ragged and whole-tile shapes and at the
benchmark size; and the same for the pair over per-route inputs against
ss2d_forward_routes and ss2d_backward_routes.  The backward_ex results themselves are checked against the float64 oracle
in tests/test_backward_gpu.py and tests/test_backward_ex_gpu.py."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import log, plan_override, to_device

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
OPTIONS = [(False, False), (True, False), (False, True), (True, True)]
OPTION_IDS = ["plain", "gate", "zoh", "gate_zoh"]
SHAPES = [(2, 70, 5, 7, 16, 4, "f32"), (2, 70, 5, 7, 16, 4, "bf16"), (1, 64, 8, 8, 4, 4, "f32"),
          (2, 40, 9, 11, 32, 4, "bf16"), (1, 33, 16, 16, 8, 4, "f32"),
          (3, 40, 1, 197, 16, 2, "bf16"), (2, 16, 1, 64, 32, 2, "f32"), (2, 24, 1, 45, 4, 2, "bf16")]


def _bits(t):
    import torch
    t = t.detach().contiguous()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(a, b):
    import torch
    return torch.equal(_bits(a), _bits(b))


def _image(g, key, wl):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(g[key + "_bf16"].view(np.int16)).view(torch.bfloat16).to(
            "cuda:0")
    return torch.from_numpy(g[key]).to("cuda:0")


def _run(wl, gate, zoh, seed, a_log="random"):
    import torch
    import selective_scan_ss2d_amd as ss
    inp = workloads.make_inputs(wl, seed=seed, a_log=a_log)
    dev = to_device(inp, wl)
    args = [dev[k] for k in ARGS]
    dy = _image(workloads.make_output_grad(wl, seed), "dy", wl)
    z = _image(workloads.make_gate(wl, seed), "z", wl) if gate else None
    fwd_ex = ss.ss2d_forward_ex if wl.K == 4 else ss.ss1d_bidir_forward_ex
    fwd_save = ss.ss2d_forward_save if wl.K == 4 else ss.ss1d_bidir_forward_save
    bwd_ex = ss.ss2d_backward_ex if wl.K == 4 else ss.ss1d_bidir_backward_ex
    bwd_saved = ss.ss2d_backward_saved if wl.K == 4 else ss.ss1d_bidir_backward_saved
    with plan_override(split=4, chunk_len=0):  # the one-pass plan the training forward runs
        y_ref = fwd_ex(*args, z=z, zoh=zoh)
    y, saved = fwd_save(*args, z=z, zoh=zoh)
    g_ref = bwd_ex(*args, dy, z=z, zoh=zoh)
    g = bwd_saved(*args, dy, saved, z=z, zoh=zoh)
    torch.cuda.synchronize()
    return y_ref, y, g_ref, g, saved


@pytest.mark.parametrize("gate,zoh", OPTIONS, ids=OPTION_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_saved_equals_recomputed(shape, gate, zoh):
    B, D, H, W, N, K, dt = shape
    wl = workloads.custom(B, D, H, W, N, K, dt)
    log(f"case saved B{B} D{D} {H}x{W} N{N} K{K} {dt} gate={gate} zoh={zoh}")
    y_ref, y, g_ref, g, _ = _run(wl, gate, zoh, seed=3)
    assert _same(y, y_ref), "forward_save's y differs from forward_ex's"
    assert set(g) == set(g_ref)
    for name in g_ref:
        assert _same(g[name], g_ref[name]), f"d{name} from the saved state differs"


def test_saved_state_is_the_checkpoints():
    """The saved state's layout: zero-free checkpoints where 8-step quarters start, and
    with the gate the fp32 route sum, whose gate product rounds to y."""
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 64, 8, 12, 16, 4, "f32")  # L = 96: three tiles, 12 quarters
    y_ref, y, _, _, saved = _run(wl, True, False, seed=5)
    L, slots = wl.H * wl.W, 12
    ck_floats = wl.B * 4 * wl.D * slots * wl.N
    assert saved.numel() * 4 == ss.saved_state_bytes(4, wl.B, wl.D, L, wl.N, True)
    ck = saved[:ck_floats].view(wl.B, 4, wl.D, slots, wl.N)
    assert torch.isfinite(ck[:, :, :, 1:]).all() and (ck[:, :, :, 1:] != 0).any()
    v = saved[ck_floats:].view(wl.B, wl.D, wl.H, wl.W)
    z = torch.from_numpy(workloads.make_gate(wl, 5)["z"]).to("cuda:0")
    gated = v * torch.nn.functional.silu(z)
    err = ((gated - y).abs().max() / y.abs().max()).item()
    log(f"  v SiLU(z) against y: {err:.2e}")
    assert err < 1e-5


@pytest.mark.parametrize("gate", [False, True], ids=["plain", "gate"])
def test_saved_full_size(gate):
    wl = workloads.workload("vmamba_t_stage1_bf16")
    log(f"case saved full size {wl.name} gate={gate}")
    y_ref, y, g_ref, g, _ = _run(wl, gate, False, seed=7, a_log="init")
    assert _same(y, y_ref)
    for name in g_ref:
        assert _same(g[name], g_ref[name]), name


def test_saved_deterministic():
    wl = workloads.custom(2, 70, 5, 7, 16, 4, "bf16")
    _, y1, _, g1, s1 = _run(wl, True, True, seed=9)
    _, y2, _, g2, s2 = _run(wl, True, True, seed=9)
    L = wl.H * wl.W
    ck = wl.B * 4 * wl.D * ((L + 7) // 8) * wl.N
    # the first quarter's checkpoint slots are not written: compare the rest, and the route sum
    c1 = s1[:ck].view(-1, (L + 7) // 8, wl.N)[:, 1:]
    c2 = s2[:ck].view(-1, (L + 7) // 8, wl.N)[:, 1:]
    assert _same(y1, y2) and _same(c1, c2) and _same(s1[ck:], s2[ck:])
    for name in g1:
        assert _same(g1[name], g2[name]), name


ROUTE_SHAPES = [(2, 70, 5, 7, 16, 4, "bf16"), (1, 64, 8, 8, 16, 4, "f32"),
                (3, 40, 1, 197, 16, 2, "bf16"), (2, 16, 1, 64, 8, 2, "f32")]


@pytest.mark.parametrize("gate,zoh", [(False, False), (True, True)], ids=["plain", "gate_zoh"])
@pytest.mark.parametrize("shape", ROUTE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_routes_saved_equals_recomputed(shape, gate, zoh):
    """The training pair of the operator over per-route inputs against ss2d_forward_routes
    and ss2d_backward_routes, bit for bit."""
    import torch
    import selective_scan_ss2d_amd as ss
    B, D, H, W, N, K, dt = shape
    wl = workloads.custom(B, D, H, W, N, K, dt)
    log(f"case routes saved B{B} D{D} {H}x{W} N{N} K{K} {dt} gate={gate} zoh={zoh}")
    inp = workloads.make_inputs(wl, seed=11, a_log="random")
    dev = to_device(inp, wl)
    r = workloads.make_route_inputs(wl, 11)
    u = (torch.from_numpy(r["u_bf16"].view(np.int16)).view(torch.bfloat16) if dt == "bf16"
         else torch.from_numpy(r["u"])).to("cuda:0")
    rest = [dev[k] for k in ARGS[1:]]
    dy = _image(workloads.make_output_grad(wl, 11), "dy", wl)
    z = _image(workloads.make_gate(wl, 11), "z", wl) if gate else None
    hw = (H, W) if K == 4 else ()
    if K == 4:
        fwd, fsave = ss.ss2d_forward_routes, ss.ss2d_forward_routes_save
        bwd, bsaved = ss.ss2d_backward_routes, ss.ss2d_backward_routes_saved
    else:
        fwd, fsave = ss.ss1d_bidir_forward_routes, ss.ss1d_bidir_forward_routes_save
        bwd, bsaved = ss.ss1d_bidir_backward_routes, ss.ss1d_bidir_backward_routes_saved
    with plan_override(split=4, chunk_len=0):
        y_ref = fwd(u, *rest, *hw, z=z, zoh=zoh)
    y, saved = fsave(u, *rest, *hw, z=z, zoh=zoh)
    g_ref = bwd(u, *rest, dy, *hw, z=z, zoh=zoh)
    g = bsaved(u, *rest, dy, saved, *hw, z=z, zoh=zoh)
    torch.cuda.synchronize()
    assert _same(y, y_ref)
    assert set(g) == set(g_ref)
    for name in g_ref:
        assert _same(g[name], g_ref[name]), name
