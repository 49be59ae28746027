"""GPU parity of the per-route front end (causal depthwise conv + SiLU, x_proj, dt_proj) and of
the operator over per-route inputs against the float64 oracle, through the C ABI: small
shapes element by element (ragged step tiles, channel counts across the 64-channel chunks,
every conv length and x_proj width the kernel supports, both element types, both route
sets, degenerate maps), the chain of both entry points, and sampled images at the VMamba-T
stage-1 size."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (TOL_DT_RAW, TOL_FRONT, assert_parity, plan_override, log, to_device,
                            to_numpy_f64)

pytestmark = pytest.mark.gpu

ARGS = ("dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
FRONT = ("conv_w", "conv_b", "x_proj_w", "dt_proj_w")
OUTS = ("u", "dt_raw", "Bs", "Cs")


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _dev(a, dtype):
    import torch
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(np.ascontiguousarray(a, np.float32))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda:0")


def _weights_dev(w):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(w[k], np.float32)).to("cuda:0")
            for k in FRONT}


def run_project(x_dev, wd, K):
    import selective_scan_ss2d_amd as ss
    fn = ss.ss2d_project if K == 4 else ss.ss1d_bidir_project
    return fn(x_dev, *[wd[k] for k in FRONT])


def check_project(orc, wl, R, KW, seed=0):
    import torch
    what = f"project B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} R{R} KW{KW} {wl.dtype}"
    log(f"case {what}")
    inp = workloads.make_inputs(wl, seed=seed)
    w = workloads.make_front_weights(wl, seed, R=R, KW=KW)
    ref = orc.project(wl.K, inp["x"], *[w[k] for k in FRONT])
    got = run_project(to_device(inp, wl)["x"], _weights_dev(w), wl.K)
    torch.cuda.synchronize()
    for k in OUTS:
        assert_parity(to_numpy_f64(got[k]), ref[k], wl.dtype, f"{what} {k}",
                      tol=TOL_DT_RAW if k == "dt_raw" else TOL_FRONT)


PROJ_SHAPES = [  # B, D, H, W, N, K, dtype, R, KW
    (1, 8, 8, 8, 4, 4, "f32", 1, 4),
    (2, 70, 5, 27, 4, 4, "f32", 3, 4),
    (2, 70, 5, 27, 4, 4, "bf16", 3, 4),
    (2, 130, 9, 11, 16, 4, "bf16", 1, 4),
    (1, 64, 7, 9, 16, 4, "f32", 6, 4),
    (1, 40, 6, 13, 16, 4, "bf16", 64, 4),     # 96 x_proj rows: the most supported
    (1, 40, 6, 13, 8, 4, "f32", 5, 1),         # KW = 1: a pointwise conv
    (1, 40, 6, 13, 8, 4, "bf16", 2, 8),        # KW = 8: the longest conv
    (1, 24, 1, 150, 4, 4, "f32", 2, 4),        # H = 1: every route along the one row
    (1, 24, 150, 1, 4, 4, "bf16", 2, 4),       # W = 1
    (1, 24, 1, 3, 4, 4, "f32", 2, 4),          # fewer steps than taps
    (2, 48, 1, 197, 16, 2, "bf16", 1, 4),      # Vim paths: 196 patches + class token
    (3, 33, 1, 65, 8, 2, "f32", 4, 3),
    # L a multiple of 4 with KW = 4: the four-steps-per-lane kernel
    (2, 70, 6, 10, 4, 4, "f32", 3, 4),         # one ragged tile, two channel chunks
    (2, 70, 6, 10, 4, 4, "bf16", 3, 4),
    (1, 130, 12, 20, 16, 4, "bf16", 1, 4),     # four tiles, the last one ragged
    (1, 40, 12, 20, 16, 4, "f32", 64, 4),      # 96 x_proj rows
    (1, 130, 12, 20, 16, 4, "bf16", 64, 4),    # dt_proj weights too large for LDS
    (2, 48, 1, 196, 16, 2, "bf16", 1, 4),      # Vim paths without the class token
    (1, 24, 4, 1, 4, 4, "f32", 2, 4),          # four steps in all
    (1, 24, 1, 5, 4, 4, "bf16", 2, 4),         # five steps: one lane holds the fifth alone
    (1, 24, 7, 1, 4, 4, "f32", 2, 4),          # seven steps (the last lane holds three)
    (2, 20, 1, 6, 4, 2, "bf16", 1, 4),         # six steps, both paths
]


@pytest.mark.parametrize("case", PROJ_SHAPES,
                         ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}_R{}_KW{}".format(*c))
def test_project_small(orc, case):
    B, D, H, W, N, K, dt, R, KW = case
    check_project(orc, workloads.custom(B, D, H, W, N, K, dt), R, KW, seed=31)


def test_project_impulse_taps(orc):
    """A unit impulse through the conv alone (x_proj, dt_proj zero): the reversed taps at the
    KW steps from the one that visits the impulse, on every route."""
    import torch
    wl = workloads.custom(1, 64, 6, 10, 4, 4, "f32")
    D, L = wl.D, wl.L
    x = np.zeros((1, D, wl.H, wl.W), np.float32)
    x[0, 5, 2, 3] = 1.0
    x[0, 63, 0, 0] = 1.0
    x[0, 17, 5, 9] = 1.0
    w = workloads.make_front_weights(wl, 5, R=2, KW=4)
    w["conv_w"] = (3.0 + np.arange(4 * D * 4, dtype=np.float32).reshape(4, D, 4) % 7)
    ref = orc.project(4, x, *[w[k] for k in FRONT])
    got = run_project(_dev(x, "f32"), _weights_dev(w), 4)
    torch.cuda.synchronize()
    assert_parity(to_numpy_f64(got["u"]), ref["u"], "f32", "impulse u")


def route_inputs_to_device(ri, wl):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(ri["u_bf16"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(ri["u"]).to("cuda:0")


def run_routes(u_dev, dev, wl, z=None, zoh=False):
    import selective_scan_ss2d_amd as ss
    if wl.K == 4:
        return ss.ss2d_forward_routes(u_dev, *[dev[k] for k in ARGS], wl.H, wl.W, z=z, zoh=zoh)
    return ss.ss1d_bidir_forward_routes(u_dev, *[dev[k] for k in ARGS], z=z, zoh=zoh)


def check_routes(orc, wl, gate, zoh, seed=0, **overrides):
    import torch
    what = (f"routes B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} {wl.dtype} gate={gate} "
            f"zoh={zoh} {overrides}")
    log(f"case {what}")
    inp = workloads.make_inputs(wl, seed=seed, a_log="random")
    ri = workloads.make_route_inputs(wl, seed)
    g = workloads.make_gate(wl, seed) if gate else None
    ref = orc.forward_routes(wl.K, ri["u"], *[inp[k] for k in ARGS], wl.H, wl.W,
                             z=g["z"] if gate else None, zoh=zoh)
    dev = to_device(inp, wl)
    z = _dev(g["z"], wl.dtype) if gate else None
    with plan_override(**overrides):
        y = run_routes(route_inputs_to_device(ri, wl), dev, wl, z=z, zoh=zoh)
    torch.cuda.synchronize()
    assert_parity(to_numpy_f64(y), ref.reshape(y.shape), wl.dtype, what)


ROUTE_SHAPES = [  # B, D, H, W, N, K, dtype
    (1, 8, 8, 8, 4, 4, "f32"),
    (2, 70, 5, 7, 16, 4, "f32"),
    (2, 70, 5, 7, 16, 4, "bf16"),
    (2, 130, 24, 24, 16, 4, "bf16"),
    (3, 100, 1, 197, 16, 2, "bf16"),
    (2, 64, 1, 320, 16, 2, "f32"),
]


@pytest.mark.parametrize("gate,zoh", [(False, False), (True, True)], ids=["plain", "gate_zoh"])
@pytest.mark.parametrize("case", ROUTE_SHAPES,
                         ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}".format(*c))
def test_routes_small(orc, case, gate, zoh):
    B, D, H, W, N, K, dt = case
    check_routes(orc, workloads.custom(B, D, H, W, N, K, dt), gate, zoh, seed=32)


@pytest.mark.parametrize("var", [dict(split=1, chunk_len=64),
                                 dict(split=4, chunk_len=96),
                                 dict(split=2, chunk_len=0)],
                         ids=["S1_C64", "S4_C96", "S2_C0"])
def test_routes_launch_variants(orc, var):
    """Chunked passes (chunk states and carries) and the lane splits on per-route inputs."""
    check_routes(orc, workloads.custom(2, 72, 13, 11, 16, 4, "f32"), True, False, seed=33,
                 **var)


@pytest.mark.parametrize("K,H,W", [(4, 9, 14), (2, 1, 130)])
def test_chain_f32(orc, K, H, W):
    """project then forward_routes on the GPU against the same chain in the oracle (the
    oracle's front-end outputs, as fp32, fed to its routes operator)."""
    import torch
    wl = workloads.custom(2, 80, H, W, 16, K, "f32")
    log(f"case chain K={K} {H}x{W}")
    inp = workloads.make_inputs(wl, seed=34, a_log="random")
    w = workloads.make_front_weights(wl, 34, R=2, KW=4)
    g = workloads.make_gate(wl, 34)
    pr = orc.project(K, inp["x"], *[w[k] for k in FRONT])
    ref = orc.forward_routes(K, pr["u"].astype(np.float32), pr["dt_raw"].astype(np.float32),
                             inp["A_log"], pr["Bs"].astype(np.float32),
                             pr["Cs"].astype(np.float32), inp["Ds"], inp["dt_bias"], H, W,
                             z=g["z"])
    dev = to_device(inp, wl)
    out = run_project(dev["x"], _weights_dev(w), K)
    dev2 = dict(dev, dt_raw=out["dt_raw"], Bs=out["Bs"], Cs=out["Cs"])
    y = run_routes(out["u"], dev2, wl, z=_dev(g["z"], "f32"))
    torch.cuda.synchronize()
    assert_parity(to_numpy_f64(y), ref.reshape(y.shape), "f32", f"chain K={K}",
                  tol=TOL_FRONT)


@pytest.mark.parametrize("name,R", [("vmamba_t_stage1_bf16", 1), ("vim_bidir_bf16", 1)])
def test_full_size_sampled_images(orc, name, R):
    """The full benchmark shapes: both entry points at full size, checked on two images
    against the oracle run on those images alone."""
    import torch
    wl = workloads.workload(name)
    log(f"case full size {name}")
    inp = workloads.make_inputs(wl, seed=35)
    w = workloads.make_front_weights(wl, 35, R=R, KW=4)
    dev = to_device(inp, wl)
    out = run_project(dev["x"], _weights_dev(w), wl.K)
    ri = workloads.make_route_inputs(wl, 35)
    y = run_routes(route_inputs_to_device(ri, wl), dev, wl)
    torch.cuda.synchronize()
    for b in (0, wl.B - 1):
        ref = orc.project(wl.K, inp["x"][b:b + 1], *[w[k] for k in FRONT])
        for k in OUTS:
            assert_parity(to_numpy_f64(out[k][b:b + 1]), ref[k], wl.dtype,
                          f"full {name} b={b} project {k}",
                          tol=TOL_DT_RAW if k == "dt_raw" else TOL_FRONT)
        sl = {k: inp[k][b:b + 1] for k in ("dt_raw", "Bs", "Cs")}
        refy = orc.forward_routes(wl.K, ri["u"][b:b + 1], sl["dt_raw"], inp["A_log"], sl["Bs"],
                                  sl["Cs"], inp["Ds"], inp["dt_bias"], wl.H, wl.W)
        assert_parity(to_numpy_f64(y[b:b + 1]), refy.reshape(y[b:b + 1].shape), wl.dtype,
                      f"full {name} b={b} routes")


# ---- dt_proj folded into the scan: the front end's R dt rows and the operator over them ----
def check_project_lr(orc, wl, R, KW, seed=0):
    import torch
    import selective_scan_ss2d_amd as ss
    what = f"project_lr B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} R{R} KW{KW} {wl.dtype}"
    log(f"case {what}")
    inp = workloads.make_inputs(wl, seed=seed)
    w = workloads.make_front_weights(wl, seed, R=R, KW=KW)
    ref = orc.project_lr(wl.K, inp["x"], w["conv_w"], w["conv_b"], w["x_proj_w"], R)
    wd = _weights_dev(w)
    fn = ss.ss2d_project_lr if wl.K == 4 else ss.ss1d_bidir_project_lr
    got = fn(to_device(inp, wl)["x"], wd["conv_w"], wd["conv_b"], wd["x_proj_w"], R)
    torch.cuda.synchronize()
    assert set(got) == {"u", "dt_lr", "Bs", "Cs"}
    for k in ("u", "dt_lr", "Bs", "Cs"):
        assert tuple(got[k].shape) == ref[k].shape, k
        assert_parity(to_numpy_f64(got[k]), ref[k], wl.dtype, f"{what} {k}", tol=TOL_FRONT)


PROJ_LR_SHAPES = [  # B, D, H, W, N, K, dtype, R, KW
    (2, 70, 5, 27, 4, 4, "f32", 3, 4),         # one step per lane
    (2, 70, 5, 27, 4, 4, "bf16", 3, 4),
    (2, 130, 6, 10, 16, 4, "bf16", 1, 4),      # four steps per lane, ragged tile
    (2, 70, 6, 10, 4, 4, "f32", 4, 4),
    (1, 40, 12, 20, 16, 4, "f32", 64, 4),      # 96 x_proj rows, 64 dt rows
    (1, 40, 6, 13, 8, 4, "bf16", 2, 8),
    (2, 48, 1, 197, 16, 2, "bf16", 1, 4),      # Vim paths
    (2, 48, 1, 196, 16, 2, "f32", 2, 4),
]


@pytest.mark.parametrize("case", PROJ_LR_SHAPES,
                         ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}_R{}_KW{}".format(*c))
def test_project_lr_small(orc, case):
    B, D, H, W, N, K, dt, R, KW = case
    check_project_lr(orc, workloads.custom(B, D, H, W, N, K, dt), R, KW, seed=36)


def run_routes_lr(u_dev, lr_dev, dtw_dev, dev, wl, z=None, zoh=False):
    import selective_scan_ss2d_amd as ss
    rest = [dev[k] for k in ARGS[1:]]
    if wl.K == 4:
        return ss.ss2d_forward_routes_lr(u_dev, lr_dev, dtw_dev, *rest, wl.H, wl.W, z=z,
                                         zoh=zoh)
    return ss.ss1d_bidir_forward_routes_lr(u_dev, lr_dev, dtw_dev, *rest, z=z, zoh=zoh)


def check_routes_lr(orc, wl, R, gate, zoh, seed=0, **overrides):
    import torch
    what = (f"routes_lr B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} R{R} {wl.dtype} "
            f"gate={gate} zoh={zoh} {overrides}")
    log(f"case {what}")
    inp = workloads.make_inputs(wl, seed=seed, a_log="random")
    ri = workloads.make_route_inputs(wl, seed)
    lr = workloads.make_lowrank_dt(wl, seed, R=R)
    g = workloads.make_gate(wl, seed) if gate else None
    ref = orc.forward_routes_lr(wl.K, ri["u"], lr["dt_lr"], lr["dt_w"],
                                *[inp[k] for k in ARGS[1:]], wl.H, wl.W,
                                z=g["z"] if gate else None, zoh=zoh)
    dev = to_device(inp, wl)
    z = _dev(g["z"], wl.dtype) if gate else None
    dtw = torch.from_numpy(lr["dt_w"]).to("cuda:0")
    with plan_override(**overrides):
        y = run_routes_lr(route_inputs_to_device(ri, wl), _dev(lr["dt_lr"], wl.dtype), dtw,
                          dev, wl, z=z, zoh=zoh)
    torch.cuda.synchronize()
    assert_parity(to_numpy_f64(y), ref.reshape(y.shape), wl.dtype, what)


ROUTE_LR_SHAPES = [  # B, D, H, W, N, K, dtype, R
    (1, 8, 8, 8, 4, 4, "f32", 1),
    (2, 70, 5, 7, 16, 4, "f32", 2),
    (2, 70, 5, 7, 16, 4, "bf16", 4),
    (2, 130, 24, 24, 16, 4, "bf16", 1),
    (1, 40, 9, 11, 32, 4, "f32", 4),           # the largest state with the most dt rows
    (1, 40, 9, 11, 1, 4, "bf16", 3),
    (3, 100, 1, 197, 16, 2, "bf16", 1),
    (2, 64, 1, 320, 16, 2, "f32", 3),
]


@pytest.mark.parametrize("gate,zoh", [(False, False), (True, True)], ids=["plain", "gate_zoh"])
@pytest.mark.parametrize("case", ROUTE_LR_SHAPES,
                         ids=lambda c: "B{}D{}_{}x{}_N{}_K{}_{}_R{}".format(*c))
def test_routes_lr_small(orc, case, gate, zoh):
    B, D, H, W, N, K, dt, R = case
    check_routes_lr(orc, workloads.custom(B, D, H, W, N, K, dt), R, gate, zoh, seed=37)


@pytest.mark.parametrize("var", [dict(split=1, chunk_len=64),
                                 dict(split=4, chunk_len=96),
                                 dict(split=2, chunk_len=0)],
                         ids=["S1_C64", "S4_C96", "S2_C0"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_routes_lr_launch_variants(orc, var, dt):
    """Chunked passes and the lane splits with dt_proj folded into the scan."""
    check_routes_lr(orc, workloads.custom(2, 72, 13, 11, 16, 4, dt), 2, True, False, seed=38,
                    **var)


@pytest.mark.parametrize("K,H,W,dt", [(4, 9, 14, "f32"), (2, 1, 130, "f32"),
                                      (4, 12, 12, "bf16")])
def test_chain_lr(orc, K, H, W, dt):
    """project_lr then forward_routes_lr on the GPU against the same chain in the oracle (its
    front-end outputs, rounded to the data type, fed to its folded operator).  The GPU's
    bf16 outputs and the oracle's rounding of its own can differ by one bf16 step where a
    value falls near a rounding boundary, so the bf16 chain is held to the bf16 bar."""
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 80, H, W, 16, K, dt)
    R = 2
    log(f"case chain_lr K={K} {H}x{W} {dt}")
    inp = workloads.make_inputs(wl, seed=39, a_log="random")
    w = workloads.make_front_weights(wl, 39, R=R, KW=4)
    g = workloads.make_gate(wl, 39)
    pr = orc.project_lr(K, inp["x"], w["conv_w"], w["conv_b"], w["x_proj_w"], R)
    rnd = (lambda a: workloads.round_bf16(a.astype(np.float32))) if dt == "bf16" else \
        (lambda a: a.astype(np.float32))
    dt_w = w["dt_proj_w"]
    ref = orc.forward_routes_lr(K, rnd(pr["u"]), rnd(pr["dt_lr"]), dt_w, inp["A_log"],
                                rnd(pr["Bs"]), rnd(pr["Cs"]), inp["Ds"], inp["dt_bias"], H, W,
                                z=g["z"] if dt == "f32" else workloads.round_bf16(g["z"]))
    dev = to_device(inp, wl)
    wd = _weights_dev(w)
    fn = ss.ss2d_project_lr if K == 4 else ss.ss1d_bidir_project_lr
    out = fn(dev["x"], wd["conv_w"], wd["conv_b"], wd["x_proj_w"], R)
    dev2 = dict(dev, Bs=out["Bs"], Cs=out["Cs"])
    y = run_routes_lr(out["u"], out["dt_lr"], wd["dt_proj_w"], dev2, wl,
                      z=_dev(g["z"], dt))
    torch.cuda.synchronize()
    assert_parity(to_numpy_f64(y), ref.reshape(y.shape), dt, f"chain_lr K={K} {dt}",
                  tol=TOL_FRONT)


def test_lr_matches_unfolded_operator(orc):
    """With dt_raw = dt_w @ dt_lr formed beforehand, the unfolded operator on the GPU and the
    folded one agree to fp32 rounding (the sum of R products taken in another order)."""
    import torch
    wl = workloads.custom(2, 96, 10, 12, 16, 4, "f32")
    log("case lr vs unfolded")
    inp = workloads.make_inputs(wl, seed=40, a_log="random")
    ri = workloads.make_route_inputs(wl, 40)
    lr = workloads.make_lowrank_dt(wl, 40, R=4)
    dt_raw = np.einsum("kdr,bkrl->bkdl", lr["dt_w"].astype(np.float64),
                       lr["dt_lr"].astype(np.float64)).astype(np.float32)
    dev = to_device(inp, wl)
    u = route_inputs_to_device(ri, wl)
    y_lr = run_routes_lr(u, _dev(lr["dt_lr"], "f32"), torch.from_numpy(lr["dt_w"]).cuda(), dev,
                         wl)
    y = run_routes(u, dict(dev, dt_raw=_dev(dt_raw, "f32")), wl)
    torch.cuda.synchronize()
    assert_parity(to_numpy_f64(y_lr), to_numpy_f64(y), "f32", "lr vs unfolded")


@pytest.mark.parametrize("name", ["vmamba_t_stage1_bf16", "vim_bidir_bf16"])
def test_full_size_lr_sampled_images(orc, name):
    """Both folded entry points at the full benchmark shapes (R = 1, the explainer's rank),
    checked on two images against the oracle run on those images alone."""
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.workload(name)
    R = 1
    log(f"case full size lr {name}")
    inp = workloads.make_inputs(wl, seed=41)
    w = workloads.make_front_weights(wl, 41, R=R, KW=4)
    dev = to_device(inp, wl)
    wd = _weights_dev(w)
    fp = ss.ss2d_project_lr if wl.K == 4 else ss.ss1d_bidir_project_lr
    out = fp(dev["x"], wd["conv_w"], wd["conv_b"], wd["x_proj_w"], R)
    ri = workloads.make_route_inputs(wl, 41)
    lr = workloads.make_lowrank_dt(wl, 41, R=R)
    y = run_routes_lr(route_inputs_to_device(ri, wl), _dev(lr["dt_lr"], wl.dtype),
                      torch.from_numpy(lr["dt_w"]).cuda(), dev, wl)
    torch.cuda.synchronize()
    for b in (0, wl.B - 1):
        ref = orc.project_lr(wl.K, inp["x"][b:b + 1], w["conv_w"], w["conv_b"], w["x_proj_w"],
                             R)
        for k in ("u", "dt_lr", "Bs", "Cs"):
            assert_parity(to_numpy_f64(out[k][b:b + 1]), ref[k], wl.dtype,
                          f"full {name} b={b} project_lr {k}", tol=TOL_FRONT)
        refy = orc.forward_routes_lr(wl.K, ri["u"][b:b + 1], lr["dt_lr"][b:b + 1], lr["dt_w"],
                                     inp["A_log"], inp["Bs"][b:b + 1], inp["Cs"][b:b + 1],
                                     inp["Ds"], inp["dt_bias"], wl.H, wl.W)
        assert_parity(to_numpy_f64(y[b:b + 1]), refy.reshape(y[b:b + 1].shape), wl.dtype,
                      f"full {name} b={b} routes_lr")
