"""bfloat16 data is fp32 arithmetic rounded once: with inputs that are bfloat16 values, the
bfloat16 entry points must return exactly the round-to-nearest-even of what the fp32 entry
points return for the same values (the kernels compute in fp32 either way, in the same
order, and round each output once).  Checked bit for bit against the host-side rounding
(`workloads.f32_to_bf16_bits`, itself pinned by the CPU tests) for the forward pass with
and without the gate and the zero-order hold, a chunked launch plan, the backward pass and
the front end's u."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import plan_override, log

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
DATA = ("x", "dt_raw", "Bs", "Cs")


def _pair(wl_bf16, seed):
    """Device inputs of one draw twice: as bfloat16 and as fp32 holding the same values."""
    import torch
    inp = workloads.make_inputs(wl_bf16, seed=seed, a_log="random")
    bf, f32 = {}, {}
    for k in DATA:
        bf[k] = torch.from_numpy(inp[k + "_bf16"].view(np.int16)).view(torch.bfloat16).cuda()
        f32[k] = torch.from_numpy(np.ascontiguousarray(inp[k], np.float32)).cuda()
    for k in ("A_log", "Ds", "dt_bias"):
        bf[k] = f32[k] = torch.from_numpy(inp[k]).cuda()
    return bf, f32


def _bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f32(t):
    return t.detach().float().cpu().numpy()


def assert_rounded(got_bf16, ref_f32, what):
    want = workloads.f32_to_bf16_bits(_f32(ref_f32))
    got = _bits(got_bf16)
    bad = int(np.count_nonzero(got != want))
    log(f"  {what}: {got.size} values, {bad} differ from the rounded fp32 result")
    assert bad == 0, f"{what}: {bad} of {got.size} bfloat16 outputs are not RNE(fp32 result)"


CASES = [  # B, D, H, W, N, K
    (2, 70, 9, 11, 16, 4),
    (2, 64, 8, 16, 8, 4),
    (3, 100, 1, 197, 16, 2),
]


@pytest.mark.parametrize("gate,zoh", [(False, False), (True, False), (False, True)],
                         ids=["plain", "gate", "zoh"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}D{}_{}x{}_N{}_K{}".format(*c))
def test_forward_bf16_is_rounded_fp32(case, gate, zoh):
    import torch
    import selective_scan_ss2d_amd as ss
    B, D, H, W, N, K = case
    wl = workloads.custom(B, D, H, W, N, K, "bf16")
    log(f"case forward rounding {case} gate={gate} zoh={zoh}")
    bf, f32 = _pair(wl, 51)
    z_bf = z_f32 = None
    if gate:
        g = workloads.make_gate(wl, 51)
        z_bf = torch.from_numpy(g["z_bf16"].view(np.int16)).view(torch.bfloat16).cuda()
        z_f32 = torch.from_numpy(np.ascontiguousarray(g["z"], np.float32)).cuda()
    fn = ss.ss2d_forward_ex if K == 4 else ss.ss1d_bidir_forward_ex
    y_bf = fn(*[bf[k] for k in ARGS], z=z_bf, zoh=zoh)
    y_32 = fn(*[f32[k] for k in ARGS], z=z_f32, zoh=zoh)
    torch.cuda.synchronize()
    assert_rounded(y_bf, y_32, "y")


def test_chunked_forward_bf16_is_rounded_fp32():
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 72, 13, 11, 16, 4, "bf16")
    log("case forward rounding, chunked plan")
    bf, f32 = _pair(wl, 52)
    with plan_override(split=4, chunk_len=64):
        y_bf = ss.ss2d_forward(*[bf[k] for k in ARGS])
        y_32 = ss.ss2d_forward(*[f32[k] for k in ARGS])
    torch.cuda.synchronize()
    assert_rounded(y_bf, y_32, "y (chunks of 64 steps)")


@pytest.mark.parametrize("K,H,W", [(4, 9, 16), (2, 1, 200)])
def test_backward_bf16_is_rounded_fp32(K, H, W):
    """Data gradients come back rounded once; parameter gradients (fp32 in both cases) are
    identical."""
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 40, H, W, 16, K, "bf16")
    log(f"case backward rounding K={K} {H}x{W}")
    bf, f32 = _pair(wl, 53)
    g = workloads.make_output_grad(wl, 53)
    dy_bf = torch.from_numpy(g["dy_bf16"].view(np.int16)).view(torch.bfloat16).cuda()
    dy_32 = torch.from_numpy(np.ascontiguousarray(g["dy"], np.float32)).cuda()
    fn = ss.ss2d_backward if K == 4 else ss.ss1d_bidir_backward
    g_bf = fn(*[bf[k] for k in ARGS], dy_bf)
    g_32 = fn(*[f32[k] for k in ARGS], dy_32)
    torch.cuda.synchronize()
    for k in DATA:
        assert_rounded(g_bf[k], g_32[k], f"d{k}")
    for k in ("A_log", "Ds", "dt_bias"):
        assert np.array_equal(_f32(g_bf[k]), _f32(g_32[k])), f"d{k} differs between data types"


@pytest.mark.parametrize("H,W", [(6, 10), (5, 27)], ids=["four_steps_per_lane", "one_step"])
def test_front_end_u_bf16_is_rounded_fp32(H, W):
    """The conv and SiLU run in fp32 for both data types; u is rounded once.  (dt_raw, Bs and
    Cs are not compared: x_proj multiplies split bf16 operands for bfloat16 data and fp32
    operands for fp32 data.)"""
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(2, 70, H, W, 8, 4, "bf16")
    log(f"case front-end rounding {H}x{W}")
    bf, f32 = _pair(wl, 54)
    w = workloads.make_front_weights(wl, 54, R=2, KW=4)
    fw = [torch.from_numpy(w[k]).cuda() for k in ("conv_w", "conv_b", "x_proj_w", "dt_proj_w")]
    o_bf = ss.ss2d_project(bf["x"], *fw)
    o_32 = ss.ss2d_project(f32["x"], *fw)
    torch.cuda.synchronize()
    assert_rounded(o_bf["u"], o_32["u"], "u")
