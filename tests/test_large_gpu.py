"""Offsets past 2^32 bytes: the benchmark batch (64 images of VMamba-T stage 1, bf16) tiled
seven times, 448 images.  The forward's fp32 per-route outputs are then 4.3 GiB, as are the
backward's fp32 per-route input gradients, so the last images' rows lie beyond every 32-bit
byte offset; dt_raw (2.2 GB) and the image tensors come close to 2^31 bytes.  Images are
independent and both batches run the same launch plan (four lanes per channel, one pass), so
every image of the large batch must reproduce its copy in the 64-image batch bit for bit:
the forward output, the gated output, and the per-image gradients (x, dt_raw, Bs, Cs).  The
parameter gradients sum over images, in a different association: within fp32 rounding of
seven times the 64-image sums.  The 64-image results themselves are checked against the
oracle elsewhere (the full-size parity tests)."""
import numpy as np
import pytest

import workloads
from tests.gpu_util import log, to_device

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
DATA = ("x", "dt_raw", "Bs", "Cs")
COPIES = 7


def _bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16 if t.dtype == torch.bfloat16
                                        else torch.int32)


def _tiled(dev):
    return {k: (v.repeat(COPIES, *([1] * (v.dim() - 1))) if k in DATA else v)
            for k, v in dev.items()}


def _assert_copies_equal(big, small, what):
    import torch
    B = small.shape[0]
    sb = _bits(small)
    bb = _bits(big)
    for i in range(COPIES):
        same = torch.equal(bb[i * B:(i + 1) * B], sb)
        assert same, f"{what}: copy {i} of the batch differs from the 64-image result"
    log(f"  {what}: {COPIES} copies of {tuple(small.shape)} bit-identical")


def test_forward_beyond_32bit_offsets():
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.workload("vmamba_t_stage1_bf16")
    log(f"case large forward: {COPIES} x {wl.B} images")
    dev = to_device(workloads.make_inputs(wl, seed=71), wl)
    g = workloads.make_gate(wl, 71)
    z = torch.from_numpy(g["z_bf16"].view(np.int16)).view(torch.bfloat16).to("cuda:0")
    y_small = ss.ss2d_forward(*[dev[k] for k in ARGS])
    yz_small = ss.ss2d_forward_ex(*[dev[k] for k in ARGS], z=z)
    big = _tiled(dev)
    zb = z.repeat(COPIES, 1, 1, 1)
    y_big = ss.ss2d_forward(*[big[k] for k in ARGS])
    yz_big = ss.ss2d_forward_ex(*[big[k] for k in ARGS], z=zb)
    torch.cuda.synchronize()
    _assert_copies_equal(y_big, y_small, "y")
    _assert_copies_equal(yz_big, yz_small, "gated y")


def test_backward_beyond_32bit_offsets():
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.workload("vmamba_t_stage1_bf16")
    log(f"case large backward: {COPIES} x {wl.B} images")
    dev = to_device(workloads.make_inputs(wl, seed=72), wl)
    dy = torch.from_numpy(workloads.make_output_grad(wl, 72)["dy_bf16"].view(np.int16)).view(
        torch.bfloat16).to("cuda:0")
    small = ss.ss2d_backward(*[dev[k] for k in ARGS], dy)
    torch.cuda.synchronize()
    small = {k: v.clone() for k, v in small.items()}
    big_in = _tiled(dev)
    big = ss.ss2d_backward(*[big_in[k] for k in ARGS], dy.repeat(COPIES, 1, 1, 1))
    torch.cuda.synchronize()
    for name in DATA:  # per-image gradients
        _assert_copies_equal(big[name], small[name], f"d{name}")
    for name in ("A_log", "Ds", "dt_bias"):  # sums over images
        got = big[name].double().cpu().numpy()
        want = COPIES * small[name].double().cpu().numpy()
        scale = np.abs(want).max()
        err = np.abs(got - want).max() / scale
        log(f"  d{name}: max |big - {COPIES} small| / max|.| = {err:.2e}")
        assert err < 1e-6, (name, err)
