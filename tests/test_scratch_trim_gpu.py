"""ss2d_scratch_trim: after the calls' streams are synchronised, trimming the library's
scratch pool hands its memory back (the reserved bytes drop), a keep_bytes above what the
pool holds releases nothing, and the next call allocates again and gives the same output
bit for bit."""
import pytest

import selective_scan_ss2d_amd as ss
import workloads
from tests.gpu_util import log, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_trim_releases_pooled_scratch_and_calls_still_match():
    import torch
    # 4 images of the stage-1 map: ~39 MB of fp32 route outputs plus the transposed x
    wl = workloads.custom(4, 192, 56, 56, 16, 4, "bf16")
    log(f"case scratch trim {wl.B}x{wl.D} {wl.H}x{wl.W} N{wl.N} {wl.dtype}")
    dev = to_device(workloads.make_inputs(wl, seed=31), wl)
    y0 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    held = ss.scratch_trim(1 << 62)  # keeps everything: reports what the pool holds
    route_bytes = wl.B * wl.K * wl.D * wl.H * wl.W * 4
    assert held >= route_bytes, (held, route_bytes)
    after = ss.scratch_trim(0)
    log(f"  pool reserved {held} bytes before the trim, {after} after")
    assert after < route_bytes, (held, after)
    assert ss.scratch_trim(0) == after  # nothing more to release
    y1 = run_gpu(dev, wl)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y0), _bits(y1))
    assert ss.scratch_trim(1 << 62) >= route_bytes
