"""CPU tests of the C ABI and the host-side logic (no GPU: nothing here launches a kernel).

Every argument error is detected before the library touches the HIP runtime, so the
status codes can be checked on a machine without a GPU, using fake (never dereferenced)
pointers.
"""
import ctypes
import os
import pathlib
import re
import subprocess

import numpy as np
import pytest

import workloads
from selective_scan_ss2d_amd import _binding as bnd

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "ss2d.h"


@pytest.fixture(scope="module")
def lib():
    # tests/test_sanitizers_cpu.py reruns this file against a build whose host code carries
    # AddressSanitizer and UBSan, named by SS2D_TEST_LIBRARY
    other = os.environ.get("SS2D_TEST_LIBRARY")
    if other:
        return bnd.load_library(other)
    if not bnd.LIBRARY_PATH.exists():
        from selective_scan_ss2d_amd import build
        build.build()
    return bnd.load_library()


def header_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    fns = header_functions()
    for name in ("ss2d_forward", "ss1d_bidir_forward", "ss2d_status_string",
                 "ss2d_abi_version", "ss2d_last_hip_error"):
        assert name in fns, name
    assert set(fns) == set(bnd.SIGNATURES), "binding signatures and header disagree"


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(bnd.LIBRARY_PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in header_functions():
        assert name in exported, f"{name} is declared in ss2d.h but not exported"
        assert getattr(lib, name) is not None


def test_abi_version_and_status_strings(lib):
    assert lib.ss2d_abi_version() == 12
    seen = set()
    for code in range(8):
        s = lib.ss2d_status_string(code)
        assert s and s not in seen
        seen.add(s)
    assert lib.ss2d_status_string(99) == b"unknown status"


# Fake device addresses: 4 KiB apart, 256-byte aligned; validation never dereferences them.
def fake_ptrs(n=8, base=1 << 40, gap=1 << 32):
    return [base + i * gap for i in range(n)]


def call2d(lib, ptrs, B=1, D=8, H=8, W=8, N=4, dtype=0):
    return lib.ss2d_forward(*ptrs, B, D, H, W, N, dtype, None)


def test_null_pointers_rejected(lib):
    ptrs = fake_ptrs()
    for i in range(8):
        p = list(ptrs)
        p[i] = None
        assert call2d(lib, p) == bnd.SS2D_ERR_NULL
        assert lib.ss1d_bidir_forward(*p, 2, 8, 16, 4, 0, None) == bnd.SS2D_ERR_NULL


@pytest.mark.parametrize("dims", [(-1, 8, 8, 8), (1, -2, 8, 8), (1, 8, 0, 8), (1, 8, 8, 0),
                                  (1, 8, 1 << 15, 1 << 15), (1 << 40, 1 << 20, 64, 64)])
def test_bad_shapes_rejected(lib, dims):
    B, D, H, W = dims
    assert call2d(lib, fake_ptrs(), B, D, H, W) == bnd.SS2D_ERR_SHAPE


@pytest.mark.parametrize("N", [0, -4])
def test_nonpositive_state_rejected(lib, N):
    assert call2d(lib, fake_ptrs(), N=N) == bnd.SS2D_ERR_SHAPE


@pytest.mark.parametrize("N", [3, 5, 12, 64])
def test_unsupported_state_size(lib, N):
    assert call2d(lib, fake_ptrs(), N=N) == bnd.SS2D_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", [-1, 2, 7])
def test_unsupported_dtype(lib, dtype):
    assert call2d(lib, fake_ptrs(), dtype=dtype) == bnd.SS2D_ERR_UNSUPPORTED


def test_empty_batch_or_channels_is_a_no_op(lib):
    nulls = [None] * 8
    assert call2d(lib, nulls, B=0) == bnd.SS2D_OK
    assert call2d(lib, nulls, D=0) == bnd.SS2D_OK
    assert lib.ss1d_bidir_forward(*nulls, 0, 8, 16, 4, 1, None) == bnd.SS2D_OK


def test_misaligned_pointers_rejected(lib):
    for i in range(8):
        p = fake_ptrs()
        p[i] += 1  # odd address: misaligned for fp32 and bf16 data and fp32 parameters
        assert call2d(lib, p, dtype=0) == bnd.SS2D_ERR_ALIGN
    p = fake_ptrs()
    p[0] += 2  # 2-byte aligned x is fine for bf16 but not for fp32
    assert call2d(lib, p, dtype=0) == bnd.SS2D_ERR_ALIGN
    import torch
    if not torch.cuda.is_available():  # past validation a GPU would run the kernels
        assert call2d(lib, p, dtype=1) == bnd.SS2D_ERR_HIP


def test_output_aliasing_an_input_rejected(lib):
    for i in range(7):
        p = fake_ptrs()
        p[7] = p[i] + 64  # y starts inside input i
        assert call2d(lib, p) == bnd.SS2D_ERR_ALIAS, i


# ---- the entry points with a gate and the zero-order-hold flag -----------------------------
def call2d_ex(lib, ptrs, z, flags=0, B=1, D=8, H=8, W=8, N=4, dtype=0):
    return lib.ss2d_forward_ex(*ptrs[:7], z, ptrs[7], B, D, H, W, N, dtype, flags, None)


def call1d_ex(lib, ptrs, z, flags=0, B=1, D=8, L=16, N=4, dtype=0):
    return lib.ss1d_bidir_forward_ex(*ptrs[:7], z, ptrs[7], B, D, L, N, dtype, flags, None)


def test_ex_unknown_flags_rejected(lib):
    z = (1 << 40) + 9 * (1 << 32)
    for flags in (2, 4, -1, 1 << 20):
        assert call2d_ex(lib, fake_ptrs(), z, flags) == bnd.SS2D_ERR_UNSUPPORTED
        assert call1d_ex(lib, fake_ptrs(), z, flags) == bnd.SS2D_ERR_UNSUPPORTED


def test_ex_null_inputs_rejected_but_null_gate_allowed(lib):
    z = (1 << 40) + 9 * (1 << 32)
    for i in range(8):
        p = fake_ptrs()
        p[i] = None
        assert call2d_ex(lib, p, z) == bnd.SS2D_ERR_NULL
        assert call1d_ex(lib, p, z, bnd.SS2D_FLAG_ZOH) == bnd.SS2D_ERR_NULL
    import torch
    if not torch.cuda.is_available():  # a NULL gate is valid: the call reaches the runtime
        assert call2d_ex(lib, fake_ptrs(), None, bnd.SS2D_FLAG_ZOH) == bnd.SS2D_ERR_HIP
        assert call1d_ex(lib, fake_ptrs(), None) == bnd.SS2D_ERR_HIP


def test_ex_gate_alignment_and_aliasing(lib):
    z = (1 << 40) + 9 * (1 << 32)
    assert call2d_ex(lib, fake_ptrs(), z + 1) == bnd.SS2D_ERR_ALIGN
    assert call2d_ex(lib, fake_ptrs(), z + 2, dtype=0) == bnd.SS2D_ERR_ALIGN
    p = fake_ptrs()
    assert call2d_ex(lib, p, p[7] + 128) == bnd.SS2D_ERR_ALIAS        # gate inside y
    assert call1d_ex(lib, p, p[7] - 64, dtype=1) == bnd.SS2D_ERR_ALIAS  # y starts inside z
    assert call2d_ex(lib, [None] * 8, None, B=0) == bnd.SS2D_OK


# ---- backward entry points ----------------------------------------------------------------
def call_bwd(lib, ptrs, B=1, D=8, H=8, W=8, N=4, dtype=0, K=4):
    if K == 4:
        return lib.ss2d_backward(*ptrs, B, D, H, W, N, dtype, None)
    return lib.ss1d_bidir_backward(*ptrs, B, D, H * W, N, dtype, None)


def test_backward_argument_errors(lib):
    ptrs = fake_ptrs(15)
    for K in (4, 2):
        for i in range(15):
            p = list(ptrs)
            p[i] = None
            assert call_bwd(lib, p, K=K) == bnd.SS2D_ERR_NULL, (K, i)
        for N in (3, 5, 64, 12):
            assert call_bwd(lib, ptrs, N=N, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        assert call_bwd(lib, ptrs, dtype=5, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        assert call_bwd(lib, ptrs, B=-1, K=K) == bnd.SS2D_ERR_SHAPE
        assert call_bwd(lib, [None] * 15, B=0, K=K) == bnd.SS2D_OK
        for i in range(15):
            p = list(ptrs)
            p[i] += 1
            assert call_bwd(lib, p, K=K) == bnd.SS2D_ERR_ALIGN, (K, i)
        for i in range(8, 15):  # an output inside an input, or inside another output
            p = list(ptrs)
            p[i] = p[i - 8] + 4
            assert call_bwd(lib, p, K=K) == bnd.SS2D_ERR_ALIAS, (K, i)
        p = list(ptrs)
        p[14] = p[8] + 128
        assert call_bwd(lib, p, K=K) == bnd.SS2D_ERR_ALIAS
    import torch
    if not torch.cuda.is_available():
        for N in (1, 2, 4, 8, 16, 32):
            assert call_bwd(lib, ptrs, N=N) == bnd.SS2D_ERR_HIP, N


def call_bwd_ex(lib, ptrs, B=1, D=8, H=8, W=8, N=4, dtype=0, K=4, flags=0):
    if K == 4:
        return lib.ss2d_backward_ex(*ptrs, B, D, H, W, N, dtype, flags, None)
    return lib.ss1d_bidir_backward_ex(*ptrs, B, D, H * W, N, dtype, flags, None)


def test_backward_ex_argument_errors(lib):
    # x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, dy | dx, ddt_raw, dA_log, dBs, dCs, dDs,
    # ddt_bias, dz
    ptrs = fake_ptrs(17)
    for K in (4, 2):
        for i in range(17):
            if i == 7:  # z = NULL: no gate
                continue
            p = list(ptrs)
            p[i] = None
            assert call_bwd_ex(lib, p, K=K) == bnd.SS2D_ERR_NULL, (K, i)
        for N in (3, 5, 64, 12):
            assert call_bwd_ex(lib, ptrs, N=N, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        assert call_bwd_ex(lib, ptrs, dtype=5, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        assert call_bwd_ex(lib, ptrs, B=-1, K=K) == bnd.SS2D_ERR_SHAPE
        assert call_bwd_ex(lib, [None] * 17, B=0, K=K) == bnd.SS2D_OK
        for i in range(17):
            p = list(ptrs)
            p[i] += 1
            assert call_bwd_ex(lib, p, K=K) == bnd.SS2D_ERR_ALIGN, (K, i)
        for i in range(9, 16):  # a gradient inside its input
            p = list(ptrs)
            p[i] = p[i - 9] + 4
            assert call_bwd_ex(lib, p, K=K) == bnd.SS2D_ERR_ALIAS, (K, i)
        for j in (7, 8, 9, 15):  # dz inside z, dy, dx or ddt_bias
            p = list(ptrs)
            p[16] = p[j] + 4
            assert call_bwd_ex(lib, p, K=K) == bnd.SS2D_ERR_ALIAS, (K, j)
        p = list(ptrs)
        p[9] = p[7] + 8  # dx inside z
        assert call_bwd_ex(lib, p, K=K) == bnd.SS2D_ERR_ALIAS
        for flags in (2, 3, -1):
            assert call_bwd_ex(lib, ptrs, K=K, flags=flags) == bnd.SS2D_ERR_UNSUPPORTED
        # without the gate, z and dz are not used: NULL is fine, so is a dz that would alias
        # or is misaligned
        p = list(ptrs)
        p[7] = None
        p[16] = p[0] + 1
        import torch
        if not torch.cuda.is_available():
            assert call_bwd_ex(lib, p, K=K) == bnd.SS2D_ERR_HIP
            assert call_bwd_ex(lib, p, K=K, flags=bnd.SS2D_FLAG_ZOH) == bnd.SS2D_ERR_HIP
    import torch
    if not torch.cuda.is_available():
        assert call_bwd_ex(lib, ptrs) == bnd.SS2D_ERR_HIP


def test_backward_routes_argument_errors(lib):
    # u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, dy | du, ddt_raw, dA_log, dBs, dCs, dDs,
    # ddt_bias, dz; u and du are (B, K, D, L)
    ptrs = fake_ptrs(17)
    for K in (4, 2):
        def call(p, **kw):
            B, D, H, W, N = kw.get("B", 1), 8, 8, 8, kw.get("N", 4)
            if K == 4:
                return lib.ss2d_backward_routes(*p, B, D, H, W, N, kw.get("dtype", 0),
                                                kw.get("flags", 0), None)
            return lib.ss1d_bidir_backward_routes(*p, B, D, H * W, N, kw.get("dtype", 0),
                                                  kw.get("flags", 0), None)
        for i in range(17):
            if i == 7:  # z = NULL: no gate
                continue
            p = list(ptrs)
            p[i] = None
            assert call(p) == bnd.SS2D_ERR_NULL, (K, i)
        assert call(ptrs, N=64) == bnd.SS2D_ERR_UNSUPPORTED
        assert call(ptrs, flags=2) == bnd.SS2D_ERR_UNSUPPORTED
        assert call(ptrs, B=-1) == bnd.SS2D_ERR_SHAPE
        assert call([None] * 17, B=0) == bnd.SS2D_OK
        for i in range(17):
            p = list(ptrs)
            p[i] += 1
            assert call(p) == bnd.SS2D_ERR_ALIGN, (K, i)
        # fp32: du (K * D * L elements) starting at u's last element, and u starting at
        # du's last route
        p = list(ptrs)
        p[9] = p[0] + 4 * (K * 8 * 64 - 1)
        assert call(p) == bnd.SS2D_ERR_ALIAS
        p = list(ptrs)
        p[0] = p[9] + 4 * (K - 1) * 8 * 64
        assert call(p) == bnd.SS2D_ERR_ALIAS


def test_backward_routes_binding_checks_steps_against_map():
    """The C entry point knows only H and W and takes rows of H * W steps; the binding must
    refuse a u whose rows are of another length before anything reaches the library."""
    import torch
    import selective_scan_ss2d_amd as ss
    B, K, D, N, H, W = 1, 4, 8, 4, 4, 5
    for L in (H * W - 1, H * W + 1):
        u = torch.zeros(B, K, D, L)
        dt = torch.zeros(B, K, D, L)
        bc = torch.zeros(B, K, N, L)
        A = torch.zeros(K, D, N)
        p = torch.zeros(K, D)
        dy = torch.zeros(B, D, H, W)
        with pytest.raises(ValueError, match="H \\* W"):
            ss.ss2d_backward_routes(u, dt, A, bc, bc, p, p, dy, H, W)
        with pytest.raises(ValueError, match="H \\* W"):
            ss.ss2d_forward_routes(u, dt, A, bc, bc, p, p, H, W)


def test_launch_plan_override_arguments(lib):
    """ss2d_set_launch_plan accepts split 0/1/2/4 and chunk_len >= -1 (below 2^30), rejects
    the rest without changing the setting, and the context manager restores automatic."""
    import selective_scan_ss2d_amd as ss
    for split in (0, 1, 2, 4):
        for chunk in (-1, 0, 32, 100):
            assert lib.ss2d_set_launch_plan(split, chunk) == bnd.SS2D_OK
    for split in (-1, 3, 8, 16):
        assert lib.ss2d_set_launch_plan(split, -1) == bnd.SS2D_ERR_UNSUPPORTED
    for chunk in (-2, 1 << 30):
        assert lib.ss2d_set_launch_plan(0, chunk) == bnd.SS2D_ERR_SHAPE
    assert lib.ss2d_set_launch_plan(0, -1) == bnd.SS2D_OK
    with pytest.raises(ss.SS2DError):
        with ss.launch_plan(3, 0):
            pass
    with ss.launch_plan(4, 64):
        pass


def test_noalloc_rejects_calls_beyond_its_scratch_before_any_hip_call(lib):
    """ss2d_forward_noalloc checks the scratch the plan needs against its fixed array
    before it touches the HIP runtime: on a machine without a GPU, a call that is too large
    returns SS2D_ERR_SCRATCH (not SS2D_ERR_HIP), and its argument errors are those of
    ss2d_forward_ex."""
    import torch
    ptrs = fake_ptrs(9)
    ptrs[7] = None  # no gate

    def call(B, D, H, W, N=16, dtype=bnd.SS2D_BF16, flags=0, p=ptrs):
        return lib.ss2d_forward_noalloc(*p, B, D, H, W, N, dtype, flags, None)
    assert call(64, 192, 56, 56) == bnd.SS2D_ERR_SCRATCH      # ~694 MB
    assert call(16, 192, 56, 56, dtype=bnd.SS2D_F32) == bnd.SS2D_ERR_SCRATCH
    assert call(1, 8, 8, 8, flags=2) == bnd.SS2D_ERR_UNSUPPORTED
    p = list(ptrs)
    p[0] = None
    assert call(1, 8, 8, 8, p=p) == bnd.SS2D_ERR_NULL
    assert call(0, 8, 8, 8) == bnd.SS2D_OK
    if not torch.cuda.is_available():  # within the limit the call reaches the runtime
        assert call(8, 192, 56, 56, dtype=bnd.SS2D_F32) == bnd.SS2D_ERR_HIP
    assert b"scratch" in lib.ss2d_status_string(bnd.SS2D_ERR_SCRATCH)


def test_library_reads_no_environment():
    """The launch plan is not steered by environment variables: the library's source holds
    no getenv."""
    for f in (ROOT / "selective_scan_ss2d_amd" / "csrc").iterdir():
        assert "getenv" not in f.read_text(), f.name


# ---- per-route front end and the operator over per-route inputs ---------------------------
def call_proj(lib, ptrs, B=1, D=8, H=8, W=8, N=4, R=2, KW=4, dtype=0, K=4):
    if K == 4:
        return lib.ss2d_project(*ptrs, B, D, H, W, N, R, KW, dtype, None)
    return lib.ss1d_bidir_project(*ptrs, B, D, H * W, N, R, KW, dtype, None)


def test_project_argument_errors(lib):
    ptrs = fake_ptrs(9)
    for K in (4, 2):
        for i in range(9):
            p = list(ptrs)
            p[i] = None
            assert call_proj(lib, p, K=K) == bnd.SS2D_ERR_NULL, (K, i)
        assert call_proj(lib, ptrs, KW=9, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        assert call_proj(lib, ptrs, R=65, N=16, K=K) == bnd.SS2D_ERR_UNSUPPORTED  # R + 2N > 96
        assert call_proj(lib, ptrs, dtype=2, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        for bad in (dict(KW=0), dict(R=0), dict(N=0), dict(B=-1), dict(H=0)):
            assert call_proj(lib, ptrs, K=K, **bad) == bnd.SS2D_ERR_SHAPE, bad
        assert call_proj(lib, [None] * 9, B=0, K=K) == bnd.SS2D_OK
        for i in range(9):
            p = list(ptrs)
            p[i] += 1
            assert call_proj(lib, p, K=K) == bnd.SS2D_ERR_ALIGN, (K, i)
        for i in range(5, 9):  # an output inside an input, or inside another output
            for j in range(0, i):
                p = list(ptrs)
                p[i] = p[j] + 4
                assert call_proj(lib, p, K=K) == bnd.SS2D_ERR_ALIAS, (K, i, j)
    import torch
    if not torch.cuda.is_available():
        assert call_proj(lib, ptrs) == bnd.SS2D_ERR_HIP
        assert call_proj(lib, ptrs, K=2, R=64, N=16) == bnd.SS2D_ERR_HIP  # R + 2N = 96
        assert call_proj(lib, ptrs, R=64, N=12, KW=8) == bnd.SS2D_ERR_HIP  # R + 2N = 88


def call_routes(lib, ptrs, z=None, flags=0, B=1, D=8, H=8, W=8, N=4, dtype=0, K=4):
    if K == 4:
        return lib.ss2d_forward_routes(*ptrs[:7], z, ptrs[7], B, D, H, W, N, dtype, flags,
                                       None)
    return lib.ss1d_bidir_forward_routes(*ptrs[:7], z, ptrs[7], B, D, H * W, N, dtype, flags,
                                         None)


def test_forward_routes_argument_errors(lib):
    z = (1 << 40) + 9 * (1 << 32)
    for K in (4, 2):
        for i in range(8):
            p = fake_ptrs()
            p[i] = None
            assert call_routes(lib, p, z, K=K) == bnd.SS2D_ERR_NULL, (K, i)
        assert call_routes(lib, fake_ptrs(), z, flags=2, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        assert call_routes(lib, fake_ptrs(), z, N=3, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        p = fake_ptrs()
        # y must not overlap u anywhere in its K planes per image (u is K times the size
        # of x): y placed after the first x-sized stretch of u still overlaps it
        p[7] = p[0] + 8 * 8 * 8 * 4 + 64
        assert call_routes(lib, p, z, K=K) == bnd.SS2D_ERR_ALIAS
        assert call_routes(lib, fake_ptrs(), fake_ptrs()[7] + 64, K=K) == bnd.SS2D_ERR_ALIAS
        assert call_routes(lib, [None] * 8, None, B=0, K=K) == bnd.SS2D_OK
    import torch
    if not torch.cuda.is_available():
        assert call_routes(lib, fake_ptrs(), None) == bnd.SS2D_ERR_HIP


def call_proj_lr(lib, ptrs, B=1, D=8, H=8, W=8, N=4, R=2, KW=4, dtype=0, K=4):
    if K == 4:
        return lib.ss2d_project_lr(*ptrs, B, D, H, W, N, R, KW, dtype, None)
    return lib.ss1d_bidir_project_lr(*ptrs, B, D, H * W, N, R, KW, dtype, None)


def test_project_lr_argument_errors(lib):
    # x, conv_w, conv_b, x_proj_w, then the outputs u, dt_lr, Bs, Cs
    ptrs = fake_ptrs(8)
    for K in (4, 2):
        for i in range(8):
            p = list(ptrs)
            p[i] = None
            assert call_proj_lr(lib, p, K=K) == bnd.SS2D_ERR_NULL, (K, i)
        assert call_proj_lr(lib, ptrs, KW=9, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        assert call_proj_lr(lib, ptrs, R=65, N=16, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        for bad in (dict(KW=0), dict(R=0), dict(N=0), dict(B=-1), dict(H=0)):
            assert call_proj_lr(lib, ptrs, K=K, **bad) == bnd.SS2D_ERR_SHAPE, bad
        assert call_proj_lr(lib, [None] * 8, B=0, K=K) == bnd.SS2D_OK
        for i in range(8):
            p = list(ptrs)
            p[i] += 1
            assert call_proj_lr(lib, p, K=K) == bnd.SS2D_ERR_ALIGN, (K, i)
        for i in range(4, 8):
            for j in range(0, i):
                p = list(ptrs)
                p[i] = p[j] + 4
                assert call_proj_lr(lib, p, K=K) == bnd.SS2D_ERR_ALIAS, (K, i, j)
        # dt_lr holds B * K * R * L elements: an output placed just past that is disjoint,
        # one placed inside it is not
        p = list(ptrs)
        p[6] = p[5] + 1 * K * 2 * 64 * 4 - 4
        assert call_proj_lr(lib, p, K=K) == bnd.SS2D_ERR_ALIAS
    import torch
    if not torch.cuda.is_available():
        assert call_proj_lr(lib, ptrs) == bnd.SS2D_ERR_HIP
        p = list(ptrs)
        p[6] = p[5] + 1 * 4 * 2 * 64 * 4
        assert call_proj_lr(lib, p) == bnd.SS2D_ERR_HIP


def call_routes_lr(lib, ptrs, z=None, flags=0, B=1, D=8, H=8, W=8, N=4, R=2, dtype=0, K=4):
    # ptrs: u, dt_lr, dt_w, A_log, Bs, Cs, Ds, dt_bias, y
    if K == 4:
        return lib.ss2d_forward_routes_lr(*ptrs[:8], z, ptrs[8], B, D, H, W, N, R, dtype,
                                          flags, None)
    return lib.ss1d_bidir_forward_routes_lr(*ptrs[:8], z, ptrs[8], B, D, H * W, N, R, dtype,
                                            flags, None)


def test_forward_routes_lr_argument_errors(lib):
    z = (1 << 40) + 10 * (1 << 32)
    for K in (4, 2):
        for i in range(9):
            p = fake_ptrs(9)
            p[i] = None
            assert call_routes_lr(lib, p, z, K=K) == bnd.SS2D_ERR_NULL, (K, i)
        for R in (0, 5, -1):
            assert call_routes_lr(lib, fake_ptrs(9), z, R=R, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        assert call_routes_lr(lib, fake_ptrs(9), z, N=3, K=K) == bnd.SS2D_ERR_UNSUPPORTED
        p = fake_ptrs(9)
        p[2] += 2  # dt_w is fp32
        assert call_routes_lr(lib, p, z, K=K) == bnd.SS2D_ERR_ALIGN
        for j in (1, 2):  # y inside dt_lr or dt_w
            p = fake_ptrs(9)
            p[8] = p[j] + 4
            assert call_routes_lr(lib, p, z, K=K) == bnd.SS2D_ERR_ALIAS, (K, j)
        assert call_routes_lr(lib, [None] * 9, None, B=0, K=K) == bnd.SS2D_OK
    import torch
    if not torch.cuda.is_available():
        for R in (1, 4):
            assert call_routes_lr(lib, fake_ptrs(9), None, R=R) == bnd.SS2D_ERR_HIP


def test_valid_call_without_gpu_reports_hip_error(lib):
    # With valid arguments the library reaches the HIP runtime; without a GPU that fails
    # cleanly with SS2D_ERR_HIP (no crash, nothing printed).
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call2d(lib, fake_ptrs()) == bnd.SS2D_ERR_HIP
    assert lib.ss2d_last_hip_error() != 0


def test_scratch_trim_without_gpu_fails_cleanly(lib):
    # No device: the HIP runtime call fails and the status says so; the reserved-bytes
    # output is written (0) whatever the outcome.
    import ctypes
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    reserved = ctypes.c_size_t(12345)
    assert lib.ss2d_scratch_trim(0, ctypes.byref(reserved)) == bnd.SS2D_ERR_HIP
    assert reserved.value == 0
    assert lib.ss2d_scratch_trim(0, None) == bnd.SS2D_ERR_HIP
    with pytest.raises(ValueError):
        bnd.scratch_trim(-1)


# ---- host logic: the input generator --------------------------------------------------
def test_bf16_rounding_is_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 2 ** -7 + 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                     -3.5, 65504.0, 3.4e38, np.inf, -np.inf, 0.0, -0.0, 1e-40], np.float32)
    got = workloads.round_bf16(vals)
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -3.5, 65536.0, np.inf, np.inf,
                     -np.inf, 0.0, -0.0], np.float32)
    assert np.array_equal(got[:11], want)
    assert np.signbit(got[10])
    nan = workloads.round_bf16(np.array([np.nan], np.float32))
    assert np.isnan(nan).all()
    # every bfloat16 pattern survives the round trip unchanged
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(workloads.f32_to_bf16_bits(f)[finite], bits[finite])


def test_workloads_are_seeded_and_shaped():
    wl = workloads.workload("tiny_f32")
    a = workloads.make_inputs(wl, seed=0)
    b = workloads.make_inputs(wl, seed=0)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (1, 8, 8, 8)
    assert a["dt_raw"].shape == (1, 4, 8, 64)
    assert a["Bs"].shape == (1, 4, 4, 64)
    assert np.allclose(a["A_log"][2, 5], np.log(np.arange(1, 5)))
    v = np.logaddexp(0.0, a["dt_bias"].astype(np.float64))  # softplus(dt_bias)
    assert (v > 0.99e-3).all() and (v < 0.1001).all()
    assert np.all(a["Ds"] == 1.0)


def test_bf16_workload_values_are_bf16_exact():
    wl = workloads.custom(B=1, D=4, H=3, W=5, N=4, dtype="bf16")
    inp = workloads.make_inputs(wl, seed=1)
    for k in ("x", "dt_raw", "Bs", "Cs"):
        assert np.array_equal(workloads.round_bf16(inp[k]), inp[k])
        assert np.array_equal(workloads.bf16_bits_to_f32(inp[k + "_bf16"]), inp[k])


def test_algorithmic_bytes_and_updates():
    # figures of the workload table: 21,248 B and 8,192 updates for the tiny case,
    # 513.86 MB and 2.466e9 updates for VMamba-T stage 1 in bf16
    tiny = workloads.workload(0)
    assert tiny.algorithmic_bytes() == 21248 and tiny.updates == 8192
    c2 = workloads.workload(2)
    assert abs(c2.algorithmic_bytes() / 1e6 - 513.86) < 0.01
    assert c2.updates == 64 * 4 * 192 * 3136 * 16
    assert workloads.workload(4).L == 197 and workloads.workload(4).K == 2
