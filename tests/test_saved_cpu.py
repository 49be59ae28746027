"""CPU tests of the training entry points' host side (no GPU: nothing here launches a
kernel): the saved-state size, and the argument checks of ss2d_forward_save and
ss2d_backward_saved, which all run before the library touches the HIP runtime (fake,
never dereferenced pointers, as in tests/test_abi_cpu.py)."""
import os

import pytest

from selective_scan_ss2d_amd import _binding as bnd


@pytest.fixture(scope="module")
def lib():
    other = os.environ.get("SS2D_TEST_LIBRARY")
    if other:
        return bnd.load_library(other)
    if not bnd.LIBRARY_PATH.exists():
        from selective_scan_ss2d_amd import build
        build.build()
    return bnd.load_library()


def fake_ptrs(n, base=1 << 40, gap=1 << 32):
    return [base + i * gap for i in range(n)]


@pytest.mark.parametrize("K,B,D,L,N", [(4, 64, 192, 3136, 16), (2, 128, 768, 197, 16),
                                       (4, 1, 8, 64, 4), (4, 3, 5, 33, 32), (2, 2, 1, 1, 8)])
def test_saved_state_bytes(lib, K, B, D, L, N):
    slots = (L + 7) // 8  # the state before every 8-step quarter, fp32
    ck = B * K * D * slots * N * 4
    assert lib.ss2d_saved_state_bytes(K, B, D, L, N, 0) == ck
    assert lib.ss2d_saved_state_bytes(K, B, D, L, N, 1) == ck + B * D * L * 4  # + route sum


@pytest.mark.parametrize("K,B,D,L,N", [(3, 1, 8, 64, 4), (4, 1, 8, 64, 2), (4, 1, 8, 64, 1),
                                       (4, 1, 8, 64, 12), (4, 1, 8, 0, 4), (4, -1, 8, 64, 4),
                                       (4, 1, 8, 1 << 30, 4)])
def test_saved_state_bytes_rejects(lib, K, B, D, L, N):
    assert lib.ss2d_saved_state_bytes(K, B, D, L, N, 0) == -1


def fwd_save(lib, p, N=4, B=1, D=8, H=8, W=8, dtype=0, flags=0):
    return lib.ss2d_forward_save(*p, B, D, H, W, N, dtype, flags, None)


def bwd_saved(lib, p, N=4, B=1, D=8, H=8, W=8, dtype=0, flags=0):
    return lib.ss2d_backward_saved(*p, B, D, H, W, N, dtype, flags, None)


# forward_save: x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, saved
def test_forward_save_checks(lib):
    p = fake_ptrs(10)
    q = list(p)
    q[9] = None
    assert fwd_save(lib, q) == bnd.SS2D_ERR_NULL
    assert fwd_save(lib, p, N=2) == bnd.SS2D_ERR_UNSUPPORTED  # checkpoints need N % 4 == 0
    assert fwd_save(lib, p, N=1) == bnd.SS2D_ERR_UNSUPPORTED
    q = list(p)
    q[9] += 4  # fp32-aligned but not 16-byte aligned
    assert fwd_save(lib, q) == bnd.SS2D_ERR_ALIGN
    for i in range(9):  # the saved state inside any other argument
        q = list(p)
        q[9] = p[i] + 64
        assert fwd_save(lib, q) == bnd.SS2D_ERR_ALIAS, i
    q = list(p)
    q[7] = None  # no gate: fine
    import torch
    if not torch.cuda.is_available():  # past the checks a GPU would run the kernels
        assert fwd_save(lib, q) == bnd.SS2D_ERR_HIP
        assert fwd_save(lib, p) == bnd.SS2D_ERR_HIP
    assert lib.ss1d_bidir_forward_save(*p[:9], None, 2, 8, 16, 4, 0, 0, None) == \
        bnd.SS2D_ERR_NULL


# backward_saved: x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, saved, dy, then the outputs dx,
# ddt_raw, dA_log, dBs, dCs, dDs, ddt_bias, dz
def test_backward_saved_checks(lib):
    p = fake_ptrs(18)
    q = list(p)
    q[8] = None
    assert bwd_saved(lib, q) == bnd.SS2D_ERR_NULL
    assert bwd_saved(lib, p, N=2) == bnd.SS2D_ERR_UNSUPPORTED
    q = list(p)
    q[8] += 4
    assert bwd_saved(lib, q) == bnd.SS2D_ERR_ALIGN
    for i in range(10, 18):  # an output inside the saved state
        q = list(p)
        q[i] = p[8] + 64
        assert bwd_saved(lib, q) == bnd.SS2D_ERR_ALIAS, i
    import torch
    if not torch.cuda.is_available():
        assert bwd_saved(lib, p) == bnd.SS2D_ERR_HIP
    assert lib.ss1d_bidir_backward_saved(*p[:8], None, *p[9:], 2, 8, 16, 4, 0, 0, None) == \
        bnd.SS2D_ERR_NULL


def test_routes_pair_checks(lib):
    p = fake_ptrs(10)
    q = list(p)
    q[9] = None
    assert lib.ss2d_forward_routes_save(*q, 1, 8, 8, 8, 4, 0, 0, None) == bnd.SS2D_ERR_NULL
    q = list(p)
    q[9] = p[0] + (1 << 12)  # inside u, which holds K routes: 4x the image's bytes
    assert lib.ss2d_forward_routes_save(*q, 1, 8, 8, 8, 4, 0, 0, None) == bnd.SS2D_ERR_ALIAS
    p = fake_ptrs(18)
    assert lib.ss2d_backward_routes_saved(*p, 1, 8, 8, 8, 2, 0, 0, None) == \
        bnd.SS2D_ERR_UNSUPPORTED
    q = list(p)
    q[8] = None
    assert lib.ss1d_bidir_backward_routes_saved(*q, 2, 8, 16, 4, 0, 0, None) == \
        bnd.SS2D_ERR_NULL
