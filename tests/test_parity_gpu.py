"""GPU parity of the HIP path (through the C ABI) against the float64 CPU oracle.

Element-by-element on sizes the oracle finishes in seconds (ragged channel counts, odd and
non-square maps, every supported state size, every launch variant forced through the
plan overrides); at the full benchmark sizes, every output element, in the launch
configuration the benchmark times.  Plus determinism, NaN propagation, streams, empty
inputs and argument errors.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (TOL, assert_parity, plan_override, log, parity_error, run_gpu,
                            to_device, to_numpy_f64)

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def oracle_full(orc, inp, wl):
    return orc.forward(wl.K, *[inp[k] for k in ARGS])


def check_case(orc, wl, a_log="init", seed=0, what=None, **overrides):
    what = what or f"{wl.name} B{wl.B} D{wl.D} {wl.H}x{wl.W} N{wl.N} K{wl.K} {wl.dtype}"
    log(f"case {what} a_log={a_log} overrides={overrides}")
    inp = workloads.make_inputs(wl, seed=seed, a_log=a_log)
    ref = oracle_full(orc, inp, wl)
    dev = to_device(inp, wl)
    import torch
    with plan_override(**overrides):
        y = run_gpu(dev, wl)
    torch.cuda.synchronize()
    return assert_parity(to_numpy_f64(y), ref, wl.dtype, what)


# ---- the tiny workload, whole output -------------------------------------------------
def test_tiny_workload(orc):
    check_case(orc, workloads.workload("tiny_f32"))


# ---- small shapes: ragged channels, odd / non-square maps, every N, both dtypes -------
SMALL = [
    # B, D, H, W, N, dtype
    (2, 70, 5, 7, 16, "f32"),
    (2, 70, 5, 7, 16, "bf16"),
    (1, 33, 3, 5, 1, "f32"),
    (1, 33, 1, 7, 2, "f32"),
    (1, 33, 7, 1, 8, "bf16"),
    (1, 20, 4, 6, 32, "f32"),
    (1, 20, 4, 6, 32, "bf16"),
    (3, 64, 17, 19, 16, "f32"),
    (2, 130, 24, 24, 16, "bf16"),
    (2, 130, 24, 24, 4, "f32"),
    (1, 1, 2, 2, 16, "f32"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}D{}_{}x{}_N{}_{}".format(*c))
def test_small_shapes(orc, case):
    B, D, H, W, N, dt = case
    check_case(orc, workloads.custom(B, D, H, W, N, 4, dt), a_log="random", seed=7)


# ---- every launch variant: lanes per channel and chunked scans ----------------------
VARIANTS = [dict(split=s, chunk_len=0) for s in (1, 2, 4)] + [
    dict(split=sp, chunk_len=c) for sp in (1, 4) for c in (32, 64, 96, 160)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: "S{}_C{}".format(
    v["split"], v["chunk_len"]))
def test_launch_variants(orc, dt, var):
    wl = workloads.custom(2, 130, 24, 24, 16, 4, dt)  # L = 576: vector loads, 3 waves/(b,k)
    check_case(orc, wl, a_log="random", seed=11, **var)
    wl = workloads.custom(2, 72, 13, 11, 16, 4, dt)   # L = 143: element loads, ragged tiles
    check_case(orc, wl, a_log="random", seed=12, **var)


# ---- bidirectional 1D variant ------------------------------------------------------
@pytest.mark.parametrize("case", [(3, 100, 197, 16, "bf16"), (2, 64, 320, 16, "f32"),
                                  (1, 65, 37, 8, "f32"), (2, 40, 64, 4, "bf16")],
                         ids=lambda c: "B{}D{}L{}N{}_{}".format(*c))
def test_bidir_small(orc, case):
    B, D, L, N, dt = case
    check_case(orc, workloads.custom(B, D, 1, L, N, 2, dt), a_log="random", seed=3)


@pytest.mark.parametrize("var", [dict(split=4, chunk_len=0),
                                 dict(split=1, chunk_len=0),
                                 dict(split=1, chunk_len=64),
                                 dict(split=4, chunk_len=96)],
                         ids=["S4", "S1", "S1_chunk64", "S4_chunk96"])
def test_bidir_variants(orc, var):
    check_case(orc, workloads.custom(2, 96, 1, 300, 16, 2, "bf16"), a_log="random", seed=5,
               **var)


# ---- full benchmark sizes, every output element, default launch plan ----------------
@pytest.mark.parametrize("name,a_log", [("tiny_f32", "init"),
                                        ("vmamba_t_stage1_f32", "init"),
                                        ("vmamba_t_stage1_bf16", "init"),
                                        ("vmamba_t_stage1_bf16", "random"),
                                        ("highres_1024px_bf16", "init"),
                                        ("vim_bidir_bf16", "init")])
def test_full_size(orc, name, a_log):
    """The whole output of every benchmark workload, in the launch plan the benchmark times,
    against the oracle's whole output (computed on all host cores)."""
    import torch
    wl = workloads.workload(name)
    log(f"case full-size {name} a_log={a_log}: generating inputs")
    inp = workloads.make_inputs(wl, seed=0, a_log=a_log)
    dev = to_device(inp, wl)
    log(f"case full-size {name}: GPU run")
    y = to_numpy_f64(run_gpu(dev, wl))
    torch.cuda.synchronize()
    del dev
    log(f"case full-size {name}: oracle")
    ref = oracle_full(orc, inp, wl)
    assert_parity(y, ref, wl.dtype, f"{name} a_log={a_log} (all {y.size} outputs)")


# ---- determinism -------------------------------------------------------------------
def test_bitwise_deterministic():
    import torch
    for wl in (workloads.workload("vmamba_t_stage1_bf16"),
               workloads.custom(2, 130, 24, 24, 16, 4, "f32")):
        log(f"case determinism {wl.name}")
        dev = to_device(workloads.make_inputs(wl, seed=2), wl)
        y1 = run_gpu(dev, wl).clone()
        y2 = run_gpu(dev, wl)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16 if wl.dtype == "bf16" else torch.int32),
                           y2.view(torch.int16 if wl.dtype == "bf16" else torch.int32))


# ---- non-finite propagation ---------------------------------------------------------
@pytest.mark.parametrize("where", ["dt_raw", "x"])
def test_nan_propagates_exactly_where_the_recurrence_carries_it(orc, where):
    import torch
    wl = workloads.custom(2, 70, 9, 13, 16, 4, "f32")
    inp = workloads.make_inputs(wl, seed=4)
    if where == "dt_raw":
        inp["dt_raw"][1, 2, 5, 40] = np.nan   # route 2, step 40 onward of channel (1, 5)
    else:
        inp["x"][0, 3, 4, 6] = np.nan          # every route of channel (0, 3) from its visit
    log(f"case NaN in {where}")
    ref = oracle_full(orc, inp, wl)
    y = to_numpy_f64(run_gpu(to_device(inp, wl), wl))
    torch.cuda.synchronize()
    assert np.array_equal(np.isnan(y), np.isnan(ref)), "NaN pattern differs from the oracle"
    assert np.isnan(ref).any() and not np.isnan(ref).all()
    ok = ~np.isnan(ref)
    e = parity_error(y[ok], ref[ok])
    assert e["gate"] <= TOL["f32"], e


# ---- streams, preallocated output, empty input, errors ------------------------------
def test_side_stream_and_preallocated_output(orc):
    import torch
    wl = workloads.custom(2, 64, 12, 10, 16, 4, "bf16")
    inp = workloads.make_inputs(wl, seed=9)
    ref = oracle_full(orc, inp, wl)
    dev = to_device(inp, wl)
    y = torch.full(tuple(dev["x"].shape), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = run_gpu(dev, wl, y=y)
    s.synchronize()
    assert out.data_ptr() == y.data_ptr()
    assert_parity(to_numpy_f64(y), ref, "bf16", "side stream")


def test_empty_batch():
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(1, 8, 4, 4, 4, 4, "f32")
    dev = to_device(workloads.make_inputs(wl), wl)
    empty = {k: (v[:0] if k in ("x", "dt_raw", "Bs", "Cs") else v) for k, v in dev.items()}
    y = ss.ss2d_forward(*[empty[k] for k in ARGS])
    torch.cuda.synchronize()
    assert y.shape == (0, 8, 4, 4)


def test_output_aliasing_input_is_rejected():
    import torch
    import selective_scan_ss2d_amd as ss
    wl = workloads.custom(1, 8, 4, 4, 4, 4, "f32")
    dev = to_device(workloads.make_inputs(wl), wl)
    with pytest.raises(ss.SS2DError) as ei:
        ss.ss2d_forward(*[dev[k] for k in ARGS], y=dev["x"])
    assert ei.value.status == ss.SS2D_ERR_ALIAS
    torch.cuda.synchronize()
