"""CPU evidence for the front end's fp32 parity bars (no GPU, no library).

A plain fp32 front end -- causal conv and SiLU rounded once per output, x_proj and dt_proj as
sequential fp32 fused multiply-adds -- is compared with the float64 oracle on the GPU suite's
own fp32 cases with R = 3 dt rows, with its channel sum taken in a few fixed orders.  x_proj's
B and C rows and u stay within the forward bar 1e-4 in every order; dt_raw, which combines R
D-term fp32 sums with either sign, crosses 1e-4 on entries that cancel below the metric's
1% floor for some orders, and stays within 2e-4.  This is the measurement behind the two
fp32 bars of the front-end GPU tests (1e-4 for u, B, C, the dt rows and the chained
forward; 2e-4 for dt_raw).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL_DT_RAW, TOL_FRONT, parity_error

F32 = np.float32
FRONT = ("conv_w", "conv_b", "x_proj_w", "dt_proj_w")


def fma(a, b, c):
    """fp32 fused multiply-add: the fp32 product is exact in float64, one rounding."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F32)


def route_sequences(x, K, H, W):
    B, D = x.shape[:2]
    flat = x.reshape(B, D, H * W)
    seqs = [flat, flat[..., ::-1]]
    if K == 4:
        cols = x.reshape(B, D, H, W).transpose(0, 1, 3, 2).reshape(B, D, H * W)
        seqs += [cols, cols[..., ::-1]]
    return [np.ascontiguousarray(s) for s in seqs]


def front_fp32(x, w, K, H, W, order):
    """Conv + SiLU, x_proj (channels summed in `order`), dt_proj, all in fp32."""
    cw, cb, xw, dw = (w[k].astype(F32) for k in FRONT)
    B, D = x.shape[:2]
    L, KW, R, M = H * W, cw.shape[-1], dw.shape[-1], xw.shape[1]
    N = (M - R) // 2
    out = {k: [] for k in ("u", "dt_raw", "Bs", "Cs")}
    for k, s in enumerate(route_sequences(x.astype(F32), K, H, W)):
        pad = np.concatenate([np.zeros((B, D, KW - 1), F32), s], axis=-1)
        v = np.broadcast_to(cb[k][None, :, None], (B, D, L)).astype(F32)
        for j in range(KW):
            v = fma(np.broadcast_to(cw[k][None, :, j, None], v.shape), pad[..., j:j + L], v)
        v64 = v.astype(np.float64)
        u = (v64 / (1.0 + np.exp(-v64))).astype(F32)  # SiLU, rounded once
        xd = np.zeros((B, M, L), F32)
        for d in order:
            xd = fma(np.broadcast_to(xw[k][None, :, d, None], xd.shape),
                     np.broadcast_to(u[:, d][:, None, :], xd.shape), xd)
        dt = np.zeros((B, D, L), F32)
        for r in range(R):
            dt = fma(np.broadcast_to(dw[k][None, :, r, None], dt.shape),
                     np.broadcast_to(xd[:, r][:, None, :], dt.shape), dt)
        for key, val in (("u", u), ("dt_raw", dt), ("Bs", xd[:, R:R + N]),
                         ("Cs", xd[:, R + N:])):
            out[key].append(val)
    return {k: np.stack(v, axis=1) for k, v in out.items()}


# (B, D, H, W, N, K, R, KW), the permutation seed of a channel order found to carry dt_raw
# past 1e-4
CASES = [((2, 70, 6, 10, 4, 4, 3, 4), 7), ((2, 70, 5, 27, 4, 4, 3, 4), 56)]


@pytest.mark.parametrize("case,perm_seed", CASES, ids=["6x10", "5x27"])
def test_plain_fp32_front_end_reaches_the_dt_raw_bar(case, perm_seed):
    B, D, H, W, N, K, R, KW = case
    wl = workloads.custom(B, D, H, W, N, K, "f32")
    inp = workloads.make_inputs(wl, seed=31)  # the GPU suite's inputs for these shapes
    w = workloads.make_front_weights(wl, 31, R=R, KW=KW)
    ref = oracle.Oracle().project(K, inp["x"], *[w[k] for k in FRONT])
    orders = {"channel order": np.arange(D), "reversed": np.arange(D)[::-1],
              f"permutation {perm_seed}": np.random.default_rng(perm_seed).permutation(D)}
    worst_dt = 0.0
    for name, order in orders.items():
        got = front_fp32(inp["x"], w, K, H, W, order)
        err = {k: parity_error(got[k], ref[k])["gate"] for k in got}
        for k in ("u", "Bs", "Cs"):
            assert err[k] <= TOL_FRONT["f32"], (name, k, err[k])
        assert err["dt_raw"] <= TOL_DT_RAW["f32"], (name, err["dt_raw"])
        worst_dt = max(worst_dt, err["dt_raw"])
    # a correct fp32 implementation does not meet 1e-4 on dt_raw in every summation order
    assert worst_dt > 1e-4, worst_dt
