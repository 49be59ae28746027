"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` handle and raises AssertionError when the handle
disagrees with the fact it checks.  ``test_oracle_pins.py`` runs them on the real oracle and
on deliberately broken copies of its source (each planted mistake must trip a pin).

What pins what:
  brute force       explicit sum over s of (prod of decays) * delta_s B_s u_s on tiny inputs
                    (the recurrence unrolled; the convolution form of the Vim summary, sec.
                    4.1, generalised to a time-varying decay)
  geometric         constant inputs: h_t = delta B u (1 - a^(t+1)) / (1 - a)
  convolve          time-invariant delta, B, C: y = u * Kbar with Kbar_j = C a^j delta B
                    (Vim summary, sec. 4.1), evaluated with numpy.convolve
  lfilter           N = 1: a first-order IIR filter, evaluated with scipy.signal.lfilter
  halving           A_log = log(log 2) and delta = 1 give a decay of exactly 1/2 per step
  small delta       delta -> 0: the state stays at zero and y = (sum_k D_k) x (the Chinese
                    VMamba article, sec. 2: a small step keeps the history)
  memoryless        a huge |A| forgets at once: y = delta <C_t, B_t> u + D u, with delta taken
                    from numpy.logaddexp (softplus) -- pins softplus and where dt_bias enters
  routes            integer-coded steps land on the positions the pages' array recipe gives
                    (flatten, flip, transpose-then-flatten, flip), on non-square maps
  flip              the reversed route equals the forward route run on the flipped input
  transpose, rot180 symmetries of the four routes under exchange of parameter sets
  linearity         y is linear in x for fixed delta, B, C
  channels          the sampled-channel entry point agrees with the full one
  gate              the optional gate against sigmoid written through tanh, z = 0, z = 40
  zoh exact         zero-order hold reproduces the exact solution of h' = A h + B u for inputs
                    held constant (Vim summary, sec. 4.1, defines the ZOH discretisation)
  backward fd       every gradient against central finite differences of the forward
  backward adjoint  <dy, y(v) - y(0)> = <grad, v> for the inputs y is affine in; dDs closed form
  backward gate     the gated output's gradients (z's included) against finite differences;
                    z = 0 and z = 40 reduce them to closed forms of the plain operator's
  backward zoh      the zero-order hold's gradients against finite differences (both sides
                    of the power series in delta A); A -> 0 reduces them to the plain ones
  backward routes   the operator over per-route inputs: fed the gathers of one x it gives
                    the plain backward exactly; its gradients against finite differences
  project impulse   a unit impulse through the per-route causal conv gives the reversed taps
                    on the KW steps from the one that visits it, the bias elsewhere
  project brute     numpy.convolve, scipy.special.expit and matrix products on tiny inputs
  project select    one-hot x_proj / dt_proj rows pick single channels: split order [dt|B|C]
                    and the weight layouts
  routes variant    per-route inputs: the gathered x reproduces the plain operator; four
                    different inputs give the route-order sum of single-route operators
  routes low rank   dt_proj folded in equals dt_raw = dt_w @ dt_lr (exact in fp32); the
                    front end without dt_proj returns x_proj's first R rows
"""
from __future__ import annotations

import math

import numpy as np
import scipy.signal

RNG_SEED = 1234


def _rng(salt: int) -> np.random.Generator:
    return np.random.default_rng(RNG_SEED + salt)


def _close(got, want, rtol, atol=0.0, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    bad = ~(err <= lim)
    if bad.any():
        worst = float(np.max(np.where(np.isnan(err), np.inf, err)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements off; worst "
                             f"|err|={worst:.3e}")


def _random_inputs(rng, B, K, D, N, L, xshape=None):
    x = rng.standard_normal(xshape or (B, D, L)).astype(np.float32)
    dt = (0.5 * rng.standard_normal((B, K, D, L))).astype(np.float32)
    Bs = rng.standard_normal((B, K, N, L)).astype(np.float32)
    Cs = rng.standard_normal((B, K, N, L)).astype(np.float32)
    A_log = rng.uniform(-0.5, 1.5, size=(K, D, N)).astype(np.float32)
    Ds = rng.standard_normal((K, D)).astype(np.float32)
    bias = rng.uniform(-3.0, -1.0, size=(K, D)).astype(np.float32)
    return x, dt, A_log, Bs, Cs, Ds, bias


def _softplus(z):
    return np.logaddexp(0.0, np.asarray(z, dtype=np.float64))


def _brute_force_scan(u, dt, bias, A_log, Bm, Cm, Dv):
    """One route in its own scan order, by the unrolled sum (pure Python loops)."""
    L = len(u)
    N = len(A_log)
    delta = [float(_softplus(float(dt[t]) + float(bias))) for t in range(L)]
    A = [-math.exp(float(A_log[n])) for n in range(N)]
    y = []
    for t in range(L):
        acc = 0.0
        for n in range(N):
            h = 0.0
            for s in range(t + 1):
                decay = 1.0
                for r in range(s + 1, t + 1):
                    decay *= math.exp(delta[r] * A[n])
                h += decay * delta[s] * float(Bm[n][s]) * float(u[s])
            acc += float(Cm[n][t]) * h
        y.append(acc + float(Dv) * float(u[t]))
    return np.array(y)


def _routes(H, W, K=4):
    """Position visited at each step of each route, built the way the pages' listings build
    the sequences: flatten row-major, flip it, transpose then flatten, flip that."""
    grid = np.arange(H * W).reshape(H, W)
    row = grid.reshape(-1)
    col = grid.T.reshape(-1)
    if K == 2:
        return [row, row[::-1]]
    return [row, row[::-1], col, col[::-1]]


# ---------------------------------------------------------------------------------------
def pin_brute_force(orc):
    rng = _rng(1)
    B, K, D, N, L = 2, 2, 3, 3, 9
    x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L)
    for keep in (0, 1):
        Cs2, Ds2 = Cs.copy(), Ds.copy()
        Cs2[:, 1 - keep] = 0.0
        Ds2[1 - keep] = 0.0
        y = orc.forward(2, x, dt, A_log, Bs, Cs2, Ds2, bias)
        want = np.zeros_like(y)
        for b in range(B):
            for d in range(D):
                order = np.arange(L) if keep == 0 else np.arange(L)[::-1]
                ys = _brute_force_scan(x[b, d, order], dt[b, keep, d], bias[keep, d],
                                       A_log[keep, d], Bs[b, keep], Cs2[b, keep], Ds2[keep, d])
                want[b, d, order] = ys
        _close(y, want, 1e-12, 1e-14, f"brute force, route {keep}")


def pin_geometric(orc):
    B, K, D, N, L = 1, 2, 2, 2, 40
    x = np.full((B, D, L), 0.75, np.float32)
    dt = np.full((B, K, D, L), -0.25, np.float32)
    bias = np.array([[-1.0, 0.5], [0.0, 0.0]], np.float32)
    A_log = np.array([[[0.0, 1.0], [-1.0, 0.5]]] * K, np.float32)
    Bs = np.empty((B, K, N, L), np.float32)
    Cs = np.empty((B, K, N, L), np.float32)
    Bs[:, :, 0], Bs[:, :, 1] = 1.5, -0.5
    Cs[:, :, 0], Cs[:, :, 1] = 0.25, 2.0
    Cs[:, 1] = 0.0
    Ds = np.array([[0.5, -1.0], [0.0, 0.0]], np.float32)
    y = orc.forward(2, x, dt, A_log, Bs, Cs, Ds, bias)
    t = np.arange(L)
    for d in range(D):
        delta = float(_softplus(-0.25 + float(bias[0, d])))
        want = np.full(L, float(Ds[0, d]) * 0.75)
        for n in range(N):
            a = math.exp(-delta * math.exp(float(A_log[0, d, n])))
            h = delta * float(Bs[0, 0, n, 0]) * 0.75 * (1.0 - a ** (t + 1)) / (1.0 - a)
            want = want + float(Cs[0, 0, n, 0]) * h
        _close(y[0, d], want, 1e-12, 0.0, f"geometric series, d={d}")


def pin_convolve(orc):
    rng = _rng(3)
    B, K, D, N, L = 1, 2, 2, 4, 50
    x = rng.standard_normal((B, D, L)).astype(np.float32)
    dt = np.zeros((B, K, D, L), np.float32)
    bias = np.array([[-2.0, -0.5], [0.0, 0.0]], np.float32)
    A_log = rng.uniform(-1.0, 1.0, size=(K, D, N)).astype(np.float32)
    bvec = rng.standard_normal(N).astype(np.float32)
    cvec = rng.standard_normal(N).astype(np.float32)
    Bs = np.broadcast_to(bvec[None, None, :, None], (B, K, N, L)).astype(np.float32)
    Cs = np.broadcast_to(cvec[None, None, :, None], (B, K, N, L)).astype(np.float32)
    Cs[:, 1] = 0.0
    Ds = np.array([[0.3, -0.7], [0.0, 0.0]], np.float32)
    y = orc.forward(2, x, dt, A_log, Bs, Cs, Ds, bias)
    j = np.arange(L)
    for d in range(D):
        delta = float(_softplus(float(bias[0, d])))
        kbar = np.zeros(L)
        for n in range(N):
            a = math.exp(-delta * math.exp(float(A_log[0, d, n])))
            kbar += float(cvec[n]) * a ** j * delta * float(bvec[n])
        kbar[0] += float(Ds[0, d])
        want = np.convolve(x[0, d].astype(np.float64), kbar)[:L]
        _close(y[0, d], want, 1e-11, 1e-13, f"convolution form, d={d}")


def pin_lfilter(orc):
    rng = _rng(4)
    B, K, D, N, L = 1, 2, 3, 1, 64
    x = rng.standard_normal((B, D, L)).astype(np.float32)
    dt = np.zeros((B, K, D, L), np.float32)
    bias = np.array([[-3.0, -1.0, 0.5], [0, 0, 0]], np.float32)
    A_log = np.array([[[-2.0], [0.0], [1.0]], [[0.0], [0.0], [0.0]]], np.float32)
    Bs = np.full((B, K, N, L), 1.25, np.float32)
    Cs = np.full((B, K, N, L), -0.5, np.float32)
    Cs[:, 1] = 0.0
    Ds = np.array([[0.0, 1.0, 2.0], [0, 0, 0]], np.float32)
    y = orc.forward(2, x, dt, A_log, Bs, Cs, Ds, bias)
    for d in range(D):
        delta = float(_softplus(float(bias[0, d])))
        a = math.exp(-delta * math.exp(float(A_log[0, d, 0])))
        h = scipy.signal.lfilter([delta * 1.25], [1.0, -a], x[0, d].astype(np.float64))
        want = -0.5 * h + float(Ds[0, d]) * x[0, d]
        _close(y[0, d], want, 1e-12, 1e-14, f"lfilter, d={d}")


def pin_halving(orc):
    B, K, D, N, L = 1, 2, 1, 1, 30
    x = np.zeros((B, D, L), np.float32)
    x[0, 0, 0] = 1.0
    # float32 cannot hold log(e - 1) or log(log 2) exactly; the expected values below use
    # the float32 numbers actually passed, and reduce to 2^-t up to that rounding.
    z = np.float32(math.log(math.e - 1.0))
    alog = np.float32(math.log(math.log(2.0)))
    dt = np.zeros((B, K, D, L), np.float32)
    bias = np.array([[z], [0.0]], np.float32)
    A_log = np.array([[[alog]], [[0.0]]], np.float32)
    Bs = np.ones((B, K, N, L), np.float32)
    Cs = np.ones((B, K, N, L), np.float32)
    Cs[:, 1] = 0.0
    Ds = np.zeros((K, D), np.float32)
    y = orc.forward(2, x, dt, A_log, Bs, Cs, Ds, bias)
    t = np.arange(L)
    _close(y[0, 0], 0.5 ** t, 5e-6, 0.0, "decay of one half per step")
    delta = math.log1p(math.exp(float(z)))
    a = math.exp(-delta * math.exp(float(alog)))
    _close(y[0, 0], delta * a ** t, 1e-13, 0.0, "impulse response")


def pin_small_delta(orc):
    rng = _rng(6)
    B, K, D, N, H, W = 2, 4, 3, 4, 3, 5
    L = H * W
    x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L, (B, D, H, W))
    dt[:] = -80.0
    y = orc.forward(4, x, dt, A_log, Bs, Cs, Ds, bias)
    want = Ds.astype(np.float64).sum(axis=0)[None, :, None, None] * x
    _close(y, want, 1e-13, 1e-30, "delta -> 0 gives (sum_k D_k) x")


def pin_memoryless(orc):
    rng = _rng(7)
    B, K, D, N, L = 2, 2, 3, 4, 11
    x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L)
    dt = rng.uniform(-3.0, 3.0, size=dt.shape).astype(np.float32)
    bias = rng.uniform(-1.0, 1.0, size=bias.shape).astype(np.float32)
    A_log[:] = 12.0  # |A| ~ 1.6e5: exp(delta * A) underflows to 0 for delta > 0.005
    y = orc.forward(2, x, dt, A_log, Bs, Cs, Ds, bias)
    want = np.zeros((B, D, L))
    routes = _routes(1, L, K=2)
    for k in range(K):
        delta = _softplus(dt[:, k].astype(np.float64) + bias[k][None, :, None])  # (B,D,L)
        cb = np.einsum("bnt,bnt->bt", Cs[:, k].astype(np.float64), Bs[:, k].astype(np.float64))
        pos = routes[k]
        u = x[:, :, pos].astype(np.float64)
        want[:, :, pos] += delta * cb[:, None, :] * u + Ds[k][None, :, None] * u
    _close(y, want, 1e-12, 1e-14, "memoryless limit")


def pin_routes(orc):
    for (H, W) in [(3, 5), (1, 7), (7, 1), (4, 6), (2, 2), (5, 3)]:
        L = H * W
        B, K, D, N = 1, 4, 1, 2
        x = np.ones((B, D, H, W), np.float32)
        dt = np.zeros((B, K, D, L), np.float32)
        bias = np.full((K, D), math.log(math.e - 1.0), np.float32)  # delta ~= 1
        A_log = np.full((K, D, N), 12.0, np.float32)  # forget at once
        Bs = np.zeros((B, K, N, L), np.float32)
        Cs = np.zeros((B, K, N, L), np.float32)
        Bs[:, :, 0, :] = 1.0
        scale = [1.0, 2.0 ** 6, 2.0 ** 12, 2.0 ** 18]  # exact in float32 times (t + 1)
        for k in range(K):
            Cs[0, k, 0, :] = scale[k] * (np.arange(L) + 1)
        Ds = np.zeros((K, D), np.float32)
        delta = float(_softplus(float(bias[0, 0])))
        routes = _routes(H, W)
        for active in range(K + 1):  # each route alone, then all four summed
            Cs2 = Cs.copy()
            if active < K:
                for k in range(K):
                    if k != active:
                        Cs2[:, k] = 0.0
            y = orc.forward(4, x, dt, A_log, Bs, Cs2, Ds, bias)
            want = np.zeros(L)
            for k in range(K):
                if active < K and k != active:
                    continue
                want[routes[k]] += delta * scale[k] * (np.arange(L) + 1)
            _close(y[0, 0].reshape(-1), want, 1e-12, 0.0, f"routes {H}x{W} active={active}")


def pin_flip(orc):
    rng = _rng(9)
    B, K, D, N, L = 2, 2, 2, 3, 13
    x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L)
    Cs1, Ds1 = Cs.copy(), Ds.copy()
    Cs1[:, 0] = 0.0
    Ds1[0] = 0.0
    y_rev = orc.forward(2, x, dt, A_log, Bs, Cs1, Ds1, bias)
    # route 1's parameters moved to route 0, run on the flipped sequence
    dt0, Bs0, Cs0 = dt.copy(), Bs.copy(), Cs1.copy()
    dt0[:, 0], Bs0[:, 0], Cs0[:, 0] = dt[:, 1], Bs[:, 1], Cs1[:, 1]
    Cs0[:, 1] = 0.0
    A0, D0, b0 = A_log.copy(), Ds1.copy(), bias.copy()
    A0[0], D0[0], b0[0] = A_log[1], Ds1[1], bias[1]
    D0[1] = 0.0
    y_fwd = orc.forward(2, np.ascontiguousarray(x[:, :, ::-1]), dt0, A0, Bs0, Cs0, D0, b0)
    _close(y_rev, y_fwd[:, :, ::-1], 1e-14, 1e-15, "reversed route == forward on flipped")


def _swap(a, pairs, axis):
    out = a.copy()
    for i, j in pairs:
        idx_i = [slice(None)] * a.ndim
        idx_j = [slice(None)] * a.ndim
        idx_i[axis], idx_j[axis] = i, j
        out[tuple(idx_i)] = a[tuple(idx_j)]
        out[tuple(idx_j)] = a[tuple(idx_i)]
    return out


def pin_transpose(orc):
    rng = _rng(10)
    B, K, D, N, H, W = 2, 4, 2, 3, 3, 5
    L = H * W
    x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L, (B, D, H, W))
    y = orc.forward(4, x, dt, A_log, Bs, Cs, Ds, bias)
    p = [(0, 2), (1, 3)]
    yt = orc.forward(4, np.ascontiguousarray(np.swapaxes(x, 2, 3)), _swap(dt, p, 1),
                     _swap(A_log, p, 0), _swap(Bs, p, 1), _swap(Cs, p, 1), _swap(Ds, p, 0),
                     _swap(bias, p, 0))
    _close(yt, np.swapaxes(y, 2, 3), 1e-12, 1e-13, "transpose symmetry")


def pin_rot180(orc):
    rng = _rng(11)
    B, K, D, N, H, W = 1, 4, 3, 2, 4, 3
    L = H * W
    x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L, (B, D, H, W))
    y = orc.forward(4, x, dt, A_log, Bs, Cs, Ds, bias)
    p = [(0, 1), (2, 3)]
    yr = orc.forward(4, np.ascontiguousarray(x[:, :, ::-1, ::-1]), _swap(dt, p, 1),
                     _swap(A_log, p, 0), _swap(Bs, p, 1), _swap(Cs, p, 1), _swap(Ds, p, 0),
                     _swap(bias, p, 0))
    _close(yr, y[:, :, ::-1, ::-1], 1e-12, 1e-13, "180-degree rotation symmetry")


def pin_linearity(orc):
    rng = _rng(12)
    B, K, D, N, H, W = 2, 4, 2, 3, 4, 4
    L = H * W
    x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L, (B, D, H, W))
    # dyadic values and power-of-two weights keep alpha*x1 + beta*x2 exact in float32
    x = (np.round(64 * x) / 64).astype(np.float32)
    x2 = (np.round(64 * rng.standard_normal(x.shape)) / 64).astype(np.float32)
    y1 = orc.forward(4, x, dt, A_log, Bs, Cs, Ds, bias)
    y2 = orc.forward(4, x2, dt, A_log, Bs, Cs, Ds, bias)
    x12 = (np.float32(0.5) * x + np.float32(-2.0) * x2).astype(np.float32)
    y12 = orc.forward(4, x12, dt, A_log, Bs, Cs, Ds, bias)
    _close(y12, 0.5 * y1 - 2.0 * y2, 1e-11, 1e-12, "linearity in x")


def pin_channels(orc):
    rng = _rng(13)
    B, K, D, N, H, W = 3, 4, 5, 2, 2, 3
    L = H * W
    x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L, (B, D, H, W))
    y = orc.forward(4, x, dt, A_log, Bs, Cs, Ds, bias)
    bi = np.array([0, 2, 1, 2])
    di = np.array([4, 0, 3, 3])
    ys = orc.forward_channels(4, x, dt, A_log, Bs, Cs, Ds, bias, bi, di)
    _close(ys, y[bi, di], 0.0, 0.0, "sampled channels")
    # a channel depends on its own inputs only
    x2 = x.copy()
    x2[1, 2] += 5.0
    y2 = orc.forward(4, x2, dt, A_log, Bs, Cs, Ds, bias)
    mask = np.ones((B, D), bool)
    mask[1, 2] = False
    _close(y2[mask], y[mask], 0.0, 0.0, "channel isolation")


def pin_gate(orc):
    """The gate multiplies every route's output, skip term included, by SiLU(z) at the image
    position: checked against the logistic function written through tanh,
    sigmoid(z) = (1 + tanh(z / 2)) / 2, and at z = 0 (output exactly zero) and z = 40
    (SiLU(z) = z to 1e-17)."""
    rng = _rng(14)
    for K, xshape in ((4, (2, 3, 4, 5)), (2, (2, 3, 7))):
        B, D = xshape[:2]
        L = int(np.prod(xshape[2:]))
        N = 4
        x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L, xshape)
        args = (K, x, dt, A_log, Bs, Cs, Ds, bias)
        y = orc.forward(*args)
        z = (2.0 * rng.standard_normal(xshape)).astype(np.float32)
        zd = z.astype(np.float64)
        _close(orc.forward(*args, z=z), y * zd * (1.0 + np.tanh(zd / 2.0)) / 2.0, 1e-12,
               1e-14, f"gate, K={K}")
        y0 = orc.forward(*args, z=np.zeros(xshape, np.float32))
        assert np.all(y0 == 0.0), "gate at z = 0"
        _close(orc.forward(*args, z=np.full(xshape, 40.0, np.float32)), 40.0 * y, 1e-14,
               1e-15, f"gate at z = 40, K={K}")
        # the gate is the same for every route: the same result whether z is read per route
        # or once; and it does not touch the plain path
        _close(orc.forward(*args, z=np.ones(xshape, np.float32)), y / (1.0 + math.exp(-1.0)),
               1e-13, 1e-15, f"gate at z = 1, K={K}")


def pin_zoh_exact(orc):
    """Zero-order hold is exact for inputs held constant over each step: with B_t, u and C
    constant in time and D = 0, route k's state after t steps is the solution of
    h' = A h + B u at time S_t = sum of its deltas, h_n = B_n u (exp(A_n S_t) - 1) / A_n,
    whatever the individual deltas are.  Checked for both routes of the 1D variant and for
    the four routes of a 2D map (constant x, so every route sees the same u)."""
    rng = _rng(15)
    for K, xshape in ((2, (1, 2, 60)), (4, (1, 2, 5, 6))):
        B, D = xshape[:2]
        L = int(np.prod(xshape[2:]))
        N = 4
        _, dt, A_log, _, _, _, bias = _random_inputs(rng, B, K, D, N, L, xshape)
        u0 = rng.uniform(0.5, 1.5, size=D).astype(np.float32)
        x = np.broadcast_to(u0[None, :, None], (B, D, L)).reshape(xshape).astype(np.float32)
        bconst = rng.standard_normal((B, K, N)).astype(np.float32)
        Bs = np.repeat(bconst[..., None], L, axis=-1).astype(np.float32)
        Cs = np.ones((B, K, N, L), np.float32)
        Ds = np.zeros((K, D), np.float32)
        got = orc.forward(K, x, dt, A_log, Bs, Cs, Ds, bias, zoh=True).reshape(B, D, L)
        want = np.zeros((B, D, L))
        routes = _routes(*(xshape[2:] if K == 4 else (1, L)), K=K)
        for d in range(D):
            for k in range(K):
                delta = _softplus(dt[0, k, d].astype(np.float64) + float(bias[k, d]))
                S = np.cumsum(delta)
                A = -np.exp(A_log[k, d].astype(np.float64))
                h = (bconst[0, k][:, None].astype(np.float64) * float(u0[d]) *
                     np.expm1(A[:, None] * S[None, :]) / A[:, None])
                want[0, d, routes[k]] += h.sum(axis=0)
        _close(got, want, 1e-11, 1e-13, f"zero-order hold, K={K}")
        # the plain path (delta * B) is not exact here
        plain = orc.forward(K, x, dt, A_log, Bs, Cs, Ds, bias).reshape(B, D, L)
        assert np.max(np.abs(plain - want)) > 1e-6 * np.max(np.abs(want)), "ZOH had no effect"


BWD_NAMES = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")


def pin_backward_fd(orc):
    """Every gradient of L = sum(dy * y), element by element, against central finite
    differences of the forward oracle (steps of 1e-3 relative, taken as the difference of the
    two float32 inputs actually used), on tiny inputs for both route sets."""
    rng = _rng(16)
    for K, xshape in ((4, (2, 2, 3, 4)), (2, (2, 2, 9))):
        B, D = xshape[:2]
        L = int(np.prod(xshape[2:]))
        N = 2
        args = list(_random_inputs(rng, B, K, D, N, L, xshape))
        dy = rng.standard_normal(xshape).astype(np.float32)
        got = orc.backward(K, *args, dy)

        def loss(a):
            return float(np.sum(orc.forward(K, *a) * dy.astype(np.float64)))

        for i, name in enumerate(BWD_NAMES):
            flat = args[i].reshape(-1)
            fd = np.empty(flat.size)
            for j in range(flat.size):
                base = float(flat[j])
                step = 1e-3 * max(1.0, abs(base))
                hi, lo = np.float32(base + step), np.float32(base - step)
                pert = [a.copy() for a in args]
                pert[i].reshape(-1)[j] = hi
                lp = loss(pert)
                pert[i].reshape(-1)[j] = lo
                lm = loss(pert)
                fd[j] = (lp - lm) / (float(hi) - float(lo))
            g = got[name].reshape(-1)
            scale = max(float(np.max(np.abs(fd))), 1e-12)
            err = float(np.max(np.abs(g - fd))) / scale
            assert err < 2e-5, f"d/d{name} (K={K}) differs from finite differences: {err:.2e}"


def pin_backward_adjoint(orc):
    """Exact identities of reverse mode: y is linear in x and affine in Bs, Cs and Ds, so
    <dy, y(v) - y(0)> = <dL/dinput, v> for any v (up to float64 rounding); and
    dDs[k, d] = sum over (b, l) of dy * x for every route k."""
    rng = _rng(17)
    for K, xshape in ((4, (2, 3, 5, 4)), (2, (2, 3, 23))):
        B, D = xshape[:2]
        L = int(np.prod(xshape[2:]))
        N = 4
        args = list(_random_inputs(rng, B, K, D, N, L, xshape))
        dy = rng.standard_normal(xshape).astype(np.float32)
        got = orc.backward(K, *args, dy)
        dyd = dy.astype(np.float64)
        for i, name in ((0, "x"), (3, "Bs"), (4, "Cs"), (5, "Ds")):
            v = rng.standard_normal(args[i].shape).astype(np.float32)
            with_v = list(args)
            with_v[i] = v
            zero = list(args)
            zero[i] = np.zeros_like(args[i])
            lhs = float(np.sum(dyd * (orc.forward(K, *with_v) - orc.forward(K, *zero))))
            rhs = float(np.sum(got[name] * v.astype(np.float64)))
            assert abs(lhs - rhs) <= 1e-10 * max(abs(lhs), 1.0), \
                f"adjoint identity for {name} (K={K}): {lhs} vs {rhs}"
        want = np.einsum("bdl,bdl->d", dyd.reshape(B, D, L),
                         args[0].astype(np.float64).reshape(B, D, L))
        _close(got["Ds"], np.broadcast_to(want, (K, D)), 1e-12, 1e-13, f"dDs closed form, K={K}")


def pin_backward_gate(orc):
    """Gradients of the gated output sum(dy * y * SiLU(z)): every input's, z's included,
    element by element against central finite differences of the gated forward oracle; and
    two closed forms against the plain operator's own (separately pinned) forward and
    backward: at z = 0 (SiLU = 0, SiLU' = 1/2) every input's gradient is exactly zero and
    dz = dy y / 2; at z = 40 (SiLU(z) = 40 and SiLU'(z) = 1 in double) the gradients are 40
    times the plain ones and dz = dy y."""
    rng = _rng(18)
    for K, xshape in ((4, (1, 2, 3, 4)), (2, (2, 2, 7))):
        B, D = xshape[:2]
        L = int(np.prod(xshape[2:]))
        N = 2
        args = list(_random_inputs(rng, B, K, D, N, L, xshape))
        dy = rng.standard_normal(xshape).astype(np.float32)
        z = (1.5 * rng.standard_normal(xshape)).astype(np.float32)
        got = orc.backward(K, *args, dy, z=z)
        dyd = dy.astype(np.float64)

        def loss(a, zz):
            return float(np.sum(orc.forward(K, *a, z=zz) * dyd))

        names = BWD_NAMES + ("z",)
        for i, name in enumerate(names):
            base_arr = z if name == "z" else args[i]
            flat = base_arr.reshape(-1)
            fd = np.empty(flat.size)
            for j in range(flat.size):
                base = float(flat[j])
                step = 1e-3 * max(1.0, abs(base))
                hi, lo = np.float32(base + step), np.float32(base - step)
                vals = []
                for v in (hi, lo):
                    pert = [a.copy() for a in args]
                    zz = z.copy()
                    (zz if name == "z" else pert[i]).reshape(-1)[j] = v
                    vals.append(loss(pert, zz))
                fd[j] = (vals[0] - vals[1]) / (float(hi) - float(lo))
            g = got[name].reshape(-1)
            scale = max(float(np.max(np.abs(fd))), 1e-12)
            err = float(np.max(np.abs(g - fd))) / scale
            assert err < 2e-5, f"gated d/d{name} (K={K}) differs from finite differences: {err:.2e}"

        y = orc.forward(K, *args)
        plain = orc.backward(K, *args, dy)
        at0 = orc.backward(K, *args, dy, z=np.zeros(xshape, np.float32))
        for name in BWD_NAMES:
            assert np.all(at0[name] == 0.0), f"gate at z = 0: d/d{name} (K={K}) not zero"
        _close(at0["z"], dyd * y / 2.0, 1e-13, 1e-15, f"gate at z = 0: dz, K={K}")
        at40 = orc.backward(K, *args, dy, z=np.full(xshape, 40.0, np.float32))
        for name in BWD_NAMES:
            _close(at40[name], 40.0 * plain[name], 1e-13, 1e-15, f"gate at z = 40: d/d{name}")
        _close(at40["z"], dyd * y, 1e-13, 1e-15, f"gate at z = 40: dz, K={K}")


def pin_backward_zoh(orc):
    """Gradients of the zero-order-hold operator: every input's (and, gated, z's) element
    by element against central finite differences of the ZOH forward oracle, with half of
    the states at |delta A| ~ 1e-3 (the power-series side of d bb / dA) and half at
    |delta A| ~ 0.1-1; and the limit A -> 0 (A_log = -30), where the hold's B term
    expm1(delta A) / A equals delta to 1e-13: every gradient but dA_log then equals the plain
    operator's (separately pinned) to that precision."""
    rng = _rng(19)
    for K, xshape, gated in ((4, (1, 2, 3, 4), True), (2, (2, 2, 7), False)):
        B, D = xshape[:2]
        L = int(np.prod(xshape[2:]))
        N = 2
        args = list(_random_inputs(rng, B, K, D, N, L, xshape))
        args[2][..., 0] = rng.uniform(-7.0, -5.0, size=(K, D)).astype(np.float32)
        dy = rng.standard_normal(xshape).astype(np.float32)
        z = (1.5 * rng.standard_normal(xshape)).astype(np.float32) if gated else None
        got = orc.backward(K, *args, dy, z=z, zoh=True)
        dyd = dy.astype(np.float64)

        def loss(a, zz):
            return float(np.sum(orc.forward(K, *a, z=zz, zoh=True) * dyd))

        names = BWD_NAMES + (("z",) if gated else ())
        for i, name in enumerate(names):
            base_arr = z if name == "z" else args[i]
            flat = base_arr.reshape(-1)
            fd = np.empty(flat.size)
            for j in range(flat.size):
                base = float(flat[j])
                step = 1e-3 * max(1.0, abs(base))
                hi, lo = np.float32(base + step), np.float32(base - step)
                vals = []
                for v in (hi, lo):
                    pert = [a.copy() for a in args]
                    zz = None if z is None else z.copy()
                    (zz if name == "z" else pert[i]).reshape(-1)[j] = v
                    vals.append(loss(pert, zz))
                fd[j] = (vals[0] - vals[1]) / (float(hi) - float(lo))
            g = got[name].reshape(-1)
            scale = max(float(np.max(np.abs(fd))), 1e-12)
            err = float(np.max(np.abs(g - fd))) / scale
            assert err < 2e-5, f"ZOH d/d{name} (K={K}) differs from finite differences: {err:.2e}"

        flat_a = list(args)
        flat_a[2] = np.full_like(args[2], -30.0)
        zoh0 = orc.backward(K, *flat_a, dy, z=z, zoh=True)
        plain0 = orc.backward(K, *flat_a, dy, z=z)
        for name in names:
            if name != "A_log":
                _close(zoh0[name], plain0[name], 1e-11, 1e-14, f"ZOH at A -> 0: d/d{name}")


def pin_backward_routes(orc):
    """Gradients of the operator over per-route inputs: fed every route's gather of one x,
    each route's du summed back at the positions it visits (in route order) is the plain
    backward's dx, and every other gradient is the plain backward's, exactly (the same
    double arithmetic), with the gate and the hold as well; and with four different inputs,
    every gradient (u's per route and step) against central finite differences of the
    routes operator."""
    for K, H, W in ((4, 3, 4), (2, 1, 7)):
        B, D, N = 2, 2, 2
        L = H * W
        rng = _rng(20 + K)
        xshape = (B, D, H, W) if K == 4 else (B, D, L)
        routes = _routes(H, W, K)
        x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L, xshape=xshape)
        dy = rng.standard_normal(xshape).astype(np.float32)
        z = (1.5 * rng.standard_normal(xshape)).astype(np.float32)
        xf = x.reshape(B, D, L)
        u = np.stack([xf[:, :, routes[k]] for k in range(K)], axis=1)
        for zoh, gate in ((False, None), (True, z)):
            want = orc.backward(K, x, dt, A_log, Bs, Cs, Ds, bias, dy, z=gate, zoh=zoh)
            got = orc.backward_routes(K, u, dt, A_log, Bs, Cs, Ds, bias, dy, H, W, z=gate,
                                      zoh=zoh)
            dx = np.zeros((B, D, L))
            for k in range(K):
                dx[:, :, routes[k]] = dx[:, :, routes[k]] + got["u"][:, k]
            _close(dx.reshape(xshape), want["x"], 0.0, 0.0, f"routes du -> dx, K={K}")
            for name in BWD_NAMES[1:] + (("z",) if gate is not None else ()):
                _close(got[name], want[name], 0.0, 0.0, f"routes d/d{name}, K={K}, zoh={zoh}")

        u = rng.standard_normal((B, K, D, L)).astype(np.float32)
        gate = z if K == 4 else None
        got = orc.backward_routes(K, u, dt, A_log, Bs, Cs, Ds, bias, dy, H, W, z=gate,
                                  zoh=True)
        args = [u, dt, A_log, Bs, Cs, Ds, bias]
        dyd = dy.astype(np.float64)

        def loss(a, zz):
            return float(np.sum(orc.forward_routes(K, a[0], *a[1:], H, W, z=zz, zoh=True)
                                * dyd))

        names = ("u",) + BWD_NAMES[1:] + (("z",) if gate is not None else ())
        for i, name in enumerate(names):
            base_arr = gate if name == "z" else args[i]
            flat = base_arr.reshape(-1)
            fd = np.empty(flat.size)
            for j in range(flat.size):
                base = float(flat[j])
                step = 1e-3 * max(1.0, abs(base))
                hi, lo = np.float32(base + step), np.float32(base - step)
                vals = []
                for v in (hi, lo):
                    pert = [a.copy() for a in args]
                    zz = None if gate is None else gate.copy()
                    (zz if name == "z" else pert[i]).reshape(-1)[j] = v
                    vals.append(loss(pert, zz))
                fd[j] = (vals[0] - vals[1]) / (float(hi) - float(lo))
            g = got[name].reshape(-1)
            scale = max(float(np.max(np.abs(fd))), 1e-12)
            err = float(np.max(np.abs(g - fd))) / scale
            assert err < 2e-5, f"routes d/d{name} (K={K}) differs from finite differences: {err:.2e}"


# ---- per-route front end (causal depthwise conv + SiLU, x_proj, dt_proj) -----------------
def _front_weights(rng, K, D, N, R, KW):
    conv_w = rng.standard_normal((K, D, KW)).astype(np.float32)
    conv_b = (0.5 * rng.standard_normal((K, D))).astype(np.float32)
    x_proj_w = (rng.standard_normal((K, R + 2 * N, D)) / np.sqrt(D)).astype(np.float32)
    dt_proj_w = rng.standard_normal((K, D, R)).astype(np.float32)
    return conv_w, conv_b, x_proj_w, dt_proj_w


def pin_project_impulse(orc):
    """A unit impulse in one channel: the route's conv output holds the taps in reverse order
    at the KW steps from the one that visits the impulse on (cross-correlation with left
    padding KW - 1, cut to the first L outputs: causal), the bias everywhere.  Taps and
    biases are >= 36, where SiLU(c) = c to 1e-15 relative, and SiLU(0) = 0 exactly."""
    for K, H, W in ((4, 3, 5), (2, 1, 7)):
        D, N, R, KW = 3, 2, 2, 4
        L = H * W
        k_, d_, j_ = np.meshgrid(np.arange(K), np.arange(D), np.arange(KW), indexing="ij")
        conv_w = (36.0 + 8.0 * j_ + 2.0 * k_ + d_).astype(np.float32)
        routes = _routes(H, W, K)
        rng = _rng(40)
        _, _, x_proj_w, dt_proj_w = _front_weights(rng, K, D, N, R, KW)
        for with_bias in (False, True):
            conv_b = (40.0 + k_[:, :, 0] + 0.25 * d_[:, :, 0]).astype(np.float32) if with_bias \
                else np.zeros((K, D), np.float32)
            for p0 in (0, L - 1, L // 2 + 1):
                x = np.zeros((1, D, L), np.float32)
                x[0, 1, p0] = 1.0
                xs = x.reshape((1, D, H, W)) if K == 4 else x
                got = orc.project(K, xs, conv_w, conv_b, x_proj_w, dt_proj_w)["u"]
                want = np.broadcast_to(conv_b.astype(np.float64)[None, :, :, None],
                                       (1, K, D, L)).copy()
                for k in range(K):
                    t0 = int(np.nonzero(routes[k] == p0)[0][0])
                    for j in range(KW):
                        if t0 + j < L:
                            want[0, k, 1, t0 + j] += conv_w[k, 1, KW - 1 - j]
                _close(got, want, 1e-13, 0.0, f"impulse K={K} p0={p0} bias={with_bias}")
        # x = 0: u = SiLU(bias).  SiLU(c) - SiLU(-c) = c, and SiLU(c) = c (1 + tanh(c / 2)) / 2
        c = rng.uniform(-4.0, 4.0, size=(K, D)).astype(np.float32)
        x = np.zeros((1, D, H, W) if K == 4 else (1, D, L), np.float32)
        up = orc.project(K, x, conv_w, c, x_proj_w, dt_proj_w)["u"]
        um = orc.project(K, x, conv_w, -c, x_proj_w, dt_proj_w)["u"]
        c64 = np.broadcast_to(c.astype(np.float64)[None, :, :, None], up.shape)
        _close(up - um, c64, 1e-14, 1e-15, f"SiLU odd part, K={K}")
        _close(up, c64 * (1.0 + np.tanh(c64 / 2.0)) / 2.0, 1e-14, 1e-15, f"SiLU, K={K}")


def _causal_xcorr(s, w):
    """sum_j w[j] s[t - (KW - 1) + j] for t < len(s), zeros before the start: numpy's full
    convolution with the reversed taps, cut to the first len(s) outputs."""
    return np.convolve(s, w[::-1])[: len(s)]


def pin_project_brute(orc):
    """Random tiny cases against numpy.convolve, scipy.special.expit and matrix products."""
    import scipy.special
    for K, H, W, KW in ((4, 3, 4, 4), (4, 2, 5, 3), (2, 1, 7, 4), (2, 1, 3, 5)):
        B, D, N, R = 2, 5, 2, 3
        L = H * W
        rng = _rng(41 + KW + K)
        x = rng.standard_normal((B, D, L)).astype(np.float32)
        conv_w, conv_b, x_proj_w, dt_proj_w = _front_weights(rng, K, D, N, R, KW)
        xs = x.reshape((B, D, H, W)) if K == 4 else x
        got = orc.project(K, xs, conv_w, conv_b, x_proj_w, dt_proj_w)
        routes = _routes(H, W, K)
        u = np.zeros((B, K, D, L))
        for b in range(B):
            for k in range(K):
                for d in range(D):
                    c = _causal_xcorr(x[b, d, routes[k]].astype(np.float64),
                                      conv_w[k, d].astype(np.float64)) + float(conv_b[k, d])
                    u[b, k, d] = c * scipy.special.expit(c)
        xd = np.matmul(x_proj_w.astype(np.float64)[None], u)        # (B, K, R + 2N, L)
        dt = np.matmul(dt_proj_w.astype(np.float64)[None], xd[:, :, :R])
        _close(got["u"], u, 1e-12, 1e-14, f"u K={K} KW={KW}")
        _close(got["dt_raw"], dt, 1e-11, 1e-13, f"dt_raw K={K} KW={KW}")
        _close(got["Bs"], xd[:, :, R:R + N], 1e-11, 1e-13, f"Bs K={K} KW={KW}")
        _close(got["Cs"], xd[:, :, R + N:], 1e-11, 1e-13, f"Cs K={K} KW={KW}")


def pin_project_select(orc):
    """One-hot x_proj and dt_proj rows pick single channels of u: the split of x_proj's
    output is [dt (R rows), B (N rows), C (N rows)], x_proj is (K, R + 2N, D) with rows as
    outputs, dt_proj is (K, D, R).  Every value is a single product with 1.0: exact."""
    K, B, D, H, W, N, R, KW = 4, 2, 6, 3, 4, 2, 3, 4
    M = R + 2 * N
    rng = _rng(45)
    x = rng.standard_normal((B, D, H, W)).astype(np.float32)
    conv_w, conv_b, _, _ = _front_weights(rng, K, D, N, R, KW)
    sel = np.array([[(m * 5 + k) % D for m in range(M)] for k in range(K)])
    x_proj_w = np.zeros((K, M, D), np.float32)
    dt_proj_w = np.zeros((K, D, R), np.float32)
    for k in range(K):
        x_proj_w[k, np.arange(M), sel[k]] = 1.0
        dt_proj_w[k, np.arange(D), (np.arange(D) + k) % R] = 1.0
    got = orc.project(K, x, conv_w, conv_b, x_proj_w, dt_proj_w)
    u = got["u"]
    for k in range(K):
        _close(got["Bs"][:, k], u[:, k, sel[k][R:R + N]], 0.0, 0.0, f"Bs rows, route {k}")
        _close(got["Cs"][:, k], u[:, k, sel[k][R + N:]], 0.0, 0.0, f"Cs rows, route {k}")
        pick = sel[k][(np.arange(D) + k) % R]
        _close(got["dt_raw"][:, k], u[:, k, pick], 0.0, 0.0, f"dt_raw rows, route {k}")


def pin_routes_variant(orc):
    """The operator over per-route inputs: fed every route's gather of one x it is the
    plain operator on x (same double arithmetic: equal), and fed four different inputs it is
    the sum, in route order, of the plain operator run on each input with the other routes'
    C and D set to zero (their terms are exact zeros)."""
    for K, H, W in ((4, 3, 5), (2, 1, 9)):
        B, D, N = 2, 3, 2
        L = H * W
        rng = _rng(46 + K)
        xshape = (B, D, H, W) if K == 4 else (B, D, L)
        routes = _routes(H, W, K)
        x, dt, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L, xshape=xshape)
        z = rng.standard_normal(xshape).astype(np.float32)
        xf = x.reshape(B, D, L)
        u = np.stack([xf[:, :, routes[k]] for k in range(K)], axis=1)
        for zoh, gate in ((False, None), (True, z)):
            want = orc.forward(K, x, dt, A_log, Bs, Cs, Ds, bias, z=gate, zoh=zoh)
            got = orc.forward_routes(K, u, dt, A_log, Bs, Cs, Ds, bias, H, W, z=gate, zoh=zoh)
            _close(got, want, 0.0, 0.0, f"gathered x, K={K}, zoh={zoh}")
        u = rng.standard_normal((B, K, D, L)).astype(np.float32)
        want = np.zeros(xshape)
        for k in range(K):
            xk = np.empty((B, D, L), np.float32)
            xk[:, :, routes[k]] = u[:, k]
            Cs_k, Ds_k = np.zeros_like(Cs), np.zeros_like(Ds)
            Cs_k[:, k], Ds_k[k] = Cs[:, k], Ds[k]
            want = want + orc.forward(K, xk.reshape(xshape), dt, A_log, Bs, Cs_k, Ds_k, bias,
                                      z=z)
        got = orc.forward_routes(K, u, dt, A_log, Bs, Cs, Ds, bias, H, W, z=z)
        _close(got, want, 0.0, 0.0, f"four inputs, K={K}")


def pin_routes_lowrank(orc):
    """dt_proj folded into the routes operator: fed dt_lr and dt_w it equals the routes
    operator fed dt_raw = dt_w @ dt_lr, with values chosen so that every product and sum is
    exact in fp32 (dt_lr on a 1/64 grid, dt_w in {±1/2, ±1, ±2}): equal results.  And the
    front end without dt_proj returns x_proj's first R rows: with dt_proj the identity on
    those rows, the full front end's dt_raw rows 0..R-1 are the same numbers."""
    rng = _rng(50)
    for K, H, W in ((4, 3, 5), (2, 1, 11)):
        B, D, N, R = 2, 3, 2, 3
        L = H * W
        xshape = (B, D, H, W) if K == 4 else (B, D, L)
        x, _, A_log, Bs, Cs, Ds, bias = _random_inputs(rng, B, K, D, N, L, xshape=xshape)
        u = rng.standard_normal((B, K, D, L)).astype(np.float32)
        dt_lr = (rng.integers(-40, 40, size=(B, K, R, L)) / 64.0).astype(np.float32)
        dt_w = rng.choice(np.array([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], np.float32),
                          size=(K, D, R))
        dt_raw = np.einsum("kdr,bkrl->bkdl", dt_w.astype(np.float64),
                           dt_lr.astype(np.float64)).astype(np.float32)
        z = rng.standard_normal(xshape).astype(np.float32)
        for zoh, gate in ((False, None), (True, z)):
            want = orc.forward_routes(K, u, dt_raw, A_log, Bs, Cs, Ds, bias, H, W, z=gate,
                                      zoh=zoh)
            got = orc.forward_routes_lr(K, u, dt_lr, dt_w, A_log, Bs, Cs, Ds, bias, H, W,
                                        z=gate, zoh=zoh)
            _close(got, want, 0.0, 0.0, f"routes low rank, K={K}, zoh={zoh}")
        conv_w, conv_b, x_proj_w, _ = _front_weights(rng, K, D, N, R, 4)
        eye = np.zeros((K, D, R), np.float32)
        for r in range(min(R, D)):
            eye[:, r, r] = 1.0
        full = orc.project(K, x, conv_w, conv_b, x_proj_w, eye)
        lr = orc.project_lr(K, x, conv_w, conv_b, x_proj_w, R)
        for key in ("u", "Bs", "Cs"):
            _close(lr[key], full[key], 0.0, 0.0, f"project without dt_proj: {key}, K={K}")
        _close(lr["dt_lr"], full["dt_raw"][:, :, :R], 0.0, 0.0, f"dt rows, K={K}")


ALL_PINS = [pin_brute_force, pin_geometric, pin_convolve, pin_lfilter, pin_halving,
            pin_small_delta, pin_memoryless, pin_routes, pin_flip, pin_transpose, pin_rot180,
            pin_linearity, pin_channels, pin_gate, pin_zoh_exact, pin_backward_fd,
            pin_backward_adjoint, pin_backward_gate, pin_backward_zoh, pin_backward_routes,
            pin_project_impulse,
            pin_project_brute,
            pin_project_select, pin_routes_variant, pin_routes_lowrank]
