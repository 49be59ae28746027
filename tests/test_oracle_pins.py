"""CPU tests of the oracle: its pins, planted mistakes that the pins must catch, thread
determinism, and the stored golden output of the smallest workload."""
import json
import os
import pathlib
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_pins

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"


@pytest.fixture(scope="module")
def orc():
    # tests/test_sanitizers_cpu.py reruns the pins against an oracle built with
    # AddressSanitizer and UBSan, named by SS2D_TEST_ORACLE_LIBRARY
    other = os.environ.get("SS2D_TEST_ORACLE_LIBRARY")
    if other:
        return oracle.Oracle(other)
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


# Planted mistakes: (what, original text in ss2d_oracle.c, replacement).  Every one of them
# must make at least one pin fail.
MUTATIONS = [
    ("drop skip term", "out[l] += (yk + Dk * u) * gate;", "out[l] += yk * gate;"),
    ("A sign", "A[n] = -exp((double)A_log[(k * D + d) * N + n]);\n            h[n] = 0.0;",
     "A[n] = exp((double)A_log[(k * D + d) * N + n]);\n            h[n] = 0.0;"),
    ("bwd: A sign in the recomputed forward",
     "A[n] = -exp((double)A_log[(k * D + d) * N + n]);\n            /* forward",
     "A[n] = exp((double)A_log[(k * D + d) * N + n]);\n            /* forward"),
    ("output before update",
     "h[n] = a * h[n] + bbar * (double)Bk[n * L + t] * u;\n"
     "                yk += (double)Ck[n * L + t] * h[n];",
     "yk += (double)Ck[n * L + t] * h[n];\n"
     "                h[n] = a * h[n] + bbar * (double)Bk[n * L + t] * u;"),
    ("no decay", "h[n] = a * h[n] +", "h[n] = h[n] +"),
    ("decay squared", "const double a = exp(delta * A[n]);",
     "const double a = exp(2.0 * delta * A[n]);"),
    ("column route transposed", "return (t % H) * W + t / H;", "return (t % W) * H + t / W;"),
    ("route 1 not reversed", "case 1:\n        return L - 1 - t;", "case 1:\n        return t;"),
    ("route 3 not reversed", "s = L - 1 - t;", "s = t;"),
    ("bias outside softplus", "const double delta = softplus(dtv + bias);",
     "const double delta = (softplus(dtv) + bias);"),
    ("no delta on B", "double bbar = delta;", "double bbar = 1.0;"),
    ("softplus wrong", "return m + log1p(exp(-fabs(z)));", "return m + log1p(exp(fabs(z)));"),
    ("C replaced by B", "yk += (double)Ck[n * L + t]", "yk += (double)Bk[n * L + t]"),
    ("B layout (L, N)", "bbar * (double)Bk[n * L + t] * u", "bbar * (double)Bk[t * N + n] * u"),
    ("delta read at image position", "                dtv = dt[t];", "                dtv = dt[l];"),
    ("backward 1D route not reversed", "return k == 0 ? t : L - 1 - t;", "return t;"),
    ("bwd gate: SiLU' without the z term", "return s * (1.0 + z * (1.0 - s));",
     "return s;"),
    ("bwd gate: routes see dy times sigmoid(z)",
     "(double)gc[l] * silu((double)zc[l]) : (double)gc[l];",
     "(double)gc[l] * sigmoid((double)zc[l]) : (double)gc[l];"),
    ("bwd gate: dz without the skip term", "ysum[l] += yroute + Dk * u;",
     "ysum[l] += yroute;"),
    ("bwd zoh: d bb / d delta taken as 1", "bb_delta = a;", "bb_delta = 1.0;"),
    ("bwd zoh: psi series coefficient", "p += xk * (double)(k + 1) / f;",
     "p += xk * (double)(k + 2) / f;"),
    ("bwd zoh: dA without the B u term", "(da * a * delta[t] + lam[n] * Bv * u * bb_A) * A[n];",
     "(da * a * delta[t]) * A[n];"),
    ("bwd zoh: psi closed form sign", "return (x * exp(x) - expm1(x)) / (x * x);",
     "return (x * exp(x) + expm1(x)) / (x * x);"),
    ("bwd routes: every route reads route 0's input",
     "const float *uk = u_routes ? u_routes + ((b * K + k) * D + d) * L : NULL;\n"
     "            for (int64_t n = 0; n < N; ++n)\n                A[n] = -exp(",
     "const float *uk = u_routes ? u_routes + ((b * K) * D + d) * L : NULL;\n"
     "            for (int64_t n = 0; n < N; ++n)\n                A[n] = -exp("),
    ("bwd routes: du written at the image position",
     "dx_b[(k * D + d) * L + t] = du; /* du per route, in scan order */",
     "dx_b[(k * D + d) * L + route_position(K, k, t, H, W)] = du;"),
    ("bwd zoh: B term of the recomputed forward left at delta",
     "                    if (zoh && A[n] != 0.0)\n                        bb = expm1(delta[t] * A[n]) / A[n];\n                    as[t * N + n] = a;",
     "                    as[t * N + n] = a;"),
    ("A_log indexed (K, N, D)", "A_log[(k * D + d) * N + n]);\n            h[n] = 0.0;",
     "A_log[(k * N + n) * D + d]);\n            h[n] = 0.0;"),
    ("Ds indexed (D, K)", "\n        const double Dk = Ds[k * D + d];",
     "\n        const double Dk = Ds[(d * K + k) % (K * D)];"),
    ("dt_bias shared by routes", "\n        const double bias = dt_bias[k * D + d];",
     "\n        const double bias = dt_bias[d];"),
    ("x ignores batch", "const float *xc = u_routes ? NULL : x + (b * D + d) * L;\n    const",
     "const float *xc = u_routes ? NULL : x + d * L;\n    const"),
    ("Cs ignores batch", "\n        const float *Ck = Cs + (b * K + k) * N * L;",
     "\n        const float *Ck = Cs + k * N * L;"),
    ("state not reset per route", "            h[n] = 0.0;\n", "\n"),
    ("gate is the sigmoid", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("gate misses the skip term", "out[l] += (yk + Dk * u) * gate;",
     "out[l] += yk * gate + Dk * u;"),
    ("gate read at the scan step", "gate = zc ? silu((double)zc[l])", "gate = zc ? silu((double)zc[t])"),
    ("ZOH without the minus one", "bbar = expm1(delta * A[n]) / A[n];",
     "bbar = exp(delta * A[n]) / A[n];"),
    ("ZOH divided by delta", "bbar = expm1(delta * A[n]) / A[n];",
     "bbar = expm1(delta * A[n]) / delta;"),
    ("ZOH ignored", "if (zoh && A[n] != 0.0)\n                    bbar =",
     "if (0)\n                    bbar ="),
    ("bwd: adjoint without decay", "lam[n] = g * (double)Ck[n * L + t] + anext * lam[n];",
     "lam[n] = g * (double)Ck[n * L + t] + lam[n];"),
    ("bwd: adjoint decays with the current step",
     "const double anext = t + 1 < L ? as[(t + 1) * N + n] : 0.0;",
     "const double anext = as[t * N + n];"),
    ("bwd: dC from the previous state", "dC_b[(k * N + n) * L + t] += g * hs[t * N + n];",
     "dC_b[(k * N + n) * L + t] += g * hprev;"),
    ("bwd: B term without delta", "double bb = delta[t], bb_delta = 1.0, bb_A = 0.0;",
     "double bb = 1.0, bb_delta = 1.0, bb_A = 0.0;"),
    ("bwd: decay derivative from the current state",
     "const double hprev = t > 0 ? hs[(t - 1) * N + n] : 0.0;\n"
     "                    const double a = as[t * N + n];",
     "const double hprev = hs[t * N + n];\n"
     "                    const double a = as[t * N + n];"),
    ("bwd: ddelta without the decay term", "ddelta += da * a * A[n] + lam[n]",
     "ddelta += lam[n]"),
    ("bwd: softplus derivative without the bias", "sigmoid((double)dt[t] + bias)",
     "sigmoid((double)dt[t])"),
    ("bwd: dA_log without the chain factor A",
     "(da * a * delta[t] + lam[n] * Bv * u * bb_A) * A[n];",
     "(da * a * delta[t] + lam[n] * Bv * u * bb_A);"),
    ("bwd: du without the skip term", "double ddelta = 0.0, du = g * Dk;",
     "double ddelta = 0.0, du = 0.0;"),
    ("bwd: dx at the scan step", "dx_b[d * L + l] += du;", "dx_b[d * L + t] += du;"),
    ("bwd: dDs from the output gradient alone", "pD[k * D + d] += g * u;", "pD[k * D + d] += g;"),
    ("bwd: bias outside softplus", "delta[t] = softplus((double)dt[t] + bias);",
     "delta[t] = (softplus((double)dt[t]) + bias);"),
    ("bwd: delta read at the image position", "delta[t] = softplus((double)dt[t] + bias);",
     "delta[t] = softplus((double)dt[route_position(K, k, t, H, W)] + bias);"),
    ("bwd: A_log indexed (K, N, D)", "A_log[(k * D + d) * N + n]);\n            /* forward",
     "A_log[(k * N + n) * D + d]);\n            /* forward"),
    ("bwd: Ds indexed (D, K)", "\n            const double Dk = Ds[k * D + d];",
     "\n            const double Dk = Ds[(d * K + k) % (K * D)];"),
    ("bwd: dt_bias shared by routes", "\n            const double bias = dt_bias[k * D + d];",
     "\n            const double bias = dt_bias[d];"),
    ("bwd: x ignores batch", "u_routes ? NULL : x + (b * D + d) * L;\n        const float *gc",
     "u_routes ? NULL : x + d * L;\n        const float *gc"),
    ("bwd: Cs ignores batch", "\n            const float *Ck = Cs + (b * K + k) * N * L;",
     "\n            const float *Ck = Cs + k * N * L;"),
    ("bwd: dy ignores batch", "const float *gc = dy + (b * D + d) * L;",
     "const float *gc = dy + d * L;"),
    ("project: conv taps in convolution order", "c += (double)w[j] * ",
     "c += (double)w[KW - 1 - j] * "),
    ("project: conv one step late", "const int64_t tau = t - (KW - 1) + j;",
     "const int64_t tau = t - KW + j;"),
    ("project: conv bias shared by routes", "double c = conv_b[(int64_t)k * D + d];",
     "double c = conv_b[d];"),
    ("project: conv taps shared by channels", "conv_w + ((int64_t)k * D + d) * KW;",
     "conv_w + ((int64_t)k * D) * KW;"),
    ("project: no SiLU", "uk[d * L + t] = silu(c);", "uk[d * L + t] = c;"),
    ("project: conv along route 0 for every route",
     "(double)xc[route_position(K, k, tau, H, W)];",
     "(double)xc[route_position(K, 0, tau, H, W)];"),
    ("project: x_proj weight read (K, D, M)", "x_proj_w[((int64_t)k * M + m) * D + d]",
     "x_proj_w[((int64_t)k * D + d) * M + m]"),
    ("project: dt_proj weight read (K, R, D)", "dt_proj_w[((int64_t)k * D + d) * R + r]",
     "dt_proj_w[((int64_t)k * R + r) * D + d]"),
    ("project: dt from the B rows", "* R + r] * xd[r];", "* R + r] * xd[R + r];"),
    ("project: B and C swapped", "Bs[(i * N + n) * L + t] = xd[R + n];",
     "Bs[(i * N + n) * L + t] = xd[R + N + n];"),
    ("routes: every route reads route 0's input",
     "u_routes + ((b * K + k) * D + d) * L : NULL;\n        for (int64_t t",
     "u_routes + ((b * K) * D + d) * L : NULL;\n        for (int64_t t"),
    ("routes: input read in reverse", "const double u = uk ? uk[t] : xc[l];",
     "const double u = uk ? uk[L - 1 - t] : xc[l];"),
    ("low rank: dt_w's first column for every r", "dtv += (double)wr[r] * (double)lr[r * L + t];",
     "dtv += (double)wr[0] * (double)lr[r * L + t];"),
    ("low rank: dt_lr of route 0", "const float *lr = dt_lr ? dt_lr + (b * K + k) * R * L : NULL;",
     "const float *lr = dt_lr ? dt_lr + (b * K) * R * L : NULL;"),
    ("low rank: dt rows from the B rows", "dt_lr[(i * R + r) * L + t] = xd[r];",
     "dt_lr[(i * R + r) * L + t] = xd[R + r];"),
]


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, what, old, new):
    src = oracle.SOURCE.read_text()
    assert src.count(old) == 1, f"mutation anchor for '{what}' not found exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(mutant_src, tmp_path / "libmutant.so")
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{what}'"


def test_thread_count_does_not_change_result(orc):
    wl = workloads.custom(B=2, D=6, H=5, W=7, N=4)
    inp = workloads.make_inputs(wl, seed=3)
    args = [inp[k] for k in ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")]
    y1 = orc.forward(4, *args, threads=1)
    y4 = orc.forward(4, *args, threads=4)
    assert np.array_equal(y1, y4)


def test_golden_tiny_workload(orc):
    """The stored output of the smallest workload (written by tests/golden/make_golden.py,
    which calls only the oracle) still matches: guards the oracle against silent drift."""
    meta = json.loads((GOLDEN / "tiny_f32.json").read_text())
    wl = workloads.workload(meta["workload"])
    inp = workloads.make_inputs(wl, seed=meta["seed"])
    y = orc.forward(wl.K, *[inp[k] for k in ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds",
                                              "dt_bias")])
    want = np.array(meta["y"], dtype=np.float64).reshape(y.shape)
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-15)


def test_gcc_present():
    assert shutil.which("gcc"), "the oracle is built with gcc"
    out = subprocess.run(["gcc", "--version"], capture_output=True, text=True)
    assert out.returncode == 0
