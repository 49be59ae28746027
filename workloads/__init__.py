"""Seeded synthetic inputs for the SS2D forward operator and its bidirectional 1D variant.

This module is shared by the CPU oracle's tests and by the GPU path's tests and benchmark.
It holds none of the operator's arithmetic: only random draws, the rounding of drawn fp32
values to bfloat16 (round to nearest even), and the recipe that turns a uniform draw into a
dt_bias value (the inverse of softplus, so that softplus(dt_bias) is the drawn value).

Workloads (shapes from the pages' models, values synthetic):
  * ``tiny_f32``              B=1,  D=8,   8x8     (L=64),    N=4,  K=4, fp32
  * ``vmamba_t_stage1_f32``   B=8,  D=192, 56x56   (L=3136),  N=16, K=4, fp32
  * ``vmamba_t_stage1_bf16``  B=64, D=192, 56x56   (L=3136),  N=16, K=4, bf16 data
  * ``highres_1024px_bf16``   B=2,  D=192, 256x256 (L=65536), N=16, K=4, bf16 data
  * ``vim_bidir_bf16``        B=128, D=768, L=197 (14x14 patches + cls), N=16, K=2, bf16

VMamba-T stage 1 is a 224x224 image at patch 4 (56x56 tokens) with 96 channels and an
expansion ratio of 2 (D=192) (Vision Mamba explainer page, VMamba backbone listing; the
Chinese VMamba article, section 4).  The high-resolution case is a 1024 px image at patch 4.
The Vim case is a 224x224 image at patch 16 plus one class token (aipaper.cc Vim summary,
section 4.2).  ImageNet and the other datasets the pages evaluate on are not used: these
seeded draws stand in for activations of those shapes.

Value recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this order, fp32):
  1. x       ~ N(0, 1)            shape (B, D, H, W)  [(B, D, L) for K=2]
  2. dt_raw  ~ N(0, 0.5**2)       shape (B, K, D, L)  (standard deviation 0.5)
  3. Bs      ~ N(0, 1)            shape (B, K, N, L)
  4. Cs      ~ N(0, 1)            shape (B, K, N, L)
  5. v       ~ U[1e-3, 1e-1)      shape (K, D), dt_bias = log(expm1(v)) in fp64, stored fp32
  6. A_log[k, d, n] = log(n + 1)  (the S4D-real initialisation the explainer's listing uses),
     or, for ``a_log="random"``, a further draw A_log ~ U[log 1, log 16) of shape (K, D, N)
  7. Ds = 1                       shape (K, D)
For bf16 workloads x, dt_raw, Bs and Cs are rounded to bfloat16 after drawing; the returned
fp32 arrays hold exactly the bfloat16 values, so every consumer sees the same numbers.
dt_raw, Bs and Cs are laid out in the scan order of each route (time innermost).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    D: int
    H: int
    W: int
    N: int
    K: int
    dtype: str  # "f32" or "bf16"

    @property
    def L(self) -> int:
        return self.H * self.W

    @property
    def updates(self) -> int:
        """State updates per forward call: one per (b, k, d, t, n)."""
        return self.B * self.K * self.D * self.L * self.N

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def algorithmic_bytes(self) -> int:
        """Bytes the operator must move: x read once, dt_raw, Bs, Cs read once, y written
        once, plus the fp32 parameters A_log, Ds, dt_bias."""
        e = self.elem_bytes
        B, K, D, L, N = self.B, self.K, self.D, self.L, self.N
        return e * (B * D * L + B * K * D * L + 2 * B * K * N * L + B * D * L) + 4 * (
            K * D * N + 2 * K * D)

    def as_dict(self) -> dict:
        return dict(name=self.name, B=self.B, D=self.D, H=self.H, W=self.W, L=self.L,
                    N=self.N, K=self.K, dtype=self.dtype)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 8, 8, 8, 4, 4, "f32"),
    "vmamba_t_stage1_f32": Workload("vmamba_t_stage1_f32", 8, 192, 56, 56, 16, 4, "f32"),
    "vmamba_t_stage1_bf16": Workload("vmamba_t_stage1_bf16", 64, 192, 56, 56, 16, 4, "bf16"),
    "highres_1024px_bf16": Workload("highres_1024px_bf16", 2, 192, 256, 256, 16, 4, "bf16"),
    "vim_bidir_bf16": Workload("vim_bidir_bf16", 128, 768, 1, 197, 16, 2, "bf16"),
}
ORDER = ["tiny_f32", "vmamba_t_stage1_f32", "vmamba_t_stage1_bf16", "highres_1024px_bf16",
         "vim_bidir_bf16"]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[ORDER[name_or_index]]
    return WORKLOADS[name_or_index]


def custom(B, D, H, W, N, K=4, dtype="f32", name="custom") -> Workload:
    return Workload(name, B, D, H, W, N, K, dtype)


# ---------------------------------------------------------------------------------------
# bfloat16 rounding of drawn values (round to nearest, ties to even; NaN stays NaN)
# ---------------------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 array holding the bfloat16 (RNE) value of each element of ``a``."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# ---------------------------------------------------------------------------------------
# Draws
# ---------------------------------------------------------------------------------------
def inverse_softplus(v: np.ndarray) -> np.ndarray:
    """z with log(1 + e^z) = v, for v > 0 (input recipe for dt_bias)."""
    return np.log(np.expm1(np.asarray(v, dtype=np.float64)))


def make_inputs(wl: Workload, seed: int = 0, a_log: str = "init") -> dict:
    """Seeded inputs for one workload, as fp32 numpy arrays (bf16-exact for bf16 workloads).

    Returns a dict with x, dt_raw, A_log, Bs, Cs, Ds, dt_bias and, for bf16 workloads, the
    raw bfloat16 bit patterns of x, dt_raw, Bs and Cs under ``<name>_bf16``.
    """
    rng = np.random.default_rng(seed)
    B, D, K, N, L = wl.B, wl.D, wl.K, wl.N, wl.L
    xshape = (B, D, L) if wl.K == 2 else (B, D, wl.H, wl.W)
    x = rng.standard_normal(xshape, dtype=np.float32)
    dt_raw = rng.standard_normal((B, K, D, L), dtype=np.float32)
    dt_raw *= np.float32(0.5)
    Bs = rng.standard_normal((B, K, N, L), dtype=np.float32)
    Cs = rng.standard_normal((B, K, N, L), dtype=np.float32)
    v = rng.uniform(1e-3, 1e-1, size=(K, D))
    dt_bias = inverse_softplus(v).astype(np.float32)
    if a_log == "init":
        A_log = np.broadcast_to(np.log(np.arange(1, N + 1, dtype=np.float64)),
                                (K, D, N)).astype(np.float32)
    elif a_log == "random":
        A_log = rng.uniform(0.0, np.log(16.0), size=(K, D, N)).astype(np.float32)
    else:
        raise ValueError(f"a_log must be 'init' or 'random', not {a_log!r}")
    Ds = np.ones((K, D), dtype=np.float32)
    out = dict(x=x, dt_raw=dt_raw, A_log=np.ascontiguousarray(A_log), Bs=Bs, Cs=Cs, Ds=Ds,
               dt_bias=dt_bias)
    if wl.dtype == "bf16":
        for key in ("x", "dt_raw", "Bs", "Cs"):
            bits = f32_to_bf16_bits(out[key])
            out[key + "_bf16"] = bits
            out[key] = bf16_bits_to_f32(bits)
    elif wl.dtype != "f32":
        raise ValueError(f"unknown dtype {wl.dtype!r}")
    return out


def make_gate(wl: Workload, seed: int = 0) -> dict:
    """Seeded gate z for the gated entry points: standard normal, the shape of x (the output
    of a linear projection, like x).  Drawn from a generator of its own so that the other
    inputs of the same seed are unchanged.  Returns z (fp32, bf16-exact for bf16 workloads)
    and, for bf16 workloads, its bit patterns under z_bf16."""
    rng = np.random.default_rng([seed, 0x9a7e])
    xshape = (wl.B, wl.D, wl.L) if wl.K == 2 else (wl.B, wl.D, wl.H, wl.W)
    z = rng.standard_normal(xshape, dtype=np.float32)
    out = dict(z=z)
    if wl.dtype == "bf16":
        bits = f32_to_bf16_bits(z)
        out["z_bf16"] = bits
        out["z"] = bf16_bits_to_f32(bits)
    return out


def make_output_grad(wl: Workload, seed: int = 0) -> dict:
    """Seeded output gradient dy for the backward entry points: standard normal, the shape of
    x and y, from a generator of its own.  Returns dy (fp32, bf16-exact for bf16 workloads)
    and, for bf16 workloads, its bit patterns under dy_bf16."""
    rng = np.random.default_rng([seed, 0xd1])
    xshape = (wl.B, wl.D, wl.L) if wl.K == 2 else (wl.B, wl.D, wl.H, wl.W)
    dy = rng.standard_normal(xshape, dtype=np.float32)
    out = dict(dy=dy)
    if wl.dtype == "bf16":
        bits = f32_to_bf16_bits(dy)
        out["dy_bf16"] = bits
        out["dy"] = bf16_bits_to_f32(bits)
    return out


def make_front_weights(wl: Workload, seed: int = 0, R: int = 1, KW: int = 4) -> dict:
    """Seeded weights of the per-route front end, fp32, from a generator of their own, each
    uniform in (-1/sqrt(fan_in), 1/sqrt(fan_in)) (the default initialisation of the conv and
    linear layers the pages' listings build without an initialiser of their own):
      conv_w    (K, D, KW)      depthwise causal conv taps, fan_in = KW
      conv_b    (K, D)          conv bias, fan_in = KW
      x_proj_w  (K, R + 2N, D)  x_proj rows [dt (R) | B (N) | C (N)], fan_in = D
      dt_proj_w (K, D, R)       dt_proj weight, fan_in = R
    R = 1 and KW = 4 are the explainer's SelectiveSSM sizes (x_proj to 2N + 1 outputs,
    dt_proj from 1 input, d_conv = 4)."""
    rng = np.random.default_rng([seed, 0xf0])
    K, D, N = wl.K, wl.D, wl.N

    def unif(shape, fan_in):
        bound = 1.0 / np.sqrt(fan_in)
        return rng.uniform(-bound, bound, size=shape).astype(np.float32)

    conv_w = unif((K, D, KW), KW)
    conv_b = unif((K, D), KW)
    x_proj_w = unif((K, R + 2 * N, D), D)
    dt_proj_w = unif((K, D, R), R)
    return dict(conv_w=conv_w, conv_b=conv_b, x_proj_w=x_proj_w, dt_proj_w=dt_proj_w)


def make_route_inputs(wl: Workload, seed: int = 0) -> dict:
    """Seeded per-route input u (B, K, D, L) for the operator whose routes each bring their
    own input (scan order of each route, time innermost): standard normal, from a generator
    of its own.  Returns u (fp32, bf16-exact for bf16 workloads) and, for bf16 workloads, its
    bit patterns under u_bf16."""
    rng = np.random.default_rng([seed, 0x0e])
    u = rng.standard_normal((wl.B, wl.K, wl.D, wl.L), dtype=np.float32)
    out = dict(u=u)
    if wl.dtype == "bf16":
        bits = f32_to_bf16_bits(u)
        out["u_bf16"] = bits
        out["u"] = bf16_bits_to_f32(bits)
    return out


def make_lowrank_dt(wl: Workload, seed: int = 0, R: int = 1) -> dict:
    """Seeded low-rank dt inputs for the operator with dt_proj folded in, from a generator of
    their own: dt_w (K, D, R) uniform in (-1/sqrt(R), 1/sqrt(R)) (dt_proj's default
    initialisation, fan_in = R) and dt_lr (B, K, R, L) ~ N(0, 3/4), so that the product
    dt_raw = dt_w @ dt_lr has variance 1/4, the standard deviation 0.5 of the dt_raw the
    other inputs use.  dt_w is fp32; dt_lr is bf16-exact for bf16 workloads, with its bit
    patterns under dt_lr_bf16."""
    rng = np.random.default_rng([seed, 0x1d])
    K, D, L = wl.K, wl.D, wl.L
    bound = 1.0 / np.sqrt(R)
    dt_w = rng.uniform(-bound, bound, size=(K, D, R)).astype(np.float32)
    dt_lr = rng.standard_normal((wl.B, K, R, L), dtype=np.float32)
    dt_lr *= np.float32(np.sqrt(0.75))
    out = dict(dt_w=dt_w, dt_lr=dt_lr)
    if wl.dtype == "bf16":
        bits = f32_to_bf16_bits(dt_lr)
        out["dt_lr_bf16"] = bits
        out["dt_lr"] = bf16_bits_to_f32(bits)
    return out
