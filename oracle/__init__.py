"""CPU oracle for the SS2D forward operator (float64).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use it; the GPU library never imports, links or calls anything here, and this
package imports nothing from the GPU package.

The arithmetic lives in ``ss2d_oracle.c`` (plain C, one sequential loop per channel and route,
every operation in double; see its header for the definition and the pages it follows).
This module only compiles it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

HERE = pathlib.Path(__file__).resolve().parent
SOURCE = HERE / "ss2d_oracle.c"
LIBRARY = HERE / "liboracle_ss2d.so"

ORACLE_ZOH = 1  # flag bit of oracle_forward_ex: zero-order hold for B

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(source: os.PathLike = SOURCE, output: os.PathLike = LIBRARY) -> pathlib.Path:
    """Compile the oracle into a shared library with gcc (IEEE double, no fast-math)."""
    output = pathlib.Path(output)
    tmp = output.with_suffix(f".so.tmp{os.getpid()}")  # concurrent builds never share a file
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-fno-fast-math", str(source), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, output)
    return output


class Oracle:
    """ctypes handle on one compiled oracle library (the tests also load planted mutants)."""

    def __init__(self, path: os.PathLike = LIBRARY):
        path = pathlib.Path(path)
        if not path.exists():
            if path != LIBRARY:
                raise FileNotFoundError(path)
            build()
        self.path = path
        lib = ctypes.CDLL(str(path))
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [ctypes.c_int] + [_f32p] * 7 + [_f64p] + \
            [ctypes.c_int64] * 5 + [ctypes.c_int]
        lib.oracle_forward_channels.restype = ctypes.c_int
        lib.oracle_forward_channels.argtypes = [ctypes.c_int] + [_f32p] * 7 + \
            [ctypes.c_int64] * 5 + [_i64p, _i64p, ctypes.c_int64, _f64p, ctypes.c_int]
        lib.oracle_forward_ex.restype = ctypes.c_int
        lib.oracle_forward_ex.argtypes = [ctypes.c_int] + [_f32p] * 8 + [ctypes.c_int, _f64p] + \
            [ctypes.c_int64] * 5 + [ctypes.c_int]
        lib.oracle_forward_channels_ex.restype = ctypes.c_int
        lib.oracle_forward_channels_ex.argtypes = [ctypes.c_int] + [_f32p] * 8 + \
            [ctypes.c_int] + [ctypes.c_int64] * 5 + [_i64p, _i64p, ctypes.c_int64, _f64p,
                                                   ctypes.c_int]
        lib.oracle_forward_routes_ex.restype = ctypes.c_int
        lib.oracle_forward_routes_ex.argtypes = lib.oracle_forward_ex.argtypes
        lib.oracle_forward_routes_lr_ex.restype = ctypes.c_int
        lib.oracle_forward_routes_lr_ex.argtypes = [ctypes.c_int] + [_f32p] * 3 + \
            [ctypes.c_int64] + [_f32p] * 6 + [ctypes.c_int, _f64p] + [ctypes.c_int64] * 5 + \
            [ctypes.c_int]
        lib.oracle_project_lr.restype = ctypes.c_int
        lib.oracle_project_lr.argtypes = [ctypes.c_int] + [_f32p] * 4 + [_f64p] * 4 + \
            [ctypes.c_int64] * 7 + [ctypes.c_int]
        lib.oracle_project.restype = ctypes.c_int
        lib.oracle_project.argtypes = [ctypes.c_int] + [_f32p] * 5 + [_f64p] * 4 + \
            [ctypes.c_int64] * 7 + [ctypes.c_int]
        lib.oracle_backward.restype = ctypes.c_int
        lib.oracle_backward.argtypes = [ctypes.c_int] + [_f32p] * 8 + [_f64p] * 7 + \
            [ctypes.c_int64] * 5 + [ctypes.c_int]
        lib.oracle_backward_ex.restype = ctypes.c_int
        lib.oracle_backward_ex.argtypes = [ctypes.c_int] + [_f32p] * 8 + [ctypes.c_int, _f32p] + \
            [_f64p] * 8 + [ctypes.c_int64] * 5 + [ctypes.c_int]
        lib.oracle_backward_routes_ex.restype = ctypes.c_int
        lib.oracle_backward_routes_ex.argtypes = lib.oracle_backward_ex.argtypes
        self.lib = lib
        self.last_threads = None

    # -- argument marshalling -----------------------------------------------------------
    @staticmethod
    def _f32(a):
        a = np.ascontiguousarray(a, dtype=np.float32)
        return a, a.ctypes.data_as(_f32p)

    def _prep(self, K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, xshape=None):
        """Checks shapes against x's (or xshape's, when x is None) and returns the dims, the
        float32 copies and their pointers (None for a missing x)."""
        shape = tuple(np.shape(x)) if x is not None else tuple(xshape)
        if K == 4:
            if len(shape) != 4:
                raise ValueError("x must be (B, D, H, W)")
            B, D, H, W = shape
        else:
            if len(shape) != 3:
                raise ValueError("x must be (B, D, L)")
            B, D, L = shape
            H, W = 1, L
        L = H * W
        N = np.asarray(A_log).shape[-1]
        shapes = dict(dt_raw=(B, K, D, L), A_log=(K, D, N), Bs=(B, K, N, L), Cs=(B, K, N, L),
                      Ds=(K, D), dt_bias=(K, D))
        arrs = dict(dt_raw=dt_raw, A_log=A_log, Bs=Bs, Cs=Cs, Ds=Ds, dt_bias=dt_bias)
        for k, shp in shapes.items():
            if tuple(np.shape(arrs[k])) != shp:
                raise ValueError(f"{k} has shape {np.shape(arrs[k])}, expected {shp}")
        keep, ptrs = [], []
        for a in (x, dt_raw, A_log, Bs, Cs, Ds, dt_bias):
            a2, p = self._f32(a) if a is not None else (None, None)
            keep.append(a2)
            ptrs.append(p)
        return (B, D, H, W, N), keep, ptrs

    def _gate(self, z, x):
        """The optional gate z (same shape as x) as a float32 pointer, or NULL."""
        if z is None:
            return None, None
        z = np.ascontiguousarray(z, dtype=np.float32)
        if z.shape != np.shape(x):
            raise ValueError(f"z has shape {z.shape}, expected {np.shape(x)}")
        return z, z.ctypes.data_as(_f32p)

    # -- public calls -----------------------------------------------------------------
    # z: optional gate (shape of x), each route's output times SiLU(z); zoh: zero-order
    # hold for B ((exp(delta A) - 1) / A * B instead of delta * B).
    def forward(self, K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, threads=0, z=None,
                zoh=False):
        (B, D, H, W, N), keep, ptrs = self._prep(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias)
        zkeep, zp = self._gate(z, x)
        y = np.empty((B, D, H * W), dtype=np.float64)
        rc = self.lib.oracle_forward_ex(K, *ptrs, zp, ORACLE_ZOH if zoh else 0,
                                        y.ctypes.data_as(_f64p), B, D, H, W, N, int(threads))
        if rc < 0:
            raise RuntimeError("oracle_forward rejected its arguments")
        self.last_threads = rc
        return y.reshape(np.shape(x))

    def forward_channels(self, K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, b_idx, d_idx,
                         threads=0, z=None, zoh=False):
        (B, D, H, W, N), keep, ptrs = self._prep(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias)
        zkeep, zp = self._gate(z, x)
        bi = np.ascontiguousarray(b_idx, dtype=np.int64)
        di = np.ascontiguousarray(d_idx, dtype=np.int64)
        if bi.shape != di.shape or bi.ndim != 1:
            raise ValueError("b_idx and d_idx must be 1-D and of equal length")
        y = np.empty((bi.size, H * W), dtype=np.float64)
        rc = self.lib.oracle_forward_channels_ex(K, *ptrs, zp, ORACLE_ZOH if zoh else 0,
                                                 B, D, H, W, N,
                                                 bi.ctypes.data_as(_i64p),
                                                 di.ctypes.data_as(_i64p), bi.size,
                                                 y.ctypes.data_as(_f64p), int(threads))
        if rc < 0:
            raise RuntimeError("oracle_forward_channels rejected its arguments")
        self.last_threads = rc
        return y.reshape((bi.size,) + tuple(np.shape(x)[2:]))

    def forward_routes(self, K, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, H, W, threads=0,
                       z=None, zoh=False):
        """y (B, D, H, W) when each route brings its own input u (B, K, D, L), in scan order
        (K = 2: H = 1, y is (B, D, W))."""
        u = np.asarray(u)
        if u.ndim != 4 or u.shape[1] != K or u.shape[3] != H * W:
            raise ValueError(f"u has shape {u.shape}, expected (B, {K}, D, {H * W})")
        B, _, D, L = u.shape
        xshape = (B, D, H, W) if K == 4 else (B, D, L)
        (_, _, _, _, N), keep, ptrs = self._prep(K, None, dt_raw, A_log, Bs, Cs, Ds, dt_bias,
                                                 xshape=xshape)
        uk, up = self._f32(u)
        zkeep, zp = self._gate(z, np.broadcast_to(np.float32(0), xshape))
        y = np.empty((B, D, L), dtype=np.float64)
        rc = self.lib.oracle_forward_routes_ex(K, up, *ptrs[1:], zp, ORACLE_ZOH if zoh else 0,
                                               y.ctypes.data_as(_f64p), B, D, H, W, N,
                                               int(threads))
        if rc < 0:
            raise RuntimeError("oracle_forward_routes_ex rejected its arguments")
        self.last_threads = rc
        return y.reshape(xshape)

    def backward_routes(self, K, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, H, W, threads=0,
                        z=None, zoh=False):
        """Gradients of sum(dy * y) for y = forward_routes(...), float64, as a dict with keys
        u (B, K, D, L: each route's own input, per step), dt_raw, A_log, Bs, Cs, Ds, dt_bias,
        and z (with the gate)."""
        u = np.asarray(u)
        if u.ndim != 4 or u.shape[1] != K or u.shape[3] != H * W:
            raise ValueError(f"u has shape {u.shape}, expected (B, {K}, D, {H * W})")
        B, _, D, L = u.shape
        xshape = (B, D, H, W) if K == 4 else (B, D, L)
        (_, _, _, _, N), keep, ptrs = self._prep(K, None, dt_raw, A_log, Bs, Cs, Ds, dt_bias,
                                                 xshape=xshape)
        uk, up = self._f32(u)
        ref = np.broadcast_to(np.float32(0), xshape)
        dyk, dyp = self._gate(dy, ref)
        if dyp is None:
            raise ValueError("dy is required")
        zk, zp = self._gate(z, ref)
        out = dict(u=np.empty((B, K, D, L)), dt_raw=np.empty((B, K, D, L)),
                   A_log=np.empty((K, D, N)), Bs=np.empty((B, K, N, L)),
                   Cs=np.empty((B, K, N, L)), Ds=np.empty((K, D)), dt_bias=np.empty((K, D)))
        order = ("u", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
        dzp = None
        if zp is not None:
            out["z"] = np.empty((B, D, L))
            dzp = out["z"].ctypes.data_as(_f64p)
        rc = self.lib.oracle_backward_routes_ex(K, up, *ptrs[1:], zp, ORACLE_ZOH if zoh else 0,
                                                dyp, *[out[k].ctypes.data_as(_f64p)
                                                       for k in order],
                                                dzp, B, D, H, W, N, int(threads))
        if rc < 0:
            raise RuntimeError("oracle_backward_routes_ex rejected its arguments")
        self.last_threads = rc
        if zp is not None:
            out["z"] = out["z"].reshape(xshape)
        return out

    def forward_routes_lr(self, K, u, dt_lr, dt_w, A_log, Bs, Cs, Ds, dt_bias, H, W,
                          threads=0, z=None, zoh=False):
        """forward_routes with dt_proj folded in: dt_raw = dt_w[k] @ dt_lr[b, k] per step,
        dt_lr (B, K, R, L) the first R rows of x_proj's output, dt_w (K, D, R)."""
        u = np.asarray(u)
        if u.ndim != 4 or u.shape[1] != K or u.shape[3] != H * W:
            raise ValueError(f"u has shape {u.shape}, expected (B, {K}, D, {H * W})")
        B, _, D, L = u.shape
        R = np.shape(dt_w)[-1]
        if tuple(np.shape(dt_w)) != (K, D, R) or tuple(np.shape(dt_lr)) != (B, K, R, L):
            raise ValueError("dt_w must be (K, D, R) and dt_lr (B, K, R, L)")
        xshape = (B, D, H, W) if K == 4 else (B, D, L)
        dt_stand_in = np.broadcast_to(np.float32(0), (B, K, D, L))
        (_, _, _, _, N), keep, ptrs = self._prep(K, None, dt_stand_in, A_log, Bs, Cs, Ds,
                                                 dt_bias, xshape=xshape)
        uk, up = self._f32(u)
        lk, lp = self._f32(dt_lr)
        wk, wp = self._f32(dt_w)
        zkeep, zp = self._gate(z, np.broadcast_to(np.float32(0), xshape))
        y = np.empty((B, D, L), dtype=np.float64)
        rc = self.lib.oracle_forward_routes_lr_ex(K, up, lp, wp, R, *ptrs[2:], zp,
                                                  ORACLE_ZOH if zoh else 0,
                                                  y.ctypes.data_as(_f64p), B, D, H, W, N,
                                                  int(threads))
        if rc < 0:
            raise RuntimeError("oracle_forward_routes_lr_ex rejected its arguments")
        self.last_threads = rc
        return y.reshape(xshape)

    def project_lr(self, K, x, conv_w, conv_b, x_proj_w, R, threads=0):
        """project without dt_proj: dict of u (B, K, D, L), dt_lr (B, K, R, L) = the first R
        rows of x_proj's output, Bs, Cs (B, K, N, L)."""
        dt_w_dummy = np.zeros((K, np.shape(x)[1], R), np.float32)
        full = self.project(K, x, conv_w, conv_b, x_proj_w, dt_w_dummy, threads=threads,
                            _lr=True)
        return full

    def project(self, K, x, conv_w, conv_b, x_proj_w, dt_proj_w, threads=0, _lr=False):
        """Per-route front end: dict of u, dt_raw (B, K, D, L) and Bs, Cs (B, K, N, L) in scan
        order, float64.  conv_w (K, D, KW), conv_b (K, D), x_proj_w (K, R + 2N, D),
        dt_proj_w (K, D, R)."""
        x = np.asarray(x)
        if K == 4:
            if x.ndim != 4:
                raise ValueError("x must be (B, D, H, W)")
            B, D, H, W = x.shape
        else:
            if x.ndim != 3:
                raise ValueError("x must be (B, D, L)")
            B, D, W = x.shape
            H = 1
        L = H * W
        KW = np.shape(conv_w)[-1]
        R = np.shape(dt_proj_w)[-1]
        M = np.shape(x_proj_w)[1]
        N = (M - R) // 2
        if N <= 0 or M != R + 2 * N:
            raise ValueError("x_proj_w must have R + 2N rows")
        shapes = dict(conv_w=(K, D, KW), conv_b=(K, D), x_proj_w=(K, M, D), dt_proj_w=(K, D, R))
        arrs = dict(conv_w=conv_w, conv_b=conv_b, x_proj_w=x_proj_w, dt_proj_w=dt_proj_w)
        for k, shp in shapes.items():
            if tuple(np.shape(arrs[k])) != shp:
                raise ValueError(f"{k} has shape {np.shape(arrs[k])}, expected {shp}")
        keep, ptrs = [], []
        for a in (x, conv_w, conv_b, x_proj_w, dt_proj_w):
            a2, p = self._f32(a)
            keep.append(a2)
            ptrs.append(p)
        if _lr:
            out = dict(u=np.empty((B, K, D, L)), dt_lr=np.empty((B, K, R, L)),
                       Bs=np.empty((B, K, N, L)), Cs=np.empty((B, K, N, L)))
            rc = self.lib.oracle_project_lr(K, *ptrs[:4],
                                            *[out[k].ctypes.data_as(_f64p)
                                              for k in ("u", "dt_lr", "Bs", "Cs")],
                                            B, D, H, W, N, R, KW, int(threads))
        else:
            out = dict(u=np.empty((B, K, D, L)), dt_raw=np.empty((B, K, D, L)),
                       Bs=np.empty((B, K, N, L)), Cs=np.empty((B, K, N, L)))
            rc = self.lib.oracle_project(K, *ptrs,
                                         *[out[k].ctypes.data_as(_f64p)
                                           for k in ("u", "dt_raw", "Bs", "Cs")],
                                         B, D, H, W, N, R, KW, int(threads))
        if rc < 0:
            raise RuntimeError("oracle_project rejected its arguments")
        self.last_threads = rc
        return out

    def backward(self, K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, threads=0, z=None,
                 zoh=False):
        """Gradients of sum(dy * y), float64, as a dict with keys x, dt_raw, A_log, Bs, Cs,
        Ds, dt_bias (each the shape of that input).  With the gate z (shape of x), y is the
        gated output and the dict also holds z's gradient under "z"; zoh: y is the
        zero-order-hold operator's output."""
        (B, D, H, W, N), keep, ptrs = self._prep(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias)
        dyk, dyp = self._gate(dy, x)
        if dyp is None:
            raise ValueError("dy is required")
        zk, zp = self._gate(z, x)
        L = H * W
        out = dict(x=np.empty((B, D, L)), dt_raw=np.empty((B, K, D, L)),
                   A_log=np.empty((K, D, N)), Bs=np.empty((B, K, N, L)),
                   Cs=np.empty((B, K, N, L)), Ds=np.empty((K, D)), dt_bias=np.empty((K, D)))
        order = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")
        outs = [out[k].ctypes.data_as(_f64p) for k in order]
        if zp is None and not zoh:
            rc = self.lib.oracle_backward(K, *ptrs, dyp, *outs, B, D, H, W, N, int(threads))
        else:
            dzp = None
            if zp is not None:
                out["z"] = np.empty((B, D, L))
                dzp = out["z"].ctypes.data_as(_f64p)
            rc = self.lib.oracle_backward_ex(K, *ptrs, zp, 1 if zoh else 0, dyp, *outs, dzp,
                                             B, D, H, W, N, int(threads))
        if rc < 0:
            raise RuntimeError("oracle_backward rejected its arguments")
        self.last_threads = rc
        out["x"] = out["x"].reshape(np.shape(x))
        if zp is not None:
            out["z"] = out["z"].reshape(np.shape(x))
        return out


_DEFAULT = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def ss2d_forward(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, threads=0, z=None, zoh=False):
    """y (B, D, H, W), float64, of the four-route SS2D forward operator."""
    return default().forward(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, threads, z=z, zoh=zoh)


def ss1d_bidir_forward(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, threads=0, z=None, zoh=False):
    """y (B, D, L), float64, of the bidirectional (forward + reversed) 1D scan."""
    return default().forward(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, threads, z=z, zoh=zoh)


def forward_channels(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, b_idx, d_idx, threads=0,
                     z=None, zoh=False):
    """Output planes of the selected (b, d) channels only."""
    return default().forward_channels(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, b_idx, d_idx,
                                      threads, z=z, zoh=zoh)


def ss2d_project(x, conv_w, conv_b, x_proj_w, dt_proj_w, threads=0):
    """Per-route front end of the four-route operator (dict u, dt_raw, Bs, Cs), float64."""
    return default().project(4, x, conv_w, conv_b, x_proj_w, dt_proj_w, threads)


def ss1d_bidir_project(x, conv_w, conv_b, x_proj_w, dt_proj_w, threads=0):
    """Per-path front end of the bidirectional 1D operator (dict u, dt_raw, Bs, Cs)."""
    return default().project(2, x, conv_w, conv_b, x_proj_w, dt_proj_w, threads)
