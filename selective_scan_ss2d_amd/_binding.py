"""ctypes binding of libss2d.so.

Argument marshalling only: shapes, dtypes and devices are checked, device pointers and the
current HIP stream are passed through, and every step of the operator runs in the library's
HIP kernels.  PyTorch supplies device memory and streams.  There is no fallback: when the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import pathlib
import threading

PKG = pathlib.Path(__file__).resolve().parent
LIBRARY_PATH = PKG / "libss2d.so"

SS2D_OK = 0
SS2D_ERR_NULL = 1
SS2D_ERR_SHAPE = 2
SS2D_ERR_UNSUPPORTED = 3
SS2D_ERR_ALIGN = 4
SS2D_ERR_HIP = 5
SS2D_ERR_ALIAS = 6
SS2D_ERR_SCRATCH = 7
SS2D_F32 = 0
SS2D_BF16 = 1
SS2D_FLAG_ZOH = 1

# Every symbol include/ss2d.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "ss2d_forward": (ctypes.c_int, [_P] * 8 + [_I64] * 5 + [ctypes.c_int, _P]),
    "ss1d_bidir_forward": (ctypes.c_int, [_P] * 8 + [_I64] * 4 + [ctypes.c_int, _P]),
    "ss2d_forward_ex": (ctypes.c_int, [_P] * 9 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss1d_bidir_forward_ex": (ctypes.c_int, [_P] * 9 + [_I64] * 4 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_forward_noalloc": (ctypes.c_int, [_P] * 9 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_backward": (ctypes.c_int, [_P] * 15 + [_I64] * 5 + [ctypes.c_int, _P]),
    "ss1d_bidir_backward": (ctypes.c_int, [_P] * 15 + [_I64] * 4 + [ctypes.c_int, _P]),
    "ss2d_backward_ex": (ctypes.c_int, [_P] * 17 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss1d_bidir_backward_ex": (ctypes.c_int, [_P] * 17 + [_I64] * 4 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_backward_routes": (ctypes.c_int, [_P] * 17 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss1d_bidir_backward_routes": (ctypes.c_int,
                                   [_P] * 17 + [_I64] * 4 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_project": (ctypes.c_int, [_P] * 9 + [_I64] * 7 + [ctypes.c_int, _P]),
    "ss1d_bidir_project": (ctypes.c_int, [_P] * 9 + [_I64] * 6 + [ctypes.c_int, _P]),
    "ss2d_forward_routes": (ctypes.c_int, [_P] * 9 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss1d_bidir_forward_routes": (ctypes.c_int,
                                  [_P] * 9 + [_I64] * 4 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_project_lr": (ctypes.c_int, [_P] * 8 + [_I64] * 7 + [ctypes.c_int, _P]),
    "ss1d_bidir_project_lr": (ctypes.c_int, [_P] * 8 + [_I64] * 6 + [ctypes.c_int, _P]),
    "ss2d_forward_routes_lr": (ctypes.c_int,
                               [_P] * 10 + [_I64] * 6 + [ctypes.c_int] * 2 + [_P]),
    "ss1d_bidir_forward_routes_lr": (ctypes.c_int,
                                     [_P] * 10 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_saved_state_bytes": (_I64, [ctypes.c_int] + [_I64] * 4 + [ctypes.c_int]),
    "ss2d_forward_save": (ctypes.c_int, [_P] * 10 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss1d_bidir_forward_save": (ctypes.c_int,
                                [_P] * 10 + [_I64] * 4 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_backward_saved": (ctypes.c_int, [_P] * 18 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss1d_bidir_backward_saved": (ctypes.c_int,
                                  [_P] * 18 + [_I64] * 4 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_forward_routes_save": (ctypes.c_int,
                                 [_P] * 10 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss1d_bidir_forward_routes_save": (ctypes.c_int,
                                       [_P] * 10 + [_I64] * 4 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_backward_routes_saved": (ctypes.c_int,
                                   [_P] * 18 + [_I64] * 5 + [ctypes.c_int] * 2 + [_P]),
    "ss1d_bidir_backward_routes_saved": (ctypes.c_int,
                                         [_P] * 18 + [_I64] * 4 + [ctypes.c_int] * 2 + [_P]),
    "ss2d_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ss2d_abi_version": (ctypes.c_int, []),
    "ss2d_last_hip_error": (ctypes.c_int, []),
    "ss2d_set_launch_plan": (ctypes.c_int, [ctypes.c_int, _I64]),
    "ss2d_scratch_trim": (ctypes.c_int, [ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]),
    "ss2d_probe_issue_rates": (ctypes.c_int, [_P, _P]),
    "ss2d_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "ss2d_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]),
}
KERNEL_KINDS = ("transpose", "scan", "chunk_agg", "carry", "merge", "checkpoint", "scan_bwd",
                "reduce", "project")


class SS2DError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None
_lock = threading.Lock()


def load_library(path: pathlib.Path | str | None = None) -> ctypes.CDLL:
    """Load libss2d.so (once) and attach signatures.  Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = pathlib.Path(path) if path is not None else LIBRARY_PATH
        if not p.exists():
            raise RuntimeError(
                f"{p} is not built; run `python -m selective_scan_ss2d_amd.build` "
                "(the SS2D operator has no fallback path)")
        lib = ctypes.CDLL(str(p))
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def abi_version() -> int:
    return load_library().ss2d_abi_version()


def scratch_trim(keep_bytes: int = 0) -> int:
    """Hand the library's pooled scratch on the current device beyond keep_bytes back to
    the driver; returns the bytes it still reserves.  Synchronise the streams of earlier
    calls first: scratch still in use stays reserved."""
    if keep_bytes < 0:
        raise ValueError("keep_bytes must be >= 0")
    reserved = ctypes.c_size_t(0)
    _check(load_library().ss2d_scratch_trim(int(keep_bytes), ctypes.byref(reserved)))
    return int(reserved.value)


def status_string(status: int) -> str:
    return load_library().ss2d_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != SS2D_OK:
        lib = load_library()
        msg = lib.ss2d_status_string(status).decode()
        if status == SS2D_ERR_HIP:
            msg += f" (hipError_t {lib.ss2d_last_hip_error()})"
        raise SS2DError(status, msg)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SS2D_F32
    if t.dtype == torch.bfloat16:
        return SS2D_BF16
    raise TypeError(f"x must be float32 or bfloat16, not {t.dtype}")


def _expect(name, t, shape, dtype, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device, stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _common(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, y, xshape, L):
    torch = _torch()
    if x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    B, D = x.shape[0], x.shape[1]
    N = A_log.shape[-1] if A_log.dim() == 3 else -1
    dt = x.dtype
    _dtype_code(x)
    dev = x.device
    _expect("x", x, xshape, dt, dev)
    _expect("dt_raw", dt_raw, (B, K, D, L), dt, dev)
    _expect("A_log", A_log, (K, D, N), torch.float32, dev)
    _expect("Bs", Bs, (B, K, N, L), dt, dev)
    _expect("Cs", Cs, (B, K, N, L), dt, dev)
    _expect("Ds", Ds, (K, D), torch.float32, dev)
    _expect("dt_bias", dt_bias, (K, D), torch.float32, dev)
    if y is None:
        y = torch.empty(xshape, dtype=dt, device=dev)
    else:
        _expect("y", y, xshape, dt, dev)
    return B, D, N, y


def ss2d_forward(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, y=None, stream=None):
    """Four-route SS2D forward on the GPU.

    x (B, D, H, W); dt_raw (B, 4, D, L); Bs, Cs (B, 4, N, L) in each route's scan order;
    A_log (4, D, N), Ds (4, D), dt_bias (4, D) fp32.  x, dt_raw, Bs, Cs (and y) share one
    dtype, float32 or bfloat16.  Returns y (B, D, H, W), enqueued on the current stream.
    """
    lib = load_library()
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    B, D, H, W = x.shape
    B, D, N, y = _common(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, y, (B, D, H, W), H * W)
    status = lib.ss2d_forward(x.data_ptr(), dt_raw.data_ptr(), A_log.data_ptr(),
                              Bs.data_ptr(), Cs.data_ptr(), Ds.data_ptr(), dt_bias.data_ptr(),
                              y.data_ptr(), B, D, H, W, N, _dtype_code(x),
                              _stream_handle(x.device, stream))
    _check(status)
    return y


def ss1d_bidir_forward(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, y=None, stream=None):
    """Bidirectional (forward + reversed) 1D selective scan on the GPU.

    x (B, D, L); dt_raw (B, 2, D, L); Bs, Cs (B, 2, N, L); A_log (2, D, N), Ds (2, D),
    dt_bias (2, D) fp32.  Returns y (B, D, L).
    """
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    B, D, L = x.shape
    B, D, N, y = _common(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, y, (B, D, L), L)
    status = lib.ss1d_bidir_forward(x.data_ptr(), dt_raw.data_ptr(), A_log.data_ptr(),
                                    Bs.data_ptr(), Cs.data_ptr(), Ds.data_ptr(),
                                    dt_bias.data_ptr(), y.data_ptr(), B, D, L, N,
                                    _dtype_code(x), _stream_handle(x.device, stream))
    _check(status)
    return y


def _gate_ptr(z, xshape, x):
    """Device pointer of the optional gate (None -> NULL), checked like the other inputs."""
    if z is None:
        return None
    _expect("z", z, xshape, x.dtype, x.device)
    return z.data_ptr()


def ss2d_forward_ex(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z=None, zoh=False, y=None,
                    stream=None):
    """ss2d_forward with the two options of the C entry point of the same name.

    z: optional gate, shape and dtype of x; the output is multiplied by SiLU(z) before its
    single rounding.  zoh: zero-order hold for B ((exp(delta A) - 1) / A * B instead of
    delta * B).
    """
    lib = load_library()
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    B, D, H, W = x.shape
    B, D, N, y = _common(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, y, (B, D, H, W), H * W)
    zp = _gate_ptr(z, (B, D, H, W), x)
    status = lib.ss2d_forward_ex(x.data_ptr(), dt_raw.data_ptr(), A_log.data_ptr(),
                                 Bs.data_ptr(), Cs.data_ptr(), Ds.data_ptr(),
                                 dt_bias.data_ptr(), zp, y.data_ptr(), B, D, H, W, N,
                                 _dtype_code(x), SS2D_FLAG_ZOH if zoh else 0,
                                 _stream_handle(x.device, stream))
    _check(status)
    return y


def ss1d_bidir_forward_ex(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z=None, zoh=False, y=None,
                          stream=None):
    """ss1d_bidir_forward with the gate z and the zero-order-hold option."""
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    B, D, L = x.shape
    B, D, N, y = _common(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, y, (B, D, L), L)
    zp = _gate_ptr(z, (B, D, L), x)
    status = lib.ss1d_bidir_forward_ex(x.data_ptr(), dt_raw.data_ptr(), A_log.data_ptr(),
                                       Bs.data_ptr(), Cs.data_ptr(), Ds.data_ptr(),
                                       dt_bias.data_ptr(), zp, y.data_ptr(), B, D, L, N,
                                       _dtype_code(x), SS2D_FLAG_ZOH if zoh else 0,
                                       _stream_handle(x.device, stream))
    _check(status)
    return y


def _routes_forward(K, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, stream, xshape,
                    dt_w=None, save=False, saved=None):
    """dt_w given: dt_raw is the low-rank dt_lr (B, K, R, L), multiplied by dt_w (K, D, R)
    inside the scan.  save: the training forward, returning (y, saved)."""
    torch = _torch()
    lib = load_library()
    if u.device.type != "cuda":
        raise ValueError("u must be a GPU tensor")
    B, D, L = xshape[0], xshape[1], u.shape[-1]
    N = A_log.shape[-1] if A_log.dim() == 3 else -1
    dt, dev = u.dtype, u.device
    _dtype_code(u)
    _expect("u", u, (B, K, D, L), dt, dev)
    if dt_w is None:
        _expect("dt_raw", dt_raw, (B, K, D, L), dt, dev)
    else:
        if dt_w.dim() != 3:
            raise ValueError("dt_w must be (K, D, R)")
        R = dt_w.shape[-1]
        _expect("dt_w", dt_w, (K, D, R), torch.float32, dev)
        _expect("dt_lr", dt_raw, (B, K, R, L), dt, dev)
    _expect("A_log", A_log, (K, D, N), torch.float32, dev)
    _expect("Bs", Bs, (B, K, N, L), dt, dev)
    _expect("Cs", Cs, (B, K, N, L), dt, dev)
    _expect("Ds", Ds, (K, D), torch.float32, dev)
    _expect("dt_bias", dt_bias, (K, D), torch.float32, dev)
    if y is None:
        y = torch.empty(xshape, dtype=dt, device=dev)
    else:
        _expect("y", y, xshape, dt, dev)
    zp = _gate_ptr(z, xshape, u)
    common = (A_log.data_ptr(), Bs.data_ptr(), Cs.data_ptr(), Ds.data_ptr(),
              dt_bias.data_ptr(), zp, y.data_ptr(), *xshape[:2], *xshape[2:], N)
    tail = (_dtype_code(u), SS2D_FLAG_ZOH if zoh else 0, _stream_handle(dev, stream))
    if save:
        saved = _saved_tensor(saved, saved_state_bytes(K, B, D, L, N, z is not None), dev)
        fn = lib.ss2d_forward_routes_save if K == 4 else lib.ss1d_bidir_forward_routes_save
        common = common[:6] + (y.data_ptr(), saved.data_ptr()) + common[7:]
        _check(fn(u.data_ptr(), dt_raw.data_ptr(), *common, *tail))
        return y, saved
    if dt_w is None:
        fn = lib.ss2d_forward_routes if K == 4 else lib.ss1d_bidir_forward_routes
        status = fn(u.data_ptr(), dt_raw.data_ptr(), *common, *tail)
    else:
        fn = lib.ss2d_forward_routes_lr if K == 4 else lib.ss1d_bidir_forward_routes_lr
        status = fn(u.data_ptr(), dt_raw.data_ptr(), dt_w.data_ptr(), *common, dt_w.shape[-1],
                    *tail)
    _check(status)
    return y


def ss2d_forward_routes(u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, H, W, z=None, zoh=False,
                        y=None, stream=None):
    """ss2d_forward_ex with each route's own input u (B, 4, D, L), in scan order, in place of
    the gathered x.  Returns y (B, D, H, W)."""
    if u.dim() != 4:
        raise ValueError("u must be (B, 4, D, L)")
    if u.shape[-1] != H * W:
        raise ValueError(f"u has {u.shape[-1]} steps, expected H * W = {H * W}")
    return _routes_forward(4, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, stream,
                           (u.shape[0], u.shape[2], H, W))


def ss1d_bidir_forward_routes(u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z=None, zoh=False,
                              y=None, stream=None):
    """ss1d_bidir_forward_ex with each path's own input u (B, 2, D, L).  Returns y (B, D, L)."""
    if u.dim() != 4:
        raise ValueError("u must be (B, 2, D, L)")
    return _routes_forward(2, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, stream,
                           (u.shape[0], u.shape[2], u.shape[3]))


def ss2d_forward_routes_lr(u, dt_lr, dt_w, A_log, Bs, Cs, Ds, dt_bias, H, W, z=None,
                           zoh=False, y=None, stream=None):
    """ss2d_forward_routes with dt_proj folded into the scan: each step's dt_raw is
    dt_w (4, D, R) fp32 times the step's column of dt_lr (B, 4, R, L).  Returns y (B, D, H, W)."""
    if u.dim() != 4:
        raise ValueError("u must be (B, 4, D, L)")
    if u.shape[-1] != H * W:
        raise ValueError(f"u has {u.shape[-1]} steps, expected H * W = {H * W}")
    return _routes_forward(4, u, dt_lr, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, stream,
                           (u.shape[0], u.shape[2], H, W), dt_w=dt_w)


def ss1d_bidir_forward_routes_lr(u, dt_lr, dt_w, A_log, Bs, Cs, Ds, dt_bias, z=None,
                                 zoh=False, y=None, stream=None):
    """ss1d_bidir_forward_routes with dt_proj folded into the scan (dt_lr (B, 2, R, L),
    dt_w (2, D, R)).  Returns y (B, D, L)."""
    if u.dim() != 4:
        raise ValueError("u must be (B, 2, D, L)")
    return _routes_forward(2, u, dt_lr, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, stream,
                           (u.shape[0], u.shape[2], u.shape[3]), dt_w=dt_w)


def _project(K, x, conv_w, conv_b, x_proj_w, dt_proj_w, stream, xshape, R=None):
    """dt_proj_w None: the low-rank variant with R dt rows, returning dt_lr for dt_raw."""
    torch = _torch()
    lib = load_library()
    if x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    B, D = xshape[0], xshape[1]
    L = 1
    for v in xshape[2:]:
        L *= v
    dt, dev = x.dtype, x.device
    _dtype_code(x)
    lr = dt_proj_w is None
    if conv_w.dim() != 3 or x_proj_w.dim() != 3 or (not lr and dt_proj_w.dim() != 3):
        raise ValueError("conv_w, x_proj_w and dt_proj_w must be 3-D")
    if not lr:
        R = dt_proj_w.shape[-1]
    KW, M = conv_w.shape[-1], x_proj_w.shape[1]
    N = (M - R) // 2
    if N < 1 or M != R + 2 * N:
        raise ValueError(f"x_proj_w has {M} rows, expected R + 2N with R = {R}")
    _expect("x", x, xshape, dt, dev)
    _expect("conv_w", conv_w, (K, D, KW), torch.float32, dev)
    _expect("conv_b", conv_b, (K, D), torch.float32, dev)
    _expect("x_proj_w", x_proj_w, (K, M, D), torch.float32, dev)
    if not lr:
        _expect("dt_proj_w", dt_proj_w, (K, D, R), torch.float32, dev)
    dt_name = "dt_lr" if lr else "dt_raw"
    out = {"u": torch.empty((B, K, D, L), dtype=dt, device=dev),
           dt_name: torch.empty((B, K, R if lr else D, L), dtype=dt, device=dev),
           "Bs": torch.empty((B, K, N, L), dtype=dt, device=dev),
           "Cs": torch.empty((B, K, N, L), dtype=dt, device=dev)}
    outs = [out[k].data_ptr() for k in ("u", dt_name, "Bs", "Cs")]
    tail = (*xshape, N, R, KW, _dtype_code(x), _stream_handle(dev, stream))
    if lr:
        fn = lib.ss2d_project_lr if K == 4 else lib.ss1d_bidir_project_lr
        status = fn(x.data_ptr(), conv_w.data_ptr(), conv_b.data_ptr(), x_proj_w.data_ptr(),
                    *outs, *tail)
    else:
        fn = lib.ss2d_project if K == 4 else lib.ss1d_bidir_project
        status = fn(x.data_ptr(), conv_w.data_ptr(), conv_b.data_ptr(), x_proj_w.data_ptr(),
                    dt_proj_w.data_ptr(), *outs, *tail)
    _check(status)
    return out


def ss2d_project(x, conv_w, conv_b, x_proj_w, dt_proj_w, stream=None):
    """Per-route front end on the GPU: causal depthwise conv + SiLU, x_proj and dt_proj of
    each of the four routes.  x (B, D, H, W) float32 or bfloat16; conv_w (4, D, KW),
    conv_b (4, D), x_proj_w (4, R + 2N, D), dt_proj_w (4, D, R) fp32.  Returns a dict of
    u, dt_raw (B, 4, D, L) and Bs, Cs (B, 4, N, L) in each route's scan order, dtype of x."""
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    return _project(4, x, conv_w, conv_b, x_proj_w, dt_proj_w, stream, tuple(x.shape))


def ss1d_bidir_project(x, conv_w, conv_b, x_proj_w, dt_proj_w, stream=None):
    """ss2d_project for the two paths (forward, reversed) of a 1D sequence x (B, D, L)."""
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    return _project(2, x, conv_w, conv_b, x_proj_w, dt_proj_w, stream, tuple(x.shape))


def ss2d_project_lr(x, conv_w, conv_b, x_proj_w, R, stream=None):
    """ss2d_project without dt_proj: returns u, Bs, Cs as there and dt_lr (B, 4, R, L), the
    R dt rows of x_proj's output, for ss2d_forward_routes_lr."""
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    return _project(4, x, conv_w, conv_b, x_proj_w, None, stream, tuple(x.shape), R=int(R))


def ss1d_bidir_project_lr(x, conv_w, conv_b, x_proj_w, R, stream=None):
    """ss1d_bidir_project without dt_proj (dt_lr (B, 2, R, L) in place of dt_raw)."""
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    return _project(2, x, conv_w, conv_b, x_proj_w, None, stream, tuple(x.shape), R=int(R))


GRAD_NAMES = ("x", "dt_raw", "A_log", "Bs", "Cs", "Ds", "dt_bias")


def _backward(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, stream, xshape, L, z=None,
              zoh=False, ex=False):
    torch = _torch()
    lib = load_library()
    B, D, N, _ = _common(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, xshape, L)
    ins = (x, dt_raw, A_log, Bs, Cs, Ds, dt_bias)
    grads = {name: torch.empty_like(t) for name, t in zip(GRAD_NAMES, ins)}
    dims = (B, D, xshape[2], xshape[3]) if K == 4 else (B, D, L)
    if not ex:
        args = [t.data_ptr() for t in ins] + [dy.data_ptr()] + \
            [grads[n].data_ptr() for n in GRAD_NAMES]
        fn = lib.ss2d_backward if K == 4 else lib.ss1d_bidir_backward
        _check(fn(*args, *dims, N, _dtype_code(x), _stream_handle(x.device, stream)))
        return grads
    if z is not None:
        _expect("z", z, xshape, x.dtype, x.device)
        grads["z"] = torch.empty_like(z)
    args = [t.data_ptr() for t in ins] + [None if z is None else z.data_ptr(), dy.data_ptr()] + \
        [grads[n].data_ptr() for n in GRAD_NAMES] + \
        [None if z is None else grads["z"].data_ptr()]
    fn = lib.ss2d_backward_ex if K == 4 else lib.ss1d_bidir_backward_ex
    _check(fn(*args, *dims, N, _dtype_code(x), SS2D_FLAG_ZOH if zoh else 0,
              _stream_handle(x.device, stream)))
    return grads


def ss2d_backward(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, stream=None):
    """Gradients of sum(dy * y) for y = ss2d_forward(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias).

    dy has the shape and dtype of x.  Returns a dict with the gradient of every input under
    its name (x, dt_raw, A_log, Bs, Cs, Ds, dt_bias), each of that input's shape and dtype.
    """
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    B, D, H, W = x.shape
    return _backward(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, stream, (B, D, H, W), H * W)


def ss1d_bidir_backward(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, stream=None):
    """Gradients of sum(dy * y) for y = ss1d_bidir_forward(...); see ss2d_backward."""
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    B, D, L = x.shape
    return _backward(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, stream, (B, D, L), L)


def ss2d_backward_ex(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, z=None, zoh=False,
                     stream=None):
    """Gradients of sum(dy * y) for y = ss2d_forward_ex(..., z=z, zoh=zoh): the dict of
    ss2d_backward, plus z's gradient under "z" (shape and dtype of z, which are x's) when
    the gate is given."""
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    B, D, H, W = x.shape
    return _backward(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, stream, (B, D, H, W), H * W,
                     z=z, zoh=zoh, ex=True)


def ss1d_bidir_backward_ex(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, z=None, zoh=False,
                           stream=None):
    """ss2d_backward_ex for y = ss1d_bidir_forward_ex(..., z=z, zoh=zoh)."""
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    B, D, L = x.shape
    return _backward(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, stream, (B, D, L), L, z=z,
                     zoh=zoh, ex=True)


def saved_state_bytes(K, B, D, L, N, gated=False) -> int:
    """Bytes of the state a training forward keeps for its backward (see ss2d_forward_save);
    raises ValueError for sizes the operator rejects or N not a multiple of 4."""
    n = load_library().ss2d_saved_state_bytes(int(K), int(B), int(D), int(L), int(N),
                                              1 if gated else 0)
    if n < 0:
        raise ValueError(f"no saved state for K={K}, B={B}, D={D}, L={L}, N={N}")
    return n


def _saved_tensor(saved, nbytes, device):
    """The saved-state buffer: fp32, contiguous, of exactly nbytes (allocated if None)."""
    torch = _torch()
    if saved is None:
        return torch.empty(nbytes // 4, dtype=torch.float32, device=device)
    _expect("saved", saved, (nbytes // 4,), torch.float32, device)
    return saved


def _forward_save(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, saved, stream, xshape,
                  L):
    lib = load_library()
    B, D, N, y = _common(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, y, xshape, L)
    zp = _gate_ptr(z, xshape, x)
    saved = _saved_tensor(saved, saved_state_bytes(K, B, D, L, N, z is not None), x.device)
    dims = (B, D, xshape[2], xshape[3]) if K == 4 else (B, D, L)
    fn = lib.ss2d_forward_save if K == 4 else lib.ss1d_bidir_forward_save
    _check(fn(x.data_ptr(), dt_raw.data_ptr(), A_log.data_ptr(), Bs.data_ptr(), Cs.data_ptr(),
              Ds.data_ptr(), dt_bias.data_ptr(), zp, y.data_ptr(), saved.data_ptr(), *dims, N,
              _dtype_code(x), SS2D_FLAG_ZOH if zoh else 0, _stream_handle(x.device, stream)))
    return y, saved


def ss2d_forward_save(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z=None, zoh=False, y=None,
                      saved=None, stream=None):
    """The training forward: y as ss2d_forward_ex(..., z=z, zoh=zoh), and the state its
    backward starts from (the scan's state before every 8-step quarter, and with the gate the
    ungated route sum), for ss2d_backward_saved.  Returns (y, saved); saved is an fp32
    tensor of saved_state_bytes(4, B, D, H * W, N, z is not None) / 4 elements."""
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    B, D, H, W = x.shape
    return _forward_save(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, saved, stream,
                         (B, D, H, W), H * W)


def ss1d_bidir_forward_save(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z=None, zoh=False, y=None,
                            saved=None, stream=None):
    """ss2d_forward_save for the bidirectional operator (K = 2)."""
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    B, D, L = x.shape
    return _forward_save(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, saved, stream,
                         (B, D, L), L)


def _backward_saved(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, saved, z, zoh, stream,
                    xshape, L):
    torch = _torch()
    lib = load_library()
    B, D, N, _ = _common(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, xshape, L)
    saved = _saved_tensor(saved, saved_state_bytes(K, B, D, L, N, z is not None), x.device)
    ins = (x, dt_raw, A_log, Bs, Cs, Ds, dt_bias)
    grads = {name: torch.empty_like(t) for name, t in zip(GRAD_NAMES, ins)}
    if z is not None:
        _expect("z", z, xshape, x.dtype, x.device)
        grads["z"] = torch.empty_like(z)
    args = [t.data_ptr() for t in ins] + [None if z is None else z.data_ptr(),
                                          saved.data_ptr(), dy.data_ptr()] + \
        [grads[n].data_ptr() for n in GRAD_NAMES] + \
        [None if z is None else grads["z"].data_ptr()]
    dims = (B, D, xshape[2], xshape[3]) if K == 4 else (B, D, L)
    fn = lib.ss2d_backward_saved if K == 4 else lib.ss1d_bidir_backward_saved
    _check(fn(*args, *dims, N, _dtype_code(x), SS2D_FLAG_ZOH if zoh else 0,
              _stream_handle(x.device, stream)))
    return grads


def ss2d_backward_saved(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, saved, z=None, zoh=False,
                        stream=None):
    """The gradients of ss2d_backward_ex(..., z=z, zoh=zoh), starting from the state that
    ss2d_forward_save kept in `saved` for the same inputs, gate and option."""
    if x.dim() != 4:
        raise ValueError("x must be (B, D, H, W)")
    B, D, H, W = x.shape
    return _backward_saved(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, saved, z, zoh, stream,
                           (B, D, H, W), H * W)


def ss1d_bidir_backward_saved(x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, saved, z=None,
                              zoh=False, stream=None):
    """ss2d_backward_saved for the bidirectional operator (K = 2)."""
    if x.dim() != 3:
        raise ValueError("x must be (B, D, L)")
    B, D, L = x.shape
    return _backward_saved(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, saved, z, zoh, stream,
                           (B, D, L), L)


def _backward_routes(K, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, xshape, z, zoh, stream,
                     saved=None):
    torch = _torch()
    lib = load_library()
    if u.device.type != "cuda":
        raise ValueError("u must be a GPU tensor")
    if u.dim() != 4 or u.shape[1] != K:
        raise ValueError(f"u must be (B, {K}, D, L)")
    B, _, D, L = u.shape
    N = A_log.shape[-1] if A_log.dim() == 3 else -1
    dt, dev = u.dtype, u.device
    _dtype_code(u)
    _expect("u", u, (B, K, D, L), dt, dev)
    _expect("dt_raw", dt_raw, (B, K, D, L), dt, dev)
    _expect("A_log", A_log, (K, D, N), torch.float32, dev)
    _expect("Bs", Bs, (B, K, N, L), dt, dev)
    _expect("Cs", Cs, (B, K, N, L), dt, dev)
    _expect("Ds", Ds, (K, D), torch.float32, dev)
    _expect("dt_bias", dt_bias, (K, D), torch.float32, dev)
    _expect("dy", dy, xshape, dt, dev)
    ins = (u, dt_raw, A_log, Bs, Cs, Ds, dt_bias)
    names = ("u",) + GRAD_NAMES[1:]
    grads = {name: torch.empty_like(t) for name, t in zip(names, ins)}
    if z is not None:
        _expect("z", z, xshape, u.dtype, u.device)
        grads["z"] = torch.empty_like(z)
    zp = [None if z is None else z.data_ptr()]
    if saved is not None:  # from the state ss2d_forward_routes_save kept
        saved = _saved_tensor(saved, saved_state_bytes(K, B, D, L, N, z is not None), dev)
        zp.append(saved.data_ptr())
        fn = lib.ss2d_backward_routes_saved if K == 4 else lib.ss1d_bidir_backward_routes_saved
    else:
        fn = lib.ss2d_backward_routes if K == 4 else lib.ss1d_bidir_backward_routes
    args = [t.data_ptr() for t in ins] + zp + [dy.data_ptr()] + \
        [grads[n].data_ptr() for n in names] + [None if z is None else grads["z"].data_ptr()]
    dims = (B, D, xshape[2], xshape[3]) if K == 4 else (B, D, L)
    _check(fn(*args, *dims, N, _dtype_code(u), SS2D_FLAG_ZOH if zoh else 0,
              _stream_handle(u.device, stream)))
    return grads


def ss2d_backward_routes(u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, H, W, z=None, zoh=False,
                         stream=None):
    """Gradients of sum(dy * y) for y = ss2d_forward_routes(u, ..., H, W, z=z, zoh=zoh): a
    dict with the gradient of every input under its name, u's per route and step (B, 4, D,
    L), and z's when the gate is given."""
    if u.dim() != 4:
        raise ValueError("u must be (B, 4, D, L)")
    if u.shape[-1] != H * W:  # the library reads and writes rows of H * W steps
        raise ValueError(f"u has {u.shape[-1]} steps, expected H * W = {H * W}")
    B, D = u.shape[0], u.shape[2]
    return _backward_routes(4, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, (B, D, H, W), z, zoh,
                            stream)


def ss1d_bidir_backward_routes(u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, z=None, zoh=False,
                               stream=None):
    """ss2d_backward_routes for y = ss1d_bidir_forward_routes(u, ...), u (B, 2, D, L)."""
    B, D, L = u.shape[0], u.shape[2], u.shape[3]
    return _backward_routes(2, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, (B, D, L), z, zoh,
                            stream)


def ss2d_forward_routes_save(u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, H, W, z=None, zoh=False,
                             y=None, saved=None, stream=None):
    """The training forward of the operator over per-route inputs: y as ss2d_forward_routes,
    and the state ss2d_backward_routes_saved starts from.  Returns (y, saved)."""
    if u.dim() != 4:
        raise ValueError("u must be (B, 4, D, L)")
    if u.shape[-1] != H * W:
        raise ValueError(f"u has {u.shape[-1]} steps, expected H * W = {H * W}")
    B, D = u.shape[0], u.shape[2]
    return _routes_forward(4, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, stream,
                           (B, D, H, W), save=True, saved=saved)


def ss1d_bidir_forward_routes_save(u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z=None, zoh=False,
                                   y=None, saved=None, stream=None):
    """ss2d_forward_routes_save for the bidirectional operator, u (B, 2, D, L)."""
    if u.dim() != 4:
        raise ValueError("u must be (B, 2, D, L)")
    B, D, L = u.shape[0], u.shape[2], u.shape[3]
    return _routes_forward(2, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, zoh, y, stream,
                           (B, D, L), save=True, saved=saved)


def ss2d_backward_routes_saved(u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, saved, H, W,
                               z=None, zoh=False, stream=None):
    """The gradients of ss2d_backward_routes, starting from the state that
    ss2d_forward_routes_save kept for the same inputs, gate and option."""
    if u.dim() != 4:
        raise ValueError("u must be (B, 4, D, L)")
    if u.shape[-1] != H * W:
        raise ValueError(f"u has {u.shape[-1]} steps, expected H * W = {H * W}")
    B, D = u.shape[0], u.shape[2]
    return _backward_routes(4, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, (B, D, H, W), z, zoh,
                            stream, saved=saved)


def ss1d_bidir_backward_routes_saved(u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, saved, z=None,
                                     zoh=False, stream=None):
    """ss2d_backward_routes_saved for the bidirectional operator, u (B, 2, D, L)."""
    B, D, L = u.shape[0], u.shape[2], u.shape[3]
    return _backward_routes(2, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, (B, D, L), z, zoh,
                            stream, saved=saved)


class launch_plan:
    """Context manager: calls made inside it from this host thread use the given lanes per
    channel (split 1, 2 or 4; 0 = automatic) and chunk length (0 = one pass, > 0 = chunks
    of that many steps, -1 = automatic) in the forward scan; the automatic plan is restored
    on exit.  For tests and tuning: the result is the operator's whatever the plan."""

    def __init__(self, split: int = 0, chunk_len: int = -1):
        self.split, self.chunk_len = int(split), int(chunk_len)

    def __enter__(self):
        _check(load_library().ss2d_set_launch_plan(self.split, self.chunk_len))
        return self

    def __exit__(self, *exc):
        load_library().ss2d_set_launch_plan(0, -1)


def probe_issue_rates(stream=None) -> dict:
    """Measured instruction rates that bound the scan (ss2d_probe_issue_rates): fused
    multiply-adds and v_exp_f32 per second (lane operations), groups of 4 fused multiply-adds
    and 1 v_exp_f32 per second (one state update's mix), the sustained shader clock (Hz) and
    the compute units.  Runs on the current device; synchronises the stream."""
    import torch
    out = (ctypes.c_double * 5)()
    st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(load_library().ss2d_probe_issue_rates(out, ctypes.c_void_p(st)))
    return {"fma_per_s": out[0], "exp_per_s": out[1], "update_mix_per_s": out[2],
            "clock_hz": out[3], "compute_units": int(out[4])}


def timing_enable(enable: bool = True) -> bool:
    """Bracket every kernel launched from this host thread with HIP events (measurement)."""
    return bool(load_library().ss2d_timing_enable(1 if enable else 0))


def timing_read() -> dict:
    """Per-kernel-kind total milliseconds and launch counts since the last read."""
    lib = load_library()
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib.ss2d_timing_read(ms, cnt))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_KINDS)}
