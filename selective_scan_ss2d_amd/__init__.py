"""SS2D operator (VMamba 2D selective scan) for MI355X / gfx950: forward, backward (also
starting from the state a training forward kept), and the per-route front end (causal conv + SiLU, x_proj, dt_proj), also with dt_proj folded into
the scan.

The operator runs in hand-written HIP kernels behind the C ABI of ``libss2d.so``
(``include/ss2d.h``); this package is its thin Python binding.  Build the library with
``python -m selective_scan_ss2d_amd.build``.
"""
from ._binding import (LIBRARY_PATH, SS2D_BF16, SS2D_ERR_ALIAS, SS2D_ERR_ALIGN, SS2D_ERR_HIP,
                       SS2D_ERR_NULL, SS2D_ERR_SHAPE, SS2D_ERR_UNSUPPORTED, SS2D_F32,
                       SS2D_FLAG_ZOH, SS2D_OK, SIGNATURES, KERNEL_KINDS, SS2DError,
                       GRAD_NAMES, abi_version, load_library, ss1d_bidir_backward,
                       ss1d_bidir_backward_ex, ss2d_backward_ex,
                       ss1d_bidir_backward_routes, ss2d_backward_routes,
                       ss1d_bidir_forward, ss1d_bidir_forward_ex, ss1d_bidir_forward_routes,
                       ss1d_bidir_forward_routes_lr, ss1d_bidir_project,
                       ss1d_bidir_project_lr, ss2d_backward, ss2d_forward, ss2d_forward_ex,
                       ss2d_forward_routes, ss2d_forward_routes_lr, ss2d_project,
                       ss2d_project_lr, status_string, timing_enable, timing_read,
                       launch_plan, probe_issue_rates, saved_state_bytes,
                       ss2d_forward_save, ss1d_bidir_forward_save, ss2d_backward_saved,
                       ss1d_bidir_backward_saved, ss2d_forward_routes_save,
                       ss1d_bidir_forward_routes_save, ss2d_backward_routes_saved,
                       ss1d_bidir_backward_routes_saved, scratch_trim)

__all__ = [
    "ss2d_forward", "ss1d_bidir_forward", "ss2d_forward_ex", "ss1d_bidir_forward_ex",
    "ss2d_backward", "ss1d_bidir_backward", "ss2d_backward_ex", "ss1d_bidir_backward_ex",
    "ss2d_backward_routes", "ss1d_bidir_backward_routes",
    "GRAD_NAMES", "ss2d_project", "ss1d_bidir_project",
    "ss2d_forward_routes", "ss1d_bidir_forward_routes", "ss2d_project_lr",
    "ss1d_bidir_project_lr", "ss2d_forward_routes_lr", "ss1d_bidir_forward_routes_lr",
    "SS2D_FLAG_ZOH", "status_string", "abi_version", "load_library",
    "SS2DError", "LIBRARY_PATH", "SIGNATURES", "SS2D_OK", "SS2D_ERR_NULL", "SS2D_ERR_SHAPE",
    "SS2D_ERR_UNSUPPORTED", "SS2D_ERR_ALIGN", "SS2D_ERR_HIP", "SS2D_ERR_ALIAS", "SS2D_F32",
    "SS2D_BF16", "KERNEL_KINDS", "timing_enable", "timing_read", "launch_plan",
    "probe_issue_rates", "saved_state_bytes", "ss2d_forward_save", "ss1d_bidir_forward_save",
    "ss2d_backward_saved", "ss1d_bidir_backward_saved", "ss2d_forward_routes_save",
    "ss1d_bidir_forward_routes_save", "ss2d_backward_routes_saved",
    "ss1d_bidir_backward_routes_saved", "scratch_trim",
]
