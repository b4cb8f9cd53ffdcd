"""ctypes view of the C ABI in include/gn.h (libgn_mi355x.so).

The library is loaded lazily, after ``torch`` so that the HIP runtime torch
already holds is the one the library binds to (both carry the SONAME
libamdhip64.so.7).  There is no fallback: if the library is missing, every
call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# GN_LIB_PATH selects another build of the same library (e.g. one compiled
# with different tile constants); by default the in-tree build is used.
LIB_PATH = os.environ.get("GN_LIB_PATH") or os.path.join(HERE, "lib", "libgn_mi355x.so")

GN_OK, GN_ERR_INVALID, GN_ERR_UNSUPPORTED, GN_ERR_WORKSPACE, GN_ERR_HIP, GN_ERR_WAIT = range(6)
GN_STATUS_WAIT_EXPIRED = 1
GN_DEBUG_UNMET_WAITS = 1
GN_DEBUG_STREAM_SPLIT = 2
GN_DEBUG_SLAB_COOP = 4
GN_SCRATCH_BYTES = 32 << 20
GN_F32, GN_F16, GN_BF16 = range(3)
GN_NCHW, GN_NHWC = range(2)
GN_GRAD_DX, GN_GRAD_DGAMMA, GN_GRAD_DBETA = 1, 2, 4
GN_PATH_AUTO, GN_PATH_GENERIC, GN_PATH_ROWS, GN_PATH_SLAB, GN_PATH_STREAM = range(5)
PATH_NAMES = {GN_PATH_AUTO: "auto", GN_PATH_GENERIC: "generic", GN_PATH_ROWS: "rows", GN_PATH_SLAB: "slab",
              GN_PATH_STREAM: "stream"}

# every symbol include/gn.h declares
EXPORTED = ("gn_forward_workspace_size", "gn_forward", "gn_backward_workspace_size", "gn_backward",
            "gn_forward_strided_workspace_size", "gn_forward_strided", "gn_backward_strided_workspace_size",
            "gn_backward_strided",
            "gn_select_path", "gn_status_string", "gn_version", "gn_rms_forward_workspace_size",
            "gn_rms_forward", "gn_rms_backward_workspace_size", "gn_rms_backward", "gn_read_status",
            "gn_backward_scratch", "gn_cooperative_state")


class PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("kernels", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("tiles", ctypes.c_int64), ("resident_cap", ctypes.c_int64), ("team", ctypes.c_int64)]


class Options(ctypes.Structure):
    _fields_ = [("force_path", ctypes.c_int32), ("max_resident_override", ctypes.c_int32),
                ("info", ctypes.POINTER(PlanInfo)), ("event_begin", ctypes.c_void_p),
                ("event_end", ctypes.c_void_p), ("kernel_begin", ctypes.c_void_p),
                ("kernel_end", ctypes.c_void_p), ("status_word", ctypes.c_void_p),
                ("spin_limit", ctypes.c_uint32), ("debug_flags", ctypes.c_uint32)]


class GNError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
    import torch  # noqa: F401  -- bind to the HIP runtime torch loaded
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz, f = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
    op = ctypes.POINTER(Options)
    L.gn_forward_workspace_size.argtypes = [i64, i64, i64, i64, i32, i32, op]
    L.gn_forward_workspace_size.restype = sz
    L.gn_backward_workspace_size.argtypes = [i64, i64, i64, i64, i32, i32, i32, op]
    L.gn_backward_workspace_size.restype = sz
    L.gn_forward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f, i32, i32, vp, sz, vp, op]
    L.gn_forward.restype = i32
    L.gn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i32, i32, vp, sz, vp, op]
    L.gn_backward.restype = i32
    pi = ctypes.POINTER(ctypes.c_int64)
    L.gn_forward_strided_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, pi, pi, op]
    L.gn_forward_strided_workspace_size.restype = sz
    L.gn_forward_strided.argtypes = [vp, pi, vp, vp, vp, pi, vp, vp, i64, i64, i64, i64, i64, f, i32, vp, sz, vp,
                                     op]
    L.gn_forward_strided.restype = i32
    L.gn_backward_strided_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, pi, pi, pi, i32, op]
    L.gn_backward_strided_workspace_size.restype = sz
    L.gn_backward_strided.argtypes = [vp, pi, vp, pi, vp, vp, vp, vp, pi, vp, vp, i32, i64, i64, i64, i64, i64, i32,
                                      vp, sz, vp, op]
    L.gn_backward_strided.restype = i32
    L.gn_select_path.argtypes = [i32, i64, i64, i64, i64, i32, i32, op]
    L.gn_select_path.restype = i32
    L.gn_rms_forward_workspace_size.argtypes = [i64, i64, i64, i32, op]
    L.gn_rms_forward_workspace_size.restype = sz
    L.gn_rms_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, f, i32, vp, sz, vp, op]
    L.gn_rms_forward.restype = i32
    L.gn_rms_backward_workspace_size.argtypes = [i64, i64, i64, i32, i32, op]
    L.gn_rms_backward_workspace_size.restype = sz
    L.gn_rms_backward.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, i32, vp, sz, vp, op]
    L.gn_rms_backward.restype = i32
    L.gn_backward_scratch.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i32, i32, vp, op]
    L.gn_backward_scratch.restype = i32
    L.gn_read_status.argtypes = [vp, vp, i32, ctypes.POINTER(ctypes.c_uint32)]
    L.gn_read_status.restype = i32
    L.gn_cooperative_state.argtypes = []
    L.gn_cooperative_state.restype = i32
    L.gn_status_string.argtypes = [i32]
    L.gn_status_string.restype = ctypes.c_char_p
    L.gn_version.restype = i32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().gn_status_string(status).decode()
