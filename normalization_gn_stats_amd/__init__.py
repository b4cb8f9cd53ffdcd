"""GroupNorm forward/backward on AMD Instinct MI355X (gfx950).

Thin binding over the C ABI of ``include/gn.h``: it checks and marshals
arguments, allocates outputs and workspace with torch, and passes torch's
current HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no CPU or PyTorch fallback -- if the library is missing or
refuses a call, these functions raise.

Tensors: x, dy are (N, C, *spatial), float32, float16 or bfloat16.  Dense
contiguous (NCHW) and channels_last (NHWC) tensors take the planner's tuned
paths; any other strides (slices, crops, permuted or broadcast views) are
passed as they are to the strided calls, which read and write them in place
-- no copy -- as long as the spatial dimensions collapse into at most two
strided ones.  gamma/beta are float32 (C,).  mean/rstd come back as float32
(N, G).
"""
from __future__ import annotations

import ctypes
import math

from . import _lib
from ._lib import (GN_BF16, GN_DEBUG_SLAB_COOP, GN_DEBUG_STREAM_SPLIT, GN_DEBUG_UNMET_WAITS, GN_ERR_WAIT,
                   GN_F16, GN_F32, GN_GRAD_DBETA, GN_GRAD_DGAMMA, GN_GRAD_DX, GN_NCHW, GN_NHWC, GN_OK,
                   GN_PATH_AUTO, GN_PATH_GENERIC, GN_PATH_ROWS, GN_PATH_SLAB, GN_PATH_STREAM, PATH_NAMES, GNError,
                   PlanInfo)

__all__ = ["forward", "backward", "forward_into", "backward_into", "backward_scratch_into", "forward_workspace_size",
           "backward_workspace_size", "forward_strided_workspace_size", "backward_strided_workspace_size",
           "strided_dims", "common_layout", "select_path", "layout_of", "GNError", "PlanInfo",
           "rms_forward", "rms_backward", "rms_forward_into", "rms_backward_into",
           "rms_forward_workspace_size", "rms_backward_workspace_size", "status_word", "read_status", "cooperative_state", "COOP_NOT_TRIED", "COOP_ACCEPTED", "COOP_REFUSED",
           "Debug", "GN_OK", "GN_ERR_WAIT", "GN_DEBUG_UNMET_WAITS", "GN_DEBUG_STREAM_SPLIT", "GN_DEBUG_SLAB_COOP",
           "GN_GRAD_DX", "GN_GRAD_DGAMMA", "GN_GRAD_DBETA", "GN_PATH_AUTO", "GN_PATH_GENERIC",
           "GN_PATH_ROWS", "GN_PATH_SLAB", "GN_PATH_STREAM", "PATH_NAMES"]

_PATHS = {None: GN_PATH_AUTO, "auto": GN_PATH_AUTO, "generic": GN_PATH_GENERIC, "rows": GN_PATH_ROWS,
          "slab": GN_PATH_SLAB, "stream": GN_PATH_STREAM}


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: GN_F32, torch.float16: GN_F16, torch.bfloat16: GN_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    return m[t.dtype]


def layout_of(t) -> int:
    """GN_NCHW if t is contiguous, GN_NHWC if it is dense channels_last."""
    torch = _torch()
    if t.dim() < 2:
        raise ValueError("expected a tensor of shape (N, C, *spatial)")
    if t.is_contiguous():
        return GN_NCHW
    if t.dim() == 4 and t.is_contiguous(memory_format=torch.channels_last):
        return GN_NHWC
    if t.dim() == 5 and t.is_contiguous(memory_format=torch.channels_last_3d):
        return GN_NHWC
    raise ValueError("tensor must be dense: contiguous (NCHW) or channels_last (NHWC)")


def _dims(t):
    N, C = t.shape[0], t.shape[1]
    HW = math.prod(t.shape[2:]) if t.dim() > 2 else 1
    return int(N), int(C), int(HW)


def common_layout(*ts):
    """The dense layout (GN_NCHW or GN_NHWC) every given tensor has, or None.
    None entries are skipped."""
    lay = None
    for t in ts:
        if t is None:
            continue
        try:
            lt = layout_of(t)
        except ValueError:
            return None
        if lay is None:
            lay = lt
        elif lt != lay:
            return None
    return lay


def strided_dims(*ts):
    """(N, C, H, W, [strides per tensor]) describing tensors of one shape
    (N, C, *spatial) for the strided calls, without a copy.

    Spatial dimensions of extent 1 are dropped; neighbours that are
    contiguous in every tensor (outer stride = inner stride * inner extent)
    are merged; at most two may remain (H, W) -- otherwise ValueError.  The
    strides are element strides (n, c, h, w); a missing h or w dimension gets
    extent 1 and stride 0."""
    ts = [t for t in ts if t is not None]
    shape = tuple(ts[0].shape)
    if len(shape) < 2:
        raise ValueError("expected tensors of shape (N, C, *spatial)")
    for t in ts:
        if tuple(t.shape) != shape:
            raise ValueError("tensors must have the same shape")
    groups = []
    for i in range(2, len(shape)):
        if shape[i] == 1:
            continue
        if groups and all(t.stride(groups[-1][-1]) == t.stride(i) * shape[i] for t in ts):
            groups[-1].append(i)
        else:
            groups.append([i])
    if len(groups) > 2:
        raise ValueError("the spatial dimensions do not collapse into two strided dimensions; "
                         "make the tensor contiguous first")
    while len(groups) < 2:
        groups.insert(0, [])
    H = math.prod(shape[i] for i in groups[0]) if groups[0] else 1
    W = math.prod(shape[i] for i in groups[1]) if groups[1] else 1
    strides = []
    for t in ts:
        hs = t.stride(groups[0][-1]) if groups[0] else 0
        ws = t.stride(groups[1][-1]) if groups[1] else 0
        strides.append((ctypes.c_int64 * 4)(t.stride(0), t.stride(1), hs, ws))
    return int(shape[0]), int(shape[1]), int(H), int(W), strides


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class Debug:
    """Failure-report knobs of gn_options (tests): spin_limit polls before a
    wait between workgroups gives up (0: the library's default); flags
    GN_DEBUG_UNMET_WAITS makes every such wait give up; GN_DEBUG_STREAM_SPLIT
    keeps the stream path in its full multi-kernel form (no fused forms);
    GN_DEBUG_SLAB_COOP keeps the slab path on its cooperative kernels."""

    def __init__(self, spin_limit: int = 0, flags: int = 0):
        self.spin_limit = int(spin_limit)
        self.flags = int(flags)


def _opts(force_path, max_resident, info, events, kernel_events=None, status=None, debug=None):
    o = _lib.Options()
    o.force_path = _PATHS[force_path] if not isinstance(force_path, int) else force_path
    o.max_resident_override = int(max_resident or 0)
    o.info = ctypes.pointer(info) if info is not None else None
    if events is not None:
        o.event_begin = ctypes.c_void_p(events[0])
        o.event_end = ctypes.c_void_p(events[1])
    if kernel_events is not None:
        o.kernel_begin = ctypes.c_void_p(kernel_events[0])
        o.kernel_end = ctypes.c_void_p(kernel_events[1])
    if status is not None:
        o.status_word = ctypes.c_void_p(_status_ptr(status))
    if debug is not None:
        o.spin_limit = debug.spin_limit
        o.debug_flags = debug.flags
    return o


def _status_ptr(t) -> int:
    torch = _torch()
    if t.device.type != "cuda" or t.dtype not in (torch.int32, torch.uint32) or t.numel() < 1:
        raise ValueError("status must be a 32-bit integer tensor of at least one element on the device")
    return t.data_ptr()


def status_word(device=None):
    """A zeroed device word for gn_options.status_word (int32 tensor of one
    element): the kernels OR their failure reports into it."""
    torch = _torch()
    return torch.zeros(1, dtype=torch.int32, device=device if device is not None else "cuda")


COOP_NOT_TRIED, COOP_ACCEPTED, COOP_REFUSED = 0, 1, 2


def cooperative_state() -> int:
    """gn_cooperative_state: COOP_NOT_TRIED, COOP_ACCEPTED or COOP_REFUSED for
    this process on the current device."""
    _torch()
    return int(_lib.lib().gn_cooperative_state())


def read_status(status, reset: bool = True, stream=None) -> int:
    """gn_read_status: waits for the stream, reads the word, returns GN_OK or
    GN_ERR_WAIT (a bounded wait gave up: that call's outputs are NaN where
    affected); zeroes the word when reset."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(status.device).cuda_stream
    w = ctypes.c_uint32()
    st = _lib.lib().gn_read_status(ctypes.c_void_p(_status_ptr(status)), ctypes.c_void_p(stream),
                                   1 if reset else 0, ctypes.byref(w))
    if st not in (GN_OK, GN_ERR_WAIT):
        raise GNError(st, "gn_read_status")
    return st


def _check_f32_vec(t, C, name):
    torch = _torch()
    if t is None:
        return
    if t.dtype != torch.float32 or t.numel() != C or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of {C} elements")


def forward_workspace_size(N, C, HW, G, dtype_code, layout, force_path=None) -> int:
    o = _opts(force_path, 0, None, None)
    return int(_lib.lib().gn_forward_workspace_size(N, C, HW, G, dtype_code, layout, ctypes.byref(o)))


def backward_workspace_size(N, C, HW, G, dtype_code, layout, mask, force_path=None) -> int:
    o = _opts(force_path, 0, None, None)
    return int(_lib.lib().gn_backward_workspace_size(N, C, HW, G, dtype_code, layout, mask, ctypes.byref(o)))


def forward_strided_workspace_size(N, C, H, W, G, dtype_code, x_strides, y_strides, force_path=None) -> int:
    o = _opts(force_path, 0, None, None)
    return int(_lib.lib().gn_forward_strided_workspace_size(N, C, H, W, G, dtype_code, x_strides, y_strides,
                                                             ctypes.byref(o)))


def backward_strided_workspace_size(N, C, H, W, G, dtype_code, dy_strides, x_strides, dx_strides, mask,
                                    force_path=None) -> int:
    o = _opts(force_path, 0, None, None)
    return int(_lib.lib().gn_backward_strided_workspace_size(N, C, H, W, G, dtype_code, dy_strides, x_strides,
                                                              dx_strides, mask, ctypes.byref(o)))


def select_path(backward: bool, N, C, HW, G, dtype_code, layout, force_path=None) -> int:
    o = _opts(force_path, 0, None, None)
    return int(_lib.lib().gn_select_path(1 if backward else 0, N, C, HW, G, dtype_code, layout, ctypes.byref(o)))


def forward_into(x, gamma, beta, num_groups, eps, y, mean, rstd, workspace, *, force_path=None,
                 max_resident=0, info=None, events=None, kernel_events=None, status=None, debug=None, stream=None):
    """gn_forward (dense x and y in one layout) or gn_forward_strided (any
    other strides) on preallocated outputs; returns nothing, raises GNError."""
    torch = _torch()
    if y is not None and (tuple(y.shape) != tuple(x.shape) or y.dtype != x.dtype):
        raise ValueError("y must match x in shape and dtype")
    layout = common_layout(x, y)
    C = int(x.shape[1])
    _check_f32_vec(gamma, C, "gamma")
    _check_f32_vec(beta, C, "beta")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    o = _opts(force_path, max_resident, info, events, kernel_events, status, debug)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if layout is not None:
        N, C, HW = _dims(x)
        st = _lib.lib().gn_forward(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), N, C, HW,
                                   int(num_groups), float(eps), _dtype_code(x), layout, _ptr(workspace), ws_bytes,
                                   ctypes.c_void_p(stream), ctypes.byref(o))
        if st != 0:
            raise GNError(st, "gn_forward")
        return
    N, C, H, W, strides = strided_dims(x, y)
    st = _lib.lib().gn_forward_strided(_ptr(x), strides[0], _ptr(gamma), _ptr(beta), _ptr(y),
                                       strides[1] if y is not None else None, _ptr(mean), _ptr(rstd), N, C, H, W,
                                       int(num_groups), float(eps), _dtype_code(x), _ptr(workspace), ws_bytes,
                                       ctypes.c_void_p(stream), ctypes.byref(o))
    if st != 0:
        raise GNError(st, "gn_forward_strided")


def forward(x, gamma, beta, num_groups: int, eps: float = 1e-5, *, compute_y: bool = True, force_path=None,
            max_resident: int = 0, info: PlanInfo | None = None, status=None, debug: Debug | None = None):
    """Returns (y, mean, rstd); y is None when compute_y is False.  status: a
    device word (``status_word()``) that receives the failure report of the
    cooperative kernels; read it with ``read_status``."""
    torch = _torch()
    if x.device.type != "cuda":
        raise ValueError("x must be on a HIP device")
    G = int(num_groups)
    with torch.cuda.device(x.device):
        # empty_like keeps x's strides when x is dense (in any dimension
        # order), and is contiguous otherwise
        y = torch.empty_like(x) if compute_y else None
        N, C = int(x.shape[0]), int(x.shape[1])
        mean = torch.empty(N * G, device=x.device, dtype=torch.float32)
        rstd = torch.empty(N * G, device=x.device, dtype=torch.float32)
        layout = common_layout(x, y)
        if layout is not None:
            wsb = forward_workspace_size(N, C, _dims(x)[2], G, _dtype_code(x), layout, force_path)
        else:
            _, _, H, W, strides = strided_dims(x, y)
            wsb = forward_strided_workspace_size(N, C, H, W, G, _dtype_code(x), strides[0],
                                                 strides[1] if y is not None else None, force_path)
        ws = torch.empty(max(wsb, 1), device=x.device, dtype=torch.uint8)
        forward_into(x, gamma, beta, G, eps, y, mean, rstd, ws, force_path=force_path,
                     max_resident=max_resident, info=info, status=status, debug=debug)
    return y, mean.view(N, G), rstd.view(N, G)


def backward_into(dy, x, mean, rstd, gamma, num_groups, mask, dx, dgamma, dbeta, workspace, *,
                  force_path=None, max_resident=0, info=None, events=None, kernel_events=None, status=None,
                  debug=None, stream=None):
    """gn_backward (dy, x, dx dense in one layout) or gn_backward_strided (any
    other strides) on preallocated outputs; returns nothing, raises GNError."""
    torch = _torch()
    if tuple(dy.shape) != tuple(x.shape) or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    if dx is not None and (tuple(dx.shape) != tuple(x.shape) or dx.dtype != x.dtype):
        raise ValueError("dx must match x in shape and dtype")
    want_dx = bool(int(mask) & GN_GRAD_DX) and dx is not None
    layout = common_layout(dy, x, dx if want_dx else None)
    C = int(x.shape[1])
    _check_f32_vec(gamma, C, "gamma")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    o = _opts(force_path, max_resident, info, events, kernel_events, status, debug)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if layout is not None:
        N, C, HW = _dims(x)
        st = _lib.lib().gn_backward(_ptr(dy), _ptr(x), _ptr(mean), _ptr(rstd), _ptr(gamma), _ptr(dx),
                                    _ptr(dgamma), _ptr(dbeta), int(mask), N, C, HW, int(num_groups),
                                    _dtype_code(x), layout, _ptr(workspace), ws_bytes, ctypes.c_void_p(stream),
                                    ctypes.byref(o))
        if st != 0:
            raise GNError(st, "gn_backward")
        return
    N, C, H, W, strides = strided_dims(dy, x, dx if want_dx else None)
    st = _lib.lib().gn_backward_strided(_ptr(dy), strides[0], _ptr(x), strides[1], _ptr(mean), _ptr(rstd),
                                        _ptr(gamma), _ptr(dx), strides[2] if want_dx else None, _ptr(dgamma),
                                        _ptr(dbeta), int(mask), N, C, H, W, int(num_groups), _dtype_code(x),
                                        _ptr(workspace), ws_bytes, ctypes.c_void_p(stream), ctypes.byref(o))
    if st != 0:
        raise GNError(st, "gn_backward_strided")


def backward_scratch_into(dy, x, mean, rstd, gamma, num_groups, mask, dx, dgamma, dbeta, *, force_path=None,
                          max_resident=0, info=None, events=None, kernel_events=None, status=None, debug=None,
                          stream=None):
    """gn_backward_scratch: gn_backward on preallocated outputs with the
    library's static device scratch instead of a workspace (dense dy, x, dx
    in one layout); returns nothing, raises GNError."""
    torch = _torch()
    if tuple(dy.shape) != tuple(x.shape) or dy.dtype != x.dtype:
        raise ValueError("dy must match x in shape and dtype")
    if dx is not None and (tuple(dx.shape) != tuple(x.shape) or dx.dtype != x.dtype):
        raise ValueError("dx must match x in shape and dtype")
    want_dx = bool(int(mask) & GN_GRAD_DX) and dx is not None
    layout = common_layout(dy, x, dx if want_dx else None)
    if layout is None:
        raise ValueError("gn_backward_scratch takes dense tensors in one layout")
    C = int(x.shape[1])
    _check_f32_vec(gamma, C, "gamma")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    o = _opts(force_path, max_resident, info, events, kernel_events, status, debug)
    N, C, HW = _dims(x)
    st = _lib.lib().gn_backward_scratch(_ptr(dy), _ptr(x), _ptr(mean), _ptr(rstd), _ptr(gamma), _ptr(dx),
                                        _ptr(dgamma), _ptr(dbeta), int(mask), N, C, HW, int(num_groups),
                                        _dtype_code(x), layout, ctypes.c_void_p(stream), ctypes.byref(o))
    if st != 0:
        raise GNError(st, "gn_backward_scratch")


def backward(dy, x, mean, rstd, gamma, num_groups: int, mask: int = GN_GRAD_DX | GN_GRAD_DGAMMA | GN_GRAD_DBETA,
             *, force_path=None, max_resident: int = 0, info: PlanInfo | None = None, status=None,
             debug: Debug | None = None):
    """Returns (dx, dgamma, dbeta), each None when not selected by mask.
    status, debug: as for ``forward``."""
    torch = _torch()
    if x.device.type != "cuda":
        raise ValueError("x must be on a HIP device")
    G = int(num_groups)
    with torch.cuda.device(x.device):
        dx = torch.empty_like(x) if mask & GN_GRAD_DX else None
        N, C = int(x.shape[0]), int(x.shape[1])
        dgamma = torch.empty(C, device=x.device, dtype=torch.float32) if mask & GN_GRAD_DGAMMA else None
        dbeta = torch.empty(C, device=x.device, dtype=torch.float32) if mask & GN_GRAD_DBETA else None
        layout = common_layout(dy, x, dx)
        if layout is not None:
            wsb = backward_workspace_size(N, C, _dims(x)[2], G, _dtype_code(x), layout, mask, force_path)
        else:
            _, _, H, W, strides = strided_dims(dy, x, dx)
            wsb = backward_strided_workspace_size(N, C, H, W, G, _dtype_code(x), strides[0], strides[1],
                                                  strides[2] if dx is not None else None, mask, force_path)
        ws = torch.empty(max(wsb, 1), device=x.device, dtype=torch.uint8)
        backward_into(dy, x, mean.reshape(-1), rstd.reshape(-1), gamma, G, mask, dx, dgamma, dbeta, ws,
                      force_path=force_path, max_resident=max_resident, info=info, status=status, debug=debug)
    return dx, dgamma, dbeta


# ---- RMSNorm over rows ([N, C] tensors; segments of C/G channels) ------------
def _rows_dims(x):
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("RMSNorm takes a contiguous [N, C] tensor")
    return int(x.shape[0]), int(x.shape[1])


def rms_forward_workspace_size(N, C, G, dtype_code, force_path=None) -> int:
    o = _opts(force_path, 0, None, None)
    return int(_lib.lib().gn_rms_forward_workspace_size(N, C, G, dtype_code, ctypes.byref(o)))


def rms_backward_workspace_size(N, C, G, dtype_code, mask, force_path=None) -> int:
    o = _opts(force_path, 0, None, None)
    return int(_lib.lib().gn_rms_backward_workspace_size(N, C, G, dtype_code, mask, ctypes.byref(o)))


def rms_forward_into(x, gamma, num_groups, eps, y, rstd, workspace, *, force_path=None, info=None, events=None,
                     kernel_events=None, stream=None):
    """gn_rms_forward on preallocated outputs; returns nothing, raises GNError."""
    torch = _torch()
    N, C = _rows_dims(x)
    _check_f32_vec(gamma, C, "gamma")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    o = _opts(force_path, 0, info, events, kernel_events)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.lib().gn_rms_forward(_ptr(x), _ptr(gamma), _ptr(y), _ptr(rstd), N, C, int(num_groups), float(eps),
                                   _dtype_code(x), _ptr(workspace), ws_bytes, ctypes.c_void_p(stream),
                                   ctypes.byref(o))
    if st != 0:
        raise GNError(st, "gn_rms_forward")


def rms_forward(x, gamma, eps: float = 1e-6, num_groups: int = 1, *, compute_y: bool = True, force_path=None,
                info: PlanInfo | None = None):
    """RMSNorm of each (row, group) segment of an [N, C] tensor.  Returns
    (y, rstd[N, G]); y is None when compute_y is False."""
    torch = _torch()
    if x.device.type != "cuda":
        raise ValueError("x must be on a HIP device")
    N, C = _rows_dims(x)
    G = int(num_groups)
    with torch.cuda.device(x.device):
        y = torch.empty_like(x) if compute_y else None
        rstd = torch.empty(N * G, device=x.device, dtype=torch.float32)
        wsb = rms_forward_workspace_size(N, C, G, _dtype_code(x), force_path)
        ws = torch.empty(max(wsb, 1), device=x.device, dtype=torch.uint8)
        rms_forward_into(x, gamma, G, eps, y, rstd, ws, force_path=force_path, info=info)
    return y, rstd.view(N, G)


def rms_backward_into(dy, x, rstd, gamma, num_groups, mask, dx, dgamma, workspace, *, force_path=None, info=None,
                      events=None, kernel_events=None, stream=None):
    """gn_rms_backward on preallocated outputs; returns nothing, raises GNError."""
    torch = _torch()
    N, C = _rows_dims(x)
    if tuple(dy.shape) != tuple(x.shape) or dy.dtype != x.dtype or not dy.is_contiguous():
        raise ValueError("dy must match x in shape and dtype")
    _check_f32_vec(gamma, C, "gamma")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    o = _opts(force_path, 0, info, events, kernel_events)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.lib().gn_rms_backward(_ptr(dy), _ptr(x), _ptr(rstd), _ptr(gamma), _ptr(dx), _ptr(dgamma), int(mask),
                                    N, C, int(num_groups), _dtype_code(x), _ptr(workspace), ws_bytes,
                                    ctypes.c_void_p(stream), ctypes.byref(o))
    if st != 0:
        raise GNError(st, "gn_rms_backward")


def rms_backward(dy, x, rstd, gamma, num_groups: int = 1, mask: int = GN_GRAD_DX | GN_GRAD_DGAMMA, *,
                 force_path=None, info: PlanInfo | None = None):
    """Returns (dx, dgamma), each None when not selected by mask."""
    torch = _torch()
    if x.device.type != "cuda":
        raise ValueError("x must be on a HIP device")
    N, C = _rows_dims(x)
    G = int(num_groups)
    with torch.cuda.device(x.device):
        dx = torch.empty_like(x) if mask & GN_GRAD_DX else None
        dgamma = torch.empty(C, device=x.device, dtype=torch.float32) if mask & GN_GRAD_DGAMMA else None
        wsb = rms_backward_workspace_size(N, C, G, _dtype_code(x), mask, force_path)
        ws = torch.empty(max(wsb, 1), device=x.device, dtype=torch.uint8)
        rms_backward_into(dy, x, rstd.reshape(-1), gamma, G, mask, dx, dgamma, ws, force_path=force_path, info=info)
    return dx, dgamma
