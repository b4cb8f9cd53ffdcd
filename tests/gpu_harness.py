"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, then compare.

Tolerances (assert_close semantics |a - b| <= atol + rtol*|ref|, as the apex
PR #2018 reproducer uses):
  y, dx      float32: rtol 1e-4, atol 1e-5; float16/bfloat16: rtol 1e-2, atol 1e-2
  mean, rstd rtol 1e-4, atol 1e-5 (float32 outputs for every dtype)
  dgamma, dbeta   ||d - d_ref||_2 / ||d_ref||_2 <= 1e-3
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import normalization_gn_stats_amd as gn
import oracle
from normalization_gn_stats_amd import inputs

TOL = {"f32": (1e-4, 1e-5), "f16": (1e-2, 1e-2), "bf16": (1e-2, 1e-2)}
STAT_TOL = (1e-4, 1e-5)
PARAM_REL_L2 = 1e-3
ALL = gn.GN_GRAD_DX | gn.GN_GRAD_DGAMMA | gn.GN_GRAD_DBETA


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def close(a, b, rtol, atol, what):
    a = np.asarray(a, np.float64).reshape(-1)
    b = np.asarray(b, np.float64).reshape(-1)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} of {a.size} outside tolerance; worst at {i}: "
                             f"got {a[i]!r}, want {b[i]!r} (rtol {rtol}, atol {atol})")


def rel_l2(a, b, what, bound=PARAM_REL_L2):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.linalg.norm(a - b)
    den = np.linalg.norm(b)
    rel = num / den if den > 0 else num
    assert rel <= bound, f"{what}: relative L2 error {rel:.3e} > {bound}"
    return rel


def img64(t: torch.Tensor, layout: str) -> np.ndarray:
    """fp64 numpy copy of a tensor's memory image (exact for f32/f16/bf16)."""
    return inputs.memory_image(t, layout).detach().to("cpu", torch.float64).numpy()


def run_gpu(wl, data, force_path=None, mask=ALL, max_resident=0, debug=None):
    """Returns dict of GPU outputs (torch tensors on the device) and the plans.
    Both calls report into a status word, which must read GN_OK afterwards
    (no bounded wait between workgroups gave up)."""
    dev = torch.device("cuda", 0)
    x = data["x"].to(dev)
    dy = data["dy"].to(dev)
    gamma = data["gamma"].to(dev)
    beta = data["beta"].to(dev)
    fi, bi = gn.PlanInfo(), gn.PlanInfo()
    status = gn.status_word(dev)
    y, mean, rstd = gn.forward(x, gamma, beta, wl.G, wl.eps, force_path=force_path, max_resident=max_resident,
                               info=fi, status=status, debug=debug)
    assert gn.read_status(status) == gn.GN_OK, f"{wl.name}: a forward wait gave up"
    dx, dg, db = gn.backward(dy, x, mean, rstd, gamma, wl.G, mask, force_path=force_path,
                             max_resident=max_resident, info=bi, status=status, debug=debug)
    assert gn.read_status(status) == gn.GN_OK, f"{wl.name}: a backward wait gave up"
    torch.cuda.synchronize()
    return dict(y=y, mean=mean, rstd=rstd, dx=dx, dgamma=dg, dbeta=db, fwd_plan=fi, bwd_plan=bi)


def check_against_oracle(wl, data, out, mask=ALL):
    rtol, atol = TOL[wl.dtype]
    x64 = img64(data["x"], wl.layout)
    dy64 = img64(data["dy"], wl.layout)
    g64 = data["gamma"].double().cpu().numpy()
    b64 = data["beta"].double().cpu().numpy()
    eps = float(np.float32(wl.eps))
    ry, rmean, rrstd = oracle.forward(x64, g64, b64, wl.N, wl.C, wl.HW, wl.G, eps, layout=wl.layout)
    close(img64(out["y"], wl.layout), ry, rtol, atol, f"{wl.name} y")
    close(out["mean"].cpu().double().numpy(), rmean, *STAT_TOL, f"{wl.name} mean")
    close(out["rstd"].cpu().double().numpy(), rrstd, *STAT_TOL, f"{wl.name} rstd")
    rdx, rdg, rdb, _, _ = oracle.backward(dy64, x64, g64, wl.N, wl.C, wl.HW, wl.G, eps, layout=wl.layout,
                                          want_dx=bool(mask & gn.GN_GRAD_DX),
                                          want_dgamma=bool(mask & gn.GN_GRAD_DGAMMA),
                                          want_dbeta=bool(mask & gn.GN_GRAD_DBETA))
    if mask & gn.GN_GRAD_DX:
        close(img64(out["dx"], wl.layout), rdx, rtol, atol, f"{wl.name} dx")
    else:
        assert out["dx"] is None
    if mask & gn.GN_GRAD_DGAMMA:
        rel_l2(out["dgamma"].cpu().numpy(), rdg, f"{wl.name} dgamma")
    if mask & gn.GN_GRAD_DBETA:
        rel_l2(out["dbeta"].cpu().numpy(), rdb, f"{wl.name} dbeta")


# ---- RMSNorm over rows --------------------------------------------------------
RMS_ALL = gn.GN_GRAD_DX | gn.GN_GRAD_DGAMMA


def rows2d(t: torch.Tensor) -> torch.Tensor:
    """[N, C, 1, 1] (or [N, C]) workload tensor as a contiguous [N, C] tensor."""
    return t.reshape(t.shape[0], t.shape[1]).contiguous()


def run_rms_gpu(wl, data, mask=RMS_ALL, affine=True):
    dev = torch.device("cuda", 0)
    x = rows2d(data["x"]).to(dev)
    dy = rows2d(data["dy"]).to(dev)
    gamma = data["gamma"].to(dev) if affine else None
    fi, bi = gn.PlanInfo(), gn.PlanInfo()
    y, rstd = gn.rms_forward(x, gamma, wl.eps, wl.G, info=fi)
    dx, dg = gn.rms_backward(dy, x, rstd, gamma, wl.G, mask, info=bi)
    torch.cuda.synchronize()
    return dict(y=y, rstd=rstd, dx=dx, dgamma=dg, fwd_plan=fi, bwd_plan=bi)


def check_rms_against_oracle(wl, data, out, mask=RMS_ALL, affine=True):
    rtol, atol = TOL[wl.dtype]
    x64 = rows2d(data["x"]).double().cpu().numpy().reshape(-1)
    dy64 = rows2d(data["dy"]).double().cpu().numpy().reshape(-1)
    g64 = data["gamma"].double().cpu().numpy() if affine else None
    eps = float(np.float32(wl.eps))
    ry, rr = oracle.rms_forward(x64, g64, wl.N, wl.C, wl.G, eps)
    close(out["y"].double().cpu().numpy(), ry, rtol, atol, f"{wl.name} rms y")
    close(out["rstd"].double().cpu().numpy(), rr, *STAT_TOL, f"{wl.name} rms rstd")
    rdx, rdg, _ = oracle.rms_backward(dy64, x64, g64, wl.N, wl.C, wl.G, eps, want_dx=bool(mask & gn.GN_GRAD_DX),
                                      want_dgamma=bool(mask & gn.GN_GRAD_DGAMMA))
    if mask & gn.GN_GRAD_DX:
        close(out["dx"].double().cpu().numpy(), rdx, rtol, atol, f"{wl.name} rms dx")
    else:
        assert out["dx"] is None
    if mask & gn.GN_GRAD_DGAMMA:
        rel_l2(out["dgamma"].cpu().numpy(), rdg, f"{wl.name} rms dgamma")
    else:
        assert out["dgamma"] is None
