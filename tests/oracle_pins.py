"""Pins of the fp64 oracle against facts it does not compute itself.

Each pin takes ``mutant`` (0 = the real oracle) and raises AssertionError when
the oracle disagrees with the fact.  The facts:

* closed forms worked by hand from the definition (a 3-element slice whose
  statistics, outputs and gradients have exact values; an NHWC two-group case);
* central finite differences of L = sum(y * w) in fp64 (pins dx, dgamma, dbeta
  against the forward);
* an independent library implementation: torch's float64 CPU group_norm,
  layer_norm (G = 1, one spatial position) and instance_norm (G = C), with
  autograd for the gradients;
* closed-form invariants: with gamma = 1, beta = 0 every slice of y has mean 0
  and variance var/(var + eps); dbeta_c is the column sum of dy; per slice
  sum(dx) = 0 and sum(dx * xhat) = rstd * B * eps / (var + eps);
* RMSNorm over rows: a hand-worked row, torch's float64 rms_norm with
  autograd, and its invariants (mean square of y, dx orthogonal to x at
  eps = 0, scale invariance, groups as independent rows);
* structure: NCHW and NHWC images of one logical tensor give the same logical
  outputs; permuting positions inside a slice permutes y and dx alike; with
  eps = 0, scaling x leaves y unchanged; a one-element slice gives y = beta and
  dx = 0; a constant slice gives y = beta and dx = eps^-1/2 * (gamma*dy minus its
  slice mean).
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _assert_close(a, b, rtol, atol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.shape != b.shape:
        raise AssertionError(f"{what}: shape {a.shape} vs {b.shape}")
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    if not np.all(err <= bound):
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: max violation at {i}: {a.flat[i]!r} vs {b.flat[i]!r}")


def _nchw_to_nhwc(a, N, C, HW):
    return np.ascontiguousarray(a.reshape(N, C, HW).transpose(0, 2, 1)).reshape(-1)


def _nhwc_to_nchw(a, N, C, HW):
    return np.ascontiguousarray(a.reshape(N, HW, C).transpose(0, 2, 1)).reshape(-1)


# ----------------------------------------------------------------------------
# hand-worked closed forms
# ----------------------------------------------------------------------------
def pin_hand_slice(mutant=0):
    """x = [-1, 0, 1], eps = 1/3: mean 0, var 2/3, var + eps = 1, rstd 1,
    xhat = x.  With gamma = 2, beta = 1/2: y = 2*x + 1/2.  With dy = [1, 0, 0]:
    A = gamma*sum(dy) = 2, B = gamma*sum(dy*xhat) = -2, M = 3, and
    dx_j = gamma*(dy_j - sum(dy)/3 - xhat_j*sum(dy*xhat)/3)
         = 2*[1 - 1/3 - 1/3, -1/3, -1/3 + 1/3] = [2/3, -2/3, 0];
    dgamma = sum(dy*xhat) = -1, dbeta = sum(dy) = 1."""
    x = np.array([-1.0, 0.0, 1.0])
    eps = 1.0 / 3.0
    y, mean, rstd = oracle.forward(x, [2.0], [0.5], 1, 1, 3, 1, eps, mutant=mutant)
    _assert_close(mean, [0.0], 0, 1e-15, "hand mean")
    _assert_close(rstd, [1.0], 1e-14, 0, "hand rstd")
    _assert_close(y, [-1.5, 0.5, 2.5], 1e-14, 1e-15, "hand y")
    dx, dg, db, _, _ = oracle.backward([1.0, 0.0, 0.0], x, [2.0], 1, 1, 3, 1, eps, mutant=mutant)
    _assert_close(dx, [2 / 3, -2 / 3, 0.0], 1e-13, 1e-14, "hand dx")
    _assert_close(dg, [-1.0], 1e-14, 0, "hand dgamma")
    _assert_close(db, [1.0], 1e-14, 0, "hand dbeta")


def pin_hand_textbook(mutant=0):
    """x = [1, 2, 3, 4], eps = 0, one group: mean 2.5, biased variance 1.25
    (the unbiased one would be 5/3), y = (x - 2.5)/sqrt(1.25)."""
    x = np.array([1.0, 2.0, 3.0, 4.0])
    y, mean, rstd = oracle.forward(x, None, None, 1, 1, 4, 1, 0.0, mutant=mutant)
    _assert_close(mean, [2.5], 0, 1e-15, "textbook mean")
    _assert_close(rstd, [1 / math.sqrt(1.25)], 1e-14, 0, "textbook rstd")
    _assert_close(y, (x - 2.5) / math.sqrt(1.25), 1e-14, 1e-15, "textbook y")


def pin_hand_nhwc_two_groups(mutant=0):
    """N=1, C=2, G=2 (one channel per group), HW=3, NHWC image
    [c0p0, c1p0, c0p1, c1p1, c0p2, c1p2] = [-1, 2, 0, 2, 1, 5], eps = 1/3.
    Group 0 = [-1, 0, 1]: mean 0, var 2/3, rstd 1.
    Group 1 = [2, 2, 5]: mean 3, deviations [-1, -1, 2], var 2, rstd sqrt(3/7).
    gamma = [1, 3], beta = [0, -1]:
    y(c0) = [-1, 0, 1]; y(c1) = 3*sqrt(3/7)*[-1, -1, 2] - 1."""
    img = np.array([-1.0, 2.0, 0.0, 2.0, 1.0, 5.0])
    y, mean, rstd = oracle.forward(img, [1.0, 3.0], [0.0, -1.0], 1, 2, 3, 2, 1 / 3, layout="nhwc", mutant=mutant)
    _assert_close(mean, [0.0, 3.0], 1e-15, 1e-15, "nhwc mean")
    _assert_close(rstd, [1.0, math.sqrt(3 / 7)], 1e-14, 0, "nhwc rstd")
    k = 3 * math.sqrt(3 / 7)
    expect = np.array([-1.0, -k - 1, 0.0, -k - 1, 1.0, 2 * k - 1])
    _assert_close(y, expect, 1e-14, 1e-14, "nhwc y")


# ----------------------------------------------------------------------------
# finite differences
# ----------------------------------------------------------------------------
def _loss(x, gamma, beta, w, N, C, HW, G, eps, layout, mutant):
    y, _, _ = oracle.forward(x, gamma, beta, N, C, HW, G, eps, layout=layout, mutant=mutant)
    return float(np.dot(y, w))


def pin_finite_differences(mutant=0):
    for layout in ("nchw", "nhwc"):
        N, C, HW, G = 2, 4, 15, 2
        r = _rng(7 if layout == "nchw" else 8)
        x = r.standard_normal(N * C * HW)
        w = r.standard_normal(N * C * HW)
        gamma = 1 + 0.3 * r.standard_normal(C)
        beta = 0.3 * r.standard_normal(C)
        eps = 1e-2
        dx, dg, db, _, _ = oracle.backward(w, x, gamma, N, C, HW, G, eps, layout=layout, mutant=mutant)

        def fd(vec, i, f):
            h = 1e-6 * max(1.0, abs(vec[i]))
            v0 = vec[i]
            vec[i] = v0 + h
            lp = f()
            vec[i] = v0 - h
            lm = f()
            vec[i] = v0
            return (lp - lm) / (2 * h)

        f = lambda: _loss(x, gamma, beta, w, N, C, HW, G, eps, layout, mutant)
        num_dx = np.array([fd(x, i, f) for i in range(x.size)])
        num_dg = np.array([fd(gamma, i, f) for i in range(C)])
        num_db = np.array([fd(beta, i, f) for i in range(C)])
        _assert_close(dx, num_dx, 1e-6, 1e-8, f"fd dx {layout}")
        _assert_close(dg, num_dg, 1e-6, 1e-8, f"fd dgamma {layout}")
        _assert_close(db, num_db, 1e-6, 1e-8, f"fd dbeta {layout}")


# ----------------------------------------------------------------------------
# torch float64 CPU library special cases
# ----------------------------------------------------------------------------
def _torch_group_norm(x4, G, gamma, beta, eps, dy4):
    xt = torch.tensor(x4, dtype=torch.float64, requires_grad=True)
    gt = torch.tensor(gamma, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(beta, dtype=torch.float64, requires_grad=True)
    y = F.group_norm(xt, G, gt, bt, eps)
    y.backward(torch.tensor(dy4, dtype=torch.float64))
    return y.detach().numpy(), xt.grad.numpy(), gt.grad.numpy(), bt.grad.numpy()


def pin_torch_group_norm(mutant=0):
    cases = [(3, 12, 5, 7, 4), (2, 8, 1, 1, 1), (1, 6, 4, 4, 6), (2, 16, 3, 9, 2)]
    for k, (N, C, H, W, G) in enumerate(cases):
        r = _rng(100 + k)
        x4 = r.standard_normal((N, C, H, W)) * 2 + 0.5
        dy4 = r.standard_normal((N, C, H, W))
        gamma = r.standard_normal(C)
        beta = r.standard_normal(C)
        eps = 1e-5
        ty, tdx, tdg, tdb = _torch_group_norm(x4, G, gamma, beta, eps, dy4)
        HW = H * W
        for layout in ("nchw", "nhwc"):
            img = x4.reshape(-1) if layout == "nchw" else _nchw_to_nhwc(x4.reshape(-1), N, C, HW)
            dimg = dy4.reshape(-1) if layout == "nchw" else _nchw_to_nhwc(dy4.reshape(-1), N, C, HW)
            y, _, _ = oracle.forward(img, gamma, beta, N, C, HW, G, eps, layout=layout, mutant=mutant)
            dx, dg, db, _, _ = oracle.backward(dimg, img, gamma, N, C, HW, G, eps, layout=layout, mutant=mutant)
            if layout == "nhwc":
                y = _nhwc_to_nchw(y, N, C, HW)
                dx = _nhwc_to_nchw(dx, N, C, HW)
            _assert_close(y, ty.reshape(-1), 1e-12, 1e-12, f"torch y {layout} {k}")
            _assert_close(dx, tdx.reshape(-1), 1e-10, 1e-11, f"torch dx {layout} {k}")
            _assert_close(dg, tdg, 1e-10, 1e-11, f"torch dgamma {layout} {k}")
            _assert_close(db, tdb, 1e-10, 1e-11, f"torch dbeta {layout} {k}")


def pin_torch_layer_norm(mutant=0):
    """G = 1 with one spatial position is LayerNorm over the channel axis."""
    N, C = 9, 40
    r = _rng(5)
    x = r.standard_normal((N, C)) * 3 - 1
    dy = r.standard_normal((N, C))
    gamma = r.standard_normal(C)
    beta = r.standard_normal(C)
    eps = 1e-5
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(gamma, requires_grad=True)
    bt = torch.tensor(beta, requires_grad=True)
    yt = F.layer_norm(xt, (C,), gt, bt, eps)
    yt.backward(torch.tensor(dy))
    y, _, _ = oracle.forward(x.reshape(-1), gamma, beta, N, C, 1, 1, eps, mutant=mutant)
    dx, dg, db, _, _ = oracle.backward(dy.reshape(-1), x.reshape(-1), gamma, N, C, 1, 1, eps, mutant=mutant)
    _assert_close(y, yt.detach().numpy().reshape(-1), 1e-12, 1e-12, "layer_norm y")
    _assert_close(dx, xt.grad.numpy().reshape(-1), 1e-10, 1e-11, "layer_norm dx")
    _assert_close(dg, gt.grad.numpy(), 1e-10, 1e-11, "layer_norm dgamma")
    _assert_close(db, bt.grad.numpy(), 1e-10, 1e-11, "layer_norm dbeta")


def pin_torch_instance_norm(mutant=0):
    """G = C is InstanceNorm with a per-channel affine."""
    N, C, H, W = 2, 5, 6, 3
    r = _rng(6)
    x = r.standard_normal((N, C, H, W))
    dy = r.standard_normal((N, C, H, W))
    gamma = r.standard_normal(C)
    beta = r.standard_normal(C)
    eps = 1e-5
    xt = torch.tensor(x, requires_grad=True)
    yt = F.instance_norm(xt, eps=eps, weight=torch.tensor(gamma), bias=torch.tensor(beta))
    yt.backward(torch.tensor(dy))
    y, _, _ = oracle.forward(x.reshape(-1), gamma, beta, N, C, H * W, C, eps, mutant=mutant)
    dx, _, _, _, _ = oracle.backward(dy.reshape(-1), x.reshape(-1), gamma, N, C, H * W, C, eps, mutant=mutant)
    _assert_close(y, yt.detach().numpy().reshape(-1), 1e-12, 1e-12, "instance_norm y")
    _assert_close(dx, xt.grad.numpy().reshape(-1), 1e-10, 1e-11, "instance_norm dx")


# ----------------------------------------------------------------------------
# closed-form invariants
# ----------------------------------------------------------------------------
def pin_invariants(mutant=0):
    N, C, H, W, G = 3, 12, 4, 6, 3
    HW = H * W
    D = C // G
    M = D * HW
    r = _rng(11)
    x = r.standard_normal(N * C * HW) * 0.05 + 2.0   # small spread: eps matters
    dy = r.standard_normal(N * C * HW)
    eps = 1e-3
    y, mean, rstd = oracle.forward(x, None, None, N, C, HW, G, eps, mutant=mutant)
    gamma = 1 + 0.2 * r.standard_normal(C)
    dx, dg, db, _, _ = oracle.backward(dy, x, gamma, N, C, HW, G, eps, mutant=mutant)
    x3 = x.reshape(N, G, M)
    y3 = y.reshape(N, G, M)
    dy3 = dy.reshape(N, G, D, HW)
    dx3 = dx.reshape(N, G, M)
    var_true = x3.var(axis=2)   # numpy's own biased variance of each slice
    _assert_close(y3.mean(axis=2), np.zeros((N, G)), 0, 1e-12, "mean(y) = 0")
    _assert_close((y3 ** 2).mean(axis=2), var_true / (var_true + eps), 1e-10, 0, "var(y) = var/(var+eps)")
    _assert_close(mean.reshape(N, G), x3.mean(axis=2), 1e-13, 1e-13, "mean = numpy mean")
    _assert_close(db, dy.reshape(N, C, HW).sum(axis=(0, 2)), 1e-12, 1e-12, "dbeta = column sum of dy")
    _assert_close(dx3.sum(axis=2), np.zeros((N, G)), 0, 1e-10, "sum dx = 0")
    xhat = (x3 - x3.mean(axis=2, keepdims=True)) / np.sqrt(var_true + eps)[..., None]
    g4 = gamma.reshape(1, G, D, 1) * dy3
    B = (g4.reshape(N, G, M) * xhat).sum(axis=2)
    rs = 1 / np.sqrt(var_true + eps)
    _assert_close((dx3 * xhat).sum(axis=2), rs * B * eps / (var_true + eps), 1e-8, 1e-10,
                  "sum dx*xhat = rstd*B*eps/(var+eps)")
    # dgamma against numpy's own xhat
    dg_np = (dy.reshape(N, C, HW) * xhat.reshape(N, C, HW)).sum(axis=(0, 2))
    _assert_close(dg, dg_np, 1e-10, 1e-11, "dgamma = sum dy*xhat")


def pin_structure(mutant=0):
    N, C, HW, G = 2, 6, 10, 3
    D = C // G
    r = _rng(21)
    x = r.standard_normal(N * C * HW)
    dy = r.standard_normal(N * C * HW)
    gamma = r.standard_normal(C)
    beta = r.standard_normal(C)
    eps = 1e-5
    # layout equivalence
    y0, m0, s0 = oracle.forward(x, gamma, beta, N, C, HW, G, eps, mutant=mutant)
    y1, m1, s1 = oracle.forward(_nchw_to_nhwc(x, N, C, HW), gamma, beta, N, C, HW, G, eps,
                                layout="nhwc", mutant=mutant)
    _assert_close(_nhwc_to_nchw(y1, N, C, HW), y0, 1e-13, 1e-13, "layout y")
    _assert_close(m1, m0, 1e-13, 1e-13, "layout mean")
    # permutation of positions inside a slice (same permutation on every channel)
    perm = r.permutation(HW)
    xp = x.reshape(N, C, HW)[:, :, perm].reshape(-1)
    dyp = dy.reshape(N, C, HW)[:, :, perm].reshape(-1)
    yp, _, _ = oracle.forward(xp, gamma, beta, N, C, HW, G, eps, mutant=mutant)
    _assert_close(yp, y0.reshape(N, C, HW)[:, :, perm].reshape(-1), 1e-12, 1e-12, "perm y")
    dx0, _, _, _, _ = oracle.backward(dy, x, gamma, N, C, HW, G, eps, mutant=mutant)
    dxp, _, _, _, _ = oracle.backward(dyp, xp, gamma, N, C, HW, G, eps, mutant=mutant)
    _assert_close(dxp, dx0.reshape(N, C, HW)[:, :, perm].reshape(-1), 1e-11, 1e-12, "perm dx")
    # scale invariance at eps = 0
    ya, _, _ = oracle.forward(x, gamma, beta, N, C, HW, G, 0.0, mutant=mutant)
    yb, _, _ = oracle.forward(x * 37.5, gamma, beta, N, C, HW, G, 0.0, mutant=mutant)
    _assert_close(yb, ya, 1e-12, 1e-12, "scale y")
    # degenerate slices: one element (M = 1) and a constant slice
    x1 = r.standard_normal(4 * 3)
    y1, _, _ = oracle.forward(x1, gamma[:3], beta[:3], 4, 3, 1, 3, eps, mutant=mutant)
    _assert_close(y1, np.tile(beta[:3], 4), 0, 1e-12, "M=1 y = beta")
    dx1, _, _, _, _ = oracle.backward(r.standard_normal(12), x1, gamma[:3], 4, 3, 1, 3, eps, mutant=mutant)
    _assert_close(dx1, np.zeros(12), 0, 1e-12, "M=1 dx = 0")
    xc = np.full(N * C * HW, 0.75)
    yc, _, sc = oracle.forward(xc, gamma, beta, N, C, HW, G, eps, mutant=mutant)
    _assert_close(yc, np.repeat(np.tile(beta, N), HW), 0, 1e-12, "constant y = beta")
    _assert_close(sc, np.full(N * G, 1 / math.sqrt(eps)), 1e-12, 0, "constant rstd = eps^-1/2")
    # constant slice: xhat = 0 and var = 0, so dx = eps^-1/2 * (gamma_c*dy - mean of gamma*dy
    # over the slice); the B term vanishes with xhat
    dxc, _, _, _, _ = oracle.backward(dy, xc, gamma, N, C, HW, G, eps, mutant=mutant)
    gdy = (gamma.reshape(1, C, 1) * dy.reshape(N, C, HW)).reshape(N, G, D * HW)
    expect = (gdy - gdy.mean(axis=2, keepdims=True)) / math.sqrt(eps)
    _assert_close(dxc, expect.reshape(-1), 1e-10, 1e-10, "constant slice dx")


# ----------------------------------------------------------------------------
# RMSNorm over rows
# ----------------------------------------------------------------------------
def pin_rms_hand(mutant=0):
    """Row [3, 4], gamma [2, 0.5], eps 0: mean square 12.5, r = 1/sqrt(12.5);
    y = [6r, 2r]; with dy = [1, 0]: B = 6r, dx = [r*(2 - 9r^2), -12r^3]
    (= [32r/25, -24r/25], the derivative of L = 2*x0*r worked by hand), and
    dgamma = [3r, 0]."""
    x = [3.0, 4.0]
    g = [2.0, 0.5]
    r = 1.0 / math.sqrt(12.5)
    y, rs = oracle.rms_forward(x, g, 1, 2, 1, 0.0, mutant=mutant)
    _assert_close(rs, [r], 1e-15, 0, "rms hand r")
    _assert_close(y, [6 * r, 2 * r], 1e-15, 0, "rms hand y")
    dx, dg, _ = oracle.rms_backward([1.0, 0.0], x, g, 1, 2, 1, 0.0, mutant=mutant)
    _assert_close(dx, [32 * r / 25, -24 * r / 25], 1e-14, 1e-15, "rms hand dx")
    _assert_close(dg, [3 * r, 0.0], 1e-15, 1e-15, "rms hand dgamma")


def pin_torch_rms_norm(mutant=0):
    """torch's float64 CPU rms_norm with autograd (the operator itself)."""
    for k, (N, C, eps, scale) in enumerate([(9, 40, 1e-5, 1.0), (5, 8, 1e-6, 0.01), (3, 256, 1e-5, 3.0)]):
        r = _rng(300 + k)
        x = r.standard_normal((N, C)) * scale + 0.3
        dy = r.standard_normal((N, C))
        gamma = r.standard_normal(C)
        xt = torch.tensor(x, requires_grad=True)
        gt = torch.tensor(gamma, requires_grad=True)
        yt = F.rms_norm(xt, (C,), gt, eps)
        yt.backward(torch.tensor(dy))
        y, _ = oracle.rms_forward(x.reshape(-1), gamma, N, C, 1, eps, mutant=mutant)
        dx, dg, _ = oracle.rms_backward(dy.reshape(-1), x.reshape(-1), gamma, N, C, 1, eps, mutant=mutant)
        _assert_close(y, yt.detach().numpy().reshape(-1), 1e-12, 1e-12, f"rms_norm y {k}")
        _assert_close(dx, xt.grad.numpy().reshape(-1), 1e-10, 1e-11, f"rms_norm dx {k}")
        _assert_close(dg, gt.grad.numpy(), 1e-10, 1e-11, f"rms_norm dgamma {k}")


def pin_rms_invariants(mutant=0):
    """gamma = 1: each row of y has mean square ms/(ms + eps); at eps = 0 each
    row's dx is orthogonal to x (sum dx*x = r*sum(dy*x)*eps/(ms + eps)) and y
    is unchanged by scaling x; rows of D = C/G channels with G > 1 are the
    G = 1 operator on each group's columns."""
    N, C, G = 6, 24, 3
    D = C // G
    r = _rng(17)
    x = r.standard_normal((N, C)) * 2 + 1
    dy = r.standard_normal((N, C))
    eps = 0.05
    y, rs = oracle.rms_forward(x.reshape(-1), None, N, C, 1, eps, mutant=mutant)
    ms = (x ** 2).mean(axis=1)
    _assert_close((y.reshape(N, C) ** 2).mean(axis=1), ms / (ms + eps), 1e-12, 1e-14, "rms mean square of y")
    dx, _, _ = oracle.rms_backward(dy.reshape(-1), x.reshape(-1), None, N, C, 1, eps, mutant=mutant)
    lhs = (dx.reshape(N, C) * x).sum(axis=1)
    rhs = rs * (dy * x).sum(axis=1) * eps / (ms + eps)
    _assert_close(lhs, rhs, 1e-10, 1e-12, "rms sum dx*x")
    y0, _ = oracle.rms_forward(x.reshape(-1), None, N, C, 1, 0.0, mutant=mutant)
    y1, _ = oracle.rms_forward((x * 37.5).reshape(-1), None, N, C, 1, 0.0, mutant=mutant)
    _assert_close(y1, y0, 1e-13, 1e-14, "rms scale invariance")
    gamma = r.standard_normal(C)
    yg, rg = oracle.rms_forward(x.reshape(-1), gamma, N, C, G, eps, mutant=mutant)
    dxg, dgg, _ = oracle.rms_backward(dy.reshape(-1), x.reshape(-1), gamma, N, C, G, eps, mutant=mutant)
    for g in range(G):
        cs = slice(g * D, (g + 1) * D)
        xs = np.ascontiguousarray(x[:, cs])
        ys, rss = oracle.rms_forward(xs.reshape(-1), gamma[cs], N, D, 1, eps, mutant=mutant)
        dxs, dgs, _ = oracle.rms_backward(np.ascontiguousarray(dy[:, cs]).reshape(-1), xs.reshape(-1), gamma[cs],
                                          N, D, 1, eps, mutant=mutant)
        _assert_close(yg.reshape(N, C)[:, cs].reshape(-1), ys, 1e-14, 0, f"rms groups y {g}")
        _assert_close(rg.reshape(N, G)[:, g], rss, 1e-15, 0, f"rms groups r {g}")
        _assert_close(dxg.reshape(N, C)[:, cs].reshape(-1), dxs, 1e-13, 1e-15, f"rms groups dx {g}")
        _assert_close(dgg[cs], dgs, 1e-13, 1e-15, f"rms groups dgamma {g}")


ALL_PINS = [pin_hand_slice, pin_hand_textbook, pin_hand_nhwc_two_groups, pin_finite_differences,
            pin_torch_group_norm, pin_torch_layer_norm, pin_torch_instance_norm, pin_invariants,
            pin_structure, pin_rms_hand, pin_torch_rms_norm, pin_rms_invariants]

# planted mistakes compiled into the oracle's mutant build (see gn_oracle.c)
MUTANTS = {
    1: "unbiased variance (M-1)",
    2: "E[x^2]-E[x]^2 written with the wrong moment",
    3: "eps dropped from rstd",
    4: "beta dropped from y",
    5: "B term dropped from dx",
    6: "sign of the B term in dx",
    7: "dgamma summed with raw x instead of xhat",
    8: "RMSNorm with the mean subtracted",
    9: "eps dropped from the RMSNorm r",
    10: "B term dropped from the RMSNorm dx",
    11: "RMSNorm dgamma summed with raw x",
}
