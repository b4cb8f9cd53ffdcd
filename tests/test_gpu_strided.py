"""Strided (non-contiguous) tensors on the GPU: crops, slices, steps,
permuted, broadcast and mixed-layout views, read and written in place by the
generic kernels, against the fp64 oracle run on the same logical values.

ROCm/pytorch PR #3564's test run includes a correctness test on
non-contiguous input; the POPCORNBENCH GroupNorm trace weighs reading
arbitrary strides against copying.  Here no copy is made: the C calls
receive the views' pointers and element strides (checked by plan info and by
sentinels around the output views).  Tolerances as in the other parity
tests (gpu_harness).
"""
import ctypes

import numpy as np
import pytest
import torch

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import _lib
import oracle
from normalization_gn_stats_amd import inputs
from gpu_harness import ALL, PARAM_REL_L2, STAT_TOL, TOL, close, rel_l2, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = 1234.0


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def _flat64(t):
    """Logical-order (NCHW) float64 numpy copy of any view."""
    return t.detach().contiguous().to("cpu", torch.float64).numpy().reshape(-1)


def _dims(x):
    N, C = int(x.shape[0]), int(x.shape[1])
    HW = int(np.prod(x.shape[2:])) if x.dim() > 2 else 1
    return N, C, HW


def _oracle(x, dy, gamma, beta, G, eps, mask):
    N, C, HW = _dims(x)
    e = float(np.float32(eps))
    g64, b64 = gamma.double().cpu().numpy(), beta.double().cpu().numpy()
    ry, rm, rr = oracle.forward(_flat64(x), g64, b64, N, C, HW, G, e)
    rdx, rdg, rdb, _, _ = oracle.backward(_flat64(dy), _flat64(x), g64, N, C, HW, G, e,
                                          want_dx=bool(mask & gn.GN_GRAD_DX),
                                          want_dgamma=bool(mask & gn.GN_GRAD_DGAMMA),
                                          want_dbeta=bool(mask & gn.GN_GRAD_DBETA))
    return ry, rm, rr, rdx, rdg, rdb


def _check(tag, dtype, out, ref, mask):
    rtol, atol = TOL[dtype]
    ry, rm, rr, rdx, rdg, rdb = ref
    close(_flat64(out["y"]), ry, rtol, atol, f"{tag} y")
    close(out["mean"].reshape(-1).cpu().double().numpy(), rm, *STAT_TOL, f"{tag} mean")
    close(out["rstd"].reshape(-1).cpu().double().numpy(), rr, *STAT_TOL, f"{tag} rstd")
    if mask & gn.GN_GRAD_DX:
        close(_flat64(out["dx"]), rdx, rtol, atol, f"{tag} dx")
    if mask & gn.GN_GRAD_DGAMMA:
        rel_l2(out["dgamma"].cpu().numpy(), rdg, f"{tag} dgamma", PARAM_REL_L2)
    if mask & gn.GN_GRAD_DBETA:
        rel_l2(out["dbeta"].cpu().numpy(), rdb, f"{tag} dbeta", PARAM_REL_L2)


def _run(x, dy, gamma, beta, G, eps=1e-5, mask=ALL):
    fi, bi = gn.PlanInfo(), gn.PlanInfo()
    y, mean, rstd = gn.forward(x, gamma, beta, G, eps, info=fi)
    dx, dg, db = gn.backward(dy, x, mean, rstd, gamma, G, mask, info=bi)
    torch.cuda.synchronize()
    return dict(y=y, mean=mean, rstd=rstd, dx=dx, dgamma=dg, dbeta=db, fwd_plan=fi, bwd_plan=bi)


# Each case: (dtype, G, builder of (x, dy) views from seeded base tensors).
def _crop_w(dt):
    return (inputs.draw((2, 32, 16, 20), dt, 11, DEV)[..., 2:18], inputs.draw((2, 32, 16, 20), dt, 12, DEV)[..., 2:18])


def _channel_slice(dt):
    return (inputs.draw((2, 64, 8, 8), dt, 13, DEV)[:, 8:40], inputs.draw((2, 64, 8, 8), dt, 14, DEV)[:, 8:40])


def _transposed(dt):
    return (inputs.draw((3, 16, 12, 10), dt, 15, DEV).transpose(2, 3),
            inputs.draw((3, 16, 12, 10), dt, 16, DEV).transpose(2, 3))


def _nhwc_crop(dt):
    return (inputs.draw((2, 24, 9, 11), dt, 17, DEV, channels_last=True)[:, :, 1:, :-2],
            inputs.draw((2, 24, 9, 11), dt, 18, DEV, channels_last=True)[:, :, 1:, :-2])


def _steps(dt):
    return (inputs.draw((2, 12, 15, 17), dt, 19, DEV)[:, :, ::2, ::3],
            inputs.draw((2, 12, 15, 17), dt, 20, DEV)[:, :, ::2, ::3])


def _rows_2d(dt):
    return inputs.draw((64, 195), dt, 21, DEV)[:, :96], inputs.draw((64, 195), dt, 22, DEV)[:, 99:195]


def _broadcast_n(dt):
    return inputs.draw((1, 16, 6, 7), dt, 23, DEV).expand(3, 16, 6, 7), inputs.draw((3, 16, 6, 7), dt, 24, DEV)


def _spatial_3d(dt):
    return (inputs.draw((2, 8, 4, 6, 10), dt, 25, DEV)[..., 1:5], inputs.draw((2, 8, 4, 6, 10), dt, 26, DEV)[..., 1:5])


def _mixed_layouts(dt):
    return inputs.draw((2, 32, 10, 12), dt, 27, DEV), inputs.draw((2, 32, 10, 12), dt, 28, DEV, channels_last=True)


def _multi_tile_nchw(dt):
    # 128x128 crops of 130x130 images: several tiles per slice and rows of 128
    return (inputs.draw((2, 64, 130, 130), dt, 29, DEV)[..., 1:-1, 1:-1],
            inputs.draw((2, 64, 130, 130), dt, 30, DEV)[..., 1:-1, 1:-1])


def _multi_tile_nhwc(dt):
    # channel-innermost crops: eight channels per group, packed rows
    return (inputs.draw((1, 32, 200, 200), dt, 31, DEV, channels_last=True)[:, :, 3:190, 5:199],
            inputs.draw((1, 32, 200, 200), dt, 32, DEV, channels_last=True)[:, :, 3:190, 5:199])


def _planes_wide(dt):
    # planes of 20x74 in unit-stride rows: the backward's plane-sum reductions
    return (inputs.draw((3, 20, 24, 80), dt, 35, DEV)[..., 2:22, 3:77],
            inputs.draw((3, 20, 24, 80), dt, 36, DEV)[..., 2:22, 3:77])


def _unaligned(dt):
    # views starting one element past a 16-byte boundary
    def mk(seed):
        flat = inputs.draw((1 + 2 * 12 * 7 * 9,), dt, seed, DEV)
        return flat[1:].view(2, 12, 7, 9)[..., :8]
    return mk(33), mk(34)


CASES = {
    "crop_w_f32": ("f32", 8, _crop_w),
    "channel_slice_bf16": ("bf16", 4, _channel_slice),
    "transposed_f16": ("f16", 4, _transposed),
    "nhwc_crop_f16": ("f16", 6, _nhwc_crop),
    "steps_f32": ("f32", 3, _steps),
    "rows_2d_bf16_g1": ("bf16", 1, _rows_2d),
    "rows_2d_f32_g4": ("f32", 4, _rows_2d),
    "broadcast_n_f32": ("f32", 4, _broadcast_n),
    "spatial_3d_bf16": ("bf16", 2, _spatial_3d),
    "mixed_layouts_f16": ("f16", 8, _mixed_layouts),
    "multi_tile_nchw_f16": ("f16", 8, _multi_tile_nchw),
    "multi_tile_nhwc_bf16": ("bf16", 4, _multi_tile_nhwc),
    "unaligned_f16": ("f16", 3, _unaligned),
    "planes_f32_g1": ("f32", 1, _planes_wide),
    "planes_bf16_g5": ("bf16", 5, _planes_wide),
    "planes_f16_g20": ("f16", 20, _planes_wide),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_strided_views_match_oracle(name):
    _need_gpu()
    dt, G, build = CASES[name]
    say(f"[strided] {name}")
    x, dy = build(dt)
    gamma, beta = inputs.draw_affine(int(x.shape[1]), 40, DEV)
    out = _run(x, dy, gamma, beta, G)
    # the backward of mixed layouts has non-dense partners; the forward of it is dense
    if name != "mixed_layouts_f16":
        assert out["fwd_plan"].path == gn.GN_PATH_GENERIC
    assert out["bwd_plan"].path == gn.GN_PATH_GENERIC
    _check(name, dt, out, _oracle(x, dy, gamma, beta, G, 1e-5, ALL), ALL)


@pytest.mark.parametrize("mask", [gn.GN_GRAD_DX, gn.GN_GRAD_DGAMMA, gn.GN_GRAD_DBETA,
                                  gn.GN_GRAD_DGAMMA | gn.GN_GRAD_DBETA])
def test_strided_masks(mask):
    _need_gpu()
    x, dy = _nhwc_crop("bf16")
    gamma, beta = inputs.draw_affine(24, 41, DEV)
    out = _run(x, dy, gamma, beta, 6, mask=mask)
    if not mask & gn.GN_GRAD_DX:
        assert out["dx"] is None
    _check(f"mask{mask}", "bf16", out, _oracle(x, dy, gamma, beta, 6, 1e-5, mask), mask)


@pytest.mark.parametrize("mask", [gn.GN_GRAD_DX, gn.GN_GRAD_DGAMMA, gn.GN_GRAD_DBETA, ALL])
def test_plane_sum_masks(mask):
    _need_gpu()
    x, dy = _planes_wide("f16")
    gamma, beta = inputs.draw_affine(20, 48, DEV)
    out = _run(x, dy, gamma, beta, 4, mask=mask)
    _check(f"planes mask{mask}", "f16", out, _oracle(x, dy, gamma, beta, 4, 1e-5, mask), mask)


def test_strided_no_affine():
    _need_gpu()
    x, dy = _crop_w("f32")
    y, mean, rstd = gn.forward(x, None, None, 8)
    dx, _, _ = gn.backward(dy, x, mean, rstd, None, 8, gn.GN_GRAD_DX)
    ones, zeros = torch.ones(32), torch.zeros(32)
    ry, rm, rr, rdx, _, _ = _oracle(x, dy, ones, zeros, 8, 1e-5, gn.GN_GRAD_DX)
    rtol, atol = TOL["f32"]
    close(_flat64(y), ry, rtol, atol, "no-affine y")
    close(_flat64(dx), rdx, rtol, atol, "no-affine dx")


def _guarded(shape, dt, index):
    """An output view `index` of a buffer filled with a sentinel, and the mask
    of the buffer's elements outside the view."""
    big = torch.full(shape, SENTINEL, device=DEV, dtype=inputs.DTYPES[dt])
    mark = torch.zeros(shape, dtype=torch.bool)
    mark[index] = True
    return big, big[index], ~mark


def test_outputs_written_in_place_and_nowhere_else():
    _need_gpu()
    dt, G = "f16", 4
    x, dy = _transposed(dt)                       # (3, 16, 10, 12)
    gamma, beta = inputs.draw_affine(16, 42, DEV)
    idx = (slice(None), slice(None), slice(1, 11), slice(2, 14))
    ybig, y, yout = _guarded((3, 16, 12, 16), dt, idx)
    dxbig, dx, dxout = _guarded((3, 16, 12, 16), dt, idx)
    mean = torch.empty(3 * G, device=DEV)
    rstd = torch.empty(3 * G, device=DEV)
    dg = torch.empty(16, device=DEV)
    db = torch.empty(16, device=DEV)
    N, C, H, W, (sx, sy) = gn.strided_dims(x, y)
    wsf = gn.forward_strided_workspace_size(N, C, H, W, G, gn.GN_F16, sx, sy)
    _, _, _, _, (sdy, sx2, sdx) = gn.strided_dims(dy, x, dx)
    wsb = gn.backward_strided_workspace_size(N, C, H, W, G, gn.GN_F16, sdy, sx2, sdx, ALL)
    ws = torch.empty(max(wsf, wsb, 1), device=DEV, dtype=torch.uint8)
    fi, bi = gn.PlanInfo(), gn.PlanInfo()
    gn.forward_into(x, gamma, beta, G, 1e-5, y, mean, rstd, ws, info=fi)
    gn.backward_into(dy, x, mean, rstd, gamma, G, ALL, dx, dg, db, ws, info=bi)
    torch.cuda.synchronize()
    assert fi.path == gn.GN_PATH_GENERIC and bi.path == gn.GN_PATH_GENERIC
    assert torch.all(ybig.cpu()[yout] == SENTINEL), "forward wrote outside the y view"
    assert torch.all(dxbig.cpu()[dxout] == SENTINEL), "backward wrote outside the dx view"
    _check("in-place views", dt, dict(y=y, mean=mean, rstd=rstd, dx=dx, dgamma=dg, dbeta=db),
           _oracle(x, dy, gamma, beta, G, 1e-5, ALL), ALL)


def test_dense_strides_take_the_dense_paths():
    _need_gpu()
    # a channels_last tensor through the strided binding helpers is the dense call
    x = inputs.draw((1, 128, 64, 130), "f16", 43, DEV, channels_last=True)
    dy = inputs.draw((1, 128, 64, 130), "f16", 44, DEV, channels_last=True)
    gamma, beta = inputs.draw_affine(128, 45, DEV)
    N, C, H, W, (sx, sy) = gn.strided_dims(x, x)
    y = torch.empty_like(x)
    mean = torch.empty(16, device=DEV)
    rstd = torch.empty(16, device=DEV)
    wsb = gn.forward_strided_workspace_size(N, C, H, W, 16, gn.GN_F16, sx, sy)
    ws = torch.empty(max(wsb, 1), device=DEV, dtype=torch.uint8)
    info = gn.PlanInfo()
    o = _lib.Options(0, 0, ctypes.pointer(info), None, None)
    st = _lib.lib().gn_forward_strided(ctypes.c_void_p(x.data_ptr()), sx, ctypes.c_void_p(gamma.data_ptr()),
                                       ctypes.c_void_p(beta.data_ptr()), ctypes.c_void_p(y.data_ptr()), sy,
                                       ctypes.c_void_p(mean.data_ptr()), ctypes.c_void_p(rstd.data_ptr()), N, C, H, W,
                                       16, 1e-5, gn.GN_F16, ctypes.c_void_p(ws.data_ptr()), wsb,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(o))
    torch.cuda.synchronize()
    assert st == 0
    assert info.path == gn.select_path(False, N, C, H * W, 16, gn.GN_F16, gn.GN_NHWC)
    assert info.path != gn.GN_PATH_GENERIC
    ry, rm, rr, _, _, _ = _oracle(x, dy, gamma, beta, 16, 1e-5, gn.GN_GRAD_DBETA)
    rtol, atol = TOL["f16"]
    close(_flat64(y), ry, rtol, atol, "dense-by-strides y")
    close(mean.cpu().double().numpy(), rm, *STAT_TOL, "dense-by-strides mean")


def test_strided_forced_paths():
    _need_gpu()
    x, dy = _crop_w("f32")
    gamma, beta = inputs.draw_affine(32, 46, DEV)
    with pytest.raises(gn.GNError):
        gn.forward(x, gamma, beta, 8, force_path="slab")
    y, m, r = gn.forward(x, gamma, beta, 8, force_path="generic")
    y2, m2, r2 = gn.forward(x, gamma, beta, 8)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(m, m2) and torch.equal(r, r2)


def test_strided_is_deterministic():
    _need_gpu()
    x, dy = _multi_tile_nhwc("bf16")
    gamma, beta = inputs.draw_affine(32, 47, DEV)
    a = _run(x, dy, gamma, beta, 4)
    b = _run(x, dy, gamma, beta, 4)
    for k in ("y", "mean", "rstd", "dx", "dgamma", "dbeta"):
        assert torch.equal(a[k], b[k]), k


def _random_view(rng, shape, dt, seed, allow_broadcast):
    """A seeded view of logical `shape` cut out of a larger dense tensor:
    dimensions permuted in memory, each given a margin (crop) and possibly a
    step, or (inputs only) broadcast along one dimension."""
    nd = len(shape)
    steps = [int(rng.choice([1, 1, 1, 2, 3])) for _ in range(nd)]
    margins = [int(rng.integers(0, 3)) for _ in range(nd)]
    base_shape = [shape[i] * steps[i] + margins[i] for i in range(nd)]
    perm = [int(v) for v in rng.permutation(nd)]
    # a dense buffer whose memory order is `perm`, viewed in logical order
    base = inputs.draw([base_shape[p] for p in perm], dt, seed, DEV)
    inv = [perm.index(i) for i in range(nd)]
    base = base.permute(*inv)
    idx = tuple(slice(margins[i], margins[i] + shape[i] * steps[i], steps[i]) for i in range(nd))
    v = base[idx]
    if allow_broadcast and rng.random() < 0.25:
        d = int(rng.integers(0, nd))
        one = [slice(None)] * nd
        one[d] = slice(0, 1)
        v = v[tuple(one)].expand(*shape)
    assert tuple(v.shape) == tuple(shape)
    return v


@pytest.mark.parametrize("case", range(24))
def test_random_strided_views(case):
    """Seeded random views for x, dy (inputs) and y, dx (outputs): permuted
    memory orders, margins, steps and broadcasts, ragged extents, every dtype,
    3-, 4- and 5-D; forward and backward against the oracle."""
    _need_gpu()
    rng = np.random.default_rng(1000 + case)
    dt = ["f32", "f16", "bf16"][case % 3]
    nd = [4, 4, 3, 5][case % 4]
    G = int(rng.choice([1, 2, 4]))
    C = G * int(rng.integers(1, 6))
    N = int(rng.integers(1, 4))
    spatial = [int(rng.integers(1, 20)) for _ in range(nd - 2)]
    if nd == 5:
        spatial = [int(rng.integers(1, 6)) for _ in range(3)]
    shape = [N, C, *spatial]
    x = _random_view(rng, shape, dt, 2 * case, True)
    dy = _random_view(rng, shape, dt, 2 * case + 1, True)
    y = _random_view(rng, shape, dt, 500 + case, False)
    dx = _random_view(rng, shape, dt, 700 + case, False)
    gamma, beta = inputs.draw_affine(C, 900 + case, DEV)
    say(f"[strided-random] case {case}: {dt} shape {shape} G={G} x.stride={x.stride()} y.stride={y.stride()}")
    try:
        gn.strided_dims(x, y, dy, dx)
    except ValueError:
        pytest.skip("these views need three spatial dimensions")   # the binding's documented limit
    mean = torch.empty(N * G, device=DEV)
    rstd = torch.empty(N * G, device=DEV)
    dg = torch.empty(C, device=DEV)
    db = torch.empty(C, device=DEV)
    ws = torch.empty(1 << 24, device=DEV, dtype=torch.uint8)
    gn.forward_into(x, gamma, beta, G, 1e-5, y, mean, rstd, ws)
    gn.backward_into(dy, x, mean, rstd, gamma, G, ALL, dx, dg, db, ws)
    torch.cuda.synchronize()
    _check(f"random {case}", dt, dict(y=y, mean=mean, rstd=rstd, dx=dx, dgamma=dg, dbeta=db),
           _oracle(x, dy, gamma, beta, G, 1e-5, ALL), ALL)
