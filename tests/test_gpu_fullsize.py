"""Full-size parity on the benchmark workloads, in the launch configuration
bench.py times (automatic path choice, default options).

* NHWC fp16 1x128x1024x2048, G=16 and rows bf16 131072x4096: every output
  against the fp64 oracle on the whole tensor.
* RMSNorm bf16 131072x4096: every output against the fp64 oracle.
* NCHW fp32 112x64x512x512, G=8 (7.5 GB per tensor), the same shape in bf16,
  and its 510x510 centre crops (the strided workload): y, dx, mean and rstd of
  sampled slices, each the oracle's result on that slice alone (a slice is its
  own GroupNorm problem with one group); dgamma/dbeta of two whole groups, the
  oracle's result on the group's sub-tensor (all samples, the group's
  channels, one group).
"""
import gc

import numpy as np
import pytest
import torch

import normalization_gn_stats_amd as gn
import oracle
from normalization_gn_stats_amd import inputs
from gpu_harness import (ALL, PARAM_REL_L2, STAT_TOL, TOL, check_rms_against_oracle, close, img64, rel_l2,
                         run_gpu, run_rms_gpu, say)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def _full_compare(wl, expect_path):
    say(f"[full] {wl.name}: generating on the device")
    data = inputs.make_inputs(wl, seed=0, device="cuda")
    out = run_gpu(wl, data)
    assert out["fwd_plan"].path == expect_path and out["bwd_plan"].path == expect_path
    say(f"[full] {wl.name}: copying to the host")
    rtol, atol = TOL[wl.dtype]
    x64 = img64(data["x"], wl.layout)
    dy64 = img64(data["dy"], wl.layout)
    g64 = data["gamma"].double().cpu().numpy()
    b64 = data["beta"].double().cpu().numpy()
    eps = float(np.float32(wl.eps))
    del data
    say(f"[full] {wl.name}: oracle forward")
    ry, rmean, rrstd = oracle.forward(x64, g64, b64, wl.N, wl.C, wl.HW, wl.G, eps, layout=wl.layout)
    close(img64(out["y"], wl.layout), ry, rtol, atol, f"{wl.name} y")
    del ry
    close(out["mean"].cpu().double().numpy(), rmean, *STAT_TOL, f"{wl.name} mean")
    close(out["rstd"].cpu().double().numpy(), rrstd, *STAT_TOL, f"{wl.name} rstd")
    say(f"[full] {wl.name}: oracle backward")
    rdx, rdg, rdb, _, _ = oracle.backward(dy64, x64, g64, wl.N, wl.C, wl.HW, wl.G, eps, layout=wl.layout)
    close(img64(out["dx"], wl.layout), rdx, rtol, atol, f"{wl.name} dx")
    rel_l2(out["dgamma"].cpu().numpy(), rdg, f"{wl.name} dgamma")
    rel_l2(out["dbeta"].cpu().numpy(), rdb, f"{wl.name} dbeta")
    say(f"[full] {wl.name}: all outputs within tolerance")
    del rdx, x64, dy64, out
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_full_nhwc_image():
    _need_gpu()
    _full_compare(inputs.NHWC_IMG, gn.GN_PATH_STREAM)


@pytest.mark.timeout(900)
def test_full_rows_bf16_131072x4096():
    _need_gpu()
    _full_compare(inputs.ROWS_BIG, gn.GN_PATH_ROWS)


@pytest.mark.timeout(900)
def test_full_nchw_sampled():
    _need_gpu()
    _nchw_sampled(inputs.NCHW_BIG, gn.GN_PATH_SLAB)


# The NCHW benchmark shape in bf16: the slab kernels' 16-bit tiles (8 chunks
# per thread) and their own loop order in the backward.
NCHW_BIG_BF16 = inputs.Workload("nchw_bf16_112x64x512x512_g8", 112, 64, 512, 512, 8, "bf16", "nchw")


@pytest.mark.timeout(900)
def test_full_nchw_bf16_sampled():
    _need_gpu()
    _nchw_sampled(NCHW_BIG_BF16, gn.GN_PATH_SLAB)


@pytest.mark.timeout(900)
def test_full_nchw_crop_sampled():
    """The strided workload bench.py times: 510x510 centre crops of the
    112x64 images, read and written in place by the generic kernels."""
    _need_gpu()
    _nchw_sampled(inputs.CROP_BIG, gn.GN_PATH_GENERIC)


def _nchw_sampled(wl, expect_path):
    say(f"[full] {wl.name}: generating on the device")
    data = inputs.make_inputs(wl, seed=0, device="cuda")
    out = run_gpu(wl, data)
    assert out["fwd_plan"].path == expect_path and out["bwd_plan"].path == expect_path
    rtol, atol = TOL[wl.dtype]
    eps = float(np.float32(wl.eps))
    D = wl.C // wl.G
    gam = data["gamma"].double().cpu().numpy()
    bet = data["beta"].double().cpu().numpy()
    rng = np.random.default_rng(11)
    slices = sorted({0, wl.N * wl.G - 1, 455} | set(int(v) for v in rng.integers(0, wl.N * wl.G, 3)))
    for s in slices:
        n, g = divmod(s, wl.G)
        say(f"[full] {wl.name}: slice n={n} g={g}")
        cs = slice(g * D, (g + 1) * D)
        xs = data["x"][n, cs].double().cpu().numpy().reshape(-1)
        dys = data["dy"][n, cs].double().cpu().numpy().reshape(-1)
        ry, rm, rr = oracle.forward(xs, gam[cs], bet[cs], 1, D, wl.HW, 1, eps)
        close(out["y"][n, cs].double().cpu().numpy().reshape(-1), ry, rtol, atol, f"y slice {s}")
        close([out["mean"].view(-1)[s].item()], rm, *STAT_TOL, f"mean slice {s}")
        close([out["rstd"].view(-1)[s].item()], rr, *STAT_TOL, f"rstd slice {s}")
        rdx, _, _, _, _ = oracle.backward(dys, xs, gam[cs], 1, D, wl.HW, 1, eps, want_dgamma=False,
                                          want_dbeta=False)
        close(out["dx"][n, cs].double().cpu().numpy().reshape(-1), rdx, rtol, atol, f"dx slice {s}")
    for g in (0, wl.G - 1):
        say(f"[full] {wl.name}: dgamma/dbeta of group {g}")
        cs = slice(g * D, (g + 1) * D)
        xg = data["x"][:, cs].contiguous().double().cpu().numpy().reshape(-1)
        dyg = data["dy"][:, cs].contiguous().double().cpu().numpy().reshape(-1)
        _, rdg, rdb, _, _ = oracle.backward(dyg, xg, gam[cs], wl.N, D, wl.HW, 1, eps, want_dx=False)
        rel_l2(out["dgamma"][cs].cpu().numpy(), rdg, f"dgamma group {g}", PARAM_REL_L2)
        rel_l2(out["dbeta"][cs].cpu().numpy(), rdb, f"dbeta group {g}", PARAM_REL_L2)
        del xg, dyg
        gc.collect()
    say(f"[full] {wl.name}: sampled outputs within tolerance")
    del data, out
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_full_rms_bf16_131072x4096():
    """RMSNorm at the rms_llm shape of the ROCm/pytorch PR #3564 table, every
    output against the fp64 oracle on the whole tensor."""
    _need_gpu()
    wl = inputs.ROWS_BIG.scaled(name="rms_bf16_131072x4096", eps=1e-6)
    say(f"[full] {wl.name}: generating on the device")
    data = inputs.make_inputs(wl, seed=0, device="cuda")
    out = run_rms_gpu(wl, data)
    assert out["fwd_plan"].path == gn.GN_PATH_ROWS and out["bwd_plan"].path == gn.GN_PATH_ROWS
    say(f"[full] {wl.name}: oracle")
    check_rms_against_oracle(wl, data, out)
    say(f"[full] {wl.name}: all outputs within tolerance")
    del data, out
    gc.collect()
    torch.cuda.empty_cache()


def test_full_sizes_are_the_benchmark_workloads():
    assert (inputs.NHWC_IMG.N, inputs.NHWC_IMG.C, inputs.NHWC_IMG.HW) == (1, 128, 1024 * 2048)
    assert (inputs.ROWS_BIG.N, inputs.ROWS_BIG.C) == (131072, 4096)
    assert (inputs.NCHW_BIG.N, inputs.NCHW_BIG.C, inputs.NCHW_BIG.HW) == (112, 64, 512 * 512)
    assert (inputs.CROP_BIG.N, inputs.CROP_BIG.C, inputs.CROP_BIG.H, inputs.CROP_BIG.W, inputs.CROP_BIG.crop) == \
        (112, 64, 510, 510, 1)
    assert ALL == 7
