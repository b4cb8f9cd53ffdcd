"""Full-size parity on the benchmark workloads.

* NHWC fp16 1x128x1024x2048, G=16 (the apex PR #2018 reproducer's image):
  every output against the fp64 oracle on the whole tensor, in the launch
  configuration bench.py times (automatic path choice: the stream kernels)
  and with the one-pass cooperative slab kernels forced, at their natural
  residency cap and at a cap of 108 workgroups (the A100's SM count in the
  apex PR's reviewer comment).  Almost every one of the image's 8192 forward
  and 16384 backward tiles is then an overflow tile: reduced in phase 1 by a
  resident workgroup and reloaded for its output after the global
  reduction -- the case that PR's reviewer notes the large regression test
  never reached.  The oracle runs once for the three.
* Rows bf16 131072x4096 and RMSNorm bf16 131072x4096: every output against
  the fp64 oracle on the whole tensor.
* NCHW fp32 112x64x512x512, G=8 (7.5 GB per tensor; the POPCORNBENCH
  GroupNorm problem's shape): every output.  The host walks the 112 samples
  one at a time (a sample is its own GroupNorm problem: its 8 slices hold
  every element that depends on it); y, dx, mean and rstd of every slice are
  compared with the oracle's result on that sample, and dgamma/dbeta of all
  64 channels with the sum over samples, in float64, of the oracle's
  per-sample dgamma/dbeta (the definition sums over n and p).
* The same shape in bf16 and the 510x510 centre crops (the strided
  workload): the same walk over every sample.
"""
import gc

import numpy as np
import pytest
import torch

import normalization_gn_stats_amd as gn
import oracle
from normalization_gn_stats_amd import inputs
from gpu_harness import (ALL, STAT_TOL, TOL, check_rms_against_oracle, close, img64, rel_l2, run_gpu,
                         run_rms_gpu, say)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def _release():
    gc.collect()
    torch.cuda.empty_cache()


def _oracle_whole(wl, data):
    """The oracle's forward and backward on the whole tensor (float64)."""
    x64 = img64(data["x"], wl.layout)
    dy64 = img64(data["dy"], wl.layout)
    g64 = data["gamma"].double().cpu().numpy()
    b64 = data["beta"].double().cpu().numpy()
    eps = float(np.float32(wl.eps))
    say(f"[full] {wl.name}: oracle forward")
    ry, rmean, rrstd = oracle.forward(x64, g64, b64, wl.N, wl.C, wl.HW, wl.G, eps, layout=wl.layout)
    say(f"[full] {wl.name}: oracle backward")
    rdx, rdg, rdb, _, _ = oracle.backward(dy64, x64, g64, wl.N, wl.C, wl.HW, wl.G, eps, layout=wl.layout)
    return dict(y=ry, mean=rmean, rstd=rrstd, dx=rdx, dgamma=rdg, dbeta=rdb)


def _compare_whole(wl, out, ref, tag):
    rtol, atol = TOL[wl.dtype]
    close(img64(out["y"], wl.layout), ref["y"], rtol, atol, f"{tag} y")
    close(out["mean"].cpu().double().numpy(), ref["mean"], *STAT_TOL, f"{tag} mean")
    close(out["rstd"].cpu().double().numpy(), ref["rstd"], *STAT_TOL, f"{tag} rstd")
    close(img64(out["dx"], wl.layout), ref["dx"], rtol, atol, f"{tag} dx")
    rel_l2(out["dgamma"].cpu().numpy(), ref["dgamma"], f"{tag} dgamma")
    rel_l2(out["dbeta"].cpu().numpy(), ref["dbeta"], f"{tag} dbeta")
    say(f"[full] {tag}: all outputs within tolerance")


# ---- the NHWC image: one oracle run, three launch configurations -------------
@pytest.fixture(scope="module")
def nhwc_image():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wl = inputs.NHWC_IMG
    say(f"[full] {wl.name}: generating on the device")
    data = inputs.make_inputs(wl, seed=0, device="cuda")
    ref = _oracle_whole(wl, data)
    yield wl, data, ref
    del data, ref
    _release()


def test_full_nhwc_image(nhwc_image):
    """The launch configuration bench.py times: the planner's stream path."""
    wl, data, ref = nhwc_image
    out = run_gpu(wl, data)
    assert out["fwd_plan"].path == gn.GN_PATH_STREAM and out["bwd_plan"].path == gn.GN_PATH_STREAM
    _compare_whole(wl, out, ref, f"{wl.name} stream")
    del out
    _release()


@pytest.mark.parametrize("cap", [0, 108], ids=lambda c: f"cap{c}")
def test_full_nhwc_image_one_pass_slab(nhwc_image, cap):
    """The one-pass cooperative forward and backward forced on the image: the
    grid holds at most `cap` workgroups (0: the occupancy limit of the
    device), far fewer than the tiles, so nearly every tile is an overflow
    tile that joins the reductions in phase 1 and is reloaded for y / dx."""
    wl, data, ref = nhwc_image
    say(f"[full] {wl.name}: slab path, cap {cap}")
    out = run_gpu(wl, data, force_path="slab", max_resident=cap)
    for kind in ("fwd_plan", "bwd_plan"):
        p = out[kind]
        assert p.path == gn.GN_PATH_SLAB
        assert p.tiles > p.grid, f"{kind}: {p.tiles} tiles, grid {p.grid}: no overflow tiles"
        if cap:
            assert p.grid <= cap
        say(f"[full] {wl.name} slab {kind}: grid {p.grid}, tiles {p.tiles}, team {p.team}, "
            f"resident cap {p.resident_cap}")
    _compare_whole(wl, out, ref, f"{wl.name} slab cap{cap}")
    del out
    _release()


# ---- rows ----------------------------------------------------------------------
@pytest.mark.timeout(900)
def test_full_rows_bf16_131072x4096():
    _need_gpu()
    wl = inputs.ROWS_BIG
    say(f"[full] {wl.name}: generating on the device")
    data = inputs.make_inputs(wl, seed=0, device="cuda")
    out = run_gpu(wl, data)
    assert out["fwd_plan"].path == gn.GN_PATH_ROWS and out["bwd_plan"].path == gn.GN_PATH_ROWS
    ref = _oracle_whole(wl, data)
    del data
    _compare_whole(wl, out, ref, wl.name)
    del out, ref
    _release()


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
    _release()


# ---- NCHW 112x64x512x512: every sample ----------------------------------------
def _nchw_every_sample(wl, expect_path):
    say(f"[full] {wl.name}: generating on the device")
    data = inputs.make_inputs(wl, seed=0, device="cuda")
    out = run_gpu(wl, data)
    assert out["fwd_plan"].path == expect_path and out["bwd_plan"].path == expect_path
    rtol, atol = TOL[wl.dtype]
    eps = float(np.float32(wl.eps))
    G = wl.G
    gam = data["gamma"].double().cpu().numpy()
    bet = data["beta"].double().cpu().numpy()
    mean = out["mean"].reshape(-1).double().cpu().numpy()
    rstd = out["rstd"].reshape(-1).double().cpu().numpy()
    dg_ref = np.zeros(wl.C, np.float64)
    db_ref = np.zeros(wl.C, np.float64)

    def host(t):   # one sample (C, H, W), logical order, float64
        return t.to("cpu").double().contiguous().numpy().reshape(-1)

    for n in range(wl.N):
        if n % 16 == 0:
            say(f"[full] {wl.name}: samples {n}..{min(n + 15, wl.N - 1)}")
        xs, dys = host(data["x"][n]), host(data["dy"][n])
        ry, rm, rr = oracle.forward(xs, gam, bet, 1, wl.C, wl.HW, G, eps)
        close(host(out["y"][n]), ry, rtol, atol, f"{wl.name} y sample {n}")
        close(mean[n * G:(n + 1) * G], rm, *STAT_TOL, f"{wl.name} mean sample {n}")
        close(rstd[n * G:(n + 1) * G], rr, *STAT_TOL, f"{wl.name} rstd sample {n}")
        rdx, rdg, rdb, _, _ = oracle.backward(dys, xs, gam, 1, wl.C, wl.HW, G, eps)
        close(host(out["dx"][n]), rdx, rtol, atol, f"{wl.name} dx sample {n}")
        dg_ref += rdg
        db_ref += rdb
    rel_l2(out["dgamma"].cpu().numpy(), dg_ref, f"{wl.name} dgamma (64 channels)")
    rel_l2(out["dbeta"].cpu().numpy(), db_ref, f"{wl.name} dbeta (64 channels)")
    say(f"[full] {wl.name}: every output of every sample within tolerance")
    del data, out
    _release()


@pytest.mark.timeout(900)
def test_full_nchw_every_sample():
    _need_gpu()
    _nchw_every_sample(inputs.NCHW_BIG, gn.GN_PATH_SLAB)


# The NCHW benchmark shape in bf16: the slab kernels' 16-bit tiles and their
# own loop order in the backward.
NCHW_BIG_BF16 = inputs.Workload("nchw_bf16_112x64x512x512_g8", 112, 64, 512, 512, 8, "bf16", "nchw")


@pytest.mark.timeout(900)
def test_full_nchw_bf16_every_sample():
    _need_gpu()
    _nchw_every_sample(NCHW_BIG_BF16, gn.GN_PATH_SLAB)


@pytest.mark.timeout(900)
def test_full_nchw_crop_every_sample():
    """The strided workload bench.py times: 510x510 centre crops of the
    112x64 images, read and written in place by the generic kernels."""
    _need_gpu()
    _nchw_every_sample(inputs.CROP_BIG, gn.GN_PATH_GENERIC)


def test_full_sizes_are_the_benchmark_workloads():
    assert (inputs.NHWC_IMG.N, inputs.NHWC_IMG.C, inputs.NHWC_IMG.HW) == (1, 128, 1024 * 2048)
    assert (inputs.ROWS_BIG.N, inputs.ROWS_BIG.C) == (131072, 4096)
    assert (inputs.NCHW_BIG.N, inputs.NCHW_BIG.C, inputs.NCHW_BIG.HW) == (112, 64, 512 * 512)
    assert (inputs.CROP_BIG.N, inputs.CROP_BIG.C, inputs.CROP_BIG.H, inputs.CROP_BIG.W, inputs.CROP_BIG.crop) == \
        (112, 64, 510, 510, 1)
    assert ALL == 7
