"""GPU parity of the stream path (NHWC as a few launches of one tile per
workgroup, or one workgroup per sample when a sample fits one tile) against
the fp64 oracle.

Cases cover every activation dtype, one and several samples (dgamma/dbeta
written by the per-group kernel or summed over the samples), a tile count
past one column-sum chunk (the two-level channel reduction), groups of
several 16-byte chunks (the merge tree across chunks), ragged last tiles and
every output mask.  Cases whose samples fit one tile, or a few tiles, run in
both forms: the fused kernels the planner picks (one workgroup per sample;
output kernels that combine the tile partials themselves), and the full
multi-kernel form forced with GN_DEBUG_STREAM_SPLIT.
"""
import pytest
import torch

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs
from gpu_harness import ALL, check_against_oracle, run_gpu, say

pytestmark = pytest.mark.gpu
W = inputs.Workload

CASES = [
    W("stream_nhwc_f16_c64_g8", 2, 64, 37, 29, 8, "f16", "nhwc"),
    W("stream_nhwc_f32_c32_g4", 3, 32, 50, 41, 4, "f32", "nhwc"),
    W("stream_nhwc_bf16_c128_g16", 1, 128, 64, 130, 16, "bf16", "nhwc", affine="n01"),
    W("stream_nhwc_f16_c512_g32", 2, 512, 9, 23, 32, "f16", "nhwc"),
    W("stream_nhwc_f16_c8_g1", 2, 8, 31, 33, 1, "f16", "nhwc"),
    # 4 chunks per group (two merge levels across chunks); one pixel per
    # iteration (256 chunks per pixel: no merge over pixel rows)
    W("stream_nhwc_f16_c64_g2", 2, 64, 33, 35, 2, "f16", "nhwc"),
    W("stream_nhwc_f16_c2048_g8", 1, 2048, 5, 9, 8, "f16", "nhwc"),
    # more than 64 backward tiles per sample: two column-sum levels
    W("stream_nhwc_f16_c64_twolevel", 2, 64, 130, 131, 8, "f16", "nhwc"),
    W("stream_nhwc_f32_c16_twolevel", 1, 16, 200, 181, 2, "f32", "nhwc"),
    # channel counts the slab kernels do not take: chunks per pixel not
    # dividing the workgroup (idle threads), groups not whole 16-byte chunks
    # (a chunk spans two or more groups), one channel per group
    W("stream_nhwc_f16_c320_g32", 2, 320, 37, 41, 32, "f16", "nhwc"),
    W("stream_nhwc_f16_c640_g32", 1, 640, 30, 33, 32, "f16", "nhwc"),
    W("stream_nhwc_bf16_c1280_g32", 2, 1280, 9, 13, 32, "bf16", "nhwc"),
    W("stream_nhwc_f32_c96_g24", 2, 96, 20, 21, 24, "f32", "nhwc"),
    W("stream_nhwc_f16_c24_g3", 3, 24, 40, 41, 3, "f16", "nhwc"),
    W("stream_nhwc_f32_c12_g12", 2, 12, 30, 31, 12, "f32", "nhwc"),
    W("stream_nhwc_f16_c2048_g1", 1, 2048, 6, 7, 1, "f16", "nhwc"),
]


# the full multi-kernel form of the stream path also where the fused forms apply
SPLIT = gn.Debug(flags=gn.GN_DEBUG_STREAM_SPLIT)
FORMS = {"auto": None, "split": SPLIT}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def _servable(wl):
    p = gn.select_path(False, wl.N, wl.C, wl.HW, wl.G, {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype],
                       gn._lib.GN_NHWC, "stream")
    return p == gn.GN_PATH_STREAM


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_stream_parity(wl, form):
    _need_gpu()
    if not _servable(wl):
        pytest.skip("shape outside the stream path (chunks per pixel must divide the workgroup)")
    if form == "split" and _tiles(wl) > 16:
        pytest.skip("samples of many tiles: both forms are the multi-kernel one")
    say(f"[stream] {wl.name} {form}")
    data = inputs.make_inputs(wl, seed=3)
    out = run_gpu(wl, data, force_path="stream", debug=FORMS[form])
    assert out["fwd_plan"].path == gn.GN_PATH_STREAM and out["bwd_plan"].path == gn.GN_PATH_STREAM
    if form == "split":
        assert out["fwd_plan"].kernels >= 3
    check_against_oracle(wl, data, out)


def _tiles(wl):
    """Statistics tiles (16 chunks per thread) per sample of wl."""
    v = 4 if wl.dtype == "f32" else 8
    tp = (256 // (wl.C // v)) * 16
    return -(-wl.HW // tp)


def _one_tile(wl):
    return _tiles(wl) == 1


# Samples that fit one tile (at most 16 chunks per thread): one workgroup per
# sample takes the whole call
ONE_TILE = [
    W("one_tile_nhwc_f32_2x32x16x16_g8", 2, 32, 16, 16, 8, "f32", "nhwc"),          # 16 chunks a thread
    W("one_tile_nhwc_f16_4x64x8x8_g8", 4, 64, 8, 8, 8, "f16", "nhwc"),              # 4 chunks a thread
    W("one_tile_nhwc_f16_c2048_g32", 1, 2048, 2, 3, 32, "f16", "nhwc"),             # 256 chunks a pixel
    W("one_tile_nhwc_f16_c320_g32", 2, 320, 9, 10, 32, "f16", "nhwc"),              # idle threads; D = 10
    W("one_tile_nhwc_f16_c96_g24", 2, 96, 8, 8, 24, "f16", "nhwc"),                 # a chunk spans two groups
    W("one_tile_nhwc_f32_n1_g1", 1, 64, 16, 16, 1, "f32", "nhwc", affine="n01"),    # dgamma/dbeta written directly
    W("one_tile_nhwc_bf16_many_n", 64, 128, 4, 4, 32, "bf16", "nhwc"),
    W("one_tile_nhwc_f32_c12_g12", 2, 12, 30, 31, 12, "f32", "nhwc"),               # one channel per group
]


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("wl", ONE_TILE, ids=lambda w: w.name)
def test_one_tile_parity(wl, form):
    _need_gpu()
    assert _one_tile(wl)
    say(f"[stream] {wl.name} {form}")
    data = inputs.make_inputs(wl, seed=13)
    out = run_gpu(wl, data, force_path="stream", debug=FORMS[form])
    fp, bp = out["fwd_plan"], out["bwd_plan"]
    assert fp.path == gn.GN_PATH_STREAM and bp.path == gn.GN_PATH_STREAM
    if form == "auto":
        assert fp.kernels == 1 and fp.grid == wl.N
        assert bp.kernels == (1 if wl.N == 1 else 2) and bp.grid == wl.N
    else:
        assert fp.kernels >= 3
    check_against_oracle(wl, data, out)


# Samples of 2 to 16 tiles: the output kernels combine the tile partials
# themselves (two launches forward; two backward, three with several samples).
FEW_TILES = [
    W("few_nhwc_f16_2x256x32x32_g32", 2, 256, 32, 32, 32, "f16", "nhwc"),           # 8 tiles
    W("few_nhwc_f32_3x32x50x41_g4", 3, 32, 50, 41, 4, "f32", "nhwc"),               # 5, ragged
    W("few_nhwc_f16_1x64x40x41_g8", 1, 64, 40, 41, 8, "f16", "nhwc", affine="n01"), # one sample
    W("few_nhwc_f16_2x320x37x41_g32", 2, 320, 37, 41, 32, "f16", "nhwc"),           # 16 tiles; D = 10
    W("few_nhwc_f32_2x96x20x21_g24", 2, 96, 20, 21, 24, "f32", "nhwc"),
    W("few_nhwc_bf16_3x24x40x41_g3", 3, 24, 40, 41, 3, "bf16", "nhwc"),
    W("many_nhwc_f16_1x64x1x8193_g8", 1, 64, 1, 8193, 8, "f16", "nhwc"),            # 17 tiles: the full form
]


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("wl", FEW_TILES, ids=lambda w: w.name)
def test_few_tiles_parity(wl, form):
    _need_gpu()
    t = _tiles(wl)
    assert 1 < t <= 17
    say(f"[stream] {wl.name} {form} tiles={t}")
    data = inputs.make_inputs(wl, seed=14)
    out = run_gpu(wl, data, force_path="stream", debug=FORMS[form])
    fp, bp = out["fwd_plan"], out["bwd_plan"]
    assert fp.path == gn.GN_PATH_STREAM and bp.path == gn.GN_PATH_STREAM
    if form == "auto" and t <= 16:
        assert fp.kernels == 2
        assert bp.kernels == (2 if wl.N == 1 else 3)
    else:
        assert fp.kernels == 3 and bp.kernels >= 4
    check_against_oracle(wl, data, out)


MASKS = [gn.GN_GRAD_DX, gn.GN_GRAD_DGAMMA, gn.GN_GRAD_DBETA, gn.GN_GRAD_DGAMMA | gn.GN_GRAD_DBETA,
         gn.GN_GRAD_DX | gn.GN_GRAD_DBETA, ALL]


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("wl", [W("stream_mask_n1", 1, 64, 40, 41, 8, "f16", "nhwc"),
                                W("stream_mask_n3", 3, 32, 30, 31, 4, "bf16", "nhwc"),        # one tile a sample
                                W("stream_mask_one_tile_n1", 1, 64, 8, 8, 8, "f16", "nhwc")],
                         ids=lambda w: w.name)
def test_stream_output_mask(wl, mask, form):
    _need_gpu()
    say(f"[stream-mask] {wl.name} mask={mask} {form}")
    data = inputs.make_inputs(wl, seed=5)
    out = run_gpu(wl, data, force_path="stream", mask=mask, debug=FORMS[form])
    assert out["bwd_plan"].path == gn.GN_PATH_STREAM
    check_against_oracle(wl, data, out, mask=mask)
    if not mask & gn.GN_GRAD_DGAMMA:
        assert out["dgamma"] is None
    if not mask & gn.GN_GRAD_DBETA:
        assert out["dbeta"] is None


def test_stream_bitwise_deterministic():
    _need_gpu()
    wl = W("stream_det", 2, 64, 130, 131, 8, "bf16", "nhwc")
    data = inputs.make_inputs(wl, seed=7)
    a = run_gpu(wl, data, force_path="stream")
    b = run_gpu(wl, data, force_path="stream")
    for k in ("y", "mean", "rstd", "dx", "dgamma", "dbeta"):
        ta, tb = a[k], b[k]
        if ta.dim() == 4:
            ta, tb = inputs.memory_image(ta, wl.layout), inputs.memory_image(tb, wl.layout)
        assert torch.equal(ta.contiguous().view(torch.uint8), tb.contiguous().view(torch.uint8)), k
