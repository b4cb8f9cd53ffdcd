"""GPU parity of the slab path (cooperative capped grid, grid-stride overflow
tiles, one-pass backward) against the fp64 oracle.

The apex PR #2018 bug was overflow tiles missing from the first accumulation
loop: dgamma/dbeta went wrong while dx stayed within tolerance.  Every case
here runs with the natural residency cap and with small forced caps, so that
most tiles are overflow tiles -- accumulated in phase 1 and reloaded for the
outputs -- and checks dgamma/dbeta as well as y and dx.
"""
import pytest
import torch

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs
from gpu_harness import check_against_oracle, run_gpu, say

pytestmark = pytest.mark.gpu
W = inputs.Workload

CASES = [
    # NHWC: chunks of 16 bytes never straddle a group; ragged last tile
    W("slab_nhwc_f16_c64_g8", 2, 64, 37, 29, 8, "f16", "nhwc"),
    W("slab_nhwc_f32_c32_g4", 3, 32, 50, 41, 4, "f32", "nhwc"),
    W("slab_nhwc_bf16_c128_g16", 1, 128, 64, 130, 16, "bf16", "nhwc", affine="n01"),
    W("slab_nhwc_f16_c512_g32", 2, 512, 9, 23, 32, "f16", "nhwc"),
    W("slab_nhwc_f16_c8_g1", 2, 8, 31, 33, 1, "f16", "nhwc"),
    # NCHW: tiles never straddle a channel plane; several tiles per plane
    W("slab_nchw_f32_c16_g4", 2, 16, 64, 70, 4, "f32", "nchw"),
    W("slab_nchw_f16_c8_g2", 2, 8, 256, 300, 2, "f16", "nchw"),
    W("slab_nchw_bf16_c12_g3", 3, 12, 40, 52, 3, "bf16", "nchw"),
    # tiles sized to small channel planes (ten channels per group, 64x64)
    W("slab_nchw_f16_c320_g32", 2, 320, 64, 64, 32, "f16", "nchw"),
    # 2, 4 (ragged last tile), 16 (the 512x512 fp32 planes) and 64 tiles per
    # channel plane, 256 and 512 tiles per slab
    W("slab_nchw_bf16_tpc2", 2, 8, 128, 256, 2, "bf16", "nchw"),
    W("slab_nchw_f32_tpc4_ragged", 2, 8, 224, 256, 2, "f32", "nchw"),
    W("slab_nchw_f32_tpc16_d8", 1, 16, 512, 512, 2, "f32", "nchw"),
    W("slab_nchw_f16_tpc64_d4", 1, 4, 1024, 1024, 1, "f16", "nchw"),
    W("slab_nchw_f16_tpc64_d8", 1, 8, 1024, 1024, 1, "f16", "nchw"),
    inputs.TINY,
]


# cap0: the planner's form at the natural cap (one workgroup per slab, the
# split form or the cooperative kernels); coop0: the cooperative kernels at
# the natural cap (GN_DEBUG_SLAB_COOP); capK: the cooperative kernels capped
# at K workgroups
@pytest.mark.parametrize("cap", [0, "coop0", 1, 3, 8], ids=lambda c: c if isinstance(c, str) else f"cap{c}")
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_slab_parity(wl, cap):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    say(f"[slab] {wl.name} cap={cap}")
    data = inputs.make_inputs(wl, seed=2)
    coop = cap == "coop0"
    cap = 0 if coop else cap
    out = run_gpu(wl, data, force_path="slab", max_resident=cap,
                  debug=gn.Debug(flags=gn.GN_DEBUG_SLAB_COOP) if coop else None)
    fp, bp = out["fwd_plan"], out["bwd_plan"]
    assert fp.path == gn.GN_PATH_SLAB and bp.path == gn.GN_PATH_SLAB
    if cap:
        assert fp.grid <= cap and bp.grid <= cap
        assert bp.resident_cap == cap
    if coop:
        assert fp.resident_cap > 0 and bp.resident_cap > 0   # the cooperative kernels ran
    check_against_oracle(wl, data, out)


# NCHW slabs of more than 1024 tiles (forced: the planner keeps the slab path
# for slabs of at most 1024): the forward's merge beyond the partials a thread
# keeps in registers, and the backward's per-channel sums over more than one
# LDS-staged chunk of tile partials; ragged last tile of every plane.
MANY_TILES = [
    W("slab_nchw_f32_d8_many_tiles", 1, 8, 150, 16384 + 40, 1, "f32", "nchw"),
    W("slab_nchw_bf16_d4_many_tiles", 1, 8, 300, 16384 + 24, 2, "bf16", "nchw"),
]


@pytest.mark.parametrize("cap", [0, 8], ids=lambda c: f"cap{c}")
@pytest.mark.parametrize("wl", MANY_TILES, ids=lambda w: w.name)
def test_slab_many_tiles(wl, cap):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    say(f"[slab] {wl.name} cap={cap}")
    data = inputs.make_inputs(wl, seed=4)
    out = run_gpu(wl, data, force_path="slab", max_resident=cap)
    fp, bp = out["fwd_plan"], out["bwd_plan"]
    assert fp.path == gn.GN_PATH_SLAB and bp.path == gn.GN_PATH_SLAB
    slabs = wl.N * wl.G
    assert fp.tiles // slabs > 1024 and bp.tiles // slabs > 1024
    check_against_oracle(wl, data, out)


# Small NCHW slabs (at most 64 KiB per tensor): one workgroup each holds the
# whole slab in registers (1 to 16 chunks per thread) and exchanges nothing;
# taken when no residency cap is forced.
SMALL_SLABS = [
    W("small_nchw_f32_r16_64kib", 2, 16, 64, 64, 4, "f32", "nchw"),      # exactly 64 KiB, 16 chunks a thread
    W("small_nchw_f16_ragged_d3", 3, 12, 24, 24, 4, "f16", "nchw"),      # 216 of 256 threads hold a chunk
    W("small_nchw_bf16_d256", 2, 256, 2, 4, 1, "bf16", "nchw"),          # one chunk per channel, one lane each
    W("small_nchw_f32_instance", 4, 8, 32, 32, 8, "f32", "nchw"),        # G = C
    W("small_nchw_f32_many_n", 64, 32, 8, 8, 8, "f32", "nchw", affine="n01"),
    W("small_nchw_f16_r2_d10", 2, 320, 16, 16, 32, "f16", "nchw"),       # ten 256-element planes, 2 chunks a thread
]


@pytest.mark.parametrize("wl", SMALL_SLABS, ids=lambda w: w.name)
def test_small_slab_parity(wl):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    say(f"[slab] {wl.name} small")
    data = inputs.make_inputs(wl, seed=9)
    out = run_gpu(wl, data, force_path="slab")
    fp, bp = out["fwd_plan"], out["bwd_plan"]
    assert fp.path == gn.GN_PATH_SLAB and bp.path == gn.GN_PATH_SLAB
    assert fp.team == 1 and fp.kernels == 1 and fp.grid == wl.N * wl.G
    check_against_oracle(wl, data, out)


@pytest.mark.parametrize("mask", [gn.GN_GRAD_DX, gn.GN_GRAD_DGAMMA, gn.GN_GRAD_DBETA,
                                  gn.GN_GRAD_DGAMMA | gn.GN_GRAD_DBETA], ids=["dx", "dgamma", "dbeta", "params"])
def test_small_slab_masks(mask):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wl = SMALL_SLABS[1]
    data = inputs.make_inputs(wl, seed=10)
    out = run_gpu(wl, data, force_path="slab", mask=mask)
    check_against_oracle(wl, data, out, mask=mask)


# Mid-size NCHW slabs (past 64 KiB, up to 256 KiB per tensor): one workgroup
# of 1024 threads each.  The forward holds 8 or 16 chunks per thread; the
# backward holds all of x and dy up to 128 KiB, and past that keeps four chunk
# rounds in registers and streams the others twice (mid_nchw_bwd).  Each case
# says whether the forward and the backward take one workgroup per slab
# (larger slabs take the split form or the cooperative kernels).
MID_SLABS = [
    (W("mid_nchw_f16_80kib", 2, 320, 64, 64, 32, "f16", "nchw"), True, True),
    (W("mid_nchw_f32_128kib", 2, 16, 64, 64, 2, "f32", "nchw"), True, True),        # all of x and dy held
    (W("mid_nchw_f16_ragged", 3, 20, 72, 80, 2, "f16", "nchw"), True, True),        # 7200 of 8192 chunk slots
    (W("mid_nchw_f16_d256", 2, 256, 16, 16, 1, "f16", "nchw"), True, True),         # four lanes per channel sum
    (W("mid_nchw_f32_175kib", 2, 30, 64, 70, 3, "f32", "nchw", affine="n01"), True, True),   # 11 rounds, 7 streamed
    (W("mid_nchw_bf16_256kib", 2, 64, 64, 64, 2, "bf16", "nchw"), True, True),      # 16 rounds: both limits
    (W("mid_nchw_f16_160kib", 2, 640, 64, 64, 32, "f16", "nchw"), True, True),      # 10 rounds: a short last batch
    (W("mid_nchw_f32_ragged_164kib", 3, 20, 60, 70, 2, "f32", "nchw"), True, True),  # 260 chunks in the last round
    (W("mid_nchw_bf16_d256_256kib", 2, 256, 16, 32, 1, "bf16", "nchw"), True, True),
    (W("mid_nchw_f32_258kib", 2, 16, 110, 150, 4, "f32", "nchw"), False, False),    # past both limits
]


@pytest.mark.parametrize("case", MID_SLABS, ids=lambda c: c[0].name)
def test_mid_slab_parity(case):
    wl, fwd_one, bwd_one = case
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    say(f"[slab] {wl.name} mid")
    data = inputs.make_inputs(wl, seed=11)
    out = run_gpu(wl, data, force_path="slab")
    fp, bp = out["fwd_plan"], out["bwd_plan"]
    assert fp.path == gn.GN_PATH_SLAB and bp.path == gn.GN_PATH_SLAB
    slabs = wl.N * wl.G
    if fwd_one:
        assert fp.team == 1 and fp.kernels == 1 and fp.grid == slabs
    else:   # the split form or the cooperative kernels
        assert fp.team != 1
    if bwd_one:
        assert bp.team == 1 and bp.grid == slabs
    else:
        assert bp.team != 1
    check_against_oracle(wl, data, out)


@pytest.mark.parametrize("case", [2, 6], ids=["held", "streamed"])
@pytest.mark.parametrize("mask", [gn.GN_GRAD_DX, gn.GN_GRAD_DGAMMA, gn.GN_GRAD_DBETA,
                                  gn.GN_GRAD_DGAMMA | gn.GN_GRAD_DBETA], ids=["dx", "dgamma", "dbeta", "params"])
def test_mid_slab_masks(mask, case):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wl = MID_SLABS[case][0]
    data = inputs.make_inputs(wl, seed=12)
    out = run_gpu(wl, data, force_path="slab", mask=mask)
    check_against_oracle(wl, data, out, mask=mask)


# NCHW tensors of at most 32 MiB (forward) or 64 MiB (backward) whose slabs
# are past 256 KiB: the split form (a statistics-tile launch, then output
# kernels that combine the slab's tile partials; two launches each way, plus
# params_over_n for dgamma/dbeta), up to 256 tiles per slab.  Each case says
# whether the forward and the backward take it.
SPLIT = [
    (W("split_nchw_f32_2x32x128x128_g4", 2, 32, 128, 128, 4, "f32", "nchw"), True, True),     # 16 tiles a slab
    (W("split_nchw_f16_1x128x256x256_g32", 1, 128, 256, 256, 32, "f16", "nchw"), True, True),  # 512 KiB slabs
    (W("split_nchw_bf16_ragged", 3, 12, 200, 200, 3, "bf16", "nchw", affine="n01"), True, True),  # short last tile
    (W("split_nchw_f16_d256", 1, 256, 32, 24, 1, "f16", "nchw"), True, True),                  # 256 one-chunk tiles
    (W("split_nchw_f32_instance", 2, 4, 400, 200, 4, "f32", "nchw"), True, True),              # G = C
    (W("split_nchw_f32_40mib", 1, 128, 256, 320, 16, "f32", "nchw"), False, True),             # backward only
    (W("split_nchw_f16_512_tiles", 1, 32, 512, 512, 1, "f16", "nchw"), False, False),          # too many tiles
]


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: c[0].name)
def test_split_parity(case):
    wl, fwd_split, bwd_split = case
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    say(f"[slab] {wl.name} split={fwd_split},{bwd_split}")
    data = inputs.make_inputs(wl, seed=15)
    out = run_gpu(wl, data, force_path="slab")
    fp, bp = out["fwd_plan"], out["bwd_plan"]
    assert fp.path == gn.GN_PATH_SLAB and bp.path == gn.GN_PATH_SLAB
    if fwd_split:
        assert fp.kernels == 2 and fp.team == 0 and fp.resident_cap == 0
    else:
        assert fp.team > 0
    if bwd_split:
        assert bp.kernels == 3 and bp.team == 0   # with dgamma/dbeta: params_over_n
    else:
        assert bp.team > 0
    check_against_oracle(wl, data, out)


@pytest.mark.parametrize("mask", [gn.GN_GRAD_DX, gn.GN_GRAD_DGAMMA, gn.GN_GRAD_DBETA,
                                  gn.GN_GRAD_DGAMMA | gn.GN_GRAD_DBETA], ids=["dx", "dgamma", "dbeta", "params"])
def test_split_masks(mask):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wl = SPLIT[2][0]
    data = inputs.make_inputs(wl, seed=16)
    out = run_gpu(wl, data, force_path="slab", mask=mask)
    check_against_oracle(wl, data, out, mask=mask)


def test_overflow_tiles_exist_under_a_cap():
    """With the cap below the tile count, members own several tiles."""
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wl = W("slab_overflow_nhwc", 1, 128, 64, 130, 16, "f16", "nhwc", affine="n01")
    data = inputs.make_inputs(wl, seed=6)
    out = run_gpu(wl, data, force_path="slab", max_resident=8)
    bp = out["bwd_plan"]
    assert bp.tiles > bp.grid          # overflow tiles: more tiles than workgroups
    assert bp.team == 8
    check_against_oracle(wl, data, out)


def test_auto_selects_slab_for_nchw():
    # NHWC streams (test_abi covers the planner); the cases above force the slab path
    assert gn.select_path(True, 1, 128, 64 * 130, 16, 1, gn._lib.GN_NHWC) == gn.GN_PATH_STREAM
    assert gn.select_path(False, 112, 64, 512 * 512, 8, 0, gn._lib.GN_NCHW) == gn.GN_PATH_SLAB
    assert gn.select_path(False, 2, 32, 256, 8, 0, gn._lib.GN_NCHW) == gn.GN_PATH_SLAB


@pytest.mark.parametrize("wl,debug", [
    (W("reuse_nchw_f32", 3, 16, 64, 70, 4, "f32", "nchw"), None),                           # one workgroup a slab
    (W("reuse_nchw_f32_coop", 3, 16, 64, 70, 4, "f32", "nchw"), gn.GN_DEBUG_SLAB_COOP),     # polled tile words
    (W("reuse_split_bf16", 3, 12, 200, 200, 3, "bf16", "nchw"), None),                      # the split form
    (W("reuse_nhwc_f16", 2, 64, 37, 29, 8, "f16", "nhwc"), None),
    (W("reuse_rows_bf16", 300, 2048, 1, 1, 2, "bf16", "nchw"), None),
], ids=lambda v: getattr(v, "name", None) or ("coop" if v else "auto"))
def test_same_workspace_new_inputs(wl, debug):
    """Back-to-back calls through the same buffers and workspace with different
    inputs: no call may see values (partial sums, counters) of the previous
    one -- identical inputs would hide that, so each call draws new ones."""
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    dev = torch.device("cuda", 0)
    first = inputs.make_inputs(wl, seed=10)
    bufs = {k: v.to(dev) for k, v in first.items()}
    N, C, HW, G = wl.N, wl.C, wl.HW, wl.G
    code = {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype]
    lay = gn.layout_of(bufs["x"])
    fws = torch.empty(gn.forward_workspace_size(N, C, HW, G, code, lay) + 1, dtype=torch.uint8, device=dev)
    bws = torch.empty(gn.backward_workspace_size(N, C, HW, G, code, lay, 7) + 1, dtype=torch.uint8, device=dev)
    out = dict(y=torch.empty_like(bufs["x"]), mean=torch.empty(N * G, device=dev), rstd=torch.empty(N * G, device=dev),
               dx=torch.empty_like(bufs["x"]), dgamma=torch.empty(C, device=dev), dbeta=torch.empty(C, device=dev))
    for seed in (11, 12, 13):
        data = inputs.make_inputs(wl, seed=seed)
        for k in bufs:
            bufs[k].copy_(data[k])
        say(f"[reuse] {wl.name} seed={seed}")
        dbg = gn.Debug(flags=debug) if debug else None
        fp, bp = gn.PlanInfo(), gn.PlanInfo()
        gn.forward_into(bufs["x"], bufs["gamma"], bufs["beta"], G, wl.eps, out["y"], out["mean"], out["rstd"], fws,
                        info=fp, debug=dbg)
        gn.backward_into(bufs["dy"], bufs["x"], out["mean"], out["rstd"], bufs["gamma"], G, 7, out["dx"],
                         out["dgamma"], out["dbeta"], bws, info=bp, debug=dbg)
        torch.cuda.synchronize()
        if wl.name.startswith("reuse_nchw"):
            # the one-workgroup kernels, or the cooperative ones with their tile words
            want = (lambda t: t > 1) if debug else (lambda t: t == 1)
            assert fp.path == bp.path == gn.GN_PATH_SLAB and want(fp.team) and want(bp.team), (fp.team, bp.team)
        elif wl.name.startswith("reuse_split"):
            assert fp.path == bp.path == gn.GN_PATH_SLAB and fp.team == bp.team == 0
        check_against_oracle(wl, data, out)
