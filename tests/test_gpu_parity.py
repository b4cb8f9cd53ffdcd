"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle,
element by element, on seeded inputs at sizes the oracle finishes in seconds.

Cases span several tiles/workgroups and ragged tails, both layouts, all three
activation dtypes, every output mask, and the degenerate shapes (one element
per slice, one sample, one channel per group, G = C, no affine parameters).
Each test also asserts which path ran.
"""
import pytest
import torch

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs
from gpu_harness import ALL, check_against_oracle, run_gpu, say

pytestmark = pytest.mark.gpu

W = inputs.Workload


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


# (workload, forced path or None, expected path)
SMALL = [
    # generic path: odd sizes, both layouts, every dtype
    (W("gen_nchw_f32", 3, 12, 7, 9, 4, "f32", "nchw"), "generic", gn.GN_PATH_GENERIC),
    (W("gen_nhwc_f32", 3, 12, 7, 9, 4, "f32", "nhwc"), "generic", gn.GN_PATH_GENERIC),
    (W("gen_nchw_f16", 2, 24, 33, 17, 6, "f16", "nchw"), "generic", gn.GN_PATH_GENERIC),
    (W("gen_nhwc_bf16", 2, 24, 33, 17, 6, "bf16", "nhwc"), "generic", gn.GN_PATH_GENERIC),
    (W("gen_multichunk_f32", 2, 8, 130, 129, 2, "f32", "nchw"), "generic", gn.GN_PATH_GENERIC),
    (W("gen_multichunk_nhwc_f16", 1, 32, 100, 101, 4, "f16", "nhwc", affine="n01"), "generic", gn.GN_PATH_GENERIC),
    # rows path (HW == 1)
    (W("rows_f16_64x1024", 64, 1024, 1, 1, 1, "f16", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_f16_100x768", 100, 768, 1, 1, 1, "f16", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_bf16_37x4096", 37, 4096, 1, 1, 1, "bf16", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_f32_50x2048", 50, 2048, 1, 1, 1, "f32", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_f32_33x40", 33, 40, 1, 1, 1, "f32", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_g4_f16_300x512", 300, 512, 1, 1, 4, "f16", "nhwc"), None, gn.GN_PATH_ROWS),
    (W("rows_g8_bf16_2100x256", 2100, 256, 1, 1, 8, "bf16", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_f16_odd_c_20x36", 20, 36, 1, 1, 1, "f16", "nchw"), None, gn.GN_PATH_GENERIC),
    # enough slices per group that the forward's waves walk several slices each
    (W("rows_walk_f16_20000x512", 20000, 512, 1, 1, 1, "f16", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_walk_f32_9001x2048", 9001, 2048, 1, 1, 1, "f32", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_walk_bf16_g4_6000x4096", 6000, 4096, 1, 1, 4, "bf16", "nhwc"), None, gn.GN_PATH_ROWS),
    # wide slices (more vectors than one wave takes): four waves per slice
    (W("rows_wide_bf16_300x8192", 300, 8192, 1, 1, 1, "bf16", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_wide_f16_129x16384", 129, 16384, 1, 1, 1, "f16", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_wide_f32_201x3072", 201, 3072, 1, 1, 1, "f32", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_wide_f32_g2_50x16384", 50, 16384, 1, 1, 2, "f32", "nhwc"), None, gn.GN_PATH_ROWS),
    # four waves per slice with at most two vectors per lane (two slices per
    # wave per block in the backward), several groups, odd slice counts
    (W("rows_cs4_bf16_g2_77x8192", 77, 8192, 1, 1, 2, "bf16", "nhwc"), None, gn.GN_PATH_ROWS),
    (W("rows_cs4_f32_g2_65x4096", 65, 4096, 1, 1, 2, "f32", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_cs4_f16_g2_31x6144", 31, 6144, 1, 1, 2, "f16", "nchw"), None, gn.GN_PATH_ROWS),
    # several blocks per backward workgroup, two or three of them (an odd count ends the walk mid-pair)
    (W("rows_cs4_bf16_2999x4096", 2999, 4096, 1, 1, 1, "bf16", "nchw"), None, gn.GN_PATH_ROWS),
    # narrow slices (at most 32 vectors): several slices per wavefront, from
    # 64 slices per wave (one vector each) to 2 (32 vectors each), with idle
    # lanes (6 vectors on 8 lanes) and ragged last row sets
    (W("rows_narrow_f16_131072x64", 131072, 64, 1, 1, 1, "f16", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_narrow_f32_5003x4", 5003, 4, 1, 1, 1, "f32", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_narrow_bf16_g2_777x96", 777, 96, 1, 1, 2, "bf16", "nhwc"), None, gn.GN_PATH_ROWS),
    (W("rows_narrow_f32_1001x128", 1001, 128, 1, 1, 1, "f32", "nchw"), None, gn.GN_PATH_ROWS),
    (W("rows_narrow_f16_g4_3000x256", 3000, 256, 1, 1, 4, "f16", "nchw"), None, gn.GN_PATH_ROWS),
    # degenerate shapes
    (W("deg_m1_f32", 5, 6, 1, 1, 6, "f32", "nchw"), None, None),         # one element per slice
    (W("deg_instance_f16", 2, 8, 5, 5, 8, "f16", "nchw"), None, None),   # G = C
    (W("deg_n1_nhwc_f32", 1, 16, 3, 3, 16, "f32", "nhwc"), None, None),
    (W("deg_one_group_f32", 2, 3, 11, 13, 1, "f32", "nchw"), None, None),
    # the small benchmark configuration
    (inputs.TINY, None, None),
]


@pytest.mark.parametrize("wl,force,expect", SMALL, ids=[c[0].name for c in SMALL])
def test_parity_small(wl, force, expect):
    _need_gpu()
    say(f"[parity] {wl.name} force={force}")
    data = inputs.make_inputs(wl, seed=0)
    out = run_gpu(wl, data, force_path=force)
    if expect is not None:
        assert out["fwd_plan"].path == expect and out["bwd_plan"].path == expect
    check_against_oracle(wl, data, out)


MASKS = [gn.GN_GRAD_DX, gn.GN_GRAD_DGAMMA, gn.GN_GRAD_DBETA, gn.GN_GRAD_DGAMMA | gn.GN_GRAD_DBETA,
         gn.GN_GRAD_DX | gn.GN_GRAD_DBETA, ALL]


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("wl", [W("mask_rows_f16", 96, 1024, 1, 1, 1, "f16", "nchw"),
                                W("mask_rows_narrow_bf16", 900, 64, 1, 1, 2, "bf16", "nchw"),
                                W("mask_gen_f32", 2, 12, 9, 10, 3, "f32", "nhwc")], ids=lambda w: w.name)
def test_output_mask(wl, mask):
    _need_gpu()
    say(f"[mask] {wl.name} mask={mask}")
    data = inputs.make_inputs(wl, seed=3)
    out = run_gpu(wl, data, mask=mask)
    check_against_oracle(wl, data, out, mask=mask)
    if not mask & gn.GN_GRAD_DGAMMA:
        assert out["dgamma"] is None
    if not mask & gn.GN_GRAD_DBETA:
        assert out["dbeta"] is None


def test_no_affine():
    """gamma = beta = NULL: gamma is 1 and beta 0; only dx can be asked for."""
    _need_gpu()
    wl = W("noaff", 3, 16, 6, 7, 4, "f32", "nchw")
    data = inputs.make_inputs(wl, seed=5)
    dev = torch.device("cuda", 0)
    x, dy = data["x"].to(dev), data["dy"].to(dev)
    y, mean, rstd = gn.forward(x, None, None, wl.G, wl.eps)
    dx, _, _ = gn.backward(dy, x, mean, rstd, None, wl.G, gn.GN_GRAD_DX)
    ones = torch.ones(wl.C)
    zeros = torch.zeros(wl.C)
    out = dict(y=y, mean=mean, rstd=rstd, dx=dx, dgamma=None, dbeta=None)
    check_against_oracle(wl, dict(data, gamma=ones, beta=zeros), out, mask=gn.GN_GRAD_DX)
    with pytest.raises(gn.GNError):
        gn.backward(dy, x, mean, rstd, None, wl.G, ALL)


def test_unaligned_pointers_take_the_generic_path():
    """A view starting 2 bytes into its storage cannot use 16-byte loads."""
    _need_gpu()
    wl = W("unaligned_rows_f16", 16, 256, 1, 1, 1, "f16", "nchw")
    data = inputs.make_inputs(wl, seed=9)
    dev = torch.device("cuda", 0)
    big = torch.empty(wl.E + 1, dtype=torch.float16, device=dev)
    x = big[1:].view(wl.N, wl.C, 1, 1)
    x.copy_(data["x"].to(dev))
    dbig = torch.empty(wl.E + 1, dtype=torch.float16, device=dev)
    dy = dbig[1:].view(wl.N, wl.C, 1, 1)
    dy.copy_(data["dy"].to(dev))
    gamma, beta = data["gamma"].to(dev), data["beta"].to(dev)
    fi, bi = gn.PlanInfo(), gn.PlanInfo()
    y, mean, rstd = gn.forward(x, gamma, beta, wl.G, wl.eps, info=fi)
    dx, dg, db = gn.backward(dy, x, mean, rstd, gamma, wl.G, ALL, info=bi)
    torch.cuda.synchronize()
    assert fi.path == gn.GN_PATH_GENERIC and bi.path == gn.GN_PATH_GENERIC
    check_against_oracle(wl, data, dict(y=y, mean=mean, rstd=rstd, dx=dx, dgamma=dg, dbeta=db))


def test_zero_extent_noop():
    _need_gpu()
    x = torch.empty(0, 8, 4, 4, device="cuda")
    g = torch.ones(8, device="cuda")
    y, mean, rstd = gn.forward(x, g, torch.zeros(8, device="cuda"), 2)
    assert y.numel() == 0 and mean.numel() == 0


@pytest.mark.parametrize("wl,force", [(inputs.ROWS_A, None), (inputs.TINY, None),
                                      (W("det_gen", 2, 16, 40, 41, 4, "bf16", "nhwc"), "generic")],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_bitwise_deterministic(wl, force):
    """Two runs give bitwise equal outputs (fixed-order reductions, no float atomics)."""
    _need_gpu()
    data = inputs.make_inputs(wl, seed=1)
    a = run_gpu(wl, data, force_path=force)
    b = run_gpu(wl, data, force_path=force)
    def bits(t):
        flat = inputs.memory_image(t, wl.layout) if t.dim() == 4 else t.reshape(-1)
        return flat.contiguous().view(torch.uint8)

    for k in ("y", "mean", "rstd", "dx", "dgamma", "dbeta"):
        assert torch.equal(bits(a[k]), bits(b[k])), k


@pytest.mark.parametrize("wl", [inputs.ROWS_A, inputs.ROWS_B], ids=lambda w: w.name)
def test_parity_row_benchmark_shapes(wl):
    """The LayerNorm-shaped workloads at their full size, every output."""
    _need_gpu()
    say(f"[parity-full] {wl.name}")
    data = inputs.make_inputs(wl, seed=0)
    out = run_gpu(wl, data)
    assert out["fwd_plan"].path == gn.GN_PATH_ROWS and out["bwd_plan"].path == gn.GN_PATH_ROWS
    check_against_oracle(wl, data, out)
