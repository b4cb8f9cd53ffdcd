"""GPU parity of RMSNorm over rows (gn_rms_forward / gn_rms_backward through
the C ABI) against the fp64 oracle.

RMSNorm runs on the rows kernels with the mean taken as 0: the cases cover
each of their shapes -- one wave per slice, several waves per slice (wide
slices, forward and backward), the slice-walking forward, several narrow
slices per wave -- every dtype, groups
of channels (G > 1), no weight, every output mask, and the RMSNorm shapes of
the ROCm/pytorch PR #3564 table at 4096 x 1024 fp16 and 131072 x 64 fp16 (the
131072 x 4096 bf16 one is in the full-size tests).
"""
import pytest
import torch

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs
from gpu_harness import RMS_ALL, check_rms_against_oracle, run_rms_gpu, say

pytestmark = pytest.mark.gpu
W = inputs.Workload

CASES = [
    W("rms_tile256_f16_4096x1024", 4096, 1024, 1, 1, 1, "f16", "nchw", eps=1e-6),
    W("rms_two_pass_f16_131072x64", 131072, 64, 1, 1, 1, "f16", "nchw", eps=1e-6),
    W("rms_bf16_37x4096", 37, 4096, 1, 1, 1, "bf16", "nchw"),
    W("rms_f32_50x2048", 50, 2048, 1, 1, 1, "f32", "nchw"),
    W("rms_f16_100x768", 100, 768, 1, 1, 1, "f16", "nchw"),
    W("rms_walk_f16_20000x512", 20000, 512, 1, 1, 1, "f16", "nchw"),
    W("rms_walk_f32_9001x2048", 9001, 2048, 1, 1, 1, "f32", "nchw"),
    W("rms_narrow_f32_5003x4", 5003, 4, 1, 1, 1, "f32", "nchw"),
    W("rms_narrow_bf16_g2_777x96", 777, 96, 1, 1, 2, "bf16", "nchw"),
    W("rms_g4_f16_300x512", 300, 512, 1, 1, 4, "f16", "nchw"),
    W("rms_g8_bf16_2100x256", 2100, 256, 1, 1, 8, "bf16", "nchw"),
    W("rms_wide_bf16_301x8192", 301, 8192, 1, 1, 1, "bf16", "nchw"),
    W("rms_wide_f32_77x6144", 77, 6144, 1, 1, 1, "f32", "nchw"),
]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_rms_parity(wl):
    _need_gpu()
    say(f"[rms] {wl.name}")
    data = inputs.make_inputs(wl, seed=8)
    out = run_rms_gpu(wl, data)
    assert out["fwd_plan"].path == gn.GN_PATH_ROWS and out["bwd_plan"].path == gn.GN_PATH_ROWS
    check_rms_against_oracle(wl, data, out)


@pytest.mark.parametrize("mask", [gn.GN_GRAD_DX, gn.GN_GRAD_DGAMMA, RMS_ALL])
@pytest.mark.parametrize("wl", [W("rms_mask_f16_96x1024", 96, 1024, 1, 1, 1, "f16", "nchw"),
                                W("rms_mask_narrow_bf16", 900, 64, 1, 1, 2, "bf16", "nchw")], ids=lambda w: w.name)
def test_rms_output_mask(wl, mask):
    _need_gpu()
    say(f"[rms-mask] {wl.name} mask={mask}")
    data = inputs.make_inputs(wl, seed=9)
    out = run_rms_gpu(wl, data, mask=mask)
    check_rms_against_oracle(wl, data, out, mask=mask)


@pytest.mark.parametrize("wl", [W("rms_noweight_f32_64x256", 64, 256, 1, 1, 1, "f32", "nchw"),
                                W("rms_noweight_f16_5000x64", 5000, 64, 1, 1, 1, "f16", "nchw")],
                         ids=lambda w: w.name)
def test_rms_without_weight(wl):
    _need_gpu()
    data = inputs.make_inputs(wl, seed=10)
    out = run_rms_gpu(wl, data, mask=gn.GN_GRAD_DX, affine=False)
    check_rms_against_oracle(wl, data, out, mask=gn.GN_GRAD_DX, affine=False)


def test_rms_bitwise_deterministic():
    _need_gpu()
    wl = W("rms_det_bf16_3000x1024", 3000, 1024, 1, 1, 1, "bf16", "nchw")
    data = inputs.make_inputs(wl, seed=11)
    a = run_rms_gpu(wl, data)
    b = run_rms_gpu(wl, data)
    for k in ("y", "rstd", "dx", "dgamma"):
        assert torch.equal(a[k].contiguous().view(torch.uint8), b[k].contiguous().view(torch.uint8)), k
