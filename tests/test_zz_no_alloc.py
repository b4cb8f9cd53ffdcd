"""gn_backward_scratch: the backward with the library's static device scratch
array in place of a caller workspace (for callers that cannot allocate).

Each case makes two calls in a row through the C ABI -- a larger input, then
a smaller one, so that the second call runs on scratch memory that still
holds the first call's counters, flags and partials -- and compares every
output with gn_backward's on the same inputs with a workspace of its own.
Both run the same kernels in the same fixed order, so the outputs must be
bitwise equal (stricter than the parity tolerances).
"""
import ctypes

import pytest
import torch

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import _lib, inputs
from gpu_harness import ALL, say

pytestmark = pytest.mark.gpu
W = inputs.Workload

# (first call, second call): the second is smaller
PAIRS = [
    (W("ns_nchw_f32_slab_a", 4, 16, 64, 70, 4, "f32", "nchw"), W("ns_nchw_f32_slab_b", 2, 16, 32, 40, 4, "f32", "nchw")),
    (W("ns_nchw_bf16_slab_a", 3, 64, 96, 96, 8, "bf16", "nchw"), W("ns_nchw_bf16_slab_b", 1, 8, 40, 52, 2, "bf16", "nchw")),
    (W("ns_nhwc_f16_slab_a", 2, 64, 37, 29, 8, "f16", "nhwc"), W("ns_nhwc_f16_slab_b", 1, 64, 9, 11, 8, "f16", "nhwc")),
    (W("ns_rows_f16_a", 4096, 1024, 1, 1, 1, "f16", "nchw"), W("ns_rows_f16_b", 1000, 768, 1, 1, 1, "f16", "nchw")),
    (W("ns_stream_f16_a", 1, 128, 256, 256, 16, "f16", "nhwc", affine="n01"),
     W("ns_stream_f16_b", 1, 128, 64, 130, 16, "f16", "nhwc", affine="n01")),
    (W("ns_generic_f32_a", 3, 12, 17, 19, 3, "f32", "nchw"), W("ns_generic_f32_b", 2, 6, 5, 7, 3, "f32", "nchw")),
    # a large slab call, then a small call on another path
    (W("ns_nchw_f32_big", 8, 64, 128, 128, 8, "f32", "nchw"), W("ns_rows_small", 64, 1024, 1, 1, 1, "f16", "nchw")),
]
FORCE = {"ns_stream_f16_a": "stream", "ns_stream_f16_b": "stream", "ns_generic_f32_a": "generic",
         "ns_generic_f32_b": "generic", "ns_nhwc_f16_slab_a": "slab", "ns_nhwc_f16_slab_b": "slab"}


def _scratch_call(L, wl, d, mean, rstd, force):
    dx = torch.full_like(d["x"], float("nan"))
    dg = torch.full((wl.C,), float("nan"), device=d["x"].device)
    db = torch.full((wl.C,), float("nan"), device=d["x"].device)
    o = _lib.Options()
    o.force_path = {None: 0, "generic": 1, "rows": 2, "slab": 3, "stream": 4}[force]
    info = _lib.PlanInfo()
    o.info = ctypes.pointer(info)
    N, C = wl.N, wl.C
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.gn_backward_scratch(P(d["dy"]), P(d["x"]), P(mean), P(rstd), P(d["gamma"]), P(dx), P(dg), P(db), ALL, N,
                               C, wl.HW, wl.G, {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype], gn.layout_of(d["x"]),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), ctypes.byref(o))
    assert st == 0, f"gn_backward_scratch: status {st}"
    return dx, dg, db, info


def _same_bits(a, b, what):
    assert a.dtype == b.dtype and a.shape == b.shape, what
    ia = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
    ib = b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
    assert torch.equal(ia, ib), f"{what}: outputs differ from gn_backward's"


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0].name}-then-{p[1].name}")
def test_scratch_backward_matches_workspace_backward(pair):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    L = _lib.lib()
    dev = torch.device("cuda", 0)
    for k, wl in enumerate(pair):
        force = FORCE.get(wl.name)
        say(f"[scratch] call {k + 1}: {wl.name} (force {force})")
        d = {n: t.to(dev) for n, t in inputs.make_inputs(wl, seed=11 + k).items()}
        _, mean, rstd = gn.forward(d["x"], d["gamma"], d["beta"], wl.G, wl.eps)
        mean, rstd = mean.reshape(-1), rstd.reshape(-1)
        ref_info = gn.PlanInfo()
        rdx, rdg, rdb = gn.backward(d["dy"], d["x"], mean, rstd, d["gamma"], wl.G, ALL, force_path=force,
                                    info=ref_info)
        dx, dg, db, info = _scratch_call(L, wl, d, mean, rstd, force)
        torch.cuda.synchronize()
        assert info.path == ref_info.path and info.grid == ref_info.grid
        _same_bits(dx, rdx, f"{wl.name} dx")
        _same_bits(dg, rdg, f"{wl.name} dgamma")
        _same_bits(db, rdb, f"{wl.name} dbeta")


def test_scratch_backward_rejects_sizes_beyond_the_array():
    """A call that would need more than GN_SCRATCH_BYTES returns
    GN_ERR_WORKSPACE before anything is enqueued (rows bf16, 262144 channels
    in 16 segments: 64 MiB of column partials)."""
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    L = _lib.lib()
    N, C, G = 65536, 262144, 16
    need = gn.backward_workspace_size(N, C, 1, G, _lib.GN_BF16, _lib.GN_NCHW, ALL)
    assert need > _lib.GN_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)   # never dereferenced: rejected on the host
    st = L.gn_backward_scratch(fake, fake, fake, fake, fake, fake, fake, fake, ALL, N, C, 1, G, _lib.GN_BF16,
                               _lib.GN_NCHW, None, None)
    assert st == _lib.GN_ERR_WORKSPACE
