"""The C-ABI calls captured into a HIP graph (as the benchmark runs them):
every replay, with eager work and synchronisations in between, must give
bitwise the eager results."""
import pytest
import torch

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs
from gpu_harness import ALL, say

pytestmark = pytest.mark.gpu
W = inputs.Workload


COOP = gn.Debug(flags=gn.GN_DEBUG_SLAB_COOP)


@pytest.mark.parametrize("wl,force,debug", [
    (W("graph_rows_f16", 512, 1024, 1, 1, 1, "f16", "nchw"), None, None),
    (W("graph_gen_bf16", 2, 16, 20, 21, 4, "bf16", "nhwc"), "generic", None),
    (inputs.TINY, None, None),                                                         # one workgroup per slab
    (W("graph_slab_nhwc_f16", 2, 64, 37, 29, 8, "f16", "nhwc"), "slab", None),
    (W("graph_slab_nchw_bf16", 2, 8, 64, 600, 2, "bf16", "nchw"), "slab", COOP),     # 12 polled tile words per slab
    (W("graph_split_nchw_bf16", 2, 8, 64, 600, 2, "bf16", "nchw"), None, None),      # the split form
    (W("graph_mid_nchw_f16", 2, 640, 64, 64, 32, "f16", "nchw"), None, None),        # 1024-thread slabs, streamed dx
    (W("graph_stream_nhwc_f16", 2, 64, 130, 131, 8, "f16", "nhwc"), "stream", None),
    (W("graph_one_tile_nhwc_f16", 4, 64, 8, 8, 8, "f16", "nhwc"), None, None),       # one workgroup per sample
    (W("graph_few_tiles_nhwc_f16", 2, 256, 32, 32, 32, "f16", "nhwc"), None, None),  # 8 tiles per sample
    (W("graph_rows_narrow_f16", 3000, 64, 1, 1, 1, "f16", "nchw"), None, None),
    (W("graph_crop_f32", 2, 16, 20, 21, 4, "f32", "nchw", crop=1), None, None),      # strided views, in place
    (W("graph_crop_planes_bf16", 2, 8, 24, 70, 2, "bf16", "nchw", crop=2), None, None),   # plane-sum backward
], ids=lambda v: getattr(v, "name", None) or ("coop" if isinstance(v, gn.Debug) else str(v)))
def test_graph_replays_match_eager(wl, force, debug):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    say(f"[graph] {wl.name}")
    dev = torch.device("cuda", 0)
    N, C, HW, G = wl.N, wl.C, wl.HW, wl.G
    code = {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype]
    if wl.crop:
        # views drawn on the device (a copy to the device would make them dense)
        d = inputs.make_inputs(wl, seed=4, device="cuda")
        y = torch.empty(d["x"].shape, dtype=d["x"].dtype, device=dev)
        dx = torch.empty_like(y)
        _, _, H_, W_, st = gn.strided_dims(d["x"], y, d["dy"], dx)
        fwb = gn.forward_strided_workspace_size(N, C, H_, W_, G, code, st[0], st[1], force)
        bwb = gn.backward_strided_workspace_size(N, C, H_, W_, G, code, st[2], st[0], st[3], ALL, force)
    else:
        d = {k: v.to(dev) for k, v in inputs.make_inputs(wl, seed=4).items()}
        lay = gn.layout_of(d["x"])
        y, dx = torch.empty_like(d["x"]), torch.empty_like(d["x"])
        fwb = gn.forward_workspace_size(N, C, HW, G, code, lay, force)
        bwb = gn.backward_workspace_size(N, C, HW, G, code, lay, ALL, force)
    fws = torch.empty(max(fwb, 1), dtype=torch.uint8, device=dev)
    bws = torch.empty(max(bwb, 1), dtype=torch.uint8, device=dev)
    out = dict(y=y, mean=torch.empty(N * G, device=dev), rstd=torch.empty(N * G, device=dev),
               dx=dx, dgamma=torch.empty(C, device=dev), dbeta=torch.empty(C, device=dev))

    def step(stream_handle):
        gn.forward_into(d["x"], d["gamma"], d["beta"], G, wl.eps, out["y"], out["mean"], out["rstd"], fws,
                        force_path=force, stream=stream_handle, debug=debug)
        gn.backward_into(d["dy"], d["x"], out["mean"], out["rstd"], d["gamma"], G, ALL, out["dx"], out["dgamma"],
                         out["dbeta"], bws, force_path=force, stream=stream_handle, debug=debug)

    step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step(torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        for v in out.values():      # eager work between replays: poison every output
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            a = inputs.memory_image(out[k], wl.layout) if out[k].dim() == 4 else out[k]
            b = inputs.memory_image(ref[k], wl.layout) if ref[k].dim() == 4 else ref[k]
            assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), (rep, k)
