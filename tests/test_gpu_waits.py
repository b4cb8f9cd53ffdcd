"""Failure report of the cooperative (slab) kernels.

Their workgroups exchange partial results inside one launch, which is only
safe while every workgroup of the grid is resident (apex PR #2018, Solution:
the cooperative grid is capped at the residency limit).  Every wait for
another workgroup is bounded.  These tests force every wait to give up from
the host -- gn_options.debug_flags = GN_DEBUG_UNMET_WAITS puts each wait's
target out of reach, and a spin limit of 64 polls ends it quickly -- so every
kernel still runs to its end.  They check that the call's status word then
reads GN_ERR_WAIT, that every output the incomplete exchange would have fed
is NaN (no finite wrong value escapes: the apex bug's failure was wrong but
finite dgamma/dbeta), and that the next call on the same workspace is
correct again.  Paths without such waits ignore the flag.
"""
import numpy as np
import pytest
import torch

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs
from gpu_harness import ALL, check_against_oracle, say

pytestmark = pytest.mark.gpu
W = inputs.Workload
FAIL = gn.Debug(spin_limit=64, flags=gn.GN_DEBUG_UNMET_WAITS)
# the slab path's cooperative kernels also where the one-workgroup or split forms would run
FAIL_COOP = gn.Debug(spin_limit=64, flags=gn.GN_DEBUG_UNMET_WAITS | gn.GN_DEBUG_SLAB_COOP)
COOP = gn.Debug(flags=gn.GN_DEBUG_SLAB_COOP)

SLAB_CASES = [
    W("wait_nchw_f32_c16_g4", 2, 16, 110, 150, 4, "f32", "nchw"),
    W("wait_nchw_bf16_c12_g3", 3, 12, 208, 160, 3, "bf16", "nchw"),
    W("wait_nhwc_f16_c64_g8", 2, 64, 37, 29, 8, "f16", "nhwc"),
    W("wait_nhwc_f32_c32_g4", 1, 32, 50, 41, 4, "f32", "nhwc"),
]


def _all_nan(t, what):
    a = t.detach().float().cpu().numpy()
    assert np.isnan(a).all(), f"{what}: {int((~np.isnan(a)).sum())} of {a.size} values are not NaN"


def _calls(wl, data, ws_f, ws_b, cap, debug, status):
    """One forward and one backward through the *_into calls on the given
    workspaces; returns the outputs.  The backward uses the saved statistics
    of a forward without failures (`data['mean']`, `data['rstd']`)."""
    dev = data["x"].device
    y = torch.empty_like(data["x"])
    mean = torch.empty(wl.N * wl.G, device=dev)
    rstd = torch.empty(wl.N * wl.G, device=dev)
    fi, bi = gn.PlanInfo(), gn.PlanInfo()
    gn.forward_into(data["x"], data["gamma"], data["beta"], wl.G, wl.eps, y, mean, rstd, ws_f, force_path="slab",
                    max_resident=cap, info=fi, status=status, debug=debug)
    fst = gn.read_status(status)
    dx = torch.empty_like(data["x"])
    dg = torch.empty(wl.C, device=dev)
    db = torch.empty(wl.C, device=dev)
    gn.backward_into(data["dy"], data["x"], data["mean"], data["rstd"], data["gamma"], wl.G, ALL, dx, dg, db, ws_b,
                     force_path="slab", max_resident=cap, info=bi, status=status, debug=debug)
    bst = gn.read_status(status)
    assert fi.path == gn.GN_PATH_SLAB and bi.path == gn.GN_PATH_SLAB
    return dict(y=y, mean=mean, rstd=rstd, dx=dx, dgamma=dg, dbeta=db, fwd_status=fst, bwd_status=bst,
                fwd_plan=fi, bwd_plan=bi)


@pytest.mark.parametrize("cap", [0, 3], ids=lambda c: f"cap{c}")
@pytest.mark.parametrize("wl", SLAB_CASES, ids=lambda w: w.name)
def test_expired_waits_are_reported_and_poison_outputs(wl, cap):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    say(f"[waits] {wl.name} cap={cap}")
    dev = torch.device("cuda", 0)
    data = {k: v.to(dev) for k, v in inputs.make_inputs(wl, seed=5).items()}
    _, m, r = gn.forward(data["x"], data["gamma"], data["beta"], wl.G, wl.eps, force_path="slab")
    data["mean"], data["rstd"] = m.reshape(-1), r.reshape(-1)
    code = {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype]
    lay = gn.layout_of(data["x"])
    ws_f = torch.empty(max(gn.forward_workspace_size(wl.N, wl.C, wl.HW, wl.G, code, lay, "slab"), 1),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(gn.backward_workspace_size(wl.N, wl.C, wl.HW, wl.G, code, lay, ALL, "slab"), 1),
                       dtype=torch.uint8, device=dev)
    status = gn.status_word(dev)

    bad = _calls(wl, data, ws_f, ws_b, cap, FAIL_COOP, status)
    assert bad["fwd_status"] == gn.GN_ERR_WAIT
    assert bad["bwd_status"] == gn.GN_ERR_WAIT
    for k in ("y", "mean", "rstd", "dx", "dgamma", "dbeta"):
        _all_nan(bad[k], f"{wl.name} {k} after expired waits")

    # the same workspaces, no forced failure: correct again, status clean
    good = _calls(wl, data, ws_f, ws_b, cap, COOP, status)
    assert good["fwd_status"] == gn.GN_OK and good["bwd_status"] == gn.GN_OK
    check_against_oracle(wl, {k: data[k].cpu() for k in ("x", "dy", "gamma", "beta")}, good)


def test_status_word_is_sticky_until_reset():
    """Reports accumulate over calls until read with reset."""
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wl = SLAB_CASES[0]
    dev = torch.device("cuda", 0)
    data = {k: v.to(dev) for k, v in inputs.make_inputs(wl, seed=6).items()}
    status = gn.status_word(dev)
    gn.forward(data["x"], data["gamma"], data["beta"], wl.G, wl.eps, force_path="slab", status=status,
               debug=FAIL_COOP)
    gn.forward(data["x"], data["gamma"], data["beta"], wl.G, wl.eps, force_path="slab", status=status, debug=COOP)
    assert gn.read_status(status, reset=False) == gn.GN_ERR_WAIT
    assert gn.read_status(status, reset=True) == gn.GN_ERR_WAIT
    assert gn.read_status(status) == gn.GN_OK


@pytest.mark.parametrize("wl,path", [
    (W("wait_rows_f16", 64, 1024, 1, 1, 1, "f16", "nchw"), "rows"),
    (W("wait_stream_f16", 1, 128, 64, 130, 16, "f16", "nhwc", affine="n01"), "stream"),
    (W("wait_generic_f32", 2, 12, 7, 9, 3, "f32", "nchw"), "generic"),
    (W("wait_small_slab_bf16", 3, 12, 40, 52, 3, "bf16", "nchw"), "slab"),   # one workgroup per slab: no waits
    (W("wait_mid_slab_f32", 2, 16, 64, 70, 4, "f32", "nchw"), "slab"),      # 70 KiB: 1024 threads per slab
], ids=lambda v: v if isinstance(v, str) else v.name)
def test_paths_without_waits_ignore_the_flag(wl, path):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    dev = torch.device("cuda", 0)
    data = inputs.make_inputs(wl, seed=7)
    d = {k: v.to(dev) for k, v in data.items()}
    status = gn.status_word(dev)
    fi, bi = gn.PlanInfo(), gn.PlanInfo()
    y, m, r = gn.forward(d["x"], d["gamma"], d["beta"], wl.G, wl.eps, force_path=path, info=fi, status=status,
                         debug=FAIL)
    dx, dg, db = gn.backward(d["dy"], d["x"], m, r, d["gamma"], wl.G, ALL, force_path=path, info=bi, status=status,
                             debug=FAIL)
    assert gn.read_status(status) == gn.GN_OK
    assert gn.PATH_NAMES[fi.path] == path and gn.PATH_NAMES[bi.path] == path
    check_against_oracle(wl, data, dict(y=y, mean=m, rstd=r, dx=dx, dgamma=dg, dbeta=db))
