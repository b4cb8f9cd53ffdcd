"""A cooperative launch the runtime refuses: while one process on the device
has made cooperative launches and still runs, another process's
hipLaunchCooperativeKernel fails (hipErrorIllegalState).  That process's slab
calls must then take the kernels that need no co-residency -- the split form
where it can tile the slabs, else the generic kernels -- and still match the
oracle.  This process makes a cooperative launch first; a child process makes
the calls (the only way to get a second process on the device), eagerly and
recorded into a graph."""
import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs

from gpu_harness import run_gpu, say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs
from gpu_harness import run_gpu, check_against_oracle
W = inputs.Workload
CASES = [   # (workload, forced path); the cooperative kernels at the natural cap
    (W("refused_nchw_f32_split", 2, 16, 64, 80, 4, "f32", "nchw"), None),        # 80 KiB slabs: split form
    (W("refused_nchw_f16_generic", 1, 64, 256, 512, 1, "f16", "nchw"), None),    # 512 tiles a slab: generic
    (W("refused_nhwc_f16_generic", 2, 64, 37, 29, 8, "f16", "nhwc"), "slab"),    # NHWC slab: generic
]
import torch
dbg = gn.Debug(flags=gn.GN_DEBUG_SLAB_COOP)
for wl, force in CASES:
    print("[refused] " + wl.name, flush=True)
    data = inputs.make_inputs(wl, seed=31)
    out = run_gpu(wl, data, force_path=force, debug=dbg)
    fp, bp = out["fwd_plan"], out["bwd_plan"]
    check_against_oracle(wl, data, out)
    # the same calls recorded into a graph: a refused cooperative launch would be
    # recorded and then skipped silently at every replay
    d = {k: v.cuda() for k, v in data.items()}
    code = {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype]
    lay = gn.layout_of(d["x"])
    y, dx = torch.empty_like(d["x"]), torch.empty_like(d["x"])
    m, r = torch.empty(wl.N * wl.G, device="cuda"), torch.empty(wl.N * wl.G, device="cuda")
    dg, db = torch.empty(wl.C, device="cuda"), torch.empty(wl.C, device="cuda")
    fws = torch.empty(gn.forward_workspace_size(wl.N, wl.C, wl.HW, wl.G, code, lay, force), dtype=torch.uint8,
                      device="cuda")
    bws = torch.empty(gn.backward_workspace_size(wl.N, wl.C, wl.HW, wl.G, code, lay, 7, force), dtype=torch.uint8,
                      device="cuda")
    gfp, gbp = gn.PlanInfo(), gn.PlanInfo()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        gn.forward_into(d["x"], d["gamma"], d["beta"], wl.G, wl.eps, y, m, r, fws, force_path=force, info=gfp,
                        debug=dbg)
        gn.backward_into(d["dy"], d["x"], m, r, d["gamma"], wl.G, 7, dx, dg, db, bws, force_path=force, info=gbp,
                         debug=dbg)
    for i in range(3):
        for t in (y, dx, m, r, dg, db):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in ((y, out["y"], "y"), (m, out["mean"].reshape(-1), "mean"),
                                (r, out["rstd"].reshape(-1), "rstd"), (dx, out["dx"], "dx"),
                                (dg, out["dgamma"], "dgamma"), (db, out["dbeta"], "dbeta")):
            assert torch.equal(got, want), (wl.name, "replay", i, name)
    print(json.dumps({"case": wl.name, "fwd": [fp.path, fp.team], "bwd": [bp.path, bp.team],
                      "graph": [gfp.path, gfp.team, gbp.path, gbp.team]}), flush=True)
"""

EXPECT = {   # path and team of the kernels that ran instead
    "refused_nchw_f32_split": [gn.GN_PATH_SLAB, 0],
    "refused_nchw_f16_generic": [gn.GN_PATH_GENERIC, None],
    "refused_nhwc_f16_generic": [gn.GN_PATH_GENERIC, None],
}


def test_refused_cooperative_launch_takes_other_kernels():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    # this process's own cooperative launch, so that the child's are refused
    wl = inputs.Workload("refused_holder_f32", 2, 16, 64, 80, 4, "f32", "nchw")
    out = run_gpu(wl, inputs.make_inputs(wl, seed=30), debug=gn.Debug(flags=gn.GN_DEBUG_SLAB_COOP))
    assert out["fwd_plan"].team > 1 and out["bwd_plan"].team > 1
    say("[refused] child process")
    env = dict(os.environ)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-u", "-c", CHILD, HERE], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=110)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    got = {d["case"]: d for d in (json.loads(l) for l in r.stdout.splitlines() if l.startswith("{"))}
    assert set(got) == set(EXPECT), out[-4000:]
    for case, (path, team) in EXPECT.items():
        for kind in ("fwd", "bwd"):
            p, t = got[case][kind]
            assert p == path and (team is None or t == team), f"{case} {kind}: path {p}, team {t}"
        fp, ft, bp, bt = got[case]["graph"]   # recorded: the same kernels as the eager calls
        assert [fp, bp] == [path, path] and (team is None or ft == bt == team), f"{case} graph: {got[case]['graph']}"


CHILD_MAX = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs
from gpu_harness import TOL, run_gpu, say
from test_gpu_maxsize import _check_params_with_oracle, _check_slice
wl = inputs.Workload("refused_max_nchw_f32", 129, 64, 512, 512, 8, "f32", "nchw")
say(f"[refused] {wl.name}: {wl.E} elements, generating on the device")
data = inputs.make_inputs(wl, seed=1, device="cuda")
out = run_gpu(wl, data)
fp, bp = out["fwd_plan"], out["bwd_plan"]
say(f"[refused] plans: forward path {fp.path} team {fp.team}, backward path {bp.path} team {bp.team}")
assert fp.path == bp.path == gn.GN_PATH_SLAB and fp.team == bp.team == 0, "the split form did not run"
rtol, atol = TOL[wl.dtype]
eps = float(np.float32(wl.eps))
for n, g in [(0, 0), (127, 7), (128, 0), (128, 7)]:
    say(f"[refused] slice ({n}, {g})")
    _check_slice(wl, data, out, n, g, eps, rtol, atol, wl.name)
_check_params_with_oracle(wl, data, out, wl.name)
say("[refused] within tolerance")
"""


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_refused_cooperative_launch_past_2to31_elements():
    """The split form as the fallback at the full 129 x 64 x 512 x 512 fp32
    size (more than 2^31 elements per tensor, offsets past 2^31): sampled
    slices and every channel's dgamma/dbeta against the oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wl = inputs.Workload("refused_holder_f32", 2, 16, 64, 80, 4, "f32", "nchw")
    out = run_gpu(wl, inputs.make_inputs(wl, seed=30), debug=gn.Debug(flags=gn.GN_DEBUG_SLAB_COOP))
    assert out["fwd_plan"].team > 1
    say("[refused] child process, 129 x 64 x 512 x 512 fp32")
    env = dict(os.environ)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    proc = subprocess.Popen([sys.executable, "-u", "-c", CHILD_MAX, HERE], cwd=ROOT, env=env,
                            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = []
    for line in proc.stdout:   # the child's progress, as it comes
        print(line, end="", flush=True)
        lines.append(line)
    rc = proc.wait(timeout=60)
    assert rc == 0, "".join(lines)[-4000:]
    assert any("within tolerance" in l for l in lines), "".join(lines)[-4000:]


CHILD_STATE = r"""
import json
import torch
import normalization_gn_stats_amd as gn
x = torch.randn(64, 1024, device="cuda", dtype=torch.float16)
gn.forward(x.view(64, 1024, 1, 1), torch.ones(1024, device="cuda"), torch.zeros(1024, device="cuda"), 1, 1e-5)
torch.cuda.synchronize()
print(json.dumps({"state": gn.cooperative_state()}), flush=True)
"""


def test_cooperative_state_and_early_launch_opt_out():
    """gn_cooperative_state in this process (accepted after its cooperative
    calls) and in child processes that make one rows call: refused by
    default (this process holds the runtime's cooperative state), not tried
    with GN_EARLY_COOP=0 (the early launch left out)."""
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wl = inputs.Workload("refused_holder_f32", 2, 16, 64, 80, 4, "f32", "nchw")
    out = run_gpu(wl, inputs.make_inputs(wl, seed=30), debug=gn.Debug(flags=gn.GN_DEBUG_SLAB_COOP))
    assert out["fwd_plan"].team > 1
    assert gn.cooperative_state() == gn.COOP_ACCEPTED
    for early, want in (("1", gn.COOP_REFUSED), ("0", gn.COOP_NOT_TRIED)):
        env = dict(os.environ)
        env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
        env["GN_EARLY_COOP"] = early
        say(f"[refused] child with GN_EARLY_COOP={early}")
        r = subprocess.run([sys.executable, "-u", "-c", CHILD_STATE], cwd=ROOT, env=env, capture_output=True,
                           text=True, timeout=110)
        assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
        got = [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
        assert got and got[-1]["state"] == want, (early, got, r.stderr[-2000:])
