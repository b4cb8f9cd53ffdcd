"""The library's one empty cooperative launch per device (gn_api.cpp): it is
skipped while the call's stream captures a graph, so a process whose very
first library call is made under capture still captures and replays
correctly, and the next eager calls, cooperative ones included, run and
match.  Runs in a child process, the only way to make the library's first
call there; when the test runner itself has made cooperative launches, the
child's are refused and take the split form (tests/test_gpu_coop_refused.py)."""
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import torch
import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs

def ref(x, G, g, b, eps):
    return torch.nn.functional.group_norm(x.float(), G, g, b, eps)

torch.manual_seed(0)
x = torch.randn(2, 32, 16, 16, device="cuda"); gam = torch.randn(32, device="cuda"); bet = torch.randn(32, device="cuda")
y = torch.empty_like(x); m = torch.empty(16, device="cuda"); r = torch.empty(16, device="cuda")
ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
torch.cuda.synchronize()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
    gn.forward_into(x, gam, bet, 8, 1e-5, y, m, r, ws)   # the process's first library call
for i in range(3):
    y.zero_()
    graph.replay()
    torch.cuda.synchronize()
    err = (y - ref(x, 8, gam, bet, 1e-5)).abs().max().item()
    assert err < 1e-5, ("replay", i, err)
print("[first_coop] capture ok", flush=True)
# eager calls afterwards: the cooperative slab kernels (forced) and the planner's choice
wl = inputs.Workload("first_coop_nchw_f16", 2, 64, 64, 80, 8, "f16", "nchw")   # 80 KiB slabs
d = {k: v.cuda() for k, v in inputs.make_inputs(wl, seed=5).items()}
for flags in (gn.GN_DEBUG_SLAB_COOP, 0):
    st = gn.status_word()
    info = gn.PlanInfo()
    yy, mu, rs = gn.forward(d["x"], d["gamma"], d["beta"], wl.G, wl.eps, force_path="slab", info=info, status=st,
                            debug=gn.Debug(flags=flags))
    assert gn.read_status(st) == gn.GN_OK
    err = (yy.float() - ref(d["x"], wl.G, d["gamma"], d["beta"], wl.eps)).abs().max().item()
    assert err < 1e-2, ("eager", flags, err)
    # with the flag the cooperative kernels, unless another process on the device holds the
    # runtime's cooperative state (the test runner, after its own cooperative calls): then the split form
    if flags:
        assert info.team > 1 or info.team == 0, info.team
    else:
        assert info.team == 1, info.team
print("[first_coop] eager ok", flush=True)
"""


def test_first_library_call_under_capture():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    env = dict(os.environ)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-u", "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=110)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "[first_coop] capture ok" in r.stdout and "[first_coop] eager ok" in r.stdout, out[-3000:]
