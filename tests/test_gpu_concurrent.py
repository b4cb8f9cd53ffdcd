"""Calls while other work runs on the same device: two cooperative slab calls
issued on two streams at once, one beside ordinary kernels on another
stream, and calls of every path from several host threads at once.  Each
team's workgroups wait for one another, so every wait must still end (a
small spin limit makes a failed wait show in the status word quickly), and
every output must equal, bit for bit, the same call made alone (the
reductions run in a fixed order)."""
import pytest

torch = pytest.importorskip("torch")

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs

from gpu_harness import say

pytestmark = pytest.mark.gpu

W = inputs.Workload
# 2 MiB slabs of 128 MiB tensors: cooperative teams of many workgroups, forward and backward
WL = W("concurrent_nchw_f16_2x512x256x256", 2, 512, 256, 256, 32, "f16", "nchw")
DBG_SPIN = 1 << 16   # polls before a wait gives up (legitimate waits here end within microseconds)


def _alone(d):
    y, m, r = gn.forward(d["x"], d["gamma"], d["beta"], WL.G, WL.eps)
    dx, dg, db = gn.backward(d["dy"], d["x"], m, r, d["gamma"], WL.G)
    torch.cuda.synchronize()
    return y, m, r, dx, dg, db


def _on(stream, d, st):
    dbg = gn.Debug(spin_limit=DBG_SPIN)
    with torch.cuda.stream(stream):
        fi, bi = gn.PlanInfo(), gn.PlanInfo()
        y, m, r = gn.forward(d["x"], d["gamma"], d["beta"], WL.G, WL.eps, status=st, debug=dbg, info=fi)
        dx, dg, db = gn.backward(d["dy"], d["x"], m, r, d["gamma"], WL.G, status=st, debug=dbg, info=bi)
    return (y, m, r, dx, dg, db), (fi, bi)


def _same(a, b, what):
    for u, v, name in zip(a, b, ("y", "mean", "rstd", "dx", "dgamma", "dbeta")):
        assert torch.equal(u, v), f"{what}: {name} differs from the lone call"


@pytest.mark.parametrize("beside", ["cooperative", "ordinary"])
def test_cooperative_calls_beside_other_streams(beside):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    say(f"[concurrent] {WL.name} beside {beside}")
    d1 = {k: v.cuda() for k, v in inputs.make_inputs(WL, seed=21).items()}
    d2 = {k: v.cuda() for k, v in inputs.make_inputs(WL, seed=22).items()}
    want1, want2 = _alone(d1), _alone(d2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    st1, st2 = gn.status_word(), gn.status_word()
    big = torch.ones(1 << 28, device="cuda")   # 1 GiB for the ordinary kernels
    torch.cuda.synchronize()
    for it in range(8):
        got1, infos = _on(s1, d1, st1)
        for info in infos:   # the cooperative kernels, forward and backward
            assert info.path == gn.GN_PATH_SLAB and info.team > 1, (info.path, info.team)
        if beside == "cooperative":
            got2, _ = _on(s2, d2, st2)
        else:
            with torch.cuda.stream(s2):
                big.mul_(1.0001).add_(1.0)
        torch.cuda.synchronize()
        assert gn.read_status(st1) == gn.GN_OK, f"iteration {it}: a wait gave up on stream 1"
        _same(got1, want1, f"iteration {it}, stream 1")
        if beside == "cooperative":
            assert gn.read_status(st2) == gn.GN_OK, f"iteration {it}: a wait gave up on stream 2"
            _same(got2, want2, f"iteration {it}, stream 2")


THREAD_SHAPES = [   # one per path: cooperative slab, one-workgroup slab, stream, rows, generic (crop)
    W("threads_nchw_f16_slab", 2, 512, 256, 256, 32, "f16", "nchw"),
    W("threads_nchw_f32_small", 4, 64, 32, 32, 8, "f32", "nchw"),
    W("threads_nhwc_f16_stream", 4, 128, 64, 64, 16, "f16", "nhwc"),
    W("threads_rows_bf16", 2048, 1024, 1, 1, 1, "bf16", "nchw"),
    W("threads_crop_f32", 2, 16, 40, 40, 4, "f32", "nchw", crop=1),
]


def test_calls_from_several_host_threads():
    """Every shape above from its own host thread and stream at once, several
    rounds: the library's host side (device facts, the early cooperative
    launch, planning) runs concurrently, since ctypes releases the
    interpreter lock; every output must equal the same call made alone."""
    import threading
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    data = [inputs.make_inputs(wl, seed=40 + i, device="cuda") for i, wl in enumerate(THREAD_SHAPES)]   # crop: views

    def call(wl, d):
        y, m, r = gn.forward(d["x"], d["gamma"], d["beta"], wl.G, wl.eps)
        dx, dg, db = gn.backward(d["dy"], d["x"], m, r, d["gamma"], wl.G)
        return y, m, r, dx, dg, db

    want = [call(wl, d) for wl, d in zip(THREAD_SHAPES, data)]
    torch.cuda.synchronize()
    for rnd in range(4):
        say(f"[threads] round {rnd}")
        got, errors = [None] * len(THREAD_SHAPES), []
        barrier = threading.Barrier(len(THREAD_SHAPES))

        def worker(i):
            try:
                s = torch.cuda.Stream()
                barrier.wait()
                with torch.cuda.stream(s):
                    got[i] = call(THREAD_SHAPES[i], data[i])
                s.synchronize()
            except Exception as e:   # reported below, in the test's own thread
                errors.append((THREAD_SHAPES[i].name, repr(e)))

        ts = [threading.Thread(target=worker, args=(i,)) for i in range(len(THREAD_SHAPES))]
        for t in ts:
            t.start()
        for t in ts:
            t.join(timeout=60)
        assert not errors, errors
        for wl, a, b in zip(THREAD_SHAPES, got, want):
            _same(a, b, f"round {rnd}, {wl.name}")
