"""GPU parity on seeded random shapes, each through the path the planner picks.

N, C, G, H, W, dtype, layout, affine parameters and output mask are drawn
from a fixed seed, with sizes chosen around the planner's boundaries: NHWC
samples of one tile or several (the stream path's one-workgroup form and its
multi-kernel form), NCHW slabs below 64 KiB, between 64 and 256 KiB and past
256 KiB (the one-workgroup kernels and the cooperative ones), spatial sizes
that are and are not whole 16-byte chunks (slab or generic), and rows (HW =
1).  Every output the mask selects is compared element by element with the
fp64 oracle at the tolerances of the other parity tests.
"""
import os
import random

import pytest
import torch

import normalization_gn_stats_amd as gn
from normalization_gn_stats_amd import inputs
from gpu_harness import ALL, check_against_oracle, run_gpu, say

pytestmark = pytest.mark.gpu
W = inputs.Workload

MASKS = [ALL, gn.GN_GRAD_DX, gn.GN_GRAD_DGAMMA | gn.GN_GRAD_DBETA, gn.GN_GRAD_DX | gn.GN_GRAD_DBETA]
# bytes per slab (NCHW) or per sample (NHWC) of each size class
TARGET = {"tiny": 3 << 10, "small": 40 << 10, "mid": 96 << 10, "mid2": 200 << 10, "large": 400 << 10}


def _cases(n=96, seed=20261202):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        dtype = rng.choice(["f32", "f16", "bf16"])
        esz = 4 if dtype == "f32" else 2
        affine = rng.choice(["default", "n01"])
        mask = rng.choice(MASKS)
        if rng.random() < 0.15:   # rows
            N, C = rng.randint(1, 300), rng.choice([40, 64, 200, 768, 1024, 2048, 4096])
            G = rng.choice([g for g in (1, 2, 4, 8) if C % g == 0])
            wl = W(f"rand{len(out)}_rows_{dtype}_{N}x{C}_g{G}", N, C, 1, 1, G, dtype, "nchw", affine=affine)
            out.append((wl, mask))
            continue
        layout = rng.choice(["nchw", "nhwc"])
        G = rng.choice([1, 2, 3, 4, 8, 16, 32])
        D = rng.choice([1, 2, 3, 4, 5, 8, 10, 16, 20, 40])
        C = G * D
        if C > 1024:
            continue
        kind = rng.choice(list(TARGET))
        per = D if layout == "nchw" else C   # channels in one slab / sample
        hw = max(1, TARGET[kind] // (per * esz))
        Wd = max(1, int((hw * rng.uniform(0.5, 2.0)) ** 0.5))
        if rng.random() < 0.7:
            Wd = max(8, Wd // 8 * 8)         # whole 16-byte chunks per plane
        H = max(1, hw // Wd)
        N = rng.choice([1, 2, 3, 5])
        if N * C * H * Wd > (3 << 20) or H * Wd == 1:
            continue
        wl = W(f"rand{len(out)}_{layout}_{dtype}_{N}x{C}x{H}x{Wd}_g{G}_{kind}", N, C, H, Wd, G, dtype, layout,
               affine=affine)
        out.append((wl, mask))
    return out


# GN_RANDOM_CASES / GN_RANDOM_SEED widen the sweep (e.g. 3000 cases, seed 9001)
CASES = _cases(n=int(os.environ.get("GN_RANDOM_CASES", "96")), seed=int(os.environ.get("GN_RANDOM_SEED", "20261202")))
# each case on the planner's path; NCHW images also on the cooperative kernels
RUNS = [(c, False) for c in CASES] + [(c, True) for c in CASES if c[0].layout == "nchw" and c[0].HW > 1]


@pytest.mark.parametrize("run", RUNS, ids=lambda r: r[0][0].name + ("-coop" if r[1] else ""))
def test_random_shape_parity(run):
    (wl, mask), coop = run
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    data = inputs.make_inputs(wl, seed=17)
    out = run_gpu(wl, data, mask=mask, debug=gn.Debug(flags=gn.GN_DEBUG_SLAB_COOP) if coop else None)
    say(f"[rand] {wl.name} mask={mask} coop={coop} fwd {gn.PATH_NAMES[out['fwd_plan'].path]} "
        f"({out['fwd_plan'].kernels} kernels) bwd {gn.PATH_NAMES[out['bwd_plan'].path]}")
    check_against_oracle(wl, data, out, mask=mask)
