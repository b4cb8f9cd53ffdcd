"""CPU model of the slab kernels' schedule (no GPU): ``schedule_model.cpp``,
built with g++ from the header the kernels and the host planner share
(``csrc/gn_slab_plan.hpp``), run over the benchmark shapes and small ragged
ones at the residency caps of apex PR #2018's Description (128 tiles per
slice against 120 resident workgroups: a cap of tiles - 8), the A100's 108
SMs of its reviewer comment, a cap of 1, the tile count itself, and the
MI355X's occupancy caps (256 CUs x 2, 3 or 4 workgroups).  Every tile must be
reduced once in phase 1 and written once in phase 2, under many
interleavings of the dynamic NHWC hand-out, and every element covered once.

Planted mistakes in a copy of the header (phase-2 draws off by one, a tile
that phase 2 never draws, the wrong last tile of a member, a wrong chunk
stride, a team larger than the cap, unclamped loads) must each make the
model fail.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "normalization_gn_stats_amd", "csrc")
SRC = os.path.join(HERE, "schedule_model.cpp")
HEADER = os.path.join(CSRC, "gn_slab_plan.hpp")

# tile chunks per thread the library uses (gn_slab.hip: GN_SLAB_NHWC_RF/RB,
# nchw_r with its per-dtype caps)
NHWC_R = {"fwd": 16, "bwd": 8}


def build(out_dir, include_dir=CSRC):
    exe = os.path.join(out_dir, "schedule_model")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-Wall", "-I", include_dir, SRC, "-o", exe])
    return exe


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    return build(str(tmp_path_factory.mktemp("sched")))


def run(exe, nhwc, N, C, HW, G, V, R, cap, seeds=8):
    r = subprocess.run([exe, str(int(nhwc)), str(N), str(C), str(HW), str(G), str(V), str(R), str(cap), str(seeds)],
                       capture_output=True, text=True, timeout=120)
    return r.returncode, r.stdout.strip()


def tiles_of(nhwc, C, HW, G, V, R):
    if nhwc:
        tp = (256 // (C // V)) * R
        return -(-HW // tp)
    te = 256 * R * V
    return (C // G) * -(-HW // te)


# (name, nhwc, N, C, HW, G, V, R)
SHAPES = [
    # the NHWC image of the apex reproducer, forward and backward tiles
    ("nhwc_f16_1x128x1024x2048_fwd", True, 1, 128, 1024 * 2048, 16, 8, NHWC_R["fwd"]),
    ("nhwc_f16_1x128x1024x2048_bwd", True, 1, 128, 1024 * 2048, 16, 8, NHWC_R["bwd"]),
    # 128 tiles per sample (the apex Description's count)
    ("nhwc_f16_1x128x128x256_fwd", True, 1, 128, 128 * 256, 16, 8, 16),
    ("nhwc_f32_3x32x50x41", True, 3, 32, 50 * 41, 4, 4, 8),
    ("nhwc_f16_2x512x9x23", True, 2, 512, 9 * 23, 32, 8, 16),
    ("nhwc_f16_2x8x31x33", True, 2, 8, 31 * 33, 1, 8, 8),
    # the NCHW configuration (fp32 forward 16 chunks, backward 8; bf16 8 and 4)
    ("nchw_f32_112x64x512x512_fwd", False, 112, 64, 512 * 512, 8, 4, 16),
    ("nchw_f32_112x64x512x512_bwd", False, 112, 64, 512 * 512, 8, 4, 8),
    ("nchw_bf16_112x64x512x512_bwd", False, 112, 64, 512 * 512, 8, 8, 4),
    # ragged last tiles of a plane, small planes, many tiles
    ("nchw_f32_2x16x64x70", False, 2, 16, 64 * 70, 4, 4, 8),
    ("nchw_f32_1x8x150x16424", False, 1, 8, 150 * 16424, 1, 4, 8),
    ("nchw_f16_2x320x64x64", False, 2, 320, 64 * 64, 32, 8, 2),
    ("nchw_f32_2x32x16x16", False, 2, 32, 16 * 16, 8, 4, 1),
]


def caps_for(T):
    caps = {1, 108, T, T + 5, 2 * T, 512, 768, 1024}
    if T > 8:
        caps.add(T - 8)
    return sorted(caps)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s[0])
def test_every_tile_reduced_and_written_once(model, shape):
    name, nhwc, N, C, HW, G, V, R = shape
    T = tiles_of(nhwc, C, HW, G, V, R)
    for cap in caps_for(T):
        rc, out = run(model, nhwc, N, C, HW, G, V, R, cap, seeds=8 if T <= 4096 else 2)
        assert rc == 0 and out.startswith("OK"), f"{name} cap {cap}: {out}"
        assert f"tiles={T} " in out, f"{name}: model plans {out}, expected {T} tiles"


def test_apex_description_case(model):
    """128 tiles per slice, 120 resident workgroups: 8 members take a second
    (overflow) tile; every tile is still reduced and written exactly once."""
    rc, out = run(model, True, 1, 128, 128 * 256, 16, 8, 16, 120, seeds=64)
    assert rc == 0 and out == "OK tiles=128 team=120 nteams=1 grid=120", out


MUTANTS = [
    # phase-2 draws off by one: the first tile is never written, a draw past the end is
    ("nhwc_phase2_tile", "return k < tiles ? tiles - 1 - k : -1;", "return k < tiles ? tiles - k : -1;",
     (True, 1, 128, 128 * 256, 16, 8, 16, 120)),
    # phase-2 draws that never name tile 0 (written only when it happens to be resident)
    ("nhwc_phase2_tile", "return k < tiles ? tiles - 1 - k : -1;", "return k < tiles - 1 ? tiles - 1 - k : -1;",
     (True, 1, 128, 128 * 256, 16, 8, 16, 100)),
    # a member's last tile one step too far
    ("nchw_last_tile", "return m + (tiles - 1 - m) / team * team;", "return m + (tiles - m) / team * team;",
     (False, 2, 16, 64 * 70 * 4, 4, 4, 8, 5)),
    # chunks of a thread one vector short of a workgroup apart (overlaps and a gap)
    ("nchw_chunk_elem", "return k0 + (int64_t)(j * kThreads + t) * V;",
     "return k0 + (int64_t)(j * (kThreads - 1) + t) * V;",
     (False, 2, 16, 64 * 70, 4, 4, 8, 3)),
    # the team ignores the cap: more workgroups than can be resident
    ("plan", "g.team = g.tiles < cap ? g.tiles : cap;", "g.team = g.tiles;",
     (False, 112, 64, 512 * 512, 8, 4, 8, 108)),
    # NHWC loads not clamped to the last pixel
    ("nhwc_pixel_load", "return p < HW - 1 ? p : HW - 1;", "return p;", (True, 3, 32, 50 * 41, 4, 4, 8, 3)),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: f"{m[0]}:{m[2][:24]}")
def test_model_catches_planted_mistakes(tmp_path, mutant):
    fn, good, bad, case = mutant
    text = open(HEADER).read()
    assert text.count(good) == 1, f"mutation anchor of {fn} not found"
    d = tmp_path / "inc"
    d.mkdir()
    (d / "gn_slab_plan.hpp").write_text(text.replace(good, bad))
    exe = build(str(tmp_path), str(d))
    rc, out = run(exe, *case, seeds=8)
    assert rc != 0 and out.startswith("FAIL"), f"planted mistake in {fn} not caught: {out}"
    good_dir = tmp_path / "good"
    good_dir.mkdir()
    rc, out = run(build(str(good_dir)), *case, seeds=8)
    assert rc == 0, f"the unmutated header fails the same case: {out}"
