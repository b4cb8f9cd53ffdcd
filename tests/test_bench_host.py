"""Host-side checks of bench.py's bookkeeping (no GPU): every kernel the
recorded byte counters name maps to the source file it is built from, and a
counter entry is used only while that file and the shared sources are
unchanged."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

TRAFFIC = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))


def test_every_recorded_kernel_has_a_source_file():
    for key in TRAFFIC["kernels"]:
        kernel = key.split("|")[1]
        fp = bench.source_fingerprint(kernel)
        assert len(fp) == 16


def test_kernel_source_table_names_existing_files():
    d = os.path.join(ROOT, "normalization_gn_stats_amd", "csrc")
    for _, f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(d, f)), f


def test_fingerprint_covers_the_included_headers_only():
    names = lambda k: {os.path.basename(p) for p in bench.source_files(k)}
    assert names("slab_nchw_bwd") == {"gn_slab.hip", "gn_device.hpp", "gn_internal.hpp", "gn_slab_plan.hpp", "gn.h"}
    assert names("small_nchw_fwd") == names("slab_nchw_bwd")
    assert names("rows_bwd_k") == {"gn_rows.hip", "gn_device.hpp", "gn_internal.hpp", "gn.h"}
    assert names("bwd_dx") == {"gn_stream.hip", "gn_device.hpp", "gn_internal.hpp", "gn.h"}
    assert names("gen_dx") == {"gn_generic.hip", "gn_device.hpp", "gn_internal.hpp", "gn.h"}
    for k in ("slab_nchw_bwd", "rows_bwd_k", "bwd_dx", "gen_dx"):
        assert all(os.path.exists(p) for p in bench.source_files(k))


def test_fingerprint_ignores_comments(tmp_path, monkeypatch):
    src = os.path.join(bench.CSRC, "gn_rows.hip")
    text = open(src).read()
    d = tmp_path / "pkg" / "csrc"   # the sources include ../../include/gn.h
    d.mkdir(parents=True)
    for f in os.listdir(bench.CSRC):
        if f.endswith((".hip", ".hpp", ".cpp")):
            (d / f).write_text(open(os.path.join(bench.CSRC, f)).read())
    inc = tmp_path / "include"
    inc.mkdir()
    (inc / "gn.h").write_text(open(os.path.join(ROOT, "include", "gn.h")).read())
    monkeypatch.setattr(bench, "CSRC", str(d))
    base = bench.source_fingerprint("rows_bwd_k")
    (d / "gn_rows.hip").write_text("// a new comment\n" + text.replace("*/", "   */", 1))
    assert bench.source_fingerprint("rows_bwd_k") == base
    (d / "gn_rows.hip").write_text(text + "\nint gn_rows_changed;\n")
    assert bench.source_fingerprint("rows_bwd_k") != base


def test_unknown_kernel_name_is_an_error():
    with pytest.raises(KeyError):
        bench.source_fingerprint("no_such_kernel")


def test_fingerprints_differ_per_source_file():
    assert bench.source_fingerprint("rows_bwd_k") != bench.source_fingerprint("slab_nchw_bwd")
    assert bench.source_fingerprint("rows_bwd_k") == bench.source_fingerprint("rows_colsum_k")


def test_stale_entry_gives_no_traffic(tmp_path, monkeypatch):
    key = next(iter(TRAFFIC["kernels"]))
    workload, kernel, grid = key.split("|")
    entry = dict(TRAFFIC["kernels"][key], source_fingerprint="0" * 16)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps({"kernels": {key: entry}}))
    csrc = tmp_path / "normalization_gn_stats_amd"
    os.symlink(os.path.join(ROOT, "normalization_gn_stats_amd"), csrc)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    assert bench.recorded_traffic(workload, kernel, grid) is None
    entry["source_fingerprint"] = bench.source_fingerprint(kernel)
    (prof / "traffic.json").write_text(json.dumps({"kernels": {key: entry}}))
    assert bench.recorded_traffic(workload, kernel, grid) == int(entry["read_bytes"] + entry["write_bytes"])


def test_oracle_sweep_lines(monkeypatch, capsys):
    """--oracle-sweep: one JSON line per configuration shape and thread count,
    with the forward and backward medians and the rate scaled to the full
    configuration by its algorithmic bytes."""
    from normalization_gn_stats_amd import inputs
    monkeypatch.setattr(bench, "ORACLE_SWEEP", (
        ("1", "tiny_nchw_f32_2x32x16x16_g8", None, "the whole workload"),
        ("4", "nchw_f32_112x64x512x512_g8", dict(N=1, H=32, W=32), "a small sample"),
    ))
    bench.oracle_sweep()
    lines = [json.loads(ln) for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert [(d["config"], d["runs"]) for d in lines][-1] == ("4", 3)
    assert {d["threads"] for d in lines if d["config"] == "1"} >= {1}
    for d in lines:
        assert d["fwd_ms"] > 0 and d["bwd_ms"] > 0
    full = inputs.WORKLOADS["nchw_f32_112x64x512x512_g8"]
    big = lines[-1]
    sample = full.scaled(N=1, H=32, W=32)
    want = big["fwd_ms"] * full.fwd_min_bytes() / sample.fwd_min_bytes()
    assert abs(big["full_fwd_ms"] - want) <= 0.01 * want + 0.01


def test_every_kernel_maps_to_its_own_source_file():
    """Each __global__ kernel under csrc/ resolves to the .hip file that defines
    it, so that a profile of any kernel can be checked against its sources."""
    import re
    d = os.path.join(ROOT, "normalization_gn_stats_amd", "csrc")
    names = {}
    for f in sorted(os.listdir(d)):
        if f.endswith(".hip"):
            pat = r"__global__\s+(?:__launch_bounds__\([^)]*\)\s+)?void\s+(\w+)\s*\("
            for m in re.finditer(pat, open(os.path.join(d, f)).read()):
                names[m.group(1)] = f
    assert len(names) > 20
    for name, f in names.items():
        mapped = [g for prefixes, g in bench.KERNEL_SOURCES if name.startswith(prefixes)]
        assert mapped and mapped[0] == f, f"{name} (in {f}) maps to {mapped}"
