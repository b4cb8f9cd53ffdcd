"""Turns raw rocprofv3 CSV output of bench.py runs into the summaries under
``profiles/``: one Markdown table per workload (kernel, workgroups,
dispatches, average duration, HBM bytes read and written per dispatch) and
the per-launch HBM byte counts in ``profiles/traffic.json`` that bench.py
reports as ``roofline.traffic``.

Inputs, per workload, three rocprofv3 runs of the same bench.py command:
  * ``--kernel-trace --stats``: durations (``*kernel_trace.csv``, ``*kernel_stats.csv``);
  * ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (KiB per dispatch,
    ``*counter_collection.csv``), each in a run of its own.
The bench command is run with ``--copy-calibration-mib M``: it copies M MiB
three times after its timed work, and the counters of those copies (the
largest copy-kernel dispatches) scale the counters, since on this part a
counter need not read the bytes a kernel moves one for one (FETCH_SIZE of a
1 GiB copy reads half of it).

Usage:
  python -m normalization_gn_stats_amd.rocprof_summary --workload W --trace DIR --fetch DIR --write DIR \\
      --copy-mib M --command "<the bench command>" [--note TEXT] [--profiles DIR]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _rows(directory: str, suffix: str) -> list[dict]:
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _get(row: dict, *names):
    low = {k.lower(): v for k, v in row.items() if k is not None}
    for n in names:
        v = low.get(n.lower())
        if v not in (None, ""):
            return v
    raise KeyError(f"none of {names} in {sorted(low)}")


def _mangled_last_name(kernel: str):
    """Last identifier of an Itanium-mangled nested name
    (_ZN2gn12_GLOBAL__N_110rows_bwd_kI... -> rows_bwd_k), or None."""
    if not kernel.startswith("_ZN"):
        return None
    i, last = 3, None
    while i < len(kernel) and kernel[i].isdigit():
        j = i
        while j < len(kernel) and kernel[j].isdigit():
            j += 1
        n = int(kernel[i:j])
        last = kernel[j:j + n]
        i = j + n
    return last


def short_name(kernel: str) -> str:
    """Kernel name without namespaces, template arguments and parameter list
    (gn::(anonymous namespace)::slab_nchw_bwd<float, 8>(...) -> slab_nchw_bwd;
    mangled names as rocprofv3 reports some template kernels likewise)."""
    m = _mangled_last_name(kernel)
    if m:
        return m
    k = kernel[5:] if kernel.startswith("void ") else kernel
    k = k.replace("(anonymous namespace)", "anonymous").split("(")[0]
    depth, base = 0, ""
    for ch in k:
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif depth == 0:
            base += ch
    base = base.strip().split("::")[-1]
    return base.strip()


def _workgroups(row: dict) -> int:
    grid = int(float(_get(row, "Grid_Size_X", "Grid_Size", "grid_size")))
    wg = int(float(_get(row, "Workgroup_Size_X", "Workgroup_Size", "workgroup_size")))
    try:
        grid *= int(float(_get(row, "Grid_Size_Y"))) * int(float(_get(row, "Grid_Size_Z")))
        wg *= int(float(_get(row, "Workgroup_Size_Y"))) * int(float(_get(row, "Workgroup_Size_Z")))
    except KeyError:
        pass
    return max(1, grid // max(1, wg))


def durations(trace_dir: str) -> dict:
    """(kernel, workgroups) -> list of durations in microseconds."""
    out: dict = {}
    for r in _rows(trace_dir, "kernel_trace.csv"):
        name = _get(r, "Kernel_Name", "kernel_name")
        t = (int(_get(r, "End_Timestamp")) - int(_get(r, "Start_Timestamp"))) / 1e3
        out.setdefault((name, _workgroups(r)), []).append(t)
    return out


def stats_table(trace_dir: str) -> list[dict]:
    """The rows of rocprofv3's own --stats summary (kernel_stats.csv)."""
    out = []
    for r in _rows(trace_dir, "kernel_stats.csv"):
        out.append(dict(name=_get(r, "Name"), calls=int(float(_get(r, "Calls"))),
                        avg_us=float(_get(r, "AverageNs")) / 1e3, total_us=float(_get(r, "TotalDurationNs")) / 1e3))
    return out


def counters(pmc_dir: str, counter: str) -> list[tuple[str, int, float]]:
    """[(kernel, workgroups, KiB)] per dispatch, in dispatch order."""
    per: dict = {}
    for r in _rows(pmc_dir, "counter_collection.csv"):
        if _get(r, "Counter_Name") != counter:
            continue
        key = int(float(_get(r, "Dispatch_Id", "Correlation_Id")))
        name = _get(r, "Kernel_Name")
        v = float(_get(r, "Counter_Value"))
        e = per.setdefault(key, [name, _workgroups(r), 0.0])
        e[2] += v   # a counter may come back split over dimensions (e.g. per XCD): their sum
    return [tuple(per[k]) for k in sorted(per)]


def calibration(values: list[tuple[str, int, float]], copy_mib: int) -> float:
    """Bytes per counter unit: copy_mib MiB over the counter of the copy
    dispatches (the three largest dispatches of a copy kernel, median)."""
    # the runtime's device-to-device blit kernel (torch's copy_ of a same-dtype
    # buffer), not other kernels whose names mention a copy (dtype conversions)
    copies = sorted((v for n, _, v in values if n.startswith("__amd_rocclr_copyBuffer")), reverse=True)[:3]
    if not copies:
        raise ValueError("no copy kernel dispatches to calibrate the counter with")
    return copy_mib * (1 << 20) / statistics.median(copies)


KERNEL_SOURCES = (
    (("rows_",), "gn_rows.hip"),
    (("slab_", "clear_words", "params_over_n"), "gn_slab.hip"),
    (("fwd_tile_stats", "fwd_finalize", "fwd_apply", "bwd_tile_sums", "col_sums", "bwd_group_ab", "bwd_dx",
      "stream_"), "gn_stream.hip"),
    (("gen_", "generic_"), "gn_generic.hip"),
)


def fingerprint(kernel: str):
    """The fingerprint bench.py compares against (its source_fingerprint)."""
    sys.path.insert(0, ROOT)
    import bench
    try:
        return bench.source_fingerprint(kernel)
    except KeyError:
        return None


def summarize(workload: str, trace: str, fetch: str, write: str, copy_mib: int, command: str, note: str,
              profiles: str) -> str:
    dur = durations(trace)
    fc = counters(fetch, "FETCH_SIZE")
    wc = counters(write, "WRITE_SIZE")
    f_scale = calibration(fc, copy_mib) / 1024.0   # bytes per KiB-unit read by the counter
    w_scale = calibration(wc, copy_mib) / 1024.0

    def per_kernel(vals):
        d: dict = {}
        for n, wg, v in vals:
            d.setdefault((n, wg), []).append(v * 1024.0)
        return d

    fk, wk = per_kernel(fc), per_kernel(wc)
    rows = []
    for (name, wg), ts in dur.items():
        s = short_name(name)
        if "copy" in name.lower() or s.startswith("__amd") or "elementwise" in name.lower() or "fill" in s.lower():
            continue   # the benchmark's own copies, fills and generators
        if not fingerprint(s):
            continue
        rd = fk.get((name, wg))
        wr = wk.get((name, wg))
        rows.append(dict(kernel=s, full=name, workgroups=wg, dispatches=len(ts), avg_us=sum(ts) / len(ts),
                         read=(statistics.mean(rd) * f_scale if rd else None),
                         write=(statistics.mean(wr) * w_scale if wr else None)))
    rows.sort(key=lambda r: -r["avg_us"] * r["dispatches"])
    mains = sorted(dict.fromkeys(r["kernel"] for r in rows[:2]))   # by name: near-equal times do not rename
    calls = call_totals(rows)
    fname = "_".join(mains) + f"__{workload}.md"
    # a workload keeps the file its first summary named, although kernels of
    # near-equal times may trade places among the two longest
    old = sorted(f for f in os.listdir(profiles) if f.endswith(f"__{workload}.md")) if os.path.isdir(profiles) else []
    if len(old) == 1:
        fname = old[0]
    lines = [f"# rocprofv3 summary: GroupNorm kernels on workload `{workload}`", "",
             "Commands (run from the repository root on one MI355X; `cd /tmp && export TMPDIR=/tmp` first):", "",
             "```",
             f"rocprofv3 --kernel-trace --stats -f csv -d <out>/trace -o run -- {command}",
             f"rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/FETCH_SIZE -o run -- {command}",
             f"rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/WRITE_SIZE -o run -- {command}",
             f"python -m normalization_gn_stats_amd.rocprof_summary --workload {workload} --trace <out>/trace "
             f"--fetch <out>/FETCH_SIZE --write <out>/WRITE_SIZE --copy-mib {copy_mib} --command '{command}'",
             "```", "",
             f"Calibration: a {copy_mib} MiB device copy reads FETCH_SIZE = {copy_mib / f_scale:.1f} MiB and "
             f"WRITE_SIZE = {copy_mib / w_scale:.1f} MiB, so FETCH_SIZE is scaled by {f_scale:.3f} and "
             f"WRITE_SIZE by {w_scale:.3f} below.", ""]
    if note:
        lines += [note, ""]
    fps = sorted({(KERNEL_SOURCES_FILE(r["kernel"]), fingerprint(r["kernel"])) for r in rows})
    lines += ["Kernel source fingerprints (sha256 of the code, comments excluded, of the kernel's .hip "
              "file and the local headers it includes): " + ", ".join(f"{f} `{h}`" for f, h in fps), "",
              "| kernel | workgroups | dispatches | avg duration (µs) | HBM read (MiB, scaled) | HBM write (MiB, scaled) |",
              "|---|---|---|---|---|---|"]
    for r in rows + calls:
        rd = f"{r['read'] / 2**20:.1f}" if r["read"] is not None else "—"
        wr = f"{r['write'] / 2**20:.1f}" if r["write"] is not None else "—"
        lines.append(f"| {r['kernel']} | {r['workgroups']} | {r['dispatches']} | {r['avg_us']:.2f} | {rd} | {wr} |")
    st = [s for s in stats_table(trace) if fingerprint(short_name(s["name"]))]
    if st:
        lines += ["", "rocprofv3 `--stats` (kernel_stats.csv), the same kernels:", "",
                  "| kernel | calls | average (µs) | total (µs) |", "|---|---|---|---|"]
        for s in st:
            lines.append(f"| {short_name(s['name'])} | {s['calls']} | {s['avg_us']:.2f} | {s['total_us']:.1f} |")
    os.makedirs(profiles, exist_ok=True)
    with open(os.path.join(profiles, fname), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    tpath = os.path.join(profiles, "traffic.json")
    try:
        traffic = json.load(open(tpath))
    except (OSError, ValueError):
        traffic = {}
    traffic["note"] = ("HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled "
                       "by the same counters on a device copy of known size; each entry carries the fingerprint "
                       "of the code (comments excluded) of the sources its kernel is compiled from (its .hip "
                       "file and the local headers it includes)")
    ks = traffic.setdefault("kernels", {})
    for k in [k for k in ks if k.startswith(f"{workload}|")]:
        del ks[k]
    for r in rows + calls:
        ks[f"{workload}|{r['kernel']}|{r['workgroups']}"] = dict(
            avg_us=round(r["avg_us"], 3), read_bytes=r["read"], write_bytes=r["write"],
            source_fingerprint=fingerprint(r["kernel"]))
    with open(tpath, "w") as fh:
        json.dump(traffic, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return os.path.join(profiles, fname)


# Kernels of one call of the multi-kernel paths (stream, generic): the first
# is the anchor whose dispatch count is the number of calls.
CALLS = {
    "stream_fwd_call": ("fwd_tile_stats", "fwd_finalize", "fwd_apply"),
    "stream_bwd_call": ("bwd_tile_sums", "col_sums", "bwd_group_ab", "params_over_n", "bwd_dx"),
    "generic_fwd_call": ("gen_stats_partial", "gen_stats_final", "gen_apply"),
    "generic_bwd_call": ("gen_dx", "gen_ab_partial", "gen_param_partial", "gen_plane_ab", "gen_plane_params",
                         "gen_plane_partial", "gen_sum_rows"),
}


def call_totals(rows: list) -> list:
    """Per call of a multi-kernel path: the sums over its kernels of the
    time and bytes per call (every dispatch of a member kernel, divided by
    the anchor's dispatch count)."""
    out = []
    for call, members in CALLS.items():
        anchor = [r for r in rows if r["kernel"] == members[0]]
        if not anchor:
            continue
        n = sum(r["dispatches"] for r in anchor)
        mem = [r for r in rows if r["kernel"] in members]
        tot = lambda k: (sum(r[k] * r["dispatches"] for r in mem) / n
                         if all(r[k] is not None for r in mem) else None)
        out.append(dict(kernel=call, full=call, workgroups="call", dispatches=n,
                        avg_us=sum(r["avg_us"] * r["dispatches"] for r in mem) / n,
                        read=tot("read"), write=tot("write")))
    return out


def KERNEL_SOURCES_FILE(kernel: str) -> str:
    for prefixes, f in KERNEL_SOURCES:
        if kernel.startswith(prefixes):
            return f
    return "?"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--note", default="")
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args(argv)
    print(summarize(a.workload, a.trace, a.fetch, a.write, a.copy_mib, a.command, a.note, a.profiles))


if __name__ == "__main__":
    main()
