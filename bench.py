#!/usr/bin/env python3
"""GroupNorm forward+backward throughput on one MI355X.

A step is one forward (statistics + normalize/affine) and one backward
(per-slice reductions, dx, dgamma/dbeta) over every shape of the workload, on
synthetic seeded inputs already resident in HBM.  The headline workload is
the NCHW float32 GroupNorm of 112 x 64 x 512 x 512 with 8 groups (the
POPCORNBENCH GroupNorm problem's shape, 7.5 GB per tensor), the largest of
the five benchmark configurations.

Prints ONE JSON line on stdout:
* ``value``: the headline step's algorithmic bytes (read x, write y,
  gamma/beta, mean/rstd; read dy, x, gamma, mean/rstd, write dx,
  dgamma/dbeta) over the measured step time, in GB/s;
* ``roofline``: the kernel that takes most of the step, timed with HIP
  events that the library records on the call's stream around that kernel;
  its rocprofv3 byte counters (``profiles/traffic.json``) as ``traffic``;
* ``configs``: the same per-call figures for each of the five benchmark
  configurations (whole-call and main-kernel microseconds, TB/s and % of the
  8 TB/s peak, forward and backward separately);
* ``cpu_baseline``: the fp64 oracle on the host cores over a bounded sample
  of the headline workload (whole samples of the tensor).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--configs all|none]
       python bench.py --rows-sweep [--steps K]   (context table, one line per shape)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "GroupNorm fwd+bwd achieved HBM GB/s (% of MI355X peak) and µs/call"
HBM_PEAK_GBS = 8000.0

# (name, workload names)
WORKLOADS = {
    "rows_f16_4096x1024+8192x768": ("rows_f16_4096x1024", "rows_f16_8192x768"),
    "tiny_nchw_f32_2x32x16x16_g8": ("tiny_nchw_f32_2x32x16x16_g8",),
    "rows_f16_4096x1024": ("rows_f16_4096x1024",),
    "rows_f16_8192x768": ("rows_f16_8192x768",),
    "nhwc_f16_1x128x1024x2048_g16": ("nhwc_f16_1x128x1024x2048_g16",),
    "nchw_f32_112x64x512x512_g8": ("nchw_f32_112x64x512x512_g8",),
    "nchw_bf16_112x64x512x512_g8": ("nchw_bf16_112x64x512x512_g8",),
    "rows_bf16_131072x4096": ("rows_bf16_131072x4096",),
    "rows_f16_131072x64": ("rows_f16_131072x64",),
    # RMSNorm over rows (gn_rms_forward / gn_rms_backward)
    "rms_f16_4096x1024": ("rms_f16_4096x1024",),
    "rms_bf16_131072x4096": ("rms_bf16_131072x4096",),
    "rms_f16_131072x64": ("rms_f16_131072x64",),
    # strided (non-contiguous) input: gn_forward_strided / gn_backward_strided
    "nchw_f32_112x64x510x510_g8_crop1": ("nchw_f32_112x64x510x510_g8_crop1",),
    "tiny_nchw_f32_2x32x14x14_g8_crop1": ("tiny_nchw_f32_2x32x14x14_g8_crop1",),
}
DEFAULT = "nchw_f32_112x64x512x512_g8"

# The five benchmark configurations, in their order: the per-config figures
# of the JSON line.
CONFIGS = (
    ("1", "tiny_nchw_f32_2x32x16x16_g8"),
    ("2", "rows_f16_4096x1024+8192x768"),
    ("3", "nhwc_f16_1x128x1024x2048_g16"),
    ("4", "nchw_f32_112x64x512x512_g8"),
    ("5", "rows_bf16_131072x4096"),
)


# The source file that defines each kernel (by name prefix) or each whole call;
# a kernel also depends on the local headers that file includes.
KERNEL_SOURCES = (
    (("rows_",), "gn_rows.hip"),
    (("slab_", "small_nchw_", "mid_nchw_", "split_nchw_", "clear_words", "params_over_n"), "gn_slab.hip"),
    (("fwd_tile_stats", "fwd_finalize", "fwd_apply", "bwd_tile_sums", "col_sums", "bwd_group_ab", "bwd_dx",
      "fwd_one_tile", "bwd_one_tile", "stream_"), "gn_stream.hip"),
    (("gen_", "generic_"), "gn_generic.hip"),
)
CSRC = os.path.join(HERE, "normalization_gn_stats_amd", "csrc")


def source_files(kernel_name: str) -> list:
    """Paths of the sources a kernel is compiled from: its .hip file and every
    local header it includes ("..." includes, followed transitively)."""
    import re
    own = [f for prefixes, f in KERNEL_SOURCES if kernel_name.startswith(prefixes)]
    if not own:
        raise KeyError(f"no source file known for kernel {kernel_name}")
    seen, todo = [], [os.path.normpath(os.path.join(CSRC, own[0]))]
    while todo:
        p = todo.pop()
        if p in seen:
            continue
        seen.append(p)
        for inc in re.findall(r'^\s*#\s*include\s+"([^"]+)"', open(p).read(), re.M):
            todo.append(os.path.normpath(os.path.join(os.path.dirname(p), inc)))
    return sorted(seen)


def code_text(path: str) -> str:
    """A source file without its comments and with runs of whitespace
    collapsed: what the compiler sees, so that a change to a comment does not
    count as a change to the kernels."""
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_fingerprint(kernel_name: str) -> str:
    """sha256 over the code of the sources a kernel is compiled from, to tell
    whether byte counters recorded in profiles/traffic.json still describe
    the kernel built now."""
    import hashlib
    h = hashlib.sha256()
    for p in source_files(kernel_name):
        h.update(os.path.relpath(p, CSRC).encode())
        h.update(code_text(p).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload, kernel_name, grid):
    """HBM bytes per launch of this kernel from profiles/traffic.json (rocprofv3
    FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None when
    missing or taken on different sources of that kernel."""
    try:
        t = json.load(open(os.path.join(HERE, "profiles", "traffic.json")))
    except (OSError, ValueError):
        return None
    e = t.get("kernels", {}).get(f"{workload}|{kernel_name}|{grid}")
    if not e or e.get("read_bytes") is None or e.get("write_bytes") is None:
        return None
    if e.get("source_fingerprint") != source_fingerprint(kernel_name):
        return None
    return int(e["read_bytes"] + e["write_bytes"])


class TimingEvents:
    """HIP events for kernel timing, created with hipEventDisableSystemFence:
    recording them performs no system-scope fence (no cache write-back and
    invalidation around the timed kernel), which on MI355X keeps the event
    pair of a microsecond-scale kernel within about a microsecond of the
    kernel's own duration (plain events read 1.5-2 us high)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch already loaded
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def new(self):
        e = self.ct.c_void_p()
        st = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {st}")
        self.made.append(e)
        return e.value

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        st = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(a), self.ct.c_void_p(b))
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return ms.value

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)
        self.made = []


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS),
                    help="rms_* workloads run RMSNorm over rows (gn_rms_forward / gn_rms_backward)")
    ap.add_argument("--configs", default="all", choices=["all", "none"],
                    help="all: also time the five benchmark configurations (per-config figures)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target duration of the oracle CPU-baseline sample (0 disables it)")
    ap.add_argument("--force-path", default=None, choices=[None, "generic", "rows", "slab", "stream"])
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB three times (a known-size "
                         "kernel that scales the rocprofv3 byte counters)")
    ap.add_argument("--rows-sweep", action="store_true",
                    help="instead of the bench line: forward/backward times of the rows shapes the pages time on "
                         "MI350X, one JSON line per shape")
    ap.add_argument("--oracle-sweep", action="store_true",
                    help="instead of the bench line: the fp64 oracle's forward and backward times on the host "
                         "cores for each benchmark configuration (a stated sample of the large ones), one JSON "
                         "line each; needs no GPU")
    ap.add_argument("--mode", default="auto", choices=["auto", "graph", "eager"],
                    help="graph: the timed steps run as one captured HIP graph (no host in the loop)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this GroupNorm engine "
              "runs on a single MI355X: slices are independent per sample, so data parallelism over N needs only "
              "an all-reduce of dgamma/dbeta, which this library leaves to the caller",
              file=sys.stderr)
        sys.exit(2)

    if args.oracle_sweep:
        oracle_sweep()
        return

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.rows_sweep:
        rows_sweep(args.steps)
        return

    K, W = args.steps, args.warmup
    log(f"headline workload {args.workload}")
    head = measure(args.workload, K, W, args.mode, args.force_path, keep_inputs=args.cpu_seconds > 0)
    value = head["bytes_per_step"] / (head["ms_per_step"] * 1e-3) / 1e9

    # ---- roofline of the dominant kernel of the headline step ----------------
    dom = max(head["calls"], key=lambda c: c["main_kernel_us"])
    traffic = None
    for kn in dom["kernel"] or ():
        traffic = recorded_traffic(args.workload, kn, dom["grid"])
        if traffic is not None:
            dom["kernel"] = kn
            break
    roofline = {"bound": "hbm", "achieved": round(dom["main_kernel_gbs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dom["main_kernel_gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "traffic_over_algorithmic": (round(traffic / dom["main_kernel_bytes"], 3) if traffic else None),
                "kernel": (f"{dom['call']} {dom['path']} " + ("call (all its kernels)"
                                                                  if dom["path"] in ("stream", "generic")
                                                                  else "main kernel") + f" on {dom['shape']}"),
                "kernel_name": (dom["kernel"] if isinstance(dom["kernel"], str) else None),
                "avg_us": round(dom["main_kernel_us"], 3), "algorithmic_bytes": dom["main_kernel_bytes"],
                "timing": ("HIP events (created without the system-scope fence) recorded by the library on "
                           "the call's stream around the main kernel "
                           "(stream and generic paths: around all kernels of the call), in a pass of K eager "
                           "steps of their own " + ("queued behind a GPU spin after the graph-timed region"
                                                    if head["mode"] == "graph" else "after the timed region"))}

    # measured device-to-device copy of 1 GiB (read + write), the practical
    # ceiling of a streaming kernel on this part: a second denominator
    copy_gbs = copy_bandwidth()
    roofline["copy_gbs"] = round(copy_gbs, 1)
    roofline["frac_of_copy"] = round(dom["main_kernel_gbs"] / copy_gbs, 4)

    if args.copy_calibration_mib > 0:
        src = torch.ones(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- oracle CPU baseline on a bounded sample --------------------------------
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(head["shapes"], args.cpu_seconds, head["bytes_per_step"])
    head["shapes"] = None
    torch.cuda.empty_cache()

    # ---- the five benchmark configurations --------------------------------------
    configs = None
    if args.configs == "all":
        configs = {}
        for label, wname in CONFIGS:
            if wname == args.workload and args.force_path is None:
                r = head
            else:
                log(f"config {label}: {wname}")
                r = measure(wname, K, W, "auto", None)
                r["shapes"] = None
                torch.cuda.empty_cache()
            configs[label] = config_summary(wname, r)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "launch": head["mode"], "shapes": head["shape_desc"],
                   "op": head["op"], "mask": head["mask"], "bytes_per_step": head["bytes_per_step"],
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "us_per_call": {f"{c['call']}:{c['shape']}": round(c["call_us"], 3) for c in head["calls"]},
        "main_kernel_us": {f"{c['call']}:{c['shape']}": round(c["main_kernel_us"], 3) for c in head["calls"]},
        "us_per_call_flushed": head["flushed"],
        "calls": [{k: (round(v, 3) if isinstance(v, float) else v) for k, v in c.items()} for c in head["calls"]],
        "roofline": roofline,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def copy_bandwidth() -> float:
    import torch
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for i in range(3):
        ce[2 * i].record(stream)
        cdst.copy_(csrc)
        ce[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    copy_ms = sorted(ce[2 * i].elapsed_time(ce[2 * i + 1]) for i in range(3))[1]
    del csrc, cdst
    return 2 * (1 << 30) / (copy_ms * 1e-3) / 1e9


def config_summary(wname, r):
    """Per-config figures: per shape, forward and backward whole-call and
    main-kernel microseconds and the call's algorithmic TB/s and % of peak."""
    shapes = {}
    for c in r["calls"]:
        d = shapes.setdefault(c["shape"], {"path": {}})
        k = c["call"]
        d["path"][k] = c["path"]
        d[f"{k}_us"] = round(c["call_us"], 3)
        d[f"{k}_main_kernel_us"] = round(c["main_kernel_us"], 3)
        d[f"{k}_bytes"] = c["call_bytes"]
        gbs = c["call_bytes"] / (c["call_us"] * 1e-6) / 1e9
        d[f"{k}_tbs"] = round(gbs / 1e3, 3)
        d[f"{k}_pct_of_peak"] = round(100 * gbs / HBM_PEAK_GBS, 2)
    out = {"workload": wname, "launch": r["mode"], "shapes": shapes}
    if r["flushed"]:
        out["us_per_call_flushed"] = r["flushed"]
    return out


def measure(workload, K, W, mode, force_path, keep_inputs=False):
    """Times K steps of one workload (all its shapes, forward then backward).

    Returns the step time, per-call whole-call and main-kernel times (from
    the library's events), the bytes per step and, for graph-timed small
    workloads, cold-cache call times."""
    import ctypes

    import torch

    import normalization_gn_stats_amd as gn
    from normalization_gn_stats_amd import inputs

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    mask = gn.GN_GRAD_DX | gn.GN_GRAD_DGAMMA | gn.GN_GRAD_DBETA
    rms_mask = gn.GN_GRAD_DX | gn.GN_GRAD_DGAMMA

    # ---- inputs resident in HBM, outputs and workspaces preallocated ----------
    shapes = []
    for name in WORKLOADS[workload]:
        wl = inputs.WORKLOADS[name]
        log(f"generating {wl.name}")
        d = inputs.make_inputs(wl, seed=0, device="cuda")
        x, dy, gamma, beta = d["x"], d["dy"], d["gamma"], d["beta"]
        code = {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype]
        if wl.op == "rms":   # [N, C] rows
            x, dy = x.reshape(wl.N, wl.C), dy.reshape(wl.N, wl.C)
            fws = gn.rms_forward_workspace_size(wl.N, wl.C, wl.G, code, force_path)
            bws = gn.rms_backward_workspace_size(wl.N, wl.C, wl.G, code, rms_mask, force_path)
        elif wl.crop:
            # views: outputs dense NCHW, inputs with their own strides
            y_, dx_ = torch.empty(x.shape, dtype=x.dtype, device=dev), torch.empty(x.shape, dtype=x.dtype, device=dev)
            _, _, H_, W_, st = gn.strided_dims(x, y_, dy, dx_)
            fws = gn.forward_strided_workspace_size(wl.N, wl.C, H_, W_, wl.G, code, st[0], st[1], force_path)
            bws = gn.backward_strided_workspace_size(wl.N, wl.C, H_, W_, wl.G, code, st[2], st[0], st[3], mask,
                                                     force_path)
        else:
            lay = gn.layout_of(x)
            fws = gn.forward_workspace_size(wl.N, wl.C, wl.HW, wl.G, code, lay, force_path)
            bws = gn.backward_workspace_size(wl.N, wl.C, wl.HW, wl.G, code, lay, mask, force_path)
        sh = dict(wl=wl, x=x, dy=dy, gamma=gamma, beta=beta, y=torch.empty_like(x), dx=torch.empty_like(x),
                  mean=torch.empty(wl.N * wl.G, device=dev), rstd=torch.empty(wl.N * wl.G, device=dev),
                  dgamma=torch.empty(wl.C, device=dev), dbeta=torch.empty(wl.C, device=dev),
                  fws=torch.empty(max(fws, 1), dtype=torch.uint8, device=dev),
                  bws=torch.empty(max(bws, 1), dtype=torch.uint8, device=dev),
                  fplan=gn.PlanInfo(), bplan=gn.PlanInfo())
        if wl.crop:
            sh.update(y=y_, dx=dx_, hw=(H_, W_), strides=st)
        shapes.append(sh)

    # Pre-marshalled C-ABI calls (the binding's checks ran once above, through
    # the size queries); a call costs one ctypes dispatch.
    L = gn._lib.lib()

    def calls_for(sh, stream_handle, evs):
        """evs: None, or per call kind ((call_begin, call_end), (kernel_begin, kernel_end)),
        either pair None."""
        wl = sh["wl"]
        code = {"f32": 0, "f16": 1, "bf16": 2}[wl.dtype]
        lay = gn.GN_NCHW if (wl.op == "rms" or wl.crop) else gn.layout_of(sh["x"])
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        out = []
        for kind in ("fwd", "bwd"):
            o = gn._lib.Options()
            o.force_path = {None: 0, "generic": 1, "rows": 2, "slab": 3, "stream": 4}[force_path]
            o.info = ctypes.pointer(sh["fplan" if kind == "fwd" else "bplan"])
            if evs is not None:
                cpair, kpair = evs[0 if kind == "fwd" else 1]
                if cpair is not None:
                    o.event_begin, o.event_end = ctypes.c_void_p(cpair[0]), ctypes.c_void_p(cpair[1])
                if kpair is not None:
                    o.kernel_begin, o.kernel_end = ctypes.c_void_p(kpair[0]), ctypes.c_void_p(kpair[1])
            if wl.op == "rms" and kind == "fwd":
                a = (P(sh["x"]), P(sh["gamma"]), P(sh["y"]), P(sh["rstd"]), wl.N, wl.C, wl.G, ctypes.c_float(wl.eps),
                     code, P(sh["fws"]), sh["fws"].numel(), ctypes.c_void_p(stream_handle), ctypes.byref(o))
                out.append((L.gn_rms_forward, a, o))
            elif wl.op == "rms":
                a = (P(sh["dy"]), P(sh["x"]), P(sh["rstd"]), P(sh["gamma"]), P(sh["dx"]), P(sh["dgamma"]), rms_mask,
                     wl.N, wl.C, wl.G, code, P(sh["bws"]), sh["bws"].numel(), ctypes.c_void_p(stream_handle),
                     ctypes.byref(o))
                out.append((L.gn_rms_backward, a, o))
            elif wl.crop and kind == "fwd":
                st = sh["strides"]
                a = (P(sh["x"]), st[0], P(sh["gamma"]), P(sh["beta"]), P(sh["y"]), st[1], P(sh["mean"]),
                     P(sh["rstd"]), wl.N, wl.C, sh["hw"][0], sh["hw"][1], wl.G, ctypes.c_float(wl.eps), code,
                     P(sh["fws"]), sh["fws"].numel(), ctypes.c_void_p(stream_handle), ctypes.byref(o))
                out.append((L.gn_forward_strided, a, o))
            elif wl.crop:
                st = sh["strides"]
                a = (P(sh["dy"]), st[2], P(sh["x"]), st[0], P(sh["mean"]), P(sh["rstd"]), P(sh["gamma"]),
                     P(sh["dx"]), st[3], P(sh["dgamma"]), P(sh["dbeta"]), mask, wl.N, wl.C, sh["hw"][0],
                     sh["hw"][1], wl.G, code, P(sh["bws"]), sh["bws"].numel(), ctypes.c_void_p(stream_handle),
                     ctypes.byref(o))
                out.append((L.gn_backward_strided, a, o))
            elif kind == "fwd":
                a = (P(sh["x"]), P(sh["gamma"]), P(sh["beta"]), P(sh["y"]), P(sh["mean"]), P(sh["rstd"]),
                     wl.N, wl.C, wl.HW, wl.G, ctypes.c_float(wl.eps), code, lay, P(sh["fws"]),
                     sh["fws"].numel(), ctypes.c_void_p(stream_handle), ctypes.byref(o))
                out.append((L.gn_forward, a, o))
            else:
                a = (P(sh["dy"]), P(sh["x"]), P(sh["mean"]), P(sh["rstd"]), P(sh["gamma"]), P(sh["dx"]),
                     P(sh["dgamma"]), P(sh["dbeta"]), mask, wl.N, wl.C, wl.HW, wl.G, code, lay, P(sh["bws"]),
                     sh["bws"].numel(), ctypes.c_void_p(stream_handle), ctypes.byref(o))
                out.append((L.gn_backward, a, o))
        return out

    def run(call_list):
        for fn, a, _o in call_list:
            st = fn(*a)
            if st != 0:
                raise gn.GNError(st, fn.__name__)

    plain = [c for sh in shapes for c in calls_for(sh, sp, None)]

    log(f"warmup {W} steps")
    t_w0 = time.perf_counter()
    for _ in range(W):
        run(plain)
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t_w0) * 1e3 / max(W, 1)

    if mode == "auto":
        mode = "graph" if warm_ms < 2.0 else "eager"

    # ---- timed region: exactly K steps between two synchronisations ----------
    graph = None
    if mode == "graph":
        # the K steps captured into one HIP graph, so that no host work sits
        # between the kernels of these microsecond-scale calls
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
            h = torch.cuda.current_stream().cuda_stream
            for i in range(K):
                for sh in shapes:
                    run(calls_for(sh, h, None))
        graph.replay()             # first replay uploads the graph
        torch.cuda.synchronize()

    # per step, per shape, per call (fwd, bwd): call events and kernel events,
    # recorded in separate passes so that neither pair brackets the other's
    # records (an event record between two kernels costs about a microsecond)
    tev = TimingEvents()

    def ev_pair():
        return (tev.new(), tev.new())

    cev = [[[ev_pair() for _ in range(2)] for _ in shapes] for _ in range(K)]
    kev = [[[ev_pair() for _ in range(2)] for _ in shapes] for _ in range(K)]
    call_pass = [[c for k, sh in enumerate(shapes)
                  for c in calls_for(sh, sp, [(cev[i][k][0], None), (cev[i][k][1], None)])] for i in range(K)]
    kern_pass = [[c for k, sh in enumerate(shapes)
                  for c in calls_for(sh, sp, [(None, kev[i][k][0]), (None, kev[i][k][1])])] for i in range(K)]

    log(f"timing {K} steps ({mode})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for cl in call_pass:   # eager: the call events ride in the timed steps
            run(cl)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    def behind_spin(passes):
        """The passes' K steps issued eagerly behind a GPU spin, so that the
        kernels run back to back (the host is not in the loop)."""
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        torch.cuda._sleep(1_000_000)
        c1.record(stream)
        torch.cuda.synchronize()
        cycles_per_ms = 1_000_000 / max(c0.elapsed_time(c1), 1e-3)
        host_ms = warm_ms * K * 3 + 20.0
        torch.cuda._sleep(int(cycles_per_ms * host_ms))
        for cl in passes:
            run(cl)
        torch.cuda.synchronize()

    if graph is not None:
        behind_spin(call_pass)
        behind_spin(kern_pass)
    else:
        for cl in kern_pass:
            run(cl)
        torch.cuda.synchronize()

    bytes_per_step = sum(sh["wl"].fwd_min_bytes() + sh["wl"].bwd_min_bytes() for sh in shapes)

    # ---- per-call durations from the library-recorded events ------------------
    calls = []
    for k, sh in enumerate(shapes):
        wl = sh["wl"]
        for c, (kind, plan) in enumerate((("fwd", sh["fplan"]), ("bwd", sh["bplan"]))):
            path = gn.PATH_NAMES[plan.path]
            call_bytes = wl.fwd_min_bytes() if kind == "fwd" else wl.bwd_min_bytes()
            if path in ("stream", "generic") or kind == "fwd":
                # stream/generic: the kernel events bracket all kernels of the call
                nbytes = call_bytes
            else:
                # the main backward kernel writes dx; dgamma/dbeta (2*C*4 bytes) are
                # written by the small column-sum kernel when one follows
                nbytes = call_bytes - (2 * wl.C * 4 if plan.kernels > 1 else 0)
            call_ms = [tev.elapsed_ms(*cev[i][k][c]) for i in range(K)]
            kern_ms = [tev.elapsed_ms(*kev[i][k][c]) for i in range(K)]
            call_avg = sum(call_ms) / K
            kern_avg = sum(kern_ms) / K
            # kernels that can be the call's main kernel (the rows path picks one of
            # several by the slice width and count; the grid tells them apart in
            # the recorded counters)
            kname = {("rows", "fwd"): ("rows_fwd_k", "rows_fwd_lds_k", "rows_fwd_narrow_k", "rows_fwd_cs_k"),
                     ("rows", "bwd"): ("rows_bwd_k", "rows_bwd_narrow_k"),
                     ("slab", "fwd"): (f"slab_{wl.layout}_fwd", "small_nchw_fwd"),
                     ("slab", "bwd"): (f"slab_{wl.layout}_bwd", "small_nchw_bwd"),
                     ("stream", "fwd"): ("stream_fwd_call",), ("stream", "bwd"): ("stream_bwd_call",),
                     ("generic", "fwd"): ("generic_fwd_call",), ("generic", "bwd"): ("generic_bwd_call",),
                     }.get((path, kind))
            whole = path in ("stream", "generic")
            calls.append(dict(shape=wl.name, call=kind, path=path, kernels=plan.kernels,
                              kernel=kname, grid=plan.grid if not whole else "call",
                              call_us=call_avg * 1e3, call_bytes=call_bytes,
                              main_kernel_us=kern_avg * 1e3, main_kernel_bytes=nbytes,
                              main_kernel_gbs=nbytes / (kern_avg * 1e-3) / 1e9))
    # ---- small (cache-resident) workloads: the calls again with the caches
    # flushed before each one -- a 512 MiB scratch fill outside the library's
    # events -- so that each call reads its inputs from HBM ----------------------
    flushed = None
    if mode == "graph":
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        reps = min(K, 20)
        fev = [[[ev_pair() for _ in range(2)] for _ in shapes] for _ in range(reps)]
        for i in range(reps):
            for k, sh in enumerate(shapes):
                for call in calls_for(sh, sp, [(fev[i][k][0], None), (fev[i][k][1], None)]):
                    scratch.fill_(i & 0xFF)
                    run([call])
        torch.cuda.synchronize()
        flushed = {}
        for k, sh in enumerate(shapes):
            for c, kind in enumerate(("fwd", "bwd")):
                d = [tev.elapsed_ms(*fev[i][k][c]) for i in range(reps)]
                flushed[f"{kind}:{sh['wl'].name}"] = round(1e3 * sum(d) / len(d), 3)
        del scratch
    tev.close()
    if graph is not None:
        del graph
    wl0 = shapes[0]["wl"]
    desc = [dict(N=s["wl"].N, C=s["wl"].C, H=s["wl"].H, W=s["wl"].W, G=s["wl"].G, dtype=s["wl"].dtype,
                 layout=s["wl"].layout,
                 **({"view": f"centre crop of ({s['wl'].H + 2 * s['wl'].crop}, "
                             f"{s['wl'].W + 2 * s['wl'].crop}) images"} if s["wl"].crop else {}))
            for s in shapes]
    return dict(mode=mode, ms_per_step=ms_per_step, bytes_per_step=bytes_per_step, calls=calls, flushed=flushed,
                shapes=shapes if keep_inputs else None, shape_desc=desc, dtype=wl0.dtype, op=wl0.op,
                mask="dx|dgamma" if wl0.op == "rms" else "dx|dgamma|dbeta")


# Rows shapes of the LayerNorm / RMSNorm backward table in ROCm/pytorch PR
# #3564 (MI350X, "Tiled+Two-pass" and "Tiled only" columns, in microseconds),
# for context on other hardware.
ROWS_SWEEP = [  # (op, N, C, dtype, pages' tiled+two-pass us, pages' tiled-only us)
    ("gn", 32, 512, "f16", 8.16, 7.94), ("gn", 96, 768, "f16", 20.78, 20.71),
    ("gn", 192, 1024, "bf16", 8.51, 8.20), ("gn", 4096, 1024, "f16", 13.12, 31.07),
    ("gn", 1024, 768, "f16", 11.05, 11.15), ("gn", 4096, 1024, "bf16", 13.10, 31.28),
    ("gn", 4096, 1024, "f32", 15.90, 30.87), ("gn", 131072, 64, "f16", 27.70, 26.48),
    ("gn", 131072, 4096, "bf16", 513.38, 509.65), ("gn", 8192, 768, "f16", 16.56, 58.22),
    ("rms", 4096, 1024, "f16", 11.18, 22.34), ("rms", 131072, 4096, "bf16", 476.03, 476.18),
    ("rms", 131072, 64, "f16", 17.29, 16.73),
]


def rows_sweep(K):
    """Forward, full backward and gamma/beta-only backward of every ROWS_SWEEP
    shape, each as a HIP graph of K back-to-back calls timed with events around
    the replay; one JSON line per shape (microseconds per call)."""
    import torch

    import normalization_gn_stats_amd as gn
    from normalization_gn_stats_amd import inputs

    dev = torch.device("cuda", 0)

    def per_call_us(fn):
        fn(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            h = torch.cuda.current_stream().cuda_stream
            for _ in range(K):
                fn(h)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) * 1e3 / K, 2)

    for op, N, C, dt, pages_2p, pages_tiled in ROWS_SWEEP:
        name = f"{op}_{dt}_{N}x{C}"
        log(f"rows sweep: {name}")
        wl = inputs.Workload(name, N, C, 1, 1, 1, dt, "nchw", eps=1e-6 if op == "rms" else 1e-5, op=op)
        d = inputs.make_inputs(wl, seed=0, device="cuda")
        code = {"f32": 0, "f16": 1, "bf16": 2}[dt]
        x, dy = d["x"].reshape(N, C), d["dy"].reshape(N, C)
        y, dx = torch.empty_like(x), torch.empty_like(x)
        mean, rstd = torch.empty(N, device=dev), torch.empty(N, device=dev)
        dg, db = torch.empty(C, device=dev), torch.empty(C, device=dev)

        def ws(nbytes):
            return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

        res = {"shape": name, "unit": "us/call"}
        if op == "gn":
            x4, dy4, y4, dx4 = (t.reshape(N, C, 1, 1) for t in (x, dy, y, dx))
            fws = ws(gn.forward_workspace_size(N, C, 1, 1, code, gn._lib.GN_NCHW))
            res["fwd"] = per_call_us(lambda h: gn.forward_into(x4, d["gamma"], d["beta"], 1, wl.eps, y4, mean, rstd,
                                                               fws, stream=h))
            masks = (("bwd", 7), ("bwd_dgamma_dbeta", 6))
            for key, mask in masks:
                bws = ws(gn.backward_workspace_size(N, C, 1, 1, code, gn._lib.GN_NCHW, mask))
                res[key] = per_call_us(lambda h: gn.backward_into(dy4, x4, mean, rstd, d["gamma"], 1, mask, dx4, dg,
                                                                  db, bws, stream=h))
        else:
            fws = ws(gn.rms_forward_workspace_size(N, C, 1, code))
            res["fwd"] = per_call_us(lambda h: gn.rms_forward_into(x, d["gamma"], 1, wl.eps, y, rstd, fws,
                                                                   stream=h))
            for key, mask in (("bwd", 3), ("bwd_dgamma", 2)):
                bws = ws(gn.rms_backward_workspace_size(N, C, 1, code, mask))
                res[key] = per_call_us(lambda h: gn.rms_backward_into(dy, x, rstd, d["gamma"], 1, mask, dx, dg, bws,
                                                                      stream=h))
        res["pages_mi350x_tiled_two_pass"] = pages_2p
        res["pages_mi350x_tiled_only"] = pages_tiled
        print(json.dumps(res), flush=True)
        del d, x, dy, y, dx
        torch.cuda.empty_cache()


def cpu_baseline(shapes, seconds, bytes_per_step):
    """The fp64 oracle (as it stands) on a bounded sample of the workload:
    whole samples n = 0, 1, ... of each shape (a sample is its own GroupNorm
    problem, N = 1 ... k), copied to the host and widened to float64 outside
    the timer, forward and backward, until about `seconds` of oracle time.
    Reported in the metric's unit: algorithmic GB/s of the samples done."""
    import numpy as np
    import torch

    import oracle

    log("cpu baseline: oracle on the host cores")
    threads = oracle.num_threads()
    done_bytes, elapsed, samples, calls = 0, 0.0, 0, 0
    per_shape = []
    for sh in shapes:
        wl = sh["wl"]
        # samples per oracle call: enough slices to occupy every thread
        chunk = max(1, min(wl.N, -(-2 * threads // wl.G)))
        frac = chunk / wl.N
        nbytes = (wl.fwd_min_bytes() + wl.bwd_min_bytes()) * frac   # this chunk's share of the step
        g = sh["gamma"].double().cpu().numpy()
        b = sh["beta"].double().cpu().numpy()
        eps = float(np.float32(wl.eps))
        per_shape.append((wl, chunk, nbytes, g, b, eps))
    budget = seconds / len(per_shape)
    for (wl, chunk, nbytes, g, b, eps), sh in zip(per_shape, shapes):
        t_shape = 0.0
        n0 = 0
        while t_shape < budget and n0 < wl.N:
            n1 = min(wl.N, n0 + chunk)
            xs = sh["x"][n0:n1]
            dys = sh["dy"][n0:n1]
            from normalization_gn_stats_amd import inputs
            x64 = inputs.memory_image(xs, wl.layout).to("cpu", torch.float64).numpy()
            dy64 = inputs.memory_image(dys, wl.layout).to("cpu", torch.float64).numpy()
            nn = n1 - n0
            t0 = time.perf_counter()
            if wl.op == "rms":
                oracle.rms_forward(x64, g, nn, wl.C, wl.G, eps)
                oracle.rms_backward(dy64, x64, g, nn, wl.C, wl.G, eps)
            else:
                oracle.forward(x64, g, b, nn, wl.C, wl.HW, wl.G, eps, layout=wl.layout)
                oracle.backward(dy64, x64, g, nn, wl.C, wl.HW, wl.G, eps, layout=wl.layout)
            dt = time.perf_counter() - t0
            t_shape += dt
            elapsed += dt
            done_bytes += nbytes * nn / chunk
            samples += nn
            calls += 1
            n0 = n1
            if n0 >= wl.N:
                n0 = 0   # small workloads: repeat the whole tensor
                if t_shape >= budget:
                    break
    wl0 = shapes[0]["wl"]
    return {"value": round(done_bytes / elapsed / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{samples} samples (n = 0, 1, ...) of {', '.join(s['wl'].name for s in shapes)} "
                       f"in {calls} oracle calls of up to {per_shape[0][1]} samples ({per_shape[0][1] * wl0.G} "
                       f"slices), forward + backward, {elapsed:.1f} s of fp64 C oracle time "
                       f"(host copies and widening excluded); {threads} OpenMP threads on {os.cpu_count()} host "
                       f"cpus, {cpu_model()}")}


# The oracle per benchmark configuration: (config, workload, sample shape or
# None for the whole workload, what the sample is).  The large configurations
# run on a sample of the same kind, whose time scales with its bytes.
ORACLE_SWEEP = (
    ("1", "tiny_nchw_f32_2x32x16x16_g8", None, "the whole workload"),
    ("2", "rows_f16_4096x1024", None, "the whole workload"),
    ("2", "rows_f16_8192x768", None, "the whole workload"),
    ("3", "nhwc_f16_1x128x1024x2048_g16", dict(H=128), "a 1x128x128x2048 image (1/8 of its rows)"),
    ("4", "nchw_f32_112x64x512x512_g8", dict(N=4), "4 of its 112 samples"),
    ("5", "rows_bf16_131072x4096", dict(N=16384), "16384 of its 131072 rows"),
)


def oracle_sweep():
    """The fp64 C oracle (as it stands) on the host cores, forward and
    backward timed separately around the oracle calls only (inputs generated
    and widened to float64 beforehand): the median of 10 runs for the small
    configurations, also on one thread, and of 3 for the large ones.  One JSON
    line per configuration shape; GB/s are algorithmic bytes of the timed
    problem, and the full configuration's time is scaled from them."""
    import statistics

    import numpy as np
    import torch

    import oracle
    from normalization_gn_stats_amd import inputs

    threads = oracle.num_threads()
    for label, name, sample, what in ORACLE_SWEEP:
        full = inputs.WORKLOADS[name]
        wl = full.scaled(**sample) if sample else full
        d = inputs.make_inputs(wl, seed=0)
        x64 = inputs.memory_image(d["x"], wl.layout).to(torch.float64).numpy()
        dy64 = inputs.memory_image(d["dy"], wl.layout).to(torch.float64).numpy()
        g = d["gamma"].double().numpy()
        b = d["beta"].double().numpy()
        eps = float(np.float32(wl.eps))
        reps = 10 if sample is None else 3
        for nthreads in ((threads, 1) if sample is None else (threads,)):
            oracle.set_num_threads(nthreads)
            tf, tb = [], []
            for _ in range(reps):
                t0 = time.perf_counter()
                oracle.forward(x64, g, b, wl.N, wl.C, wl.HW, wl.G, eps, layout=wl.layout)
                t1 = time.perf_counter()
                oracle.backward(dy64, x64, g, wl.N, wl.C, wl.HW, wl.G, eps, layout=wl.layout)
                t2 = time.perf_counter()
                tf.append(t1 - t0)
                tb.append(t2 - t1)
            f, bw = statistics.median(tf), statistics.median(tb)
            scale_f = full.fwd_min_bytes() / wl.fwd_min_bytes()
            scale_b = full.bwd_min_bytes() / wl.bwd_min_bytes()
            print(json.dumps({"config": label, "workload": name, "timed": what, "threads": nthreads,
                              "runs": reps, "fwd_ms": round(f * 1e3, 3), "bwd_ms": round(bw * 1e3, 3),
                              "fwd_gbs": round(wl.fwd_min_bytes() / f / 1e9, 3),
                              "bwd_gbs": round(wl.bwd_min_bytes() / bw / 1e9, 3),
                              "full_fwd_ms": round(f * scale_f * 1e3, 2), "full_bwd_ms": round(bw * scale_b * 1e3, 2),
                              "cpu": f"{os.cpu_count()} host cpus, {cpu_model()}"}), flush=True)
        oracle.set_num_threads(threads)


if __name__ == "__main__":
    main()
