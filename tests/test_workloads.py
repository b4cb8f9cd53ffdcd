"""Workload shapes agree with the cases the pages fix (tests/golden/page_cases.json)."""
import json
import os

from normalization_gn_stats_amd import inputs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_cases.json")))


def test_nhwc_workload_is_the_apex_reproducer():
    g = GOLD["apex_pr2018_reproducer"]
    w = inputs.NHWC_IMG
    assert (w.N, w.C, w.G, w.H, w.W, w.dtype, w.layout, w.eps) == (
        g["N"], g["C"], g["G"], g["H"], g["W"], g["dtype"], g["layout"], g["eps"])
    assert w.affine == "n01"  # weight and bias drawn with randn there


def test_nchw_workload_is_the_popcornbench_problem():
    g = GOLD["popcornbench_groupnorm_forward"]
    w = inputs.NCHW_BIG
    assert (w.N, w.C, w.G, w.H, w.W, w.dtype, w.layout) == (g["N"], g["C"], g["G"], g["H"], g["W"], g["dtype"], g["layout"])


def test_row_workloads_are_the_rocm_table_shapes():
    g = GOLD["rocm_pytorch_3564_shapes"]
    for w, key in ((inputs.ROWS_A, "tile256_large"), (inputs.ROWS_B, "gpt2_style"), (inputs.ROWS_BIG, "llm_hidden_4096"),
                   (inputs.ROWS_NARROW, "two_pass_huge_M")):
        assert (w.N, w.C, w.dtype, w.G, w.HW) == (g[key]["rows"], g[key]["cols"], g[key]["dtype"], 1, 1)


def test_rms_workloads_are_the_rocm_table_shapes():
    g = GOLD["rocm_pytorch_3564_shapes"]
    for w, key in ((inputs.RMS_A, "rms_tile256"), (inputs.RMS_BIG, "rms_llm"), (inputs.RMS_NARROW, "rms_two_pass")):
        assert (w.N, w.C, w.dtype, w.G, w.HW, w.op) == (g[key]["rows"], g[key]["cols"], g[key]["dtype"], 1, 1, "rms")
        assert g[key]["op"] == "rms_norm"
    w = inputs.RMS_A
    assert w.fwd_min_bytes() == 2 * w.E * 2 + w.C * 4 + w.N * 4
    assert w.bwd_min_bytes() == 3 * w.E * 2 + w.C * 4 + w.N * 4 + w.C * 4


def test_inputs_are_seeded_and_quantised():
    w = inputs.TINY
    a = inputs.make_inputs(w, seed=0)
    b = inputs.make_inputs(w, seed=0)
    for k in a:
        assert (a[k] == b[k]).all()
    assert a["x"].dtype == w.torch_dtype and a["gamma"].dtype.is_floating_point
    n = inputs.make_inputs(inputs.Workload("t", 2, 8, 3, 5, 2, "f16", "nhwc"), seed=1)
    assert n["x"].is_contiguous(memory_format=__import__("torch").channels_last)


def test_min_bytes_formula():
    w = inputs.NHWC_IMG
    assert w.fwd_min_bytes() == 2 * w.E * 2 + 2 * 128 * 4 + 2 * 16 * 4
    assert w.bwd_min_bytes() == 3 * w.E * 2 + 128 * 4 + 2 * 16 * 4 + 2 * 128 * 4
