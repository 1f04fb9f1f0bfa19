"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the choice of the roofline kernel, and
the per-launch statistics.  The plan query behind the kernel names is host code in the library."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import fp8_blockwise_quantized_amd as fq  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       env=dict(os.environ, **env), timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _decoder_like_ops():
    """fprop, dgrad and wgrad of two 16384-token linears whose fprop and dgrad plans are unsplit
    256x256 tiles; the wgrad of the first is split (that call also launches a reduction pass)."""
    ops = []
    for name, K, N in [("a", 2048, 2560), ("b", 2048, 11264)]:
        M = 16384
        f = 2 * M * N * K
        ops += [dict(name=f"{name}.quant", kind="quant_dual", flops=0, bytes=M * K * 4),
                dict(name=f"{name}.fprop", kind="fprop", flops=f, bytes=0, plan=(fq.OP_FPROP, M, N, K), kid=(0, 0)),
                dict(name=f"{name}.dgrad", kind="dgrad", flops=f, bytes=0, plan=(fq.OP_DGRAD_WT, M, N, K), kid=(1, 0)),
                dict(name=f"{name}.wgrad", kind="wgrad", flops=f, bytes=0, plan=(fq.OP_WGRAD, M, N, K), kid=(2, 1))]
    return ops


def test_roofline_kernel_is_the_one_with_most_time():
    ops = _decoder_like_ops()
    # dgrad slower than fprop: the dgrad symbol carries the most time; faster: the fprop symbol
    for scale, kop, names in ((1.3, 1, ["a.dgrad", "b.dgrad"]), (0.7, 0, ["a.fprop", "b.fprop"])):
        dur = [0.05 if o["kind"] == "quant_dual" else (0.2 * scale if o["kind"] == "dgrad" else 0.2) for o in ops]
        r = bench.roofline(fq, ops, dur, with_traffic=False)
        assert r["kernel"].startswith(f"void fp8bq::gemm_tn_kernel<{kop}, 256, 256, 2, 4, 2, 0, ")
        assert r["launches"] == names
        fl = sum(o["flops"] for o in ops if o["name"] in names) / 2
        ms = 0.2 * (scale if kop == 1 else 1.0)
        assert r["flops_per_launch"] == fl
        assert abs(r["achieved"] - round(fl / (ms * 1e-3) / 1e12, 1)) < 0.05
        assert abs(r["frac"] - r["achieved"] / bench.FP8_PEAK_TFLOPS) < 1e-4


def test_split_calls_are_left_out_of_the_kernel_but_counted_in_their_kind():
    ops = _decoder_like_ops()
    # only the wgrads carry time: the split call (a.wgrad, GEMM + reduction pass) cannot stand for its
    # kernel, the unsplit one (b.wgrad) can; the wgrad kind counts both
    dur = [1.0 if o["kind"] == "wgrad" else 0.1 for o in ops]
    r = bench.roofline(fq, ops, dur, with_traffic=False)
    for name in r["launches"]:
        o = next(x for x in ops if x["name"] == name)
        assert fq.fp8bq_gemm_plan(*o["plan"])[2] == 1
    assert r["launches"] == ["b.wgrad"]
    w = r["by_kind"]["wgrad"]
    fl = sum(o["flops"] for o in ops if o["kind"] == "wgrad")
    assert w["launches"] == 2 and w["with_reduction_pass"] == ["a.wgrad"]
    assert abs(w["achieved"] - round(fl / 2e-3 / 1e12, 1)) < 0.05 and w["unit"] == "TFLOP/s"
    assert set(r["by_kind"]) == {"fprop", "dgrad", "wgrad", "quantize"}
    q = r["by_kind"]["quantize"]
    assert q["bound"] == "hbm" and q["peak"] == bench.HBM_PEAK_GBS and "copy_gbs" not in q
    r2 = bench.roofline(fq, ops, dur, with_traffic=False, copy_gbs=6000.0, torch_copy_gbs=5000.0)
    q2 = r2["by_kind"]["quantize"]
    assert abs(q2["frac_of_copy"] - q2["achieved"] / 6000.0) < 1e-4 and q2["torch_copy_gbs"] == 5000.0


def test_per_launch_statistics():
    ops = _decoder_like_ops()[:2]
    mean, med, mn = [0.05, 0.2], [0.049, 0.19], [0.048, 0.18]
    b = bench.summarize(ops, mean, med, mn)
    assert b["per_launch"][1] == {"op": "a.fprop", "ms": 0.2, "ms_median": 0.19, "ms_min": 0.18,
                                  "tflops": round(ops[1]["flops"] / 0.2e-3 / 1e12, 1)}
    assert b["fprop"]["launches"] == 1 and b["quant_dual"]["gbs"] == round(ops[0]["bytes"] / 0.05e-3 / 1e9, 1)


def test_planner_summary_compares_like_with_like():
    """The planner check counts a product as planned well when the forced run with the planner's own
    plan is within 3% of the fastest forced run (so noise between processes does not count); the
    planner's own timing only stands in when no forced tile reproduces its plan."""
    n = len(bench.PLANNER_SHAPES)
    tiles = {"64x64": [64, 64, 1], "128x128": [128, 128, 1], "256x256": [256, 256, 1]}
    got = {name: [{"plan": plan, "us": 10.0} for _ in range(n)] for name, plan in tiles.items()}
    got["planner"] = [{"plan": [128, 128, 1], "us": 12.0} for _ in range(n)]  # slower process, same plan
    got["64x64"][0]["us"] = 9.0       # product 0: a faster tile than the planned one (11% off)
    got["256x256"][1]["us"] = 9.8     # product 1: faster by 2%, still within 3%
    got["planner"][2]["plan"] = [32, 32, 1]  # product 2: no forced tile has that plan -> planner's time
    value, points = bench.planner_summary(got)
    assert points[0]["fastest_forced"] == "64x64" and points[0]["planned_tile"] == "128x128"
    assert abs(points[0]["planner_over_fastest"] - 10.0 / 9.0) < 1e-3
    assert points[1]["planner_over_fastest"] == round(10.0 / 9.8, 3)
    assert points[2]["planned_tile"] is None and points[2]["planner_over_fastest"] == 1.2
    assert all(p["planner_over_fastest"] == 1.0 for p in points[3:])
    assert value == round((n - 2) / n, 3)
