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
    256x256 tiles; the wgrad of the first is split (so its kernel is not isolated)."""
    ops = []
    for name, K, N in [("a", 2048, 2560), ("b", 2048, 11264)]:
        M = 16384
        f = 2 * M * N * K
        ops += [dict(name=f"{name}.quant", kind="quant_dual", flops=0, bytes=M * K * 4),
                dict(name=f"{name}.fprop", kind="fprop", flops=f, bytes=0, plan=(fq.OP_FPROP, M, N, K), kid=(0, 0)),
                dict(name=f"{name}.dgrad", kind="dgrad", flops=f, bytes=0, plan=(fq.OP_DGRAD_WT, M, N, K), kid=(1, 0)),
                dict(name=f"{name}.wgrad", kind="wgrad", flops=f, bytes=0, plan=(fq.OP_WGRAD, M, N, K), kid=(2, 1))]
    return ops


def test_roofline_kernel_is_chosen_by_flops_not_timing():
    ops = _decoder_like_ops()
    # dgrad launches slower than fprop, then faster: the choice stays on the first symbol in step order
    for scale in (1.3, 0.7):
        dur = [0.05 if o["kind"] == "quant_dual" else (0.2 * scale if o["kind"] == "dgrad" else 0.2) for o in ops]
        r = bench.roofline(fq, ops, dur, with_traffic=False)
        assert r["kernel"].startswith("void fp8bq::gemm_tn_kernel<0, 256, 256, 2, 4, 2, 0, ")
        assert r["launches"] == ["a.fprop", "b.fprop"]
        fl = sum(o["flops"] for o in ops if o["kind"] == "fprop") / 2
        assert r["flops_per_launch"] == fl
        assert abs(r["achieved"] - round(fl / 0.2e-3 / 1e12, 1)) < 0.05
        assert abs(r["frac"] - r["achieved"] / bench.FP8_PEAK_TFLOPS) < 1e-4


def test_split_symbol_is_not_eligible():
    ops = _decoder_like_ops()
    # only the wgrads carry time: the wgrad symbol of the split call is excluded, the other one is not
    # eligible either if any call of it splits; the result falls back to an isolated symbol
    dur = [1.0 if o["kind"] == "wgrad" else 0.1 for o in ops]
    r = bench.roofline(fq, ops, dur, with_traffic=False)
    for name in r["launches"]:
        o = next(x for x in ops if x["name"] == name)
        assert fq.fp8bq_gemm_plan(*o["plan"])[2] == 1


def test_per_launch_statistics():
    ops = _decoder_like_ops()[:2]
    mean, med, mn = [0.05, 0.2], [0.049, 0.19], [0.048, 0.18]
    b = bench.summarize(ops, mean, med, mn)
    assert b["per_launch"][1] == {"op": "a.fprop", "ms": 0.2, "ms_median": 0.19, "ms_min": 0.18,
                                  "tflops": round(ops[1]["flops"] / 0.2e-3 / 1e12, 1)}
    assert b["fprop"]["launches"] == 1 and b["quant_dual"]["gbs"] == round(ops[0]["bytes"] / 0.05e-3 / 1e9, 1)
