#!/usr/bin/env python3
"""Benchmark of the FP8 blockwise-quantized linear layer's hot path on one MI355X.

One step = the whole path for one synthetic 2B-class decoder block at M = 16384 tokens (hidden
2048; QKV 2048->2560, O 2048->2048, gate+up 2048->11264, down 5632->2048).  Per linear:
    quantize X both ways (1x128 for fprop, 128x1 for wgrad) in one pass, quantize W 128x128
    (codes also written transposed for dgrad), fprop Y = X W^T,
    quantize dY both ways in one pass, dgrad dX = dY W, wgrad dW = dY^T X
i.e. 12 quantize passes and 12 GEMMs, all E4M3, BF16 in and out, inputs resident in HBM.

    python bench.py [--steps K] [--warmup W] [--workload decoder|delayed|hyperball|linear|sweep|qerror]
                    [--no-cpu-baseline]

`--workload delayed` runs the same decoder-block step with per-tensor delayed scaling instead (one
running amax and one scale per tensor, X / W / dY each quantized once with transposed codes, the
three GEMMs with per-tensor scales): the pages' own alternative recipe, as a comparison point.
`--workload qerror` is not a timing: on the heavy-tailed gradient workload it reports the relative
Frobenius error of dgrad and wgrad against float64 products of the unquantized BF16 inputs, with dY
in E5M2 and in E4M3 (sampled rows / columns).
`--workload hyperball` times the Hyperball update (with the fixed-radius projection) of the decoder
block's four FP32 master weights from BF16 gradients, and reports GB/s.
`--workload planner` checks the tile planner: each GEMM of a fixed list (small-token fprops and
dgrads, split and decoder-block wgrads) is timed under the library's plan and under every tile shape
forced in turn (one child process per tile, since the override is read once per process), and the
line reports for how many the planned tile (timed with the forced runs) is within 3% of the fastest.

Prints ONE JSON line on stdout.  `value` = GEMM FLOPs of the step / wall time of the step (the
quantize passes are inside the timed step).  `breakdown` holds per-product TFLOP/s and per-pass GB/s
from HIP events recorded on the launch stream.  `roofline` is for the GEMM kernel with the most time
per step, with `by_kind` entries for fprop, dgrad, wgrad (each against the FP8 peak) and the quantize
passes (against HBM, beside the same run's streaming-copy and torch-copy bandwidths; `scrubbed` times
each quantize launch again on its own after a 512 MiB read that evicts the caches, so that no launch
reads from the caches or pays for the write-back of an earlier kernel's output, each beside a streaming
copy of its own byte count timed the same way).  After the timed steps, `configs`
times the other workloads: the single 8192 x 8192 x 2048 linear, the token sweep K = N = 2048 with its
knee, and the heavy-tailed gradients (dgrad / wgrad with dY in E5M2 and E4M3, and their quantization
error).  `cpu_baseline` times the CPU oracle on a bounded sample of the same path (first 4096 tokens)
and, per workload and operation, quantize GB/s and GEMM GFLOP/s on samples.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, published
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
METRIC = "FP8 blockwise GEMM TFLOP/s (fprop/dgrad/wgrad) + % of MI355X FP8 peak; quant GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", choices=["decoder", "delayed", "hyperball", "linear", "sweep", "qerror",
                                          "planner", "planner-child"], default="decoder")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the single-linear, token-sweep and heavy-tailed workloads after the decoder step")
    p.add_argument("--cpu-tokens", type=int, default=4096)
    p.add_argument("--calibrate", action="store_true",
                   help="first run one plain elementwise kernel over 256 MiB in / 256 MiB out, so a "
                        "rocprofv3 counter run can scale FETCH_SIZE / WRITE_SIZE")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the GEMMs would shard by tokens, with one all-reduce of dW per step).", file=sys.stderr)
        sys.exit(2)

    if args.workload == "planner":
        return run_planner(args)  # spawns the timing children before this process touches the GPU

    import numpy as np
    import torch

    import fp8_blockwise_quantized_amd as fq
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fq.lib()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate:
        a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)  # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del a, b

    if args.workload == "decoder":
        ops, bufs, desc = build_decoder(torch, fq, synth, dev)
    elif args.workload == "delayed":
        ops, bufs, desc = build_delayed(torch, fq, synth, dev)
    elif args.workload == "hyperball":
        return run_hyperball(args, torch, fq, synth, dev)
    elif args.workload == "qerror":
        return run_qerror(torch, fq, synth, dev)
    elif args.workload == "linear":
        ops, bufs, desc = build_linear(torch, fq, synth, dev)
    elif args.workload == "planner-child":
        return run_planner_child(args, torch, fq, synth, dev)
    else:
        return run_sweep(args, torch, fq, synth, dev)

    step_flops = sum(o["flops"] for o in ops)
    step_bytes = sum(o["bytes"] for o in ops)
    stream = torch.cuda.current_stream(dev)

    def step(record=None):
        for i, o in enumerate(ops):
            if record is not None:
                record[i][0].record(stream)
            o["fn"]()
            if record is not None:
                record[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, wall clock, synchronized on both sides
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps

    # per-launch durations with HIP events on the launch stream (separate pass over the same steps)
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in ops]
          for _ in range(args.steps)]
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    per = np.array([[ev[k][i][0].elapsed_time(ev[k][i][1]) for i in range(len(ops))] for k in range(args.steps)])
    dur_ms = per.mean(axis=0)  # mean per launch

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    breakdown = summarize(ops, dur_ms, np.median(per, axis=0), per.min(axis=0))
    copies = copy_ceiling(torch, fq, dev) if args.workload == "decoder" else {}
    roof = roofline(fq, ops, dur_ms, with_traffic=args.workload == "decoder", copy_gbs=copies.get("stream"),
                    torch_copy_gbs=copies.get("torch"))
    if roof and "quantize" in roof["by_kind"] and args.workload == "decoder":
        roof["by_kind"]["quantize"]["scrubbed"] = quant_scrubbed(torch, dev, ops, copies.get("stream"), fq=fq)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded, shapes and distributions of the workload)",
        "config": dict(desc, accumulate="fp32", inputs_and_outputs="bf16"),
        "step_gemm_flops": step_flops,
        "step_quant_bytes": step_bytes,
        "pct_fp8_peak_step": round(100 * value / FP8_PEAK_TFLOPS, 2),
        "breakdown": breakdown,
        "roofline": roof,
        "cpu_baseline": None,
    }
    del bufs
    if args.workload == "decoder" and not args.no_configs:
        out["configs"] = run_configs(torch, fq, synth, dev, steps=min(args.steps, 20))
    if not args.no_cpu_baseline and args.workload == "decoder":
        out["cpu_baseline"] = cpu_baseline(args.cpu_tokens, desc)
    print(json.dumps(out), flush=True)


# -----------------------------------------------------------------------------------------------
# workloads
# -----------------------------------------------------------------------------------------------

def _q1x128_bytes(R, C, in_bytes=2):
    return R * C * in_bytes + R * C + R * (C // 128) * 4


def _q128x1_bytes(R, C, in_bytes=2):
    return R * C * in_bytes + R * C + (R // 128) * C * 4


def _qw_bytes(N, K, in_bytes=2):
    return N * K * in_bytes + N * K + (N // 128) * (K // 128) * 4


def _alloc_1x128(torch, R, C, dev):
    return (torch.empty((R, C), dtype=torch.uint8, device=dev),
            torch.empty((C // 128, (R + 3) // 4 * 4), dtype=torch.float32, device=dev)[:, :R])


def _alloc_128x1(torch, R, C, dev):
    return (torch.empty((C, R), dtype=torch.uint8, device=dev),
            torch.empty((R // 128, (C + 3) // 4 * 4), dtype=torch.float32, device=dev)[:, :C])


def _qdual_bytes(R, C, in_bytes=2):
    return R * C * in_bytes + 2 * R * C + R * (C // 128) * 4 + (R // 128) * C * 4


def linear_ops(torch, fq, name, X, W, dY, dev, with_backward=True, weight_jobs=None):
    """Closures for one linear's hot path; every output buffer is preallocated.  With the backward
    pass, X and dY are each quantized both ways (1x128 and 128x1) in one pass.  With weight_jobs (a
    list), W's quantization (codes, scales, W^T codes) is appended there as a job of one batched launch
    for all weights instead of being an op of this linear."""
    M, K = X.shape
    N = W.shape[0]
    E4 = fq.E4M3
    qx, sx = _alloc_1x128(torch, M, K, dev)
    qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws_f = fq._workspace(fq.OP_FPROP, M, N, K, dev)
    bufs = [qx, sx, qw, sw, y, ws_f]
    if with_backward:
        qxt, sxt = _alloc_128x1(torch, M, K, dev)
        qwt = torch.empty((K, N), dtype=torch.uint8, device=dev)
        bufs += [qxt, sxt, qwt]
        quant_x = dict(name=f"{name}.quant_x_dual", kind="quant_dual", bytes=_qdual_bytes(M, K), flops=0,
                       fn=fq.prepare(fq.fp8bq_quantize_act_dual, X, E4, qx, sx, E4, qxt, sxt))
        quant_w = dict(name=f"{name}.quant_w_dual", kind="quant_w_dual", bytes=_qw_bytes(N, K) + N * K, flops=0,
                       fn=fq.prepare(fq.fp8bq_quantize_weight_dual, W, E4, qw, sw, qwt))
    else:
        quant_x = dict(name=f"{name}.quant_x_1x128", kind="quant_1x128", bytes=_q1x128_bytes(M, K), flops=0,
                       fn=fq.prepare(fq.fp8bq_quantize_act_1x128, X, E4, qx, sx))
        quant_w = dict(name=f"{name}.quant_w_128x128", kind="quant_128x128", bytes=_qw_bytes(N, K), flops=0,
                       fn=fq.prepare(fq.fp8bq_quantize_weight_128x128, W, E4, qw, sw))
    if weight_jobs is not None and with_backward:
        weight_jobs.append((W, qw, sw, qwt))
        quant_w = None
    ops = [op for op in (quant_x, quant_w) if op is not None] + [
        dict(name=f"{name}.fprop", kind="fprop", bytes=0, flops=2 * M * N * K, plan=(fq.OP_FPROP, M, N, K), kid=(0, 0),
             fn=fq.prepare(fq.fp8bq_gemm_fprop, qx, sx, E4, qw, sw, E4, y, ws_f)),
    ]
    if with_backward:
        qdy, sdy = _alloc_1x128(torch, M, N, dev)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        qdyt, sdyt = _alloc_128x1(torch, M, N, dev)
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        ws_d = fq._workspace(fq.OP_DGRAD_WT, M, N, K, dev)
        ws_w = fq._workspace(fq.OP_WGRAD, M, N, K, dev)
        ops += [
            dict(name=f"{name}.quant_dy_dual", kind="quant_dual", bytes=_qdual_bytes(M, N), flops=0,
                 fn=fq.prepare(fq.fp8bq_quantize_act_dual, dY, E4, qdy, sdy, E4, qdyt, sdyt)),
            dict(name=f"{name}.dgrad", kind="dgrad", bytes=0, flops=2 * M * N * K, plan=(fq.OP_DGRAD_WT, M, N, K),
                 kid=(1, 0), fn=fq.prepare(fq.fp8bq_gemm_dgrad_wt, qdy, sdy, E4, qwt, sw, E4, dx, ws_d)),
            dict(name=f"{name}.wgrad", kind="wgrad", bytes=0, flops=2 * M * N * K, plan=(fq.OP_WGRAD, M, N, K),
                 kid=(2, 1), fn=fq.prepare(fq.fp8bq_gemm_wgrad, qdyt, sdyt, E4, qxt, sxt, E4, dw, ws_w)),
        ]
        bufs += [qdy, sdy, dx, qdyt, sdyt, dw, ws_d, ws_w]
    return ops, bufs


def build_decoder(torch, fq, synth, dev):
    log("generating the decoder-block inputs ...")
    ops, bufs, wjobs = [], [], []
    for name, K, N in synth.DECODER_LINEARS:
        c = synth.decoder_linear(name)
        X, W, dY = c["X"].to(dev), c["W"].to(dev), c["dY"].to(dev)
        o, b = linear_ops(torch, fq, name, X, W, dY, dev, weight_jobs=wjobs)
        ops += o
        bufs += b + [X, W, dY]
    # all four weights are known when the step starts: one launch quantizes them (codes, scales, W^T codes)
    wbytes = sum(_qw_bytes(*w.shape) + w.numel() for w, _, _, _ in wjobs)
    ops.insert(0, dict(name="weights.quant_w_dual", kind="quant_w_dual", bytes=wbytes, flops=0,
                       fn=fq.prepare(fq.fp8bq_quantize_weights_dual, wjobs, fq.E4M3)))
    desc = {
        "workload": "decoder block fprop+dgrad+wgrad, M=16384 tokens, hidden 2048, GQA 16q/2kv x128 "
                    "(QKV 2048->2560, O 2048->2048), SwiGLU gate+up 2048->11264, down 5632->2048; "
                    "E4M3 act 1x128 / weight 128x128 / wgrad 128x1 (X and dY quantized both ways in one pass "
                    "each, the four weights with their W^T codes in one launch); BF16 in/out",
        "tokens": synth.DECODER_M,
        "linears": [[n, k, nn] for n, k, nn in synth.DECODER_LINEARS],
        "gemms_per_step": 12,
        "quant_passes_per_step": 12,
        "quant_launches_per_step": 9,
    }
    return ops, bufs, desc


def _qtensor_bytes(R, C, transpose, in_bytes=2):
    # algorithmic: one read of the input and the codes (twice with the transposed copy); the
    # kernels read the input a second time, after the whole-tensor amax is known
    return R * C * in_bytes + R * C * (2 if transpose else 1) + 8


def delayed_linear_ops(torch, fq, name, X, W, dY, dev):
    """One linear's step with per-tensor delayed scaling: X, W and dY each quantized once (codes and
    their transpose) against their running amax (beta 0.99), then fprop, dgrad and wgrad as per-tensor
    GEMMs on those codes."""
    M, K = X.shape
    N = W.shape[0]
    E4 = fq.E4M3
    u8 = lambda r, c: torch.empty((r, c), dtype=torch.uint8, device=dev)
    one = lambda: torch.ones(1, dtype=torch.float32, device=dev)
    qx, qxt, qw, qwt, qdy, qdyt = u8(M, K), u8(K, M), u8(N, K), u8(K, N), u8(M, N), u8(N, M)
    ax, aw, ady, sx, sw, sdy = one(), one(), one(), one(), one(), one()
    wsq = torch.empty(max(fq.fp8bq_quantize_tensor_workspace_size(M, max(K, N)), 16), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    ws_f = fq._workspace(fq.OP_TENSOR, M, N, K, dev)
    ws_d = fq._workspace(fq.OP_TENSOR, M, K, N, dev)
    ws_w = fq._workspace(fq.OP_TENSOR, N, K, M, dev)
    ops = [
        dict(name=f"{name}.quant_x_tensor", kind="quant_tensor", bytes=_qtensor_bytes(M, K, True), flops=0,
             fn=fq.prepare(fq.fp8bq_quantize_tensor_delayed, X, E4, ax, 0.99, qx, qxt, sx, wsq)),
        dict(name=f"{name}.quant_w_tensor", kind="quant_tensor", bytes=_qtensor_bytes(N, K, True), flops=0,
             fn=fq.prepare(fq.fp8bq_quantize_tensor_delayed, W, E4, aw, 0.99, qw, qwt, sw, wsq)),
        dict(name=f"{name}.fprop", kind="fprop", bytes=0, flops=2 * M * N * K, plan=(fq.OP_TENSOR, M, N, K),
             kid=(0, 0), fn=fq.prepare(fq.fp8bq_gemm_tensor, qx, sx, E4, qw, sw, E4, y, ws_f)),
        dict(name=f"{name}.quant_dy_tensor", kind="quant_tensor", bytes=_qtensor_bytes(M, N, True), flops=0,
             fn=fq.prepare(fq.fp8bq_quantize_tensor_delayed, dY, E4, ady, 0.99, qdy, qdyt, sdy, wsq)),
        dict(name=f"{name}.dgrad", kind="dgrad", bytes=0, flops=2 * M * N * K, plan=(fq.OP_TENSOR, M, K, N),
             kid=(0, 0), fn=fq.prepare(fq.fp8bq_gemm_tensor, qdy, sdy, E4, qwt, sw, E4, dx, ws_d)),
        dict(name=f"{name}.wgrad", kind="wgrad", bytes=0, flops=2 * M * N * K, plan=(fq.OP_TENSOR, N, K, M),
             kid=(0, 0), fn=fq.prepare(fq.fp8bq_gemm_tensor, qdyt, sdy, E4, qxt, sx, E4, dw, ws_w)),
    ]
    bufs = [qx, qxt, qw, qwt, qdy, qdyt, ax, aw, ady, sx, sw, sdy, wsq, y, dx, dw, ws_f, ws_d, ws_w]
    return ops, bufs


def build_delayed(torch, fq, synth, dev):
    log("generating the decoder-block inputs ...")
    ops, bufs = [], []
    for name, K, N in synth.DECODER_LINEARS:
        c = synth.decoder_linear(name)
        X, W, dY = c["X"].to(dev), c["W"].to(dev), c["dY"].to(dev)
        o, b = delayed_linear_ops(torch, fq, name, X, W, dY, dev)
        ops += o
        bufs += b + [X, W, dY]
    desc = {
        "workload": "decoder block fprop+dgrad+wgrad, M=16384 tokens, shapes as the blockwise step; per-tensor "
                    "delayed scaling (running amax, beta 0.99, one scale per tensor), E4M3, X / W / dY each "
                    "quantized once with transposed codes; BF16 in/out",
        "tokens": synth.DECODER_M,
        "linears": [[n, k, nn] for n, k, nn in synth.DECODER_LINEARS],
        "gemms_per_step": 12,
        "quant_calls_per_step": 12,
    }
    return ops, bufs, desc


def run_hyperball(args, torch, fq, synth, dev):
    """Hyperball update with projection of the four decoder weights (FP32 masters, BF16 gradients),
    all four in one batched call per step (per weight and one call per weight for comparison).
    Algorithmic bytes per element: the norms (of g, of w and of their product) must be known before
    any element is written, so g and w are read once for them (2 + 4) and then read again and w
    written in one update pass (2 + 4 + 4) = 16."""
    import numpy as np
    items = []
    for name, K, N in synth.DECODER_LINEARS:
        w = synth.random_f32((N, K), seed=7 + N, std=0.02).to(dev)
        g = synth.random_bf16((N, K), seed=8 + N, std=1e-3).to(dev)
        radius = float(torch.linalg.vector_norm(w.double()).item())
        norms = torch.empty(2, dtype=torch.float32, device=dev)
        ws = torch.empty(fq.fp8bq_hyperball_workspace_size(N, K), dtype=torch.uint8, device=dev)
        items.append((name, w, g, radius, norms, ws, 16 * N * K))

    calls = [fq.prepare(fq.fp8bq_hyperball_step, w, g, 1e-4, 0.1, 1e-8, radius, norms, ws)
             for _, w, g, radius, norms, ws, _ in items]
    wsb = torch.empty(fq.fp8bq_hyperball_batch_workspace_size(len(items)), dtype=torch.uint8, device=dev)
    batched = fq.prepare(fq.fp8bq_hyperball_step_batch, [(w, g, radius, norms) for _, w, g, radius, norms, _, _ in items],
                         1e-4, 0.1, 1e-8, wsb)

    def one_by_one():
        for c in calls:
            c()

    def timed(step):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / args.steps

    ms = timed(batched)  # the step: all four weights in one batched call (two launches)
    ms_single = timed(one_by_one)  # for comparison: one call (two launches) per weight
    total = sum(it[-1] for it in items)
    gbs = total / (ms * 1e-3) / 1e9
    stream = torch.cuda.current_stream(dev)
    per = []
    for (name, w, g, radius, norms, ws, nbytes), call in zip(items, calls):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / args.steps
        per.append({"weight": name, "shape": list(w.shape), "ms": round(t, 5),
                    "gbs": round(nbytes / (t * 1e-3) / 1e9, 1)})
    print(json.dumps({"metric": "Hyperball update with fixed-radius projection, GB/s (16 B per weight element)",
                      "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(ms, 4),
                      "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "steps": args.steps,
                      "step": "the four weights in one fp8bq_hyperball_step_batch call (two launches)",
                      "one_call_per_weight": {"ms_per_step": round(ms_single, 4),
                                              "gbs": round(total / (ms_single * 1e-3) / 1e9, 1)},
                      "config": {"workload": "decoder-block weights (QKV, O, gate+up, down), FP32 masters, "
                                             "BF16 gradients"},
                      "per_weight": per}), flush=True)


def time_calls(torch, fns, steps, warmup=3):
    """Mean ms per call of each function, HIP events around every call on the launch stream."""
    import numpy as np
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(steps)]
    for k in range(steps):
        for (e0, e1), f in zip(ev[k], fns):
            e0.record(stream)
            f()
            e1.record(stream)
    torch.cuda.synchronize()
    return [float(np.mean([ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(steps)])) for i in range(len(fns))]


def _rate(flops_or_bytes, ms, scale):
    return round(flops_or_bytes / (ms * 1e-3) / scale, 1)


def run_configs(torch, fq, synth, dev, steps):
    """The other workloads, timed after the decoder step (not part of `value`):
    single_linear  X[8192, 2048] (outlier columns) and W[8192, 2048]: quantize X 1x128, W 128x128, fprop;
    token_sweep    fprop with K = N = 2048 for M = 512 .. 32768 (TFLOP/s against M, and the knee: the
                   smallest M within 10% of the best rate);
    heavy_tailed   dY[16384, 5632] Student-t(3) * 1e-3, X[16384, 2048], W[5632, 2048]: dgrad and wgrad with
                   dY in E5M2 and in E4M3, and the quantization-error report of each."""
    E4, E5 = fq.E4M3, fq.E5M2
    out = {}
    log("configs: single linear ...")
    c = synth.single_linear()
    X, W = c["X"].to(dev), c["W"].to(dev)
    ops, bufs = linear_ops(torch, fq, "linear", X, W, None, dev, with_backward=False)
    ms = time_calls(torch, [o["fn"] for o in ops], steps)
    out["single_linear"] = {
        "workload": "X[8192, 2048] BF16 N(0,1), 1% outlier columns x50; W[8192, 2048] N(0,0.02); E4M3",
        "fprop_tflops": _rate(ops[2]["flops"], ms[2], 1e12), "fprop_ms": round(ms[2], 5),
        "fprop_pct_fp8_peak": round(100 * ops[2]["flops"] / (ms[2] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 1),
        "quant_x_1x128_gbs": _rate(ops[0]["bytes"], ms[0], 1e9), "quant_w_128x128_gbs": _rate(ops[1]["bytes"], ms[1], 1e9),
        "plan": list(fq.fp8bq_gemm_plan(fq.OP_FPROP, 8192, 8192, 2048)),
    }
    del ops, bufs, X, W, c

    log("configs: token sweep ...")
    Wd = synth.sweep_weight().to(dev)
    pts = []
    for M in synth.SWEEP_M:
        Xd = synth.sweep_x(M).to(dev)
        ops, bufs = linear_ops(torch, fq, f"M{M}", Xd, Wd, None, dev, with_backward=False)
        ms = time_calls(torch, [ops[2]["fn"]], max(steps, 20))[0]
        pts.append({"M": M, "us": round(1e3 * ms, 2), "tflops": _rate(ops[2]["flops"], ms, 1e12),
                    "plan": list(fq.fp8bq_gemm_plan(fq.OP_FPROP, M, 2048, 2048))})
        del ops, bufs, Xd
    best = max(p["tflops"] for p in pts)
    out["token_sweep"] = {"workload": "fprop, K = N = 2048, X[M, 2048] N(0,1), W N(0,0.02)", "points": pts,
                          "knee_M": next(p["M"] for p in pts if p["tflops"] >= 0.9 * best)}
    del Wd

    log("configs: heavy-tailed gradients ...")
    c = synth.heavy_tailed()
    dY, X, W = c["dY"].to(dev), c["X"].to(dev), c["W"].to(dev)
    M, N, K = dY.shape[0], dY.shape[1], X.shape[1]
    qw, sw, qwt = fq.quantize_weight_dual(W, E4)
    qxt, sxt = fq.quantize_act_128x1(X, E4)
    res = {"workload": "dY[16384, 5632] Student-t(3) * 1e-3, X[16384, 2048] (outlier columns), W[5632, 2048]; "
                       "X and W in E4M3"}
    fl = 2 * M * N * K
    for name, fmt in (("e5m2", E5), ("e4m3", E4)):
        q, sq, qt, sqt = fq.quantize_act_dual(dY, fmt, fmt)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        wsd = fq._workspace(fq.OP_DGRAD_WT, M, N, K, dev)
        wsw = fq._workspace(fq.OP_WGRAD, M, N, K, dev)
        ms = time_calls(torch, [fq.prepare(fq.fp8bq_gemm_dgrad_wt, q, sq, fmt, qwt, sw, E4, dx, wsd),
                                fq.prepare(fq.fp8bq_gemm_wgrad, qt, sqt, fmt, qxt, sxt, E4, dw, wsw)], steps)
        res[f"dy_{name}"] = {"dgrad_tflops": _rate(fl, ms[0], 1e12), "wgrad_tflops": _rate(fl, ms[1], 1e12),
                             "dgrad_ms": round(ms[0], 5), "wgrad_ms": round(ms[1], 5)}
        del q, sq, qt, sqt, dx, dw, wsd, wsw
    res["quantization_error"] = qerror_report(torch, fq, c, dev)
    out["heavy_tailed"] = res
    return out


def qerror_report(torch, fq, c, dev):
    """Relative Frobenius error of the FP8 dgrad and wgrad (FP32 out) against float64 products of
    the unquantized BF16 inputs, dY in E5M2 and in E4M3 (X, W in E4M3), on 256 sampled rows of dX and
    128 x 128 sampled entries of dW.  Reported, not graded: the pages give no expected value."""
    import numpy as np
    dY, X, W = c["dY"], c["X"], c["W"]
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(dY.shape[0], 256, replace=False))
    ncols = np.sort(rng.choice(dY.shape[1], 128, replace=False))
    kcols = np.sort(rng.choice(X.shape[1], 128, replace=False))
    f64 = lambda t: t.float().numpy().astype(np.float64)
    ref_dx = f64(dY[rows]) @ f64(W)
    ref_dw = f64(dY[:, ncols]).T @ f64(X[:, kcols])
    dYd, Xd, Wd = dY.to(dev), X.to(dev), W.to(dev)
    qw, sw, qwt = fq.quantize_weight_dual(Wd, fq.E4M3)
    qxt, sxt = fq.quantize_act_128x1(Xd, fq.E4M3)
    out = {}
    rel = lambda got, ref: float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    for name, fmt in (("e5m2", fq.E5M2), ("e4m3", fq.E4M3)):
        q, s, qt, st = fq.quantize_act_dual(dYd, fmt, fmt)
        dx = fq.gemm_dgrad_wt(q, s, qwt, sw, fmt, fq.E4M3, out_dtype=torch.float32)
        dw = fq.gemm_wgrad(qt, st, qxt, sxt, fmt, fq.E4M3, out_dtype=torch.float32)
        torch.cuda.synchronize()
        got_dx = dx[torch.from_numpy(rows).to(dev)].double().cpu().numpy()
        got_dw = dw.double().cpu().numpy()[np.ix_(ncols, kcols)]
        out[name] = {"dgrad_rel_frobenius": rel(got_dx, ref_dx), "wgrad_rel_frobenius": rel(got_dw, ref_dw)}
    return out


def run_qerror(torch, fq, synth, dev):
    """The quantization-error report of the heavy-tailed gradient workload alone (see qerror_report)."""
    out = qerror_report(torch, fq, synth.heavy_tailed(), dev)
    for name, r in out.items():
        log(name, r)
    print(json.dumps({"report": "quantization error, heavy-tailed gradients (dY Student-t(3) * 1e-3), "
                                "FP8 GEMM (FP32 out) vs float64 of the unquantized BF16 inputs",
                      "dy_format": out, "x_w_format": "e4m3",
                      "sample": "256 rows of dX [16384, 2048]; 128 x 128 entries of dW [5632, 2048]"}), flush=True)


def build_linear(torch, fq, synth, dev):
    c = synth.single_linear()
    X, W = c["X"].to(dev), c["W"].to(dev)
    ops, bufs = linear_ops(torch, fq, "linear", X, W, None, dev, with_backward=False)
    desc = {"workload": "single fprop linear X[8192,2048] W[8192,2048], E4M3 act 1x128 / weight 128x128",
            "tokens": 8192}
    return ops, bufs + [X, W], desc


def run_sweep(args, torch, fq, synth, dev):
    W = synth.sweep_weight().to(dev)
    res = []
    for M in synth.SWEEP_M:
        X = synth.sweep_x(M).to(dev)
        ops, bufs = linear_ops(torch, fq, f"M{M}", X, W, None, dev, with_backward=False)
        g = ops[2]
        for _ in range(args.warmup):
            g["fn"]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            g["fn"]()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        tf = g["flops"] / (ms * 1e-3) / 1e12
        res.append({"M": M, "ms": round(ms, 5), "tflops": round(tf, 1), "pct_peak": round(100 * tf / FP8_PEAK_TFLOPS, 1)})
        log(res[-1])
    print(json.dumps({"workload": "square-weight fprop sweep K=N=2048", "points": res}))


# (op, M, N, K) in the C-ABI's meaning of each product: the small end of the token sweep, small and
# split products, and the decoder block's GEMMs at 16384 tokens
PLANNER_SHAPES = [
    ("fprop", 512, 2048, 2048), ("fprop", 1024, 2048, 2048), ("fprop", 2048, 2048, 2048), ("fprop", 4096, 2048, 2048),
    ("fprop", 2048, 512, 4096), ("fprop", 8192, 256, 2048), ("fprop", 16384, 2560, 2048), ("fprop", 16384, 11264, 2048),
    ("dgrad", 512, 2048, 2048), ("dgrad", 1024, 2048, 2048), ("dgrad", 4096, 4096, 256), ("dgrad", 4096, 2048, 512),
    ("dgrad", 16384, 2048, 5632),
    ("wgrad", 8192, 256, 2048), ("wgrad", 4096, 2048, 512), ("wgrad", 16384, 256, 256), ("wgrad", 4096, 1024, 1024),
    ("wgrad", 16384, 2048, 2048), ("wgrad", 16384, 2560, 2048), ("wgrad", 16384, 2048, 5632),
    ("wgrad", 16384, 11264, 2048),
]
PLANNER_TILES = [("planner", None), ("64x64", 4), ("128x128", 0), ("256x256", 3)]  # FP8BQ_GEMM_TILE values


def run_planner(args):
    """Parent of the planner check: one child per tile choice, then the comparison."""
    import subprocess
    got = {}
    for name, tile in PLANNER_TILES:
        env = dict(os.environ)
        env.pop("FP8BQ_GEMM_TILE", None)
        if tile is not None:
            env["FP8BQ_GEMM_TILE"] = str(tile)
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", "planner-child",
               "--steps", str(args.steps), "--warmup", str(args.warmup)]
        r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900)
        if r.returncode != 0:
            log(r.stderr[-3000:])
            sys.exit(r.returncode)
        got[name] = json.loads(r.stdout.strip().splitlines()[-1])["points"]
        log(f"planner check: {name} timed")
    value, points = planner_summary(got)
    print(json.dumps({
        "metric": "GEMM tile planner: share of products whose planned tile is within 3% of the fastest tile",
        "value": value, "unit": "fraction", "n_gpus": 1, "higher_is_better": True,
        "steps": args.steps, "warmup": args.warmup, "dtype": "fp8_e4m3",
        "data": "synthetic (N(0,1) activations, N(0,0.02) weights, N(0,1e-3) gradients, drawn on the device)",
        "config": {"workload": "GEMM planner check: each product timed under the plan and under each forced "
                               "tile shape (its own best split), median of per-call HIP events"},
        "worst_planner_over_fastest": max(p["planner_over_fastest"] for p in points),
        "points": points}), flush=True)


def planner_summary(got):
    """(share within 3%, per-product records) from the children's points, keyed by PLANNER_TILES name."""
    points, within = [], 0
    for i, (op, M, N, K) in enumerate(PLANNER_SHAPES):
        us = {name: got[name][i]["us"] for name, _ in PLANNER_TILES}
        forced = {name: v for name, v in us.items() if name != "planner"}
        plans = {name: got[name][i]["plan"] for name in forced}
        best = min(forced, key=forced.get)
        # the planner's plan is one of the forced tiles' plans (that tile with its own best split):
        # compare the timings of the same process kind, so process-to-process noise does not count
        chosen = next((n for n in forced if plans[n] == got["planner"][i]["plan"]), None)
        ratio = (forced[chosen] if chosen else us["planner"]) / forced[best]
        within += ratio <= 1.03
        points.append({"op": op, "shape": [M, N, K], "plan": got["planner"][i]["plan"], "us": us,
                       "forced_plans": plans, "fastest_forced": best, "planned_tile": chosen,
                       "planner_over_fastest": round(ratio, 3)})
    return round(within / len(points), 3), points


def run_planner_child(args, torch, fq, synth, dev):
    """Times each product of PLANNER_SHAPES under this process's plan (FP8BQ_GEMM_TILE forces a tile)."""
    import numpy as np
    E4 = fq.E4M3
    res = []
    for i, (op, M, N, K) in enumerate(PLANNER_SHAPES):
        if op == "fprop":
            qa, sa = fq.quantize_act_1x128(synth.device_normal_bf16((M, K), 500 + i, dev))
            qb, sb = fq.quantize_weight_128x128(synth.device_normal_bf16((N, K), 600 + i, dev, std=0.02))
            out, code = torch.empty((M, N), dtype=torch.bfloat16, device=dev), fq.OP_FPROP
            fn = fq.prepare(fq.fp8bq_gemm_fprop, qa, sa, E4, qb, sb, E4, out, fq._workspace(code, M, N, K, dev))
        elif op == "dgrad":
            qa, sa = fq.quantize_act_1x128(synth.device_normal_bf16((M, N), 700 + i, dev, std=1e-3))
            _, sb, qb = fq.quantize_weight_dual(synth.device_normal_bf16((N, K), 800 + i, dev, std=0.02))
            out, code = torch.empty((M, K), dtype=torch.bfloat16, device=dev), fq.OP_DGRAD_WT
            fn = fq.prepare(fq.fp8bq_gemm_dgrad_wt, qa, sa, E4, qb, sb, E4, out, fq._workspace(code, M, N, K, dev))
        else:
            qa, sa = fq.quantize_act_128x1(synth.device_normal_bf16((M, N), 900 + i, dev, std=1e-3))
            qb, sb = fq.quantize_act_128x1(synth.device_normal_bf16((M, K), 1000 + i, dev))
            out, code = torch.empty((N, K), dtype=torch.bfloat16, device=dev), fq.OP_WGRAD
            fn = fq.prepare(fq.fp8bq_gemm_wgrad, qa, sa, E4, qb, sb, E4, out, fq._workspace(code, M, N, K, dev))
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
        res.append({"op": op, "shape": [M, N, K], "plan": list(fq.fp8bq_gemm_plan(code, M, N, K)), "us": round(us, 2)})
        log(res[-1])
        del qa, sa, qb, sb, out, fn
    print(json.dumps({"points": res}), flush=True)


# -----------------------------------------------------------------------------------------------
# reporting
# -----------------------------------------------------------------------------------------------

def summarize(ops, dur_ms, med_ms=None, min_ms=None):
    """Per kind (quantize / fprop / dgrad / wgrad) sums of the mean launch durations, and per launch
    the mean (`ms`, which all rates use), with the median and minimum over the steps beside it."""
    kinds = {}
    for o, d in zip(ops, dur_ms):
        k = kinds.setdefault(o["kind"], {"ms": 0.0, "flops": 0, "bytes": 0, "launches": 0})
        k["ms"] += float(d)
        k["flops"] += o["flops"]
        k["bytes"] += o["bytes"]
        k["launches"] += 1
    out = {}
    for name, k in kinds.items():
        r = {"ms_per_step": round(k["ms"], 4), "launches": k["launches"]}
        if k["flops"]:
            tf = k["flops"] / (k["ms"] * 1e-3) / 1e12
            r.update(tflops=round(tf, 1), pct_fp8_peak=round(100 * tf / FP8_PEAK_TFLOPS, 1))
        if k["bytes"]:
            gbs = k["bytes"] / (k["ms"] * 1e-3) / 1e9
            r.update(gbs=round(gbs, 1), pct_hbm_peak=round(100 * gbs / HBM_PEAK_GBS, 1))
        out[name] = r
    out["per_launch"] = []
    for i, (o, d) in enumerate(zip(ops, dur_ms)):
        r = {"op": o["name"], "ms": round(float(d), 5)}
        if med_ms is not None:
            r.update(ms_median=round(float(med_ms[i]), 5), ms_min=round(float(min_ms[i]), 5))
        r.update({"tflops": round(o["flops"] / (d * 1e-3) / 1e12, 1)} if o["flops"] else
                 {"gbs": round(o["bytes"] / (d * 1e-3) / 1e9, 1)})
        out["per_launch"].append(r)
    return out


# Kernel instance names as profilers print them: gemm_tn_kernel<OP, BM, BN, waves_m, waves_n, LDS
# stages, scale mode, fmtA, fmtB, f32 out>; the tile shape comes from the library's plan query.
_TILE_ARGS = {(64, 64): "64, 64, 4, 1, 2", (128, 128): "128, 128, 2, 2, 2", (128, 256): "128, 256, 2, 4, 2",
              (256, 128): "256, 128, 4, 2, 2", (256, 256): "256, 256, 2, 4, 2"}
def gemm_kernel(fq, o):
    """(kernel name, isolated) of a GEMM call: o["plan"] is its plan query (op, M, N, K) and o["kid"]
    the kernel's (OP, scale mode) template arguments.  Isolated when the call launches that one kernel
    (a split contraction adds a reduction pass after it)."""
    tm, tn, split = fq.fp8bq_gemm_plan(*o["plan"])
    kop, sbm = o["kid"]
    name = (f"void fp8bq::gemm_tn_kernel<{kop}, {_TILE_ARGS[(tm, tn)]}, {sbm}, "
            f"0, 0, 0>(fp8bq::GemmDesc, unsigned int, unsigned int, int, float*)")
    return name, split == 1


def _traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic_decoder_block.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
        src = open(os.path.join(ROOT, "fp8_blockwise_quantized_amd", "csrc", "gemm.hip"), "rb").read()
        if t.get("gemm_hip_sha256") != hashlib.sha256(src).hexdigest():
            return None
        k = t.get("kernels", {}).get(kernel)
        return k.get("bytes_per_launch") if k else None
    except (OSError, ValueError):
        return None


def roofline(fq, ops, dur_ms, with_traffic=True, copy_gbs=None, torch_copy_gbs=None):
    """The dominant GEMM kernel and one entry per product kind.

    Dominant kernel: the kernel symbol with the most time per step over the calls that launch it
    alone (a split contraction adds a reduction pass to a call, so such calls are left out of the
    symbol's figures); achieved = its algorithmic FLOPs per launch / its mean launch duration (HIP
    events on the launch stream, one pair per call).

    by_kind: fprop, dgrad and wgrad each as a whole (every call of that kind, reduction passes
    included: what the product costs the step), and the quantize passes against HBM (algorithmic
    bytes), with the same run's copy bandwidths beside them when measured: copy_gbs, the library's
    streaming copy (the fastest plain copy measured on this GPU, the ceiling frac_of_copy is taken
    against), and torch_copy_gbs, torch's device copy, for context."""
    groups = {}
    for o, d in zip(ops, dur_ms):
        if not o["flops"]:
            continue
        name, isolated = gemm_kernel(fq, o)
        g = groups.setdefault(name, [])
        if isolated:
            g.append((o, float(d)))
    eligible = [(sum(d for _, d in sel), -i, name, sel) for i, (name, sel) in enumerate(groups.items()) if sel]
    if not eligible:
        return None
    _, _, name, sel = max(eligible, key=lambda e: (e[0], e[1]))
    t = sum(d for _, d in sel)
    flops_per_launch = sum(o["flops"] for o, _ in sel) / len(sel)
    ms_per_launch = t / len(sel)
    achieved = flops_per_launch / (ms_per_launch * 1e-3) / 1e12
    by_kind = {}
    for kind in ("fprop", "dgrad", "wgrad"):
        sel_k = [(o, float(d)) for o, d in zip(ops, dur_ms) if o["kind"] == kind]
        if not sel_k:
            continue
        tk = sum(d for _, d in sel_k)
        ak = sum(o["flops"] for o, _ in sel_k) / (tk * 1e-3) / 1e12
        split = [o["name"] for o, _ in sel_k if not gemm_kernel(fq, o)[1]]
        by_kind[kind] = {"bound": "mfma", "achieved": round(ak, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ak / FP8_PEAK_TFLOPS, 4), "ms_per_step": round(tk, 4),
                         "launches": len(sel_k), "with_reduction_pass": split}
    q = [(o, float(d)) for o, d in zip(ops, dur_ms) if o["bytes"]]
    if q:
        tq = sum(d for _, d in q)
        gq = sum(o["bytes"] for o, _ in q) / (tq * 1e-3) / 1e9
        by_kind["quantize"] = {"bound": "hbm", "achieved": round(gq, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(gq / HBM_PEAK_GBS, 4), "ms_per_step": round(tq, 4), "launches": len(q)}
        if copy_gbs:
            by_kind["quantize"].update(copy_gbs=round(copy_gbs, 1), frac_of_copy=round(gq / copy_gbs, 4))
        if torch_copy_gbs:
            by_kind["quantize"].update(torch_copy_gbs=round(torch_copy_gbs, 1))
    return {
        "bound": "mfma",
        "kernel": name,
        "achieved": round(achieved, 1),
        "peak": FP8_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
        "traffic": _traffic(name) if with_traffic else None,
        "selection": "kernel with the most time per step over calls that launch it alone",
        "launches_per_step": len(sel),
        "launches": [o["name"] for o, _ in sel],
        "flops_per_launch": flops_per_launch,
        "mean_launch_ms": round(ms_per_launch, 5),
        "by_kind": by_kind,
    }


def quant_scrubbed(torch, dev, ops, copy_gbs=None, reps=5, scrub_mib=512, fq=None):
    """Each quantize launch of the step timed on its own with cold caches: before every timed launch a
    read of `scrub_mib` MiB (twice the 256 MB Infinity Cache) evicts them, writing back what the
    earlier kernels left dirty, outside the event pair.  In the step a launch also pays for the
    write-back of the outputs of the kernels before it; here it does not.  GB/s at the algorithmic
    bytes, over all launches (total bytes / total time) and per launch (mean of `reps`).
    With `fq`, the library's streaming copy of each launch's own byte count (half read, half written)
    is timed the same way beside it: a copy's bandwidth depends on its size (the launch ramp weighs
    on the shorter ones), so that is the like-for-like ceiling of each launch."""
    import numpy as np
    q = [o for o in ops if o["bytes"]]
    scrub = torch.ones(scrub_mib << 18, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    runs = [o["fn"] for o in q]
    if fq is not None:
        for o in q:
            n = (o["bytes"] // 2) // 16 * 16
            a = torch.ones(n, dtype=torch.uint8, device=dev)
            runs.append(fq.prepare(fq.fp8bq_stream_copy, a, torch.empty_like(a)))
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in runs]
          for _ in range(reps)]
    sink = []
    for r in range(reps):
        for (e0, e1), fn in zip(ev[r], runs):
            sink.append(scrub.sum())
            e0.record(stream)
            fn()
            e1.record(stream)
    torch.cuda.synchronize()
    times = np.array([[e0.elapsed_time(e1) for e0, e1 in row] for row in ev]).mean(axis=0)
    ms, cms = times[:len(q)], times[len(q):]
    del scrub, sink, runs
    gbs = sum(o["bytes"] for o in q) / (ms.sum() * 1e-3) / 1e9
    out = {"achieved": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
           "method": f"each launch alone after a {scrub_mib} MiB read that evicts the caches (mean of {reps})",
           "per_launch": [{"op": o["name"], "ms": round(float(m), 5), "gbs": _rate(o["bytes"], float(m), 1e9)}
                          for o, m in zip(q, ms)]}
    if copy_gbs:
        out["frac_of_copy"] = round(gbs / copy_gbs, 4)
    if len(cms):
        for r, c in zip(out["per_launch"], cms):
            r.update(same_bytes_copy_ms=round(float(c), 5), frac_of_same_bytes_copy=round(float(c) / float(r["ms"]), 4))
        out["same_bytes_copy_gbs"] = round(sum(o["bytes"] for o in q) / (cms.sum() * 1e-3) / 1e9, 1)
        out["frac_of_same_bytes_copy"] = round(float(cms.sum()) / float(ms.sum()), 4)
    return out


def copy_ceiling(torch, fq, dev, mib=1024, reps=10):
    """GB/s (bytes read + written) of two device copies of `mib` MiB, timed with HIP events on the
    launch stream: "stream", the library's streaming copy (16-byte non-temporal accesses), the
    bandwidth a streaming kernel can reach on this GPU; "torch", torch's device copy."""
    a = torch.empty(mib << 18, dtype=torch.float32, device=dev)
    a.fill_(1.0)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    out = {}
    for name, fn in (("stream", fq.prepare(fq.fp8bq_stream_copy, a, b)), ("torch", lambda: b.copy_(a))):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = 2 * (mib << 20) / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del a, b
    return out


# -----------------------------------------------------------------------------------------------
# CPU oracle baseline
# -----------------------------------------------------------------------------------------------

def cpu_baseline(tokens, desc):
    """The oracle (as it stands) on the same path for the first `tokens` tokens of every linear:
    quantize X, W, dY (1x128, 128x128, 1x128, 128x1, 128x1), fprop, dgrad, wgrad, BF16 rounding."""
    import numpy as np

    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        threads = 1
    E4 = oracle.E4M3
    flops = 0
    t_total = 0.0
    for name, K, N in synth.DECODER_LINEARS:
        c = synth.decoder_linear(name)
        X = c["X"][:tokens].float().numpy()
        dY = c["dY"][:tokens].float().numpy()
        W = c["W"].float().numpy()
        t0 = time.perf_counter()
        qx, sx = oracle.quant_act_1x128(X, E4)
        qw, sw = oracle.quant_weight_128x128(W, E4)
        oracle.to_bf16_rne(oracle.gemm_fprop(qx, sx, E4, qw, sw, E4))
        qdy, sdy = oracle.quant_act_1x128(dY, E4)
        oracle.to_bf16_rne(oracle.gemm_dgrad(qdy, sdy, E4, qw, sw, E4))
        qdyt, sdyt = oracle.quant_act_128x1(dY, E4)
        qxt, sxt = oracle.quant_act_128x1(X, E4)
        oracle.to_bf16_rne(oracle.gemm_wgrad(qdyt, sdyt, E4, qxt, sxt, E4))
        t_total += time.perf_counter() - t0
        flops += 3 * 2 * tokens * N * K
        log(f"cpu oracle {name}: {t_total:.1f} s so far")
    per_config = cpu_per_config()
    return {
        "value": round(flops / t_total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the same decoder-block path (4 linears x quantize 5 ways + fprop/dgrad/wgrad + BF16 "
                  f"rounding) on the first {tokens} of {desc.get('tokens')} tokens, full weights; "
                  f"NumPy quantizers on 1 core, float64 BLAS GEMMs on {threads} threads; "
                  f"{t_total:.1f} s wall",
        "seconds": round(t_total, 2),
        "cpu_model": _cpu_model(),
        "cpu_count": os.cpu_count(),
        "affinity": len(os.sched_getaffinity(0)),
        "per_config": per_config,
    }


def cpu_per_config():
    """The oracle per workload and operation on bounded samples: quantize GB/s (vectorized NumPy, one
    core; algorithmic bytes as on the GPU) and GEMM GFLOP/s (float64 BLAS on all the process's threads,
    BF16 rounding included)."""
    import numpy as np

    import oracle
    import synth
    E4, E5 = oracle.E4M3, oracle.E5M2

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    def qrate(nbytes, sec):
        return {"gbs": round(nbytes / sec / 1e9, 4), "seconds": round(sec, 3)}

    def grate(fl, sec):
        return {"gflops": round(fl / sec / 1e9, 2), "seconds": round(sec, 3)}

    out = {}
    # tiny check (whole workload; FP32 inputs: 4 B in + 1 B code + scales)
    c = synth.tiny_check()
    A, W, dY = c["A"].numpy(), c["W"].numpy(), c["dY"].numpy()
    (qa, sa), t1 = timed(lambda: oracle.quant_act_1x128(A, E4))
    (qw, sw), t2 = timed(lambda: oracle.quant_weight_128x128(W, E4))
    _, t3 = timed(lambda: oracle.to_bf16_rne(oracle.gemm_fprop(qa, sa, E4, qw, sw, E4)))
    out["tiny_check"] = {"sample": "whole workload (256 x 256 x 256)",
                         "quant_1x128": qrate(A.size * 5 + A.size // 128 * 4, t1),
                         "quant_128x128": qrate(W.size * 5 + 16, t2), "fprop": grate(2 * 256 ** 3, t3)}
    # single linear: 512 rows of X, 256 rows of W for the quantizers; 512 rows of Y for the GEMM
    c = synth.single_linear()
    X, Wl = c["X"][:512].float().numpy(), c["W"].float().numpy()
    (qx, sx), t1 = timed(lambda: oracle.quant_act_1x128(X, E4))
    (qw, sw), t2 = timed(lambda: oracle.quant_weight_128x128(Wl, E4))
    _, t3 = timed(lambda: oracle.to_bf16_rne(oracle.gemm_fprop(qx, sx, E4, qw, sw, E4)))
    out["single_linear"] = {"sample": "X rows 0..511 (Y[512, 8192]); all of W",
                            "quant_1x128": qrate(X.size * 3 + X.size // 128 * 4, t1),
                            "quant_128x128": qrate(Wl.size * 3 + Wl.size // 16384 * 4, t2),
                            "fprop": grate(2 * 512 * 8192 * 2048, t3)}
    # token sweep at its smallest M (whole)
    Ws, Xs = synth.sweep_weight().float().numpy(), synth.sweep_x(512).float().numpy()
    (qx, sx), t1 = timed(lambda: oracle.quant_act_1x128(Xs, E4))
    qw, sw = oracle.quant_weight_128x128(Ws, E4)
    _, t3 = timed(lambda: oracle.to_bf16_rne(oracle.gemm_fprop(qx, sx, E4, qw, sw, E4)))
    out["token_sweep_M512"] = {"sample": "whole workload at M = 512",
                               "quant_1x128": qrate(Xs.size * 3 + Xs.size // 128 * 4, t1),
                               "fprop": grate(2 * 512 * 2048 * 2048, t3)}
    # heavy-tailed gradients: the first 512 tokens
    c = synth.heavy_tailed()
    dYh, Xh, Wh = c["dY"][:512].float().numpy(), c["X"][:512].float().numpy(), c["W"].float().numpy()
    (qd, sd), t1 = timed(lambda: oracle.quant_act_1x128(dYh, E5))
    (qdt, sdt), t2 = timed(lambda: oracle.quant_act_128x1(dYh, E5))
    qxt, sxt = oracle.quant_act_128x1(Xh, E4)
    qw, sw = oracle.quant_weight_128x128(Wh, E4)
    _, t3 = timed(lambda: oracle.to_bf16_rne(oracle.gemm_dgrad(qd, sd, E5, qw, sw, E4)))
    _, t4 = timed(lambda: oracle.to_bf16_rne(oracle.gemm_wgrad(qdt, sdt, E5, qxt, sxt, E4)))
    fl = 2 * 512 * 5632 * 2048
    out["heavy_tailed"] = {"sample": "tokens 0..511, dY in E5M2",
                           "quant_1x128_e5m2": qrate(dYh.size * 3 + dYh.size // 128 * 4, t1),
                           "quant_128x1_e5m2": qrate(dYh.size * 3 + dYh.size // 128 * 4, t2),
                           "dgrad": grate(fl, t3), "wgrad": grate(fl, t4)}
    log(f"cpu oracle per workload done")
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
