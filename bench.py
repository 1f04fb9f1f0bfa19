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

Prints ONE JSON line on stdout.  `value` = GEMM FLOPs of the step / wall time of the step (the
quantize passes are inside the timed step).  `breakdown` holds per-product TFLOP/s and per-pass GB/s
from HIP events recorded on the launch stream; `roofline` is for the dominant GEMM kernel;
`cpu_baseline` times the CPU oracle on a bounded sample of the same path (first 4096 tokens).
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
    p.add_argument("--workload", choices=["decoder", "delayed", "hyperball", "linear", "sweep", "qerror"],
                   default="decoder")
    p.add_argument("--no-cpu-baseline", action="store_true")
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
    roof = roofline(fq, ops, dur_ms, with_traffic=args.workload == "decoder")
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
                       fn=lambda: fq.fp8bq_quantize_act_dual(X, E4, qx, sx, E4, qxt, sxt))
        quant_w = dict(name=f"{name}.quant_w_dual", kind="quant_w_dual", bytes=_qw_bytes(N, K) + N * K, flops=0,
                       fn=lambda: fq.fp8bq_quantize_weight_dual(W, E4, qw, sw, qwt))
    else:
        quant_x = dict(name=f"{name}.quant_x_1x128", kind="quant_1x128", bytes=_q1x128_bytes(M, K), flops=0,
                       fn=lambda: fq.fp8bq_quantize_act_1x128(X, E4, qx, sx))
        quant_w = dict(name=f"{name}.quant_w_128x128", kind="quant_128x128", bytes=_qw_bytes(N, K), flops=0,
                       fn=lambda: fq.fp8bq_quantize_weight_128x128(W, E4, qw, sw))
    if weight_jobs is not None and with_backward:
        weight_jobs.append((W, qw, sw, qwt))
        quant_w = None
    ops = [op for op in (quant_x, quant_w) if op is not None] + [
        dict(name=f"{name}.fprop", kind="fprop", bytes=0, flops=2 * M * N * K, plan=(fq.OP_FPROP, M, N, K), kid=(0, 0),
             fn=lambda: fq.fp8bq_gemm_fprop(qx, sx, E4, qw, sw, E4, y, ws_f)),
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
                 fn=lambda: fq.fp8bq_quantize_act_dual(dY, E4, qdy, sdy, E4, qdyt, sdyt)),
            dict(name=f"{name}.dgrad", kind="dgrad", bytes=0, flops=2 * M * N * K, plan=(fq.OP_DGRAD_WT, M, N, K),
                 kid=(1, 0), fn=lambda: fq.fp8bq_gemm_dgrad_wt(qdy, sdy, E4, qwt, sw, E4, dx, ws_d)),
            dict(name=f"{name}.wgrad", kind="wgrad", bytes=0, flops=2 * M * N * K, plan=(fq.OP_WGRAD, M, N, K),
                 kid=(2, 1), fn=lambda: fq.fp8bq_gemm_wgrad(qdyt, sdyt, E4, qxt, sxt, E4, dw, ws_w)),
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
                       fn=lambda: fq.fp8bq_quantize_weights_dual(wjobs, fq.E4M3)))
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
             fn=lambda: fq.fp8bq_quantize_tensor_delayed(X, E4, ax, 0.99, qx, qxt, sx, wsq)),
        dict(name=f"{name}.quant_w_tensor", kind="quant_tensor", bytes=_qtensor_bytes(N, K, True), flops=0,
             fn=lambda: fq.fp8bq_quantize_tensor_delayed(W, E4, aw, 0.99, qw, qwt, sw, wsq)),
        dict(name=f"{name}.fprop", kind="fprop", bytes=0, flops=2 * M * N * K, plan=(fq.OP_TENSOR, M, N, K),
             kid=(0, 0), fn=lambda: fq.fp8bq_gemm_tensor(qx, sx, E4, qw, sw, E4, y, ws_f)),
        dict(name=f"{name}.quant_dy_tensor", kind="quant_tensor", bytes=_qtensor_bytes(M, N, True), flops=0,
             fn=lambda: fq.fp8bq_quantize_tensor_delayed(dY, E4, ady, 0.99, qdy, qdyt, sdy, wsq)),
        dict(name=f"{name}.dgrad", kind="dgrad", bytes=0, flops=2 * M * N * K, plan=(fq.OP_TENSOR, M, K, N),
             kid=(0, 0), fn=lambda: fq.fp8bq_gemm_tensor(qdy, sdy, E4, qwt, sw, E4, dx, ws_d)),
        dict(name=f"{name}.wgrad", kind="wgrad", bytes=0, flops=2 * M * N * K, plan=(fq.OP_TENSOR, N, K, M),
             kid=(0, 0), fn=lambda: fq.fp8bq_gemm_tensor(qdyt, sdy, E4, qxt, sx, E4, dw, ws_w)),
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
    """Hyperball update with projection of the four decoder weights (FP32 masters, BF16 gradients).
    Algorithmic bytes per element: gradient read 2 + weight read and write 8 + the projection's second
    weight read and write 8 (it needs the whole updated tensor's norm first) = 18."""
    import numpy as np
    items = []
    for name, K, N in synth.DECODER_LINEARS:
        w = synth.random_f32((N, K), seed=7 + N, std=0.02).to(dev)
        g = synth.random_bf16((N, K), seed=8 + N, std=1e-3).to(dev)
        radius = float(torch.linalg.vector_norm(w.double()).item())
        norms = torch.empty(2, dtype=torch.float32, device=dev)
        ws = torch.empty(fq.fp8bq_hyperball_workspace_size(N, K), dtype=torch.uint8, device=dev)
        items.append((name, w, g, radius, norms, ws, 18 * N * K))

    def step():
        for _, w, g, radius, norms, ws, _ in items:
            fq.fp8bq_hyperball_step(w, g, 1e-4, 0.1, 1e-8, radius, norms, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    total = sum(it[-1] for it in items)
    gbs = total / (ms * 1e-3) / 1e9
    stream = torch.cuda.current_stream(dev)
    per = []
    for name, w, g, radius, norms, ws, nbytes in items:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fq.fp8bq_hyperball_step(w, g, 1e-4, 0.1, 1e-8, radius, norms, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / args.steps
        per.append({"weight": name, "shape": list(w.shape), "ms": round(t, 5),
                    "gbs": round(nbytes / (t * 1e-3) / 1e9, 1)})
    print(json.dumps({"metric": "Hyperball update with fixed-radius projection, GB/s (18 B per weight element)",
                      "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(ms, 4),
                      "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "steps": args.steps,
                      "config": {"workload": "decoder-block weights (QKV, O, gate+up, down), FP32 masters, "
                                             "BF16 gradients"},
                      "per_weight": per}), flush=True)


def run_qerror(torch, fq, synth, dev):
    """Quantization error of the heavy-tailed gradient workload (dY Student-t(3) * 1e-3 [16384, 5632],
    X [16384, 2048] with outlier columns, W [5632, 2048]): relative Frobenius error of the FP8 dgrad
    (dY . W) and wgrad (dY^T . X) against float64 products of the unquantized BF16 inputs, for dY in
    E5M2 and in E4M3 (X and W in E4M3), on 256 sampled rows of dX and 128 x 128 sampled entries of dW."""
    import numpy as np
    c = synth.heavy_tailed()
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
        log(name, out[name])
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
_TILE_ARGS = {(128, 128): "128, 128, 2, 2, 2", (128, 256): "128, 256, 2, 4, 2", (256, 128): "256, 128, 4, 2, 2",
              (256, 256): "256, 256, 2, 4, 2"}
def gemm_kernel(fq, o):
    """(kernel name, isolated) of a GEMM op: o["plan"] is its plan query (op, M, N, K) and o["kid"]
    the kernel's (OP, scale mode) template arguments.  Isolated when the call launches that one kernel
    (a split contraction adds a reduction pass)."""
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


def roofline(fq, ops, dur_ms, with_traffic=True):
    """The dominant GEMM kernel among those whose every launch in the step is that kernel alone, by
    FLOPs per step (the first in step order on a tie, so the choice does not depend on timing noise):
    achieved = its algorithmic FLOPs per launch / its mean launch duration (HIP events on the launch
    stream, one pair per call), over all of its launches in the step."""
    groups = {}
    for o, d in zip(ops, dur_ms):
        if not o["flops"]:
            continue
        name, isolated = gemm_kernel(fq, o)
        g = groups.setdefault(name, {"ok": True, "sel": []})
        g["ok"] &= isolated
        g["sel"].append((o, float(d)))
    eligible = [(sum(o["flops"] for o, _ in g["sel"]), -i, name, g["sel"])
                for i, (name, g) in enumerate(groups.items()) if g["ok"]]
    if not eligible:
        return None
    _, _, name, sel = max(eligible, key=lambda e: (e[0], e[1]))
    t = sum(d for _, d in sel)
    flops_per_launch = sum(o["flops"] for o, _ in sel) / len(sel)
    ms_per_launch = t / len(sel)
    achieved = flops_per_launch / (ms_per_launch * 1e-3) / 1e12
    return {
        "bound": "mfma",
        "kernel": name,
        "achieved": round(achieved, 1),
        "peak": FP8_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
        "traffic": _traffic(name) if with_traffic else None,
        "launches_per_step": len(sel),
        "launches": [o["name"] for o, _ in sel],
        "flops_per_launch": flops_per_launch,
        "mean_launch_ms": round(ms_per_launch, 5),
    }


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
    }


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
