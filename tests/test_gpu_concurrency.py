"""Re-entrancy: the entry points keep no mutable state beyond a per-device property cache, so
several host threads, each enqueueing on its own stream, must get exactly the results of a serial
run (every kernel is deterministic).  ctypes releases the interpreter lock during the calls, so
the library really is entered concurrently."""

import threading

import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _chain(X, W, dY):
    """The hot path of one linear (quantize X, W, dY; fprop, dgrad, wgrad) on the current stream."""
    q, s, qt, st = fq.quantize_act_dual(X)
    qw, sw, qwt = fq.quantize_weight_dual(W)
    y = fq.gemm_fprop(q, s, qw, sw)
    qd, sd, qdt, sdt = fq.quantize_act_dual(dY)
    dx = fq.gemm_dgrad_wt(qd, sd, qwt, sw)
    dw = fq.gemm_wgrad(qdt, sdt, qt, st)
    return [q, s, qw, sw, y, dx, dw]


def test_threads_on_separate_streams_match_serial():
    shapes = [(1024, 512, 768), (512, 1280, 256), (2048, 256, 1024), (768, 768, 512)]
    inputs = []
    for i, (M, N, K) in enumerate(shapes):
        inputs.append((synth.random_bf16((M, K), seed=500 + i, outliers=True).to(DEV),
                       synth.random_bf16((N, K), seed=510 + i, std=0.02).to(DEV),
                       synth.random_bf16((M, N), seed=520 + i, std=1e-3).to(DEV)))
    serial = [_chain(*inp) for inp in inputs]
    torch.cuda.synchronize()

    results, errors = [None] * len(inputs), []
    start = threading.Barrier(len(inputs))

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait()
                for _ in range(5):
                    out = _chain(*inputs[i])
            s.synchronize()
            results[i] = out
        except Exception as e:  # surfaced in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(inputs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (got, want) in enumerate(zip(results, serial)):
        assert got is not None, f"thread {i} did not finish"
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"thread {i}: results differ from the serial run"


def test_batched_weight_quantization_threads_match_serial():
    """Several host threads, each quantizing its own set of weights in one batched launch on its own
    stream, get exactly the serial results (the launch keeps its job table in kernel arguments, so
    concurrent calls share nothing)."""
    sets = [[synth.random_bf16((128 * (1 + (i + j) % 4), 128 * (1 + j % 3)), seed=700 + 10 * i + j, std=0.3).to(DEV)
             for j in range(5)] for i in range(4)]
    serial = [fq.quantize_weights_dual(ws) for ws in sets]
    torch.cuda.synchronize()
    results, errors = [None] * len(sets), []
    start = threading.Barrier(len(sets))

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait()
                for _ in range(10):
                    out = fq.quantize_weights_dual(sets[i])
            s.synchronize()
            results[i] = out
        except Exception as e:  # surfaced in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(sets))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (got, want) in enumerate(zip(results, serial)):
        assert got is not None, f"thread {i} did not finish"
        for g, w in zip(got, want):
            for a, b in zip(g, w):
                assert torch.equal(a, b), f"thread {i}: batched results differ from the serial run"
