"""One linear's hot path captured in a HIP graph through the same C-ABI calls (torch.cuda.CUDAGraph
records them on its capture stream).  The entry points allocate nothing, never synchronize and
launch only kernels (no memset nodes), so every replay must reproduce the eager results bit for bit.
The replays are interleaved with eager work of the program and synchronizations, and each replay
starts from outputs overwritten with a sentinel."""

import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _u8(r, c):
    return torch.empty((r, c), dtype=torch.uint8, device=DEV)


def _f32(r, c):
    return torch.empty((r, c), dtype=torch.float32, device=DEV)


def test_linear_step_graph_replays_match_eager():
    M, N, K = 1024, 768, 512
    E4, E5 = fq.E4M3, fq.E5M2
    X = synth.random_bf16((M, K), seed=61, outliers=True).to(DEV)
    W = synth.random_bf16((N, K), seed=62, std=0.02).to(DEV)
    W2 = synth.random_bf16((256, K), seed=63, std=0.02).to(DEV)  # a second weight in the same batch
    dY = synth.random_bf16((M, N), seed=64, std=1e-3).to(DEV)
    q, s, qt, st = _u8(M, K), _f32(K // 128, M), _u8(K, M), _f32(M // 128, K)
    qw, sw, qwt = _u8(N, K), _f32(N // 128, K // 128), _u8(K, N)
    qw2, sw2, qwt2 = _u8(256, K), _f32(2, K // 128), _u8(K, 256)
    qd, sd, qdt, sdt = _u8(M, N), _f32(N // 128, M), _u8(N, M), _f32(M // 128, N)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dw = torch.empty((N, K), dtype=torch.float32, device=DEV)
    ws_f = fq._workspace(fq.OP_FPROP, M, N, K, DEV)
    ws_d = fq._workspace(fq.OP_DGRAD_WT, M, N, K, DEV)
    ws_w = fq._workspace(fq.OP_WGRAD, M, N, K, DEV)
    outs = [q, s, qt, st, qw, sw, qwt, qw2, sw2, qwt2, qd, sd, qdt, sdt, y, dx, dw]

    def step():
        fq.fp8bq_quantize_act_dual(X, E4, q, s, E4, qt, st)
        fq.fp8bq_quantize_weights_dual([(W, qw, sw, qwt), (W2, qw2, sw2, qwt2)], E4)
        fq.fp8bq_gemm_fprop(q, s, E4, qw, sw, E4, y, ws_f)
        fq.fp8bq_quantize_act_dual(dY, E5, qd, sd, E5, qdt, sdt)
        fq.fp8bq_gemm_dgrad_wt(qd, sd, E5, qwt, sw, E4, dx, ws_d)
        fq.fp8bq_gemm_wgrad(qdt, sdt, E5, qt, st, E4, dw, ws_w)

    def scramble():
        for t in outs:
            t.fill_(77 if t.dtype == torch.uint8 else -7.0)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    other = torch.randn(512, 512, device=DEV)
    for r in range(4):
        scramble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs from the eager run"
        other = other @ other.t() / 512.0  # the program's own eager work between replays
        torch.cuda.synchronize()
