"""On a real device, a call that fails validation returns its status and enqueues nothing: outputs
(and inputs) keep the bytes they held.  The status codes themselves are checked without a GPU in
test_abi.py; here the point is that no kernel ran."""

import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPE, WORKSPACE, OVERLAP = 2, 7, 10


def _operands(M, N, K):
    X = synth.random_bf16((M, K), seed=M + K, std=1.0).to(DEV)
    W = synth.random_bf16((N, K), seed=N + K, std=0.02).to(DEV)
    dY = synth.random_bf16((M, N), seed=M + N, std=1e-3).to(DEV)
    q, s = fq.quantize_act_1x128(X)
    qw, sw = fq.quantize_weight_128x128(W)
    qd, sd = fq.quantize_act_1x128(dY)
    return q, s, qw, sw, qd, sd


def _status(call):
    with pytest.raises(fq.Fp8bqError) as e:
        call()
    return e.value.status


def test_gemm_errors_enqueue_nothing():
    M, N, K = 384, 512, 1024
    q, s, qw, sw, qd, sd = _operands(M, N, K)
    torch.cuda.synchronize()
    # dgrad on row-major weight codes needs a transpose buffer of N*K bytes: 16 bytes are too few
    dx = torch.full((M, K), -3.0, dtype=torch.bfloat16, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    assert _status(lambda: fq.fp8bq_gemm_dgrad(qd, sd, fq.E4M3, qw, sw, fq.E4M3, dx, small)) == WORKSPACE
    # an output laid over the A codes (K = 2N, so the BF16 [M, N] output is exactly their bytes): the
    # codes must survive the refused call
    buf = torch.empty(M * K, dtype=torch.uint8, device=DEV)
    qa = buf.view(M, K)
    qa.copy_(q)
    y = buf.view(torch.bfloat16).view(M, N)
    before = buf.clone()
    assert _status(lambda: fq.fp8bq_gemm_fprop(qa, s, fq.E4M3, qw, sw, fq.E4M3, y)) == OVERLAP
    torch.cuda.synchronize()
    assert bool((dx == -3.0).all()), "dgrad wrote its output despite the error"
    assert torch.equal(buf, before), "fprop wrote over its input despite the error"


def test_quantizer_errors_enqueue_nothing():
    x = synth.random_bf16((256, 256), seed=5, std=1.0).to(DEV)
    q = torch.full((256, 200), 0x77, dtype=torch.uint8, device=DEV)
    s = torch.full((1, 256), 5.0, dtype=torch.float32, device=DEV)
    assert _status(lambda: fq.fp8bq_quantize_act_1x128(x[:, :200], fq.E4M3, q, s)) == SHAPE  # C % 128 != 0
    qt = torch.full((256, 256), 0x66, dtype=torch.uint8, device=DEV)
    s2 = torch.full((2, 256), 5.0, dtype=torch.float32, device=DEV)
    st = torch.full((2, 256), 6.0, dtype=torch.float32, device=DEV)
    # both code layouts into one array
    assert _status(lambda: fq.fp8bq_quantize_act_dual(x, fq.E4M3, qt, s2, fq.E4M3, qt, st)) == OVERLAP
    torch.cuda.synchronize()
    assert bool((q == 0x77).all()) and bool((s == 5.0).all())
    assert bool((qt == 0x66).all()) and bool((s2 == 5.0).all()) and bool((st == 6.0).all())


def test_binding_refuses_mismatched_tensors_on_the_device():
    """The binding's own checks on device tensors: an output with too few rows, scales of another
    element type, a scale array left on the host, a workspace on the host.  Nothing runs."""
    M, N, K = 384, 512, 1024
    q, s, qw, sw, qd, sd = _operands(M, N, K)
    y = torch.full((M, N), -2.0, dtype=torch.bfloat16, device=DEV)
    short = torch.full((M - 128, N), -2.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fq.fp8bq_gemm_fprop(q, s, fq.E4M3, qw, sw, fq.E4M3, short)
    with pytest.raises(TypeError):
        fq.fp8bq_gemm_fprop(q, s.to(torch.bfloat16), fq.E4M3, qw, sw, fq.E4M3, y)
    with pytest.raises(ValueError):
        fq.fp8bq_gemm_fprop(q, s.cpu(), fq.E4M3, qw, sw, fq.E4M3, y)
    with pytest.raises(ValueError):
        fq.fp8bq_gemm_fprop(q, s, fq.E4M3, qw, sw, fq.E4M3, y, torch.zeros(1 << 20, dtype=torch.uint8))
    torch.cuda.synchronize()
    assert bool((y == -2.0).all()) and bool((short == -2.0).all())


def test_prepared_calls_match_direct_calls():
    """fq.prepare keeps a call's marshalled arguments: repeated launches give the direct call's output."""
    M, N, K = 384, 512, 1024
    q, s, qw, sw, qd, sd = _operands(M, N, K)
    y1 = torch.full((M, N), -2.0, dtype=torch.bfloat16, device=DEV)
    y2 = torch.full((M, N), -3.0, dtype=torch.bfloat16, device=DEV)
    fq.fp8bq_gemm_fprop(q, s, fq.E4M3, qw, sw, fq.E4M3, y1)
    launch = fq.prepare(fq.fp8bq_gemm_fprop, q, s, fq.E4M3, qw, sw, fq.E4M3, y2)
    launch()
    launch()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_stream_copy_copies_every_byte():
    """The bandwidth reference copies exactly: sizes that leave a partial last iteration, a size
    past one grid stride, and an overlap refused with nothing written."""
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    for nbytes in (16, 4096 + 48, 3 << 20, (257 << 20) + 16 * 7):
        src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
        dst = torch.zeros_like(src)
        fq.fp8bq_stream_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), nbytes
    buf = torch.arange(4096, dtype=torch.uint8, device=DEV)
    before = buf.clone()
    with pytest.raises(fq.Fp8bqError) as e:
        fq.fp8bq_stream_copy(buf[:2048], buf[1024:3072])
    assert e.value.status == 10  # FP8BQ_ERR_OVERLAP
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
