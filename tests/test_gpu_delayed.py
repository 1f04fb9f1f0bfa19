"""GPU parity of the per-tensor delayed-scaling path against the oracle.

Quantizer: over several steps of one running amax, the updated amax, the scale and every code
(and its transpose, when asked for) must be bit-identical to the oracle's.  The GEMM of two
per-tensor-scaled operands is held to the blockwise GEMM's bound: |err| <= 2e-3 ||a_i|| ||b_j||
and a relative Frobenius error <= 1e-3 against the BF16-rounded float64 product.
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import oracle
import synth
from parity import FP, check_gemm, f32_bits, row_norms, say, to_np_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
E4, E5 = oracle.E4M3, oracle.E5M2


def _input(shape, seed, dtype, mag):
    if dtype == torch.float32:
        return synth.random_f32(shape, seed, std=mag)
    return synth.random_bf16(shape, seed, std=mag)


def _steps(shape, dtype, fmt, transpose, beta=0.99, mags=(1.0, 40.0, 0.05), seed=0):
    amax_d = torch.ones(1, dtype=torch.float32, device=DEV)
    a = np.float32(1.0)
    for step, mag in enumerate(mags):
        x = _input(shape, seed + 17 * step + shape[0], dtype, mag)
        q, s, qt = fq.quantize_tensor_delayed(x.to(DEV), amax_d, beta, FP[fmt], transpose)
        torch.cuda.synchronize()
        oq, os_, a = oracle.quant_tensor_delayed(x.float().numpy(), a, beta, fmt,
                                                 "bf16" if dtype == torch.bfloat16 else "f32")
        assert f32_bits(amax_d.cpu().numpy())[0] == f32_bits(a), f"step {step}: running amax"
        assert f32_bits(s.cpu().numpy())[0] == f32_bits(os_), f"step {step}: scale"
        got = q.cpu().numpy()
        bad = np.argwhere(got != oq)
        assert bad.size == 0, f"step {step}: {len(bad)} codes differ, first at {bad[0].tolist()}"
        if transpose:
            assert np.array_equal(qt.cpu().numpy(), got.T), f"step {step}: transposed codes"
    return a


@pytest.mark.parametrize("fmt", [E4, E5])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape,transpose", [((256, 384), True), ((200, 256), False), ((1, 128), False),
                                             ((1024, 2048), True), ((4099, 640), False)])
def test_running_amax_steps(fmt, dtype, shape, transpose):
    a = _steps(shape, dtype, fmt, transpose)
    say(f"delayed {fmt} {dtype} {shape} T={transpose}: running amax {float(a):.6g}")


@pytest.mark.parametrize("beta", [0.0, 1.0, 0.5])
def test_beta_extremes(beta):
    _steps((384, 256), torch.bfloat16, E4, True, beta=beta, mags=(3.0, 0.01))


def test_bf16_copy_of_fp32_input():
    """The double-rounding case: 1 + 2^-4 + 2^-9 quantizes through its BF16 copy (a tie) to 0x38."""
    x = torch.zeros((128, 128), dtype=torch.float32)
    x[0, 0] = 448.0
    x[5, 7] = 1 + 2.0 ** -4 + 2.0 ** -9
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    q, s, qt = fq.quantize_tensor_delayed(x.to(DEV), amax, 0.0, fq.E4M3, transpose=True)
    torch.cuda.synchronize()
    assert float(s.item()) == 1.0 and float(amax.item()) == 448.0
    assert int(q[0, 0]) == 0x7E and int(q[5, 7]) == 0x38 and int(qt[7, 5]) == 0x38


def test_strided_input_and_empty():
    big = synth.random_bf16((256, 512), seed=9, std=2.0).to(DEV)
    x = big[:, 128:384]
    amax = torch.full((1,), 5.0, dtype=torch.float32, device=DEV)
    q, s, qt = fq.quantize_tensor_delayed(x, amax, 0.99, fq.E4M3, transpose=True)
    torch.cuda.synchronize()
    oq, os_, a = oracle.quant_tensor_delayed(x.float().cpu().numpy(), np.float32(5.0), 0.99, E4, "bf16")
    assert np.array_equal(q.cpu().numpy(), oq) and f32_bits(s.cpu().numpy())[0] == f32_bits(os_)
    # no rows: nothing is enqueued, the running amax and the scale keep their values
    s0 = torch.full((1,), 7.0, dtype=torch.float32, device=DEV)
    e = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    qe = torch.empty((0, 256), dtype=torch.uint8, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    fq.fp8bq_quantize_tensor_delayed(e, fq.E4M3, amax, 0.5, qe, None, s0, ws)
    torch.cuda.synchronize()
    assert f32_bits(amax.cpu().numpy())[0] == f32_bits(a) and float(s0.item()) == 7.0


def test_activation_size_sampled():
    """A 16384 x 2048 activation: the running amax and scale exactly, codes on sampled rows."""
    c = synth.decoder_linear("qkv")
    X = c["X"]
    amax = torch.ones(1, dtype=torch.float32, device=DEV)
    q, s, qt = fq.quantize_tensor_delayed(X.to(DEV), amax, 0.99, fq.E4M3, transpose=True)
    torch.cuda.synchronize()
    xf = X.float().numpy()
    a = oracle.amax_ema_update(np.float32(1.0), xf, 0.99, "bf16")
    os_ = oracle.tensor_scale(a, E4)
    assert f32_bits(amax.cpu().numpy())[0] == f32_bits(a)
    assert f32_bits(s.cpu().numpy())[0] == f32_bits(os_)
    rows = np.unique(np.concatenate([[0, 16383], np.random.default_rng(1).choice(16384, 96, replace=False)]))
    oq = oracle.quant_tensor(xf[rows], os_, E4)
    assert np.array_equal(q.cpu().numpy()[rows], oq)
    assert np.array_equal(qt.cpu().numpy()[:, rows], oq.T)


# ------------------------------------------------------------------------------------------
# GEMM with per-tensor scales
# ------------------------------------------------------------------------------------------

def _quant_both(x, fmt, transpose=False):
    amax = torch.ones(1, dtype=torch.float32, device=DEV)
    q, s, qt = fq.quantize_tensor_delayed(x.to(DEV), amax, 0.0, FP[fmt], transpose)
    return q, s, qt


def _check(got, qa, sa, fa, qb, sb, fb, what, out_f32=False, rows=None):
    """qa/qb: numpy codes, sa/sb: numpy float32 scales; rows: optional row sample of qa."""
    a = oracle.dequant_tensor(qa if rows is None else qa[rows], sa, fa)
    b = oracle.dequant_tensor(qb, sb, fb)
    y64 = a @ b.T
    worst, fro = check_gemm(got, y64, row_norms(a), row_norms(b), out_f32=out_f32, what=what)
    say(f"{what}: max|err|/(|a||b|) = {worst:.2e}, rel Frobenius = {fro:.2e}")


@pytest.mark.parametrize("shape", [(256, 256, 256), (200, 384, 640), (1000, 1024, 2048), (256, 256, 4096)])
@pytest.mark.parametrize("fa,fb", [(E4, E4), (E5, E4)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_tensor_parity(shape, fa, fb, out_dtype):
    M, N, K = shape
    X = synth.random_bf16((M, K), seed=M + K, outliers=True)
    W = synth.random_bf16((N, K), seed=N + K + 1, std=0.02)
    qa, sa, _ = _quant_both(X, fa)
    qb, sb, _ = _quant_both(W, fb)
    y = fq.gemm_tensor(qa, sa, qb, sb, FP[fa], FP[fb], out_dtype=out_dtype)
    torch.cuda.synchronize()
    _check(to_np_f64(y), qa.cpu().numpy(), sa.cpu().numpy()[0], fa, qb.cpu().numpy(), sb.cpu().numpy()[0], fb,
           f"tensor gemm {shape} {fa}x{fb}", out_f32=out_dtype == torch.float32)


def test_gemm_tensor_three_products():
    """fprop, dgrad and wgrad of one linear, each through the transposed codes the quantizer writes."""
    M, N, K = 512, 384, 256
    X = synth.random_bf16((M, K), seed=41, outliers=True)
    W = synth.random_bf16((N, K), seed=42, std=0.02)
    dY = synth.random_bf16((M, N), seed=43, std=1e-3)
    qx, sx, qxt = _quant_both(X, E4, transpose=True)
    qw, sw, qwt = _quant_both(W, E4, transpose=True)
    qdy, sdy, qdyt = _quant_both(dY, E5, transpose=True)
    y = fq.gemm_tensor(qx, sx, qw, sw)                       # Y = X W^T       [M, N]
    dx = fq.gemm_tensor(qdy, sdy, qwt, sw, fq.E5M2, fq.E4M3)  # dX = dY W       [M, K]
    dw = fq.gemm_tensor(qdyt, sdy, qxt, sx, fq.E5M2, fq.E4M3)  # dW = dY^T X     [N, K]
    torch.cuda.synchronize()
    n = lambda t: t.cpu().numpy()
    _check(to_np_f64(y), n(qx), n(sx)[0], E4, n(qw), n(sw)[0], E4, "tensor fprop")
    _check(to_np_f64(dx), n(qdy), n(sdy)[0], E5, n(qwt), n(sw)[0], E4, "tensor dgrad")
    _check(to_np_f64(dw), n(qdyt), n(sdy)[0], E5, n(qxt), n(sx)[0], E4, "tensor wgrad")


def test_gemm_tensor_full_size_sampled():
    c = synth.decoder_linear("gate_up")
    X, W = c["X"], c["W"]
    qa, sa, _ = _quant_both(X, E4)
    qb, sb, _ = _quant_both(W, E4)
    y = fq.gemm_tensor(qa, sa, qb, sb)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 16383], np.random.default_rng(2).choice(16384, 64, replace=False)]))
    got = to_np_f64(y[torch.from_numpy(rows).to(DEV)])
    _check(got, qa.cpu().numpy(), sa.cpu().numpy()[0], E4, qb.cpu().numpy(), sb.cpu().numpy()[0], E4,
           "tensor gemm 16384x11264x2048 (sampled rows)", rows=rows)
