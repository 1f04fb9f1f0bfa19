"""Operands and outputs past 4 GiB: a token count of 2,200,064 (2^21 + 102,912; a multiple of 128)
puts the activation codes (4.5 GB), the BF16 activations (9.0 GB), the fprop output (4.5 GB) and
wgrad's transposed codes (4.5 GB) beyond 32-bit byte offsets.  Every quantizer and GEMM addresses
these through 64-bit tile bases plus 32-bit in-tile offsets and buffer ranges; this checks that rows
near the end (byte offsets above 2^32) come out right.  Codes and scales of sampled rows are compared
bit for bit with the oracle, GEMM outputs on sampled rows / columns to the usual bound, and the dual
quantizer's two outputs are compared with the separate quantizers on the device.
"""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import oracle
import synth
from parity import check_gemm, f32_bits, row_norms, say, to_np_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
E4 = oracle.E4M3
M = 2_200_064


def _rows():
    rng = np.random.default_rng(5)
    tail = np.arange(M - 3, M)
    edge = np.array([(1 << 31) // 2048 - 1, (1 << 31) // 2048, (1 << 32) // 2048 - 1, (1 << 32) // 2048])
    return np.unique(np.concatenate([[0], edge, tail, rng.choice(M, 40, replace=False)]))


def test_fprop_beyond_4gib():
    K, N = 2048, 1024
    X = synth.device_normal_bf16((M, K), seed=901, device=DEV)
    W = synth.random_bf16((N, K), seed=902, std=0.02)
    qx, sx = fq.quantize_act_1x128(X)
    qw, sw = fq.quantize_weight_128x128(W.to(DEV))
    y = fq.gemm_fprop(qx, sx, qw, sw)  # [M, 1024] BF16: 4.5 GB
    torch.cuda.synchronize()
    rows = _rows()
    ridx = torch.from_numpy(rows).to(DEV)
    xs = X[ridx].float().cpu().numpy()
    oq, os_ = oracle.quant_act_1x128(xs, E4)
    assert np.array_equal(qx[ridx].cpu().numpy(), oq)
    assert np.array_equal(f32_bits(sx[:, ridx].cpu().numpy().T), f32_bits(os_))
    oqw, osw = oracle.quant_weight_128x128(W.float().numpy(), E4)
    a = oracle.dequant_act_1x128(oq, os_, E4)
    b = oracle.dequant_weight_128x128(oqw, osw, E4)
    worst, fro = check_gemm(to_np_f64(y[ridx]), a @ b.T, row_norms(a), row_norms(b), what="fprop M=2.2M")
    say(f"fprop M={M}: max|err|/(|a||b|) = {worst:.2e}, rel Frobenius = {fro:.2e}")


def test_dual_and_wgrad_beyond_4gib():
    K, N = 2048, 256
    X = synth.device_normal_bf16((M, K), seed=903, device=DEV)
    dY = synth.device_normal_bf16((M, N), seed=904, device=DEV, std=1e-3)
    qxt, sxt = fq.quantize_act_128x1(X)  # [K, M]: 4.5 GB
    q, s, qt, st = fq.quantize_act_dual(X)
    qx, sx = fq.quantize_act_1x128(X)
    torch.cuda.synchronize()
    assert torch.equal(q, qx) and torch.equal(s, sx)
    assert torch.equal(qt, qxt) and torch.equal(st, sxt)
    del q, s, qt, st, qx, sx
    qdyt, sdyt = fq.quantize_act_128x1(dY)
    dw = fq.gemm_wgrad(qdyt, sdyt, qxt, sxt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    kc = np.sort(rng.choice(K, 12, replace=False))
    nc = np.sort(rng.choice(N, 12, replace=False))
    xk = X[:, torch.from_numpy(kc).to(DEV)].float().cpu().numpy()
    dyn = dY[:, torch.from_numpy(nc).to(DEV)].float().cpu().numpy()
    oqx, osx = oracle.quant_act_128x1(xk, E4)
    oqd, osd = oracle.quant_act_128x1(dyn, E4)
    # the transposed codes of those columns, all 2.2M tokens, bit for bit (the last ones past 4 GiB)
    assert np.array_equal(qxt[torch.from_numpy(kc).to(DEV)].cpu().numpy(), oqx.T)
    assert np.array_equal(f32_bits(sxt[:, torch.from_numpy(kc).to(DEV)].cpu().numpy()), f32_bits(osx))
    a = oracle.dequant_act_128x1(oqd, osd, E4)
    b = oracle.dequant_act_128x1(oqx, osx, E4)
    got = dw.cpu().numpy().astype(np.float64)[np.ix_(nc, kc)]
    worst, _ = check_gemm(got, a.T @ b, row_norms(a.T), row_norms(b.T), out_f32=True, what="wgrad M=2.2M")
    say(f"wgrad over {M} tokens (split {fq.fp8bq_gemm_plan(fq.OP_WGRAD, M, N, K)[2]}): "
        f"max|err|/(|a||b|) = {worst:.2e}")


def test_more_than_65535_row_blocks():
    """8,388,864 rows (65,538 blocks of 128): the quantizers' tile grids are one-dimensional, so a
    row-block count past the short grid dimensions' limit is still covered exactly once."""
    R, C = 8_388_864, 128
    X = synth.device_normal_bf16((R, C), seed=905, device=DEV)
    q, s, qt, st = fq.quantize_act_dual(X)
    qw, sw, qwt = fq.quantize_weight_dual(X)
    amax = torch.ones(1, dtype=torch.float32, device=DEV)
    qd, sd, qdt = fq.quantize_tensor_delayed(X, amax, 0.99, fq.E4M3, transpose=True)
    torch.cuda.synchronize()
    # 1x128 codes of sampled rows, with rows of the last blocks
    rows = np.unique(np.concatenate([[0, R - 1, R - 128, R - 129], np.random.default_rng(7).choice(R, 40, replace=False)]))
    ridx = torch.from_numpy(rows).to(DEV)
    xs = X[ridx].float().cpu().numpy()
    oq, os_ = oracle.quant_act_1x128(xs, E4)
    assert np.array_equal(q[ridx].cpu().numpy(), oq)
    assert np.array_equal(f32_bits(s[:, ridx].cpu().numpy().T), f32_bits(os_))
    # 128x1 codes of two whole columns (every row block)
    for c in (0, C - 1):
        col = X[:, c:c + 1].float().cpu().numpy()
        oqc, osc = oracle.quant_act_128x1(col, E4)
        assert np.array_equal(qt[c].cpu().numpy(), oqc[:, 0]), c
        assert np.array_equal(f32_bits(st[:, c].cpu().numpy()), f32_bits(osc[:, 0])), c
    # 128x128 weight codes of the first and last tiles, and their transpose
    for r0 in (0, R - 128):
        tile = X[r0:r0 + 128].float().cpu().numpy()
        oqw, osw = oracle.quant_weight_128x128(tile, E4)
        assert np.array_equal(qw[r0:r0 + 128].cpu().numpy(), oqw), r0
        assert f32_bits(sw[r0 // 128].cpu().numpy())[0] == f32_bits(osw)[0, 0], r0
        assert np.array_equal(qwt[:, r0:r0 + 128].cpu().numpy(), oqw.T), r0
    # per-tensor codes and their transpose on the same rows
    a = oracle.amax_ema_update(np.float32(1.0), X.float().abs().max().cpu().numpy().reshape(1), 0.99, "bf16")
    os_d = oracle.tensor_scale(a, E4)
    assert f32_bits(sd.cpu().numpy())[0] == f32_bits(os_d)
    oqd = oracle.quant_tensor(xs, os_d, E4)
    assert np.array_equal(qd[ridx].cpu().numpy(), oqd)
    assert np.array_equal(qdt[:, ridx].cpu().numpy(), oqd.T)
    say(f"{R} rows ({R // 128} row blocks): 1x128, 128x1, 128x128 and per-tensor codes exact")
