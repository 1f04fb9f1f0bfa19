"""Pins for the oracle's GEMMs and BF16 output rounding (CPU only).

What pins them, independent of the GEMM code:
* BF16 round-to-nearest-even closed forms (ties, carries, double-rounding
  traps, subnormals) and PyTorch's fp32->bf16 cast on values exact in fp32;
* hand-computable products: one-hot activation rows of amplitude 448 give
  scale 1 and code 0x7E, so each output is 448 times one dequantized weight;
* exact rational brute force (Python Fractions, its own bit-field decoder)
  on tiny fprop, dgrad and wgrad problems;
* the per-block form of the contraction (scales applied per 128 block)
  against the dequantize-then-matmul form;
* invariants: a consistent permutation of 128-blocks along the contraction
  leaves the result unchanged; dgrad equals fprop against the transposed
  weight; wgrad(a, b) is the transpose of wgrad(b, a).
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import (
    E4M3,
    E5M2,
    bf16_bits_to_f64,
    gemm_dgrad,
    gemm_dgrad_blockloops,
    gemm_fprop,
    gemm_fprop_blockloops,
    gemm_wgrad,
    gemm_wgrad_blockloops,
    quant_act_128x1,
    quant_act_1x128,
    quant_weight_128x128,
    dequant_weight_128x128,
    to_bf16_rne,
)


# --------------------------------------------------------------------------
# BF16 rounding
# --------------------------------------------------------------------------

def test_bf16_closed_forms():
    cases = [
        (1.0, 1.0),
        (1 + 2.0 ** -8, 1.0),  # tie -> even (mantissa 0)
        (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),  # tie -> even (mantissa 2)
        (1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -7),  # just above the tie
        (1 + 2.0 ** -8 - 2.0 ** -40, 1.0),
        (2 - 2.0 ** -9, 2.0),  # carry into the exponent
        (-(1 + 3 * 2.0 ** -8), -(1 + 2.0 ** -6)),
        (1.5 * 2.0 ** -133, 2.0 ** -132),  # subnormal tie -> even
        (2.0 ** -134, 0.0),  # subnormal tie -> zero
        (3.0 * 2.0 ** -126, 3.0 * 2.0 ** -126),
        (0.0, 0.0),
    ]
    for v, exp in cases:
        assert to_bf16_rne(np.float64(v)) == exp, v


def test_bf16_matches_torch_on_fp32_values():
    x = synth.random_f32((1 << 20,), seed=21).numpy() * np.float32(1e3)
    x = np.concatenate([x, x * np.float32(1e-30), x * np.float32(1e30)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(to_bf16_rne(x.astype(np.float64)), bf16_bits_to_f64(ref))


def test_bf16_bits_decode():
    assert bf16_bits_to_f64(np.uint16(0x3F80)) == 1.0
    assert bf16_bits_to_f64(np.uint16(0xC000)) == -2.0
    assert bf16_bits_to_f64(np.uint16(0x0001)) == 2.0 ** -133


# --------------------------------------------------------------------------
# hand-computable products
# --------------------------------------------------------------------------

def test_fprop_one_hot_rows():
    K, N = 256, 128
    w = synth.random_bf16((N, K), seed=22, std=0.02).float().numpy()
    qw, sw = quant_weight_128x128(w, E4M3)
    wdq = dequant_weight_128x128(qw, sw, E4M3)
    ks = [0, 5, 127, 128, 200, 255]
    x = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        x[i, k] = 448.0
    qx, sx = quant_act_1x128(x, E4M3)
    for i, k in enumerate(ks):
        assert qx[i, k] == 0x7E
        assert sx[i, k // 128] == 1.0
    y = gemm_fprop(qx, sx, E4M3, qw, sw, E4M3)
    for i, k in enumerate(ks):
        assert np.array_equal(y[i], 448.0 * wdq[:, k])


# --------------------------------------------------------------------------
# exact rational brute force
# --------------------------------------------------------------------------

def _frac_decode(code, fmt):
    """Bit-field decode into an exact Fraction (its own implementation)."""
    ebits, mbits, bias = (4, 3, 7) if fmt == E4M3 else (5, 2, 15)
    sign = -1 if code & 0x80 else 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    f = code & ((1 << mbits) - 1)
    if e == 0:
        return sign * Fraction(f, 1 << mbits) * Fraction(2) ** (1 - bias)
    return sign * (1 + Fraction(f, 1 << mbits)) * Fraction(2) ** (e - bias)


def _exact_matmul(a_q, a_s_full, fa, b_q, b_s_full, fb):
    """Exact sum_k (dec(a)*sa)[i,k] * (dec(b)*sb)[j,k] with Fractions."""
    I, K = a_q.shape
    J = b_q.shape[0]
    A = [[_frac_decode(int(a_q[i, k]), fa) * Fraction(float(a_s_full[i, k])) for k in range(K)] for i in range(I)]
    B = [[_frac_decode(int(b_q[j, k]), fb) * Fraction(float(b_s_full[j, k])) for k in range(K)] for j in range(J)]
    return [[sum(A[i][k] * B[j][k] for k in range(K)) for j in range(J)] for i in range(I)]


def _close(y64, exact, rel=1e-14):
    for i, row in enumerate(exact):
        for j, v in enumerate(row):
            assert abs(Fraction(float(y64[i, j])) - v) <= rel * (abs(v) + Fraction(1, 10 ** 30)), (i, j)


def test_fprop_exact_rational():
    x = synth.random_bf16((2, 256), seed=23, outliers=True).float().numpy()
    w = synth.random_bf16((128, 256), seed=24, std=0.02).float().numpy()
    qx, sx = quant_act_1x128(x, E4M3)
    qw, sw = quant_weight_128x128(w, E4M3)
    y = gemm_fprop(qx, sx, E4M3, qw, sw, E4M3)
    cols = [0, 1, 77, 127]
    sxf = np.repeat(sx, 128, axis=1)
    swf = np.repeat(np.repeat(sw, 128, axis=0), 128, axis=1)
    exact = _exact_matmul(qx, sxf, E4M3, qw[cols], swf[cols], E4M3)
    _close(y[:, cols], exact)


def test_dgrad_exact_rational():
    dy = synth.random_bf16((2, 256), seed=25, std=1e-3).float().numpy()
    w = synth.random_bf16((256, 128), seed=26, std=0.02).float().numpy()
    qdy, sdy = quant_act_1x128(dy, E5M2)
    qw, sw = quant_weight_128x128(w, E4M3)
    y = gemm_dgrad(qdy, sdy, E5M2, qw, sw, E4M3)
    cols = [0, 3, 64, 127]
    sdyf = np.repeat(sdy, 128, axis=1)
    swf = np.repeat(np.repeat(sw, 128, axis=0), 128, axis=1)
    # dX[m, k] = sum_n dY[m, n] W[n, k]: contract over n, so B rows are W columns
    exact = _exact_matmul(qdy, sdyf, E5M2, qw.T[cols], swf.T[cols], E4M3)
    _close(y[:, cols], exact)


def test_wgrad_exact_rational():
    dy = synth.random_bf16((256, 3), seed=27, std=1e-3).float().numpy()
    x = synth.random_bf16((256, 4), seed=28, outliers=True).float().numpy()
    qdy, sdy = quant_act_128x1(dy, E4M3)
    qx, sx = quant_act_128x1(x, E4M3)
    y = gemm_wgrad(qdy, sdy, E4M3, qx, sx, E4M3)
    sdyf = np.repeat(sdy, 128, axis=0)
    sxf = np.repeat(sx, 128, axis=0)
    exact = _exact_matmul(qdy.T, sdyf.T, E4M3, qx.T, sxf.T, E4M3)
    _close(y, exact)


# --------------------------------------------------------------------------
# per-block form vs dequantize-then-matmul (the 256 x 256 tiny-check sizes)
# --------------------------------------------------------------------------

def _rel(a, b):
    return np.max(np.abs(a - b)) / np.max(np.abs(b))


def test_blockloops_agree_tiny_check():
    c = synth.tiny_check()
    A, W, dY = c["A"].numpy(), c["W"].numpy(), c["dY"].numpy()
    qa, sa = quant_act_1x128(A, E4M3)
    qw, sw = quant_weight_128x128(W, E4M3)
    assert _rel(gemm_fprop_blockloops(qa, sa, E4M3, qw, sw, E4M3), gemm_fprop(qa, sa, E4M3, qw, sw, E4M3)) <= 1e-12
    qdy, sdy = quant_act_1x128(dY, E5M2)
    assert _rel(gemm_dgrad_blockloops(qdy, sdy, E5M2, qw, sw, E4M3), gemm_dgrad(qdy, sdy, E5M2, qw, sw, E4M3)) <= 1e-12
    qdyt, sdyt = quant_act_128x1(dY, E4M3)
    qat, sat = quant_act_128x1(A, E4M3)
    assert _rel(gemm_wgrad_blockloops(qdyt, sdyt, E4M3, qat, sat, E4M3), gemm_wgrad(qdyt, sdyt, E4M3, qat, sat, E4M3)) <= 1e-12


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_kblock_permutation_invariance():
    x = synth.random_bf16((64, 512), seed=29, outliers=True).float().numpy()
    w = synth.random_bf16((256, 512), seed=30, std=0.02).float().numpy()
    qx, sx = quant_act_1x128(x, E4M3)
    qw, sw = quant_weight_128x128(w, E4M3)
    y = gemm_fprop(qx, sx, E4M3, qw, sw, E4M3)
    for perm in list(itertools.permutations(range(4)))[1:6]:
        cols = np.concatenate([np.arange(p * 128, (p + 1) * 128) for p in perm])
        yp = gemm_fprop(qx[:, cols], sx[:, list(perm)], E4M3, qw[:, cols], sw[:, list(perm)], E4M3)
        assert _rel(yp, y) <= 1e-13
    # quantizing the permuted inputs gives the permuted codes and scales
    cols = np.concatenate([np.arange(p * 128, (p + 1) * 128) for p in (2, 0, 3, 1)])
    qx2, sx2 = quant_act_1x128(x[:, cols], E4M3)
    assert np.array_equal(qx2, qx[:, cols]) and np.array_equal(sx2, sx[:, [2, 0, 3, 1]])


def test_dgrad_is_fprop_against_transposed_weight():
    dy = synth.random_bf16((96, 256), seed=31, std=1e-3).float().numpy()
    w = synth.random_bf16((256, 384), seed=32, std=0.02).float().numpy()
    qdy, sdy = quant_act_1x128(dy, E4M3)
    qw, sw = quant_weight_128x128(w, E4M3)
    qwt, swt = quant_weight_128x128(np.ascontiguousarray(w.T), E4M3)
    assert np.array_equal(qwt, qw.T) and np.array_equal(swt, sw.T)
    assert _rel(gemm_dgrad(qdy, sdy, E4M3, qw, sw, E4M3), gemm_fprop(qdy, sdy, E4M3, qwt, swt, E4M3)) <= 1e-13


def test_wgrad_transpose_symmetry():
    a = synth.random_bf16((384, 40), seed=33, std=1e-3).float().numpy()
    b = synth.random_bf16((384, 24), seed=34).float().numpy()
    qa, sa = quant_act_128x1(a, E5M2)
    qb, sb = quant_act_128x1(b, E4M3)
    assert _rel(gemm_wgrad(qa, sa, E5M2, qb, sb, E4M3).T, gemm_wgrad(qb, sb, E4M3, qa, sa, E5M2)) <= 1e-13
