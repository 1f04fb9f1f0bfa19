"""Shared helpers for the GPU parity tests: device transfers and the GEMM acceptance rule.

GEMM acceptance (for every sampled output element (i, j)):
  * |Y_gpu - Y64| <= 2e-3 * ||A_dq[i, :]||_2 * ||B_dq[j, :]||_2, where Y64 is the oracle's unrounded
    float64 result and A_dq / B_dq are the oracle's dequantized contraction vectors;
  * ||Y_gpu - bf16(Y64)||_F / ||bf16(Y64)||_F <= 1e-3 over the sample (the reference is rounded to
    BF16 because BF16 output rounding alone is about 1.65e-3 relative to unrounded float64).
FP32 outputs are held to 1e-4 of the same Cauchy-Schwarz bound: the FP8 MFMA's internal sum of a
128-long block is not a correctly rounded FP32 sum (about 2.5e-5 of the bound was seen on same-sign
data), and the per-block fold adds FP32 rounding.

For degenerate inputs whose rows are parallel (|y| close to ||a|| ||b||), rounding the output to BF16
alone (up to 2^-8 relative) exceeds 2e-3 ||a|| ||b||, so no BF16-output GEMM can meet the first rule
there; such cases are held to the same bound on the error beyond the output rounding,
|Y_gpu - bf16(Y64)| <= 2e-3 ||a|| ||b|| (check_gemm(..., beyond_rounding=True)).
"""

import sys

import numpy as np
import torch

import oracle

FP = {oracle.E4M3: 0, oracle.E5M2: 1}
GEMM_ABS = 2e-3
GEMM_FRO = 1e-3
F32_ABS = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def to_np_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        t.detach().cpu().numpy().astype(np.float64)


def check_gemm(y_gpu, y64, a_norm, b_norm, out_f32=False, what="", beyond_rounding=False):
    """y_gpu, y64: float64 [I, J]; a_norm [I], b_norm [J] (L2 norms of the dequantized operands)."""
    bound = np.outer(a_norm, b_norm)
    err = np.abs(y_gpu - (oracle.to_bf16_rne(y64) if beyond_rounding else y64))
    lim = (F32_ABS if out_f32 else GEMM_ABS) * bound
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    assert np.all(err <= lim), f"{what}: max |err| / (|a||b|) = {worst:.3e}"
    if out_f32:
        return worst, 0.0
    ref = oracle.to_bf16_rne(y64)
    den = np.linalg.norm(ref)
    fro = float(np.linalg.norm(y_gpu - ref) / den) if den > 0 else float(np.linalg.norm(y_gpu - ref))
    assert fro <= GEMM_FRO, f"{what}: relative Frobenius {fro:.3e}"
    return worst, fro


def row_norms(m):
    return np.sqrt(np.sum(np.asarray(m, np.float64) ** 2, axis=1))
