"""Seeded synthetic inputs for the FP8 blockwise linear layer.

This module only draws random numbers and rounds them to the input dtype.
It holds none of the method's arithmetic (no amax, scale, division, FP8
encoding or GEMM), so both the HIP path and the CPU oracle can consume its
tensors.

Every tensor comes from its own NumPy PCG64 stream, spawned from
``np.random.SeedSequence(seed)`` in a fixed order; fp32 draws are rounded to
BF16 (round-to-nearest-even) where the workload is BF16.  Distributions:
"N(0, s)" has standard deviation s; "outliers" multiplies floor(1% of the
columns), chosen by a seeded permutation, by 50 before BF16 rounding;
Student-t uses nu = 3.

Workloads (shapes follow a 2B-class decoder: hidden 2048, GQA with 16 query
and 2 key/value heads of 128, SwiGLU intermediate 5632):

1. tiny check, seed 0: A[256, 256] fp32 N(0,1), W[256, 256] fp32 N(0,0.02),
   dY[256, 256] fp32 N(0,1e-3);
2. single fprop linear, seed 1: X[8192, 2048] bf16 N(0,1) with outliers,
   W[8192, 2048] bf16 N(0,0.02);
3. one decoder block at M = 16384 tokens, seed 2: per linear X[M, K] N(0,1),
   W[N, K] N(0,0.02), dY[M, N] N(0,1e-3), for QKV 2048->2560, O 2048->2048,
   gate+up 2048->11264, down 5632->2048;
4. square-weight sweep, seed 3: W[2048, 2048] N(0,0.02), X[M, 2048] N(0,1)
   for M in 512 .. 32768;
5. heavy-tailed gradients, seed 4: dY[16384, 5632] Student-t(3) * 1e-3,
   X[16384, 2048] N(0,1) with outliers, W[5632, 2048] N(0,0.02).

Tensors too large to draw on the host (the beyond-4-GiB tests) come from
``device_normal_bf16``: torch's seeded generator on the device, N(0, s) in
fp32 rounded to BF16.
"""

import numpy as np
import torch

SEEDS = {"tiny": 0, "single": 1, "decoder": 2, "sweep": 3, "heavy": 4}

DECODER_LINEARS = (
    # name, K (in), N (out)
    ("qkv", 2048, 2560),
    ("o", 2048, 2048),
    ("gate_up", 2048, 11264),
    ("down", 5632, 2048),
)
DECODER_M = 16384
SWEEP_M = (512, 1024, 2048, 4096, 8192, 16384, 32768)


def _streams(seed, n):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _to_torch(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t


def normal(rng, shape, std, dtype=torch.bfloat16):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return _to_torch(a, dtype)


def normal_outliers(rng, shape, std, dtype=torch.bfloat16, frac=0.01, factor=50.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    ncols = shape[1]
    k = int(np.floor(frac * ncols))
    cols = rng.permutation(ncols)[:k]
    a[:, cols] *= np.float32(factor)
    return _to_torch(a, dtype)


def student_t(rng, shape, nu, scale, dtype=torch.bfloat16):
    a = rng.standard_t(nu, size=shape).astype(np.float32)
    a *= np.float32(scale)
    return _to_torch(a, dtype)


def tiny_check():
    r = _streams(SEEDS["tiny"], 3)
    return {
        "A": normal(r[0], (256, 256), 1.0, torch.float32),
        "W": normal(r[1], (256, 256), 0.02, torch.float32),
        "dY": normal(r[2], (256, 256), 1e-3, torch.float32),
    }


def single_linear():
    r = _streams(SEEDS["single"], 2)
    return {
        "X": normal_outliers(r[0], (8192, 2048), 1.0),
        "W": normal(r[1], (8192, 2048), 0.02),
    }


def decoder_linear(name, M=DECODER_M):
    """X, W, dY of one linear of the decoder block (independent streams)."""
    names = [n for n, _, _ in DECODER_LINEARS]
    i = names.index(name)
    _, K, N = DECODER_LINEARS[i]
    r = _streams(SEEDS["decoder"], 3 * len(DECODER_LINEARS))[3 * i: 3 * i + 3]
    return {
        "X": normal(r[0], (M, K), 1.0),
        "W": normal(r[1], (N, K), 0.02),
        "dY": normal(r[2], (M, N), 1e-3),
    }


def decoder_block(M=DECODER_M):
    return {n: decoder_linear(n, M) for n, _, _ in DECODER_LINEARS}


def sweep_weight():
    return normal(_streams(SEEDS["sweep"], 1 + len(SWEEP_M))[0], (2048, 2048), 0.02)


def sweep_x(M):
    i = SWEEP_M.index(M)
    return normal(_streams(SEEDS["sweep"], 1 + len(SWEEP_M))[1 + i], (M, 2048), 1.0)


def heavy_tailed():
    r = _streams(SEEDS["heavy"], 3)
    return {
        "dY": student_t(r[0], (16384, 5632), 3, 1e-3),
        "X": normal_outliers(r[1], (16384, 2048), 1.0),
        "W": normal(r[2], (5632, 2048), 0.02),
    }


def random_bf16(shape, seed, std=1.0, outliers=False):
    """Small ad-hoc inputs for tests (ragged shapes, edge cases)."""
    rng = _streams(seed, 1)[0]
    if outliers:
        return normal_outliers(rng, shape, std)
    return normal(rng, shape, std)


def random_f32(shape, seed, std=1.0):
    rng = _streams(seed, 1)[0]
    return normal(rng, shape, std, torch.float32)


def device_normal_bf16(shape, seed, device, std=1.0, chunk_rows=1 << 18):
    """N(0, std) BF16 tensor drawn on `device` by torch's generator seeded with `seed`, one block of
    rows at a time (for tensors of several GiB); the same seed gives the same tensor."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = (torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device) * std).to(torch.bfloat16)
    return out
