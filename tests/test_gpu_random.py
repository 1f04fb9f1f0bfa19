"""Seeded random shapes for the whole path, against the oracle: token counts that are not multiples
of 128 (fprop, dgrad), feature sizes that are, both FP8 formats for the gradient, BF16 and FP32
outputs.  Each case checks the dual activation quantizer bit for bit (both layouts) and all three
GEMMs to the GEMM acceptance rule, so odd combinations of tile shape, contraction split and ragged
edges chosen by the planner are all exercised."""

import numpy as np
import pytest
import torch

import fp8_blockwise_quantized_amd as fq
import oracle
import synth
from parity import FP, f32_bits, say
from test_gpu_gemm import checked, run_dgrad, run_fprop, run_wgrad

pytestmark = pytest.mark.gpu
DEV = "cuda"
E4, E5 = oracle.E4M3, oracle.E5M2


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.integers(1, 1600))
    N = 128 * int(rng.integers(1, 13))
    K = 128 * int(rng.integers(1, 13))
    fdy = E5 if rng.integers(2) else E4
    out = torch.float32 if rng.integers(3) == 0 else torch.bfloat16
    return M, N, K, fdy, out


@pytest.mark.parametrize("seed", range(48))
def test_random_shapes(seed):
    M, N, K, fdy, out = _case(seed)
    X = synth.random_bf16((M, K), seed=3 * seed + 1, outliers=seed % 2 == 0)
    W = synth.random_bf16((N, K), seed=3 * seed + 2, std=0.02)
    dY = synth.random_bf16((M, N), seed=3 * seed + 3, std=1e-3)
    f32 = out == torch.float32
    what = f"seed {seed}: M={M} N={N} K={K} dY {fdy} {'f32' if f32 else 'bf16'}"
    say(what)
    checked(run_fprop(X, W, out_dtype=out), what + " fprop", out_f32=f32)
    checked(run_dgrad(dY, W, fdy=fdy, out_dtype=out), what + " dgrad", out_f32=f32)
    # wgrad and the 128x1 groups need whole 128-token blocks
    Mw = max(128, (M // 128) * 128)
    Xw = synth.random_bf16((Mw, K), seed=3 * seed + 4)
    dYw = synth.random_bf16((Mw, N), seed=3 * seed + 5, std=1e-3)
    checked(run_wgrad(dYw, Xw, fdy=fdy, out_dtype=out), what + f" wgrad (M={Mw})", out_f32=f32)
    q, s, qt, st = fq.quantize_act_dual(Xw.to(DEV), FP[E4], FP[fdy])
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_act_1x128(Xw.float().numpy(), E4)
    oqt, ost = oracle.quant_act_128x1(Xw.float().numpy(), fdy)
    # device layouts: s is [C/128, R] (group-major), qt is [C, R] (tokens contiguous)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(f32_bits(s.cpu().numpy().T), f32_bits(os_))
    assert np.array_equal(qt.cpu().numpy().T, oqt) and np.array_equal(f32_bits(st.cpu().numpy()), f32_bits(ost))
