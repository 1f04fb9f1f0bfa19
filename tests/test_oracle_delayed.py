"""Pins for the oracle's per-tensor delayed-scaling functions (CPU only).

What pins them, independent of the code under test:
* the fp32 bit patterns of the update's two multipliers for the listing's beta = 0.99
  (0.99 -> 0x3F7D70A4; 1 - 0.99 formed in double -> 0x3C23D70A, not fp32(1 - fp32(0.99)));
* an exact-rational recomputation (Python Fractions) of the update with one fp32 rounding per
  product and one for the sum, and for a BF16 tensor one more rounding of the weighted current
  amax to BF16 (the product has the tensor's type in the listing);
* the closed form of the recurrence under a constant input, c + (a0 - c) beta^n;
* the special cases beta = 0 (the running amax is the current amax, so the per-tensor rule is the
  blockwise rule with the whole tensor as one group) and beta = 1 (the amax never moves);
* a hand-computed double-rounding case that only the BF16 copy of the input produces;
* the pages' listing run verbatim in CPU PyTorch on FP32 and on BF16 tensors (current amax of the
  tensor as given, in-place decay and add on a one-element fp32 buffer, amax / fmt_max,
  clamp(min=1e-12), BF16 copy, divide, clamp, cast), step by step;
* that the BF16 rounding of the weighted current amax matters: on BF16 tensors the update without
  it disagrees with the listing;
* for the GEMM: equality with the blockwise oracle GEMM under uniform scales, a hand-computable
  product and exact linearity in the scales.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import (
    E4M3,
    E5M2,
    SCALE_FLOOR,
    amax_ema_update,
    decode,
    ema_constants,
    fmt_max,
    gemm_fprop,
    gemm_tensor,
    quant_tensor,
    quant_tensor_delayed,
    quant_weight_128x128,
    quantize_group_rows,
    tensor_scale,
)

TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def bits(v):
    return int(np.asarray(v, dtype=np.float32).view(np.uint32))


def _rn_f32(fr: Fraction, mant: int = 23) -> Fraction:
    """Round an exact rational to the nearest binary value with `mant` fraction bits (fp32: 23,
    BF16: 7), ties to even, normal range only."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (e - mant)
    fl = a // quantum
    rem = a / quantum - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def test_multipliers_for_the_listing_beta():
    b1, b2 = ema_constants(0.99)
    assert bits(b1) == 0x3F7D70A4
    assert bits(b2) == 0x3C23D70A  # fp32(0.010000000000000009), the double 1 - 0.99 rounded once


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta", [0.99, 0.9, 0.5])
def test_update_matches_exact_rational(beta, in_dtype):
    rng = np.random.default_rng(3)
    b1, b2 = (Fraction(float(c)) for c in ema_constants(beta))
    for _ in range(200):
        a0 = np.float32(rng.uniform(0.01, 100.0))
        x = (rng.standard_normal(64) * rng.uniform(0.01, 50.0)).astype(np.float32)
        if in_dtype == "bf16":  # BF16-valued elements (truncate to 8 significant bits: exact)
            x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
        cur = max(abs(Fraction(float(v))) for v in x)
        fresh = _rn_f32(cur * b2)
        if in_dtype == "bf16":
            fresh = _rn_f32(fresh, 7)
        want = _rn_f32(_rn_f32(Fraction(float(a0)) * b1) + fresh)
        assert Fraction(float(amax_ema_update(a0, x, beta, in_dtype))) == want


@pytest.mark.parametrize("a0,c", [(1.0, 448.0), (1000.0, 3.5), (2.0, 2.0)])
def test_constant_input_follows_the_closed_form(a0, c):
    beta = 0.99
    a = np.float32(a0)
    x = np.array([c, -c / 2], np.float32)
    for n in range(1, 501):
        a = amax_ema_update(a, x, beta, "f32")
        exact = c + (a0 - c) * beta ** n
        # each step adds at most 1.5 fp32 ulps, and beta shrinks earlier errors: <= 150 ulps in all
        assert abs(float(a) - exact) <= 150 * 2.0 ** -23 * max(a0, c), (n, float(a), exact)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_beta_zero_is_the_rule_with_one_group(fmt):
    x = synth.random_bf16((64, 256), seed=21, outliers=True).float().numpy()
    q, s, a = quant_tensor_delayed(x, np.float32(7.0), 0.0, fmt, "bf16")
    qg, sg = quantize_group_rows(x.reshape(1, -1), fmt)
    assert bits(a) == bits(np.max(np.abs(x)))
    assert bits(s) == bits(sg[0])
    assert np.array_equal(q, qg.reshape(x.shape))
    # and it agrees with the blockwise quantizers on a single 128x128 tile
    t = x[:, :128].copy()
    t = np.concatenate([t, t], axis=0)  # 128 x 128
    qt, st, _ = quant_tensor_delayed(t, np.float32(1.0), 0.0, fmt, "bf16")
    qw, sw = quant_weight_128x128(t, fmt)
    assert np.array_equal(qt, qw) and bits(st) == bits(sw[0, 0])


def test_beta_one_keeps_the_running_amax():
    x = np.array([[3.0, -900.0]], np.float32)
    assert bits(amax_ema_update(np.float32(12.5), x, 1.0, "f32")) == bits(12.5)
    assert bits(amax_ema_update(np.float32(12.5), x, 1.0, "bf16")) == bits(12.5)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("j", [-20, -3, 0, 5])
def test_power_of_two_scale(fmt, j):
    a = np.float32(fmt_max(fmt) * 2.0 ** j)
    s = tensor_scale(a, fmt)
    assert bits(s) == bits(np.float32(2.0 ** j))
    q = quant_tensor(np.array([[a, -a]], np.float32), s, fmt)
    top = 0x7E if fmt == E4M3 else 0x7B
    assert q.tolist() == [[top, top | 0x80]]


def test_scale_floor_for_a_zero_amax():
    assert bits(tensor_scale(np.float32(0.0), E4M3)) == bits(SCALE_FLOOR) == 0x2B8CBCCC


def test_bf16_copy_decides_a_tie():
    """1 + 2^-4 + 2^-9 (fp32) lies just above the E4M3 midpoint between 1.0 and 1.125, but its BF16
    copy is 1 + 2^-4 exactly: the midpoint, which goes to the even code 1.0 (0x38).  The element 448
    fixes amax = 448 and s = 1 with beta = 0."""
    x = np.array([[448.0, 1 + 2.0 ** -4 + 2.0 ** -9]], np.float32)
    q, s, a = quant_tensor_delayed(x, np.float32(1.0), 0.0, E4M3, "f32")
    assert bits(s) == bits(1.0) and bits(a) == bits(448.0)
    assert q.tolist() == [[0x7E, 0x38]]  # without the BF16 copy the second code would be 0x39


def _listing_steps(xs, fmt, beta=0.99):
    """The listing's _update_amax and _quantize, verbatim in CPU torch, over the tensors xs (one
    running amax buffer, initialized to one as the listing registers it).  Yields (buffer, scale,
    codes) after each tensor."""
    fm = fmt_max(fmt)
    buf = torch.ones(1)
    for xt in xs:
        current_amax = xt.abs().max().detach()
        buf.mul_(beta).add_(current_amax * (1 - beta))
        scale = (buf / fm).clamp(min=1e-12)
        codes = (xt.bfloat16() / scale).clamp(-fm, fm).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
        yield buf.numpy()[0].copy(), scale.numpy()[0].copy(), codes


def _listing_inputs(src_dtype, n=3, shape=(32, 256), mags=(1.0, 40.0, 0.05)):
    return [(torch.from_numpy(np.random.default_rng(step).standard_normal(shape).astype(np.float32))
             * mags[step % len(mags)]).to(src_dtype) for step in range(n)]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("src_dtype", [torch.float32, torch.bfloat16])
def test_matches_the_listing_in_torch(fmt, src_dtype):
    """Three steps of the listing's running-amax update and quantization, verbatim in CPU PyTorch
    on an FP32 or a BF16 tensor, against the oracle told the tensor's type."""
    xs = _listing_inputs(src_dtype)
    in_dtype = "bf16" if src_dtype == torch.bfloat16 else "f32"
    a = np.float32(1.0)
    for step, (xt, (buf, scale, codes)) in enumerate(zip(xs, _listing_steps(xs, fmt))):
        q, s, a = quant_tensor_delayed(xt.float().numpy(), a, 0.99, fmt, in_dtype)
        assert bits(a) == bits(buf), step
        assert bits(s) == bits(scale), step
        assert np.array_equal(q, codes), step


def test_bf16_rounding_of_the_weighted_amax_matters():
    """Over 200 BF16 tensors the listing's running amax equals the oracle's BF16 reading at every
    step, while an update that keeps the weighted current amax in fp32 departs from it."""
    xs = _listing_inputs(torch.bfloat16, n=200, shape=(8, 128), mags=(1.0, 3.0, 0.3, 17.0, 0.02))
    a_bf16 = a_f32 = np.float32(1.0)
    departs = 0
    for step, (xt, (buf, _, _)) in enumerate(zip(xs, _listing_steps(xs, E4M3))):
        xf = xt.float().numpy()
        a_bf16 = amax_ema_update(a_bf16, xf, 0.99, "bf16")
        assert bits(a_bf16) == bits(buf), step
        a_f32 = amax_ema_update(a_f32, xf, 0.99, "f32")
        departs += bits(a_f32) != bits(buf)
    assert departs > 100


def test_gemm_equals_blockwise_gemm_with_uniform_scales():
    X = synth.random_bf16((96, 256), seed=31, outliers=True).float().numpy()
    W = synth.random_bf16((128, 256), seed=32, std=0.02).float().numpy()
    qx, sx, _ = quant_tensor_delayed(X, np.float32(1.0), 0.5, E4M3, "bf16")
    qw, sw, _ = quant_tensor_delayed(W, np.float32(1.0), 0.5, E4M3, "bf16")
    y = gemm_tensor(qx, sx, E4M3, qw, sw, E4M3)
    yb = gemm_fprop(qx, np.full((96, 2), sx, np.float32), E4M3, qw, np.full((1, 2), sw, np.float32), E4M3)
    assert np.array_equal(y, yb)


def test_gemm_hand_computed():
    # A rows 448 e_k with scale 1 are code 0x7E at column k: Y[i, j] = 448 * B_dq[j, k_i]
    qa = np.zeros((3, 128), np.uint8)
    ks = [0, 77, 127]
    for i, k in enumerate(ks):
        qa[i, k] = 0x7E
    qb = np.random.default_rng(5).integers(0, 0x7E, size=(4, 128)).astype(np.uint8)
    y = gemm_tensor(qa, np.float32(1.0), E4M3, qb, np.float32(0.25), E4M3)
    bq = decode(qb, E4M3) * 0.25
    for i, k in enumerate(ks):
        assert np.array_equal(y[i], 448.0 * bq[:, k])


def test_gemm_linear_in_the_scales():
    rng = np.random.default_rng(6)
    qa = rng.integers(0, 0x7E, size=(8, 256)).astype(np.uint8)
    qb = rng.integers(0, 0x7B, size=(16, 256)).astype(np.uint8)
    y1 = gemm_tensor(qa, np.float32(0.5), E4M3, qb, np.float32(3.0), E5M2)
    y2 = gemm_tensor(qa, np.float32(1.0), E4M3, qb, np.float32(3.0), E5M2)
    assert np.array_equal(2.0 * y1, y2)
