"""Pins for the oracle's blockwise quantizers (CPU only).

What pins them, independent of the quantizer code:
* hand-computed single-group examples (tests/golden/quant_examples.txt);
* closed forms of the scale rule (powers of two, the 1e-12 floor);
* an exact-rational recomputation (Python Fractions) of both fp32 divisions
  with round-to-nearest-even, and of the cast by nearest-value search;
* the pages' own listing run in CPU PyTorch (its amax / 448, clamp(min=1e-12),
  divide, clamp, cast), applied group by group with explicit Python loops
  over the 1x128, 128x1 and 128x128 geometries;
* invariants: full-scale code at the amax position, sign symmetry,
  power-of-two equivariance, and the FP8 rounding-error bound.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import (
    E4M3,
    E5M2,
    SCALE_FLOOR,
    decode,
    fmt_max,
    quant_act_128x1,
    quant_act_1x128,
    quant_weight_128x128,
    quantize_group_rows,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_examples.txt")
TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
MAXCODE = {E4M3: 0x7E, E5M2: 0x7B}


def f32_bits(x):
    return int(np.float32(x).view(np.uint32))


# --------------------------------------------------------------------------
# golden examples
# --------------------------------------------------------------------------

def _golden_examples():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, s_hex, vals, codes = [p.strip() for p in line.split(";")]
            x = np.zeros(128, np.float32)
            for tok in vals.split():
                i, v = tok.split(":")
                x[int(i)] = np.float32(float(v))
            exp = {int(tok.split(":")[0]): int(tok.split(":")[1], 16) for tok in codes.split()}
            out.append((fmt, int(s_hex, 16), x, exp))
    return out


@pytest.mark.parametrize("case", range(4))
def test_golden_examples(case):
    fmt, s_bits, x, exp = _golden_examples()[case]
    q, s = quantize_group_rows(x[None, :], fmt)
    assert f32_bits(s[0]) == s_bits
    for i, c in exp.items():
        assert int(q[0, i]) == c, (i, hex(int(q[0, i])), hex(c))


def test_floor_bits_from_golden():
    with open(os.path.join(os.path.dirname(__file__), "golden", "fp8_formats.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    floor = [r for r in rows if r[0] == "floor"][0]
    assert f32_bits(SCALE_FLOOR) == int(floor[2], 16)
    assert float(SCALE_FLOOR) == float(np.float32(float(floor[1])))


# --------------------------------------------------------------------------
# closed forms of the scale rule
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_scale_power_of_two_closed_form(fmt):
    m = fmt_max(fmt)
    for j in range(-20, 21):
        x = np.zeros((1, 128), np.float32)
        x[0, 17] = np.float32(m * 2.0 ** j)
        x[0, 3] = np.float32(-m * 2.0 ** j / 3)
        q, s = quantize_group_rows(x, fmt)
        assert float(s[0]) == 2.0 ** j
        assert int(q[0, 17]) == MAXCODE[fmt]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_scale_floor(fmt):
    # all-zero group and a group whose amax/fmt_max is below 1e-12
    for amax in (0.0, 1e-13):
        x = np.zeros((1, 128), np.float32)
        x[0, 5] = np.float32(amax)
        q, s = quantize_group_rows(x, fmt)
        assert f32_bits(s[0]) == 0x2B8CBCCC
    # -0.0 entries keep their sign
    x = np.full((1, 128), -0.0, np.float32)
    q, s = quantize_group_rows(x, fmt)
    assert np.all(q == 0x80)


# --------------------------------------------------------------------------
# exact-rational recomputation of the fp32 divisions and the cast
# --------------------------------------------------------------------------

def _rn_f32(fr: Fraction) -> Fraction:
    """Round a rational to the nearest fp32 value, ties to even (finite range)."""
    if fr == 0:
        return Fraction(0)
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** max(e - 23, -149)
    n = a / quantum
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    return -r if neg else r


def _nearest_code(y: Fraction, fmt) -> int:
    tab = decode(np.arange(256, dtype=np.uint8), fmt)
    best, bestd = None, None
    for c in range(128):
        v = tab[c]
        if not np.isfinite(v):
            continue
        d = abs(abs(y) - Fraction(v))
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best | (0x80 if y < 0 else 0)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_exact_rational_recomputation(fmt):
    fm = Fraction(int(fmt_max(fmt)))
    floor = Fraction(float(SCALE_FLOOR))
    x = synth.random_bf16((3, 128), seed=11, outliers=True).float().numpy()
    x[2] *= np.float32(1e-3)
    q, s = quantize_group_rows(x, fmt)
    for g in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in x[g])
        sg = max(_rn_f32(amax / fm), floor)
        assert Fraction(float(s[g])) == sg
        for i in range(0, 128, 3):
            y = _rn_f32(Fraction(float(x[g, i])) / sg)
            y = max(min(y, fm), -fm)
            c = _nearest_code(y, fmt)
            if y == 0 and np.signbit(x[g, i]):
                c = 0x80
            assert int(q[g, i]) == c, (g, i, float(x[g, i]))


# --------------------------------------------------------------------------
# the pages' listing, run in CPU torch, group by group
# --------------------------------------------------------------------------

def listing_quantize(group_t: torch.Tensor, fmt):
    """The listing's per-tensor rule applied to one group (a torch tensor of
    bf16 or fp32 values): amax in an fp32 buffer, amax / max clamped at 1e-12,
    divide, clamp, cast."""
    m = fmt_max(fmt)
    amax = group_t.abs().max().detach().float().reshape(1)
    scale = (amax / m).clamp(min=1e-12)
    y = (group_t / scale).clamp(-m, m)
    return y.to(TORCH_DT[fmt]).view(torch.uint8), scale


def test_listing_dtype_promotion_is_fp32():
    x = torch.ones(4, dtype=torch.bfloat16)
    scale = torch.ones(1)
    assert (x / scale).dtype == torch.float32


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_1x128_matches_listing_loops(fmt, dtype):
    R, C = 5, 384
    xt = synth.random_bf16((R, C), seed=3, outliers=True) if dtype == "bf16" else synth.random_f32((R, C), seed=3)
    xt[1, 128:256] = 0
    q, s = quant_act_1x128(xt.float().numpy(), fmt)
    assert q.shape == (R, C) and s.shape == (R, C // 128)
    for r in range(R):
        for g in range(C // 128):
            qq, ss = listing_quantize(xt[r, g * 128:(g + 1) * 128], fmt)
            assert np.array_equal(q[r, g * 128:(g + 1) * 128], qq.numpy())
            assert f32_bits(s[r, g]) == f32_bits(ss.item())


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_128x1_matches_listing_loops(fmt):
    R, C = 256, 7
    xt = synth.random_bf16((R, C), seed=4, outliers=True)
    q, s = quant_act_128x1(xt.float().numpy(), fmt)
    assert q.shape == (R, C) and s.shape == (R // 128, C)
    for rb in range(R // 128):
        for c in range(C):
            qq, ss = listing_quantize(xt[rb * 128:(rb + 1) * 128, c], fmt)
            assert np.array_equal(q[rb * 128:(rb + 1) * 128, c], qq.numpy())
            assert f32_bits(s[rb, c]) == f32_bits(ss.item())


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_128x128_matches_listing_loops(fmt):
    N, K = 256, 384
    wt = synth.random_bf16((N, K), seed=5, std=0.02)
    q, s = quant_weight_128x128(wt.float().numpy(), fmt)
    assert s.shape == (2, 3)
    for nb in range(N // 128):
        for kb in range(K // 128):
            blk = wt[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            qq, ss = listing_quantize(blk, fmt)
            assert np.array_equal(q[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128], qq.numpy())
            assert f32_bits(s[nb, kb]) == f32_bits(ss.item())


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_full_scale_code_at_amax(fmt):
    x = synth.random_bf16((64, 256), seed=6, outliers=True).float().numpy()
    q, s = quant_act_1x128(x, fmt)
    xg = np.abs(x.reshape(64, 2, 128))
    qg = q.reshape(64, 2, 128) & 0x7F
    at_max = xg == xg.max(axis=2, keepdims=True)
    assert np.all(qg[at_max] == MAXCODE[fmt])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_sign_symmetry(fmt):
    x = synth.random_bf16((32, 256), seed=7).float().numpy()
    q1, s1 = quant_act_1x128(x, fmt)
    q2, s2 = quant_act_1x128(-x, fmt)
    assert np.array_equal(s1, s2)
    assert np.array_equal(q1 ^ 0x80, q2)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_power_of_two_equivariance(fmt):
    x = synth.random_bf16((32, 256), seed=8).float().numpy()
    q0, s0 = quant_act_1x128(x, fmt)
    for j in (-12, -3, 1, 9):
        qj, sj = quant_act_1x128(x * np.float32(2.0 ** j), fmt)
        assert np.array_equal(qj, q0)
        assert np.array_equal(sj, s0 * np.float32(2.0 ** j))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_rounding_error_bound(fmt):
    x = synth.random_bf16((128, 512), seed=9, outliers=True).float().numpy().astype(np.float64)
    q, s = quant_act_1x128(x.astype(np.float32), fmt)
    dq = decode(q, fmt) * np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(dq - x)
    mbits = 3 if fmt == E4M3 else 2
    min_normal = 2.0 ** -6 if fmt == E4M3 else 2.0 ** -14
    sub_q = 2.0 ** -9 if fmt == E4M3 else 2.0 ** -16
    sfull = np.repeat(s.astype(np.float64), 128, axis=1)
    y = np.abs(x) / sfull
    normal = y >= min_normal
    # half a unit in the last place, plus a small allowance for the fp32 division
    rel = 2.0 ** -(mbits + 1) * (1 + 1e-6) + 1e-6
    assert np.all(err[normal] <= rel * np.abs(x[normal]))
    assert np.all(err[~normal] <= (sub_q / 2) * sfull[~normal] * (1 + 1e-5) + 1e-6 * np.abs(x[~normal]))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_1x128_matches_listing_vectorized(fmt):
    """The listing's rule with one fp32 amax buffer per group, over 2M values
    (enough that a reciprocal-multiply or wrong-rounding mistake, which moves
    a few codes in ten thousand, is certain to show)."""
    xt = synth.random_bf16((1024, 2048), seed=10, outliers=True)
    q, s = quant_act_1x128(xt.float().numpy(), fmt)
    m = fmt_max(fmt)
    g = xt.reshape(-1, 128)
    amax = g.abs().amax(dim=1, keepdim=True).float()
    scale = (amax / m).clamp(min=1e-12)
    ref = (g / scale).clamp(-m, m).to(TORCH_DT[fmt]).view(torch.uint8).reshape(1024, 2048)
    assert np.array_equal(q, ref.numpy())
    assert np.array_equal(s.reshape(-1).view(np.uint32), scale.reshape(-1).numpy().view(np.uint32))
