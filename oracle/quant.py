"""Blockwise FP8 quantizers: 1x128 (activations), 128x1 (token axis, for
wgrad) and 128x128 (weights).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The per-group rule is the one [HL] gives in ``FP8Linear._quantize`` (section
"核心挑战：Scale Factor 管理") and again in section "常见错误：直接转换而不加
Scale":

1. amax = max |x| over the group (exact, order-free);
2. s = amax / fmt_max, computed as an IEEE fp32 division rounded to nearest
   even (the listing keeps its amax buffers in fp32 and torch promotes a
   bf16/fp32 division by them to fp32);
3. s = max(s, fp32(1e-12))  (the listing's ``clamp(min=1e-12)``);
4. y = x / s, again an IEEE fp32 division (the listing divides; it does not
   multiply by a reciprocal);
5. y = clamp(y, -fmt_max, fmt_max) (this clamp is what saturates: the cast
   itself does not);
6. q = the nearest FP8 code of y, ties to even (the cast to
   ``float8_e4m3fn`` / ``float8_e5m2``).

Dequantization is decode(q) * s ([HL] ``forward``).

The pages use one scale per tensor with a running amax; the recipe of
[XZY] and [APD] replaces that with one scale per block taken from the
block's own amax: 1x128 groups for activations (consecutive elements of a
row, along the contraction axis), 128x128 tiles for weights.  The 128x1
geometry (128 consecutive rows of one column) is the same 1-D group laid
along the token axis, which wgrad contracts over; it is quantized from the
original high-precision tensor, not from the 1x128 codes (the pages are
silent; this reading avoids double rounding).

Inputs are float32 NumPy arrays (bf16 inputs are widened to fp32 exactly
before they get here).  Scales are returned as float32 in logical
coordinates: s[r, g] for 1x128, s[rb, c] for 128x1, s[nb, kb] for 128x128.
"""

import numpy as np

from .fp8_codec import encode, fmt_max

# fp32(1e-12): the listing's clamp floor for the scale.
SCALE_FLOOR = np.float32(1e-12)

GROUP = 128


def quantize_group_rows(xg, fmt):
    """Quantize each row of xg[G, n] (float32) as one group.

    Returns (codes uint8[G, n], scales float32[G]).
    """
    xg = np.asarray(xg, dtype=np.float32)
    if xg.ndim != 2:
        raise ValueError("quantize_group_rows expects a 2-D array")
    fmax = np.float32(fmt_max(fmt))
    amax = np.max(np.abs(xg), axis=1) if xg.shape[1] else np.zeros(xg.shape[0], np.float32)
    s = (amax.astype(np.float32) / fmax).astype(np.float32)  # IEEE fp32 divide
    s = np.maximum(s, SCALE_FLOOR).astype(np.float32)
    y = (xg / s[:, None]).astype(np.float32)  # IEEE fp32 divide
    y = np.minimum(np.maximum(y, -fmax), fmax).astype(np.float32)
    q = encode(y, fmt)
    return q, s


def _check_2d(x, name):
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError(f"{name} must be 2-D")
    return x


def quant_act_1x128(x, fmt):
    """x[R, C] -> (q[R, C] uint8, s[R, C/128] float32).

    One group = 128 consecutive elements of one row, starting at column 0.
    """
    x = _check_2d(x, "x")
    R, C = x.shape
    if C % GROUP:
        raise ValueError("C must be a multiple of 128")
    g = C // GROUP
    q, s = quantize_group_rows(x.reshape(R * g, GROUP), fmt)
    return q.reshape(R, C), s.reshape(R, g)


def quant_act_128x1(x, fmt):
    """x[R, C] -> (q[R, C] uint8, s[R/128, C] float32), codes in x's orientation.

    One group = 128 consecutive rows of one column, starting at row 0.
    """
    x = _check_2d(x, "x")
    R, C = x.shape
    if R % GROUP:
        raise ValueError("R must be a multiple of 128")
    rb = R // GROUP
    # (rb, 128, C) -> (rb, C, 128): each (rb, c) is one group
    xg = x.reshape(rb, GROUP, C).transpose(0, 2, 1).reshape(rb * C, GROUP)
    q, s = quantize_group_rows(xg, fmt)
    q = q.reshape(rb, C, GROUP).transpose(0, 2, 1).reshape(R, C)
    return np.ascontiguousarray(q), s.reshape(rb, C)


def quant_weight_128x128(w, fmt):
    """w[N, K] -> (q[N, K] uint8, s[N/128, K/128] float32).

    One group = one aligned 128x128 tile.
    """
    w = _check_2d(w, "w")
    N, K = w.shape
    if N % GROUP or K % GROUP:
        raise ValueError("N and K must be multiples of 128")
    nb, kb = N // GROUP, K // GROUP
    wg = w.reshape(nb, GROUP, kb, GROUP).transpose(0, 2, 1, 3).reshape(nb * kb, GROUP * GROUP)
    q, s = quantize_group_rows(wg, fmt)
    q = q.reshape(nb, kb, GROUP, GROUP).transpose(0, 2, 1, 3).reshape(N, K)
    return np.ascontiguousarray(q), s.reshape(nb, kb)
