"""FP8 E4M3 / E5M2 codec, written from the bit-field definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[HL] section "Blackwell 的 FP8 Tensor Core" names the two formats by their
PyTorch dtypes, ``float8_e4m3fn`` (1 sign, 4 exponent, 3 mantissa bits,
largest value 448) and ``float8_e5m2`` (1, 5, 2 bits, largest value 57344).
Those dtype names pin the OCP variants:

* E4M3 "fn": exponent bias 7, no infinities, NaN only at S.1111.111,
  so the largest finite magnitude is 1.75 * 2**8 = 448;
* E5M2: exponent bias 15, IEEE-like, +-Inf at S.11111.00 and NaN at
  S.11111.{01,10,11}, largest finite magnitude 1.75 * 2**15 = 57344.

Both keep subnormals (exponent field 0).

``encode`` is round-to-nearest, ties-to-even, on finite fp32 inputs whose
magnitude is at most the format maximum (the quantizer clamps before it
encodes, [HL] "_quantize").  The sign bit is copied from the input even when
the magnitude rounds to zero.
"""

import numpy as np

E4M3 = "e4m3"
E5M2 = "e5m2"

# (exponent bits, mantissa bits, exponent bias, has_inf)
FORMATS = {
    E4M3: (4, 3, 7, False),
    E5M2: (5, 2, 15, True),
}


def _decode_one(code: int, fmt: str) -> float:
    """Value of one 8-bit code, from its sign, exponent and mantissa fields."""
    ebits, mbits, bias, has_inf = FORMATS[fmt]
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    f = code & ((1 << mbits) - 1)
    emax_field = (1 << ebits) - 1
    if has_inf:
        if e == emax_field:
            return sign * float("inf") if f == 0 else float("nan")
    else:
        if e == emax_field and f == (1 << mbits) - 1:
            return float("nan")
    if e == 0:
        # subnormal: 0.f * 2**(1 - bias)
        return sign * (f / float(1 << mbits)) * 2.0 ** (1 - bias)
    return sign * (1.0 + f / float(1 << mbits)) * 2.0 ** (e - bias)


def decode_table(fmt: str) -> np.ndarray:
    """float64[256]: the value of every code (NaN where the code is NaN)."""
    return np.array([_decode_one(c, fmt) for c in range(256)], dtype=np.float64)


_TABLES = {f: decode_table(f) for f in FORMATS}


def decode(codes, fmt: str) -> np.ndarray:
    """Elementwise value (float64) of uint8 codes."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLES[fmt][codes]


def _positive_ladder(fmt: str):
    """Codes 0x00.. upward while finite, and their float64 magnitudes.

    For both formats the positive codes are ordered by value, so the finite
    non-negative magnitudes are a sorted ladder indexed by the code itself.
    """
    tab = _TABLES[fmt]
    n = 0
    while n < 128 and np.isfinite(tab[n]):
        n += 1
    mags = tab[:n].copy()
    return mags


_LADDERS = {f: _positive_ladder(f) for f in FORMATS}


def fmt_max(fmt: str) -> float:
    """Largest finite magnitude of the format (448 or 57344)."""
    return float(_LADDERS[fmt][-1])


def encode(y, fmt: str) -> np.ndarray:
    """Round finite fp32 values with |y| <= fmt_max to the nearest code.

    Ties go to the code with a zero least-significant bit.  The comparison is
    against the exact midpoint of the two neighbouring magnitudes; both the
    fp32 input and that midpoint are exact in float64, so the decision is
    exact.  Raises on NaN, Inf or |y| > fmt_max (the caller clamps first).
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    mags = _LADDERS[fmt]
    if not np.all(np.isfinite(a)):
        raise ValueError("encode: non-finite input")
    if a.size and a.max() > mags[-1]:
        raise ValueError("encode: magnitude above the format maximum")
    # hi = first ladder index with mags[hi] >= a
    hi = np.searchsorted(mags, a, side="left")
    hi = np.minimum(hi, len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    exact = mags[hi] == a
    mid = 0.5 * (mags[lo] + mags[hi])
    pick_hi = a > mid
    tie = a == mid
    hi_even = (hi & 1) == 0
    pick_hi = np.where(tie, hi_even, pick_hi)
    mag_code = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    return (mag_code | sign).astype(np.uint8)
