"""Pins for the oracle's FP8 codec (CPU only).

What pins it, independent of the codec itself:
* the maxima and bit widths the pages print (tests/golden/fp8_formats.txt);
* brute-force enumeration of all 256 codes of each format (round trip,
  ordering, NaN/Inf placement, extreme values);
* PyTorch's CPU casts to float8_e4m3fn / float8_e5m2 (the cast the pages'
  listing uses), on a dense structured sweep of fp32 inputs covering every
  rounding decision point, plus all midpoints (ties) and their neighbours;
  an exhaustive sweep over every fp32 pattern runs with FP8BQ_EXHAUSTIVE=1.
"""

import os

import numpy as np
import pytest
import torch

from oracle import E4M3, E5M2, decode, decode_table, encode, fmt_max

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_formats.txt")
TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def _golden_formats():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows[parts[0]] = parts[1:]
    return rows


def torch_cast_codes(y_f32, fmt):
    t = torch.from_numpy(np.ascontiguousarray(y_f32, dtype=np.float32))
    return t.to(TORCH_DT[fmt]).view(torch.uint8).numpy()


def test_pages_maxima_and_widths():
    g = _golden_formats()
    for fmt in (E4M3, E5M2):
        ebits, mbits, vmax, code_hex = g[fmt]
        assert fmt_max(fmt) == float(vmax)
        assert decode(int(code_hex, 16), fmt) == float(vmax)
        # the largest finite magnitude is 1.75 * 2**(emax) with the given widths
        tab = decode_table(fmt)
        fin = tab[np.isfinite(tab)]
        assert fin.max() == float(vmax)
        # exponent/mantissa widths: the number of distinct positive normal
        # binades is 2**ebits - 1 (E4M3 uses the top binade) or - 2 (E5M2 not)
        pos = fin[fin > 0]
        normals = pos[pos >= pos[pos > 0].min() * 2 ** int(mbits)]
        binades = len(np.unique(np.floor(np.log2(normals))))
        assert binades == (2 ** int(ebits) - 1 if fmt == E4M3 else 2 ** int(ebits) - 2)
        # 2**mbits values per binade; E4M3's top binade gives its last code to NaN
        counts = np.unique(np.floor(np.log2(normals)), return_counts=True)[1]
        assert np.all(counts[:-1] == 2 ** int(mbits))
        assert counts[-1] == (2 ** int(mbits) - 1 if fmt == E4M3 else 2 ** int(mbits))


def test_specials_and_counts():
    t4, t5 = decode_table(E4M3), decode_table(E5M2)
    assert np.isnan(t4[0x7F]) and np.isnan(t4[0xFF])
    assert np.isfinite(t4).sum() == 254
    assert not np.isinf(t4).any()
    assert t5[0x7C] == np.inf and t5[0xFC] == -np.inf
    for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF):
        assert np.isnan(t5[c])
    assert np.isfinite(t5).sum() == 248


def test_extreme_values():
    assert decode(0x01, E4M3) == 2.0 ** -9
    assert decode(0x08, E4M3) == 2.0 ** -6
    assert decode(0x07, E4M3) == 7 * 2.0 ** -9
    assert decode(0x01, E5M2) == 2.0 ** -16
    assert decode(0x04, E5M2) == 2.0 ** -14
    assert decode(0x38, E4M3) == 1.0 and decode(0x3C, E5M2) == 1.0
    for fmt in (E4M3, E5M2):
        z = decode(0x80, fmt)
        assert z == 0.0 and np.signbit(z)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_matches_torch(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()
    mine = decode_table(fmt)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    assert np.array_equal(ref[fin], mine[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(mine[fin]))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_roundtrip_every_code(fmt):
    tab = decode_table(fmt)
    for c in range(256):
        v = tab[c]
        if not np.isfinite(v):
            continue
        assert int(encode(np.float32(v), fmt)) == c, hex(c)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_positive_codes_monotone_and_mirrored(fmt):
    tab = decode_table(fmt)
    fin = [c for c in range(128) if np.isfinite(tab[c])]
    vals = tab[fin]
    assert np.all(np.diff(vals) > 0)
    assert fin == list(range(len(fin)))
    for c in fin:
        assert tab[c | 0x80] == -tab[c]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_midpoints_tie_to_even(fmt):
    tab = decode_table(fmt)
    n = int(np.isfinite(tab[:128]).sum())
    for c in range(n - 1):
        lo, hi = tab[c], tab[c + 1]
        mid = np.float32(0.5 * (lo + hi))
        assert float(mid) == 0.5 * (lo + hi)  # exact in fp32
        even = c if c % 2 == 0 else c + 1
        assert int(encode(mid, fmt)) == even
        assert int(encode(-mid, fmt)) == even | 0x80
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert int(encode(below, fmt)) == c
        assert int(encode(above, fmt)) == c + 1
        # and torch agrees on all three
        ys = np.array([mid, below, above, -mid], np.float32)
        assert np.array_equal(encode(ys, fmt), torch_cast_codes(ys, fmt))


def test_sign_of_zero_kept():
    for fmt in (E4M3, E5M2):
        assert int(encode(np.float32(-1e-30), fmt)) == 0x80
        assert int(encode(np.float32(-0.0), fmt)) == 0x80
        assert int(encode(np.float32(0.0), fmt)) == 0x00
        assert int(encode(np.float32(1e-30), fmt)) == 0x00


def test_encode_rejects_out_of_contract():
    for fmt in (E4M3, E5M2):
        m = np.float32(fmt_max(fmt))
        with pytest.raises(ValueError):
            encode(np.nextafter(m, np.float32(np.inf)), fmt)
        with pytest.raises(ValueError):
            encode(np.float32(np.nan), fmt)


def _structured_fp32(fmt):
    """Every fp32 exponent up to the format maximum x every top-13 mantissa
    pattern x 8 low-bit patterns (zeros, ones, the half-way bit, neighbours)."""
    emax_field = 127 + int(np.floor(np.log2(fmt_max(fmt))))
    exps = np.arange(0, emax_field + 1, dtype=np.uint32)
    top = np.arange(1 << 13, dtype=np.uint32) << np.uint32(10)
    low = np.array([0, 1, 0x1FF, 0x200, 0x201, 0x3FE, 0x3FF, 0x155], dtype=np.uint32)
    bits = (exps[:, None, None] << np.uint32(23)) | top[None, :, None] | low[None, None, :]
    y = bits.reshape(-1).view(np.float32)
    y = y[np.abs(y) <= np.float32(fmt_max(fmt))]
    return np.concatenate([y, -y])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_matches_torch_structured(fmt):
    y = _structured_fp32(fmt)
    assert y.size > 10_000_000
    mine = encode(y, fmt)
    ref = torch_cast_codes(y, fmt)
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, (y[bad[:5]], mine[bad[:5]], ref[bad[:5]])


@pytest.mark.exhaustive
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_matches_torch_exhaustive(fmt):
    lim = np.float32(fmt_max(fmt)).view(np.uint32)
    step = 1 << 24
    for start in range(0, int(lim) + 1, step):
        bits = np.arange(start, min(start + step, int(lim) + 1), dtype=np.uint32)
        y = bits.view(np.float32)
        for s in (y, -y):
            assert np.array_equal(encode(s, fmt), torch_cast_codes(s, fmt)), hex(start)
