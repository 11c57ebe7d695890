"""Pins for the oracle's element codecs (E2M1, E4M3, E8M0).

Each check uses something other than the oracle's own formula: bit-field
decoding vs the oracle's tables, torch's float8 dtypes (an independent library
conversion), brute-force nearest search with exact rationals, and hand-worked
fixtures under tests/golden/.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden_lines

E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]


def test_e2m1_decode_from_bitfields(orc):
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = (m * 0.5) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert orc.e2m1_value(c) == (-mag if s else mag)


def test_e4m3_decode_vs_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], got[~nan])
    assert orc.e4m3_value(0x7E) == 448.0 and orc.e4m3_value(0x01) == 2.0 ** -9


def test_e8m0_decode_vs_torch(orc):
    codes = torch.arange(255, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([orc.e8m0_value(c) for c in range(255)])
    assert np.array_equal(ref, got)
    assert np.isnan(orc.e8m0_value(255))


def _nearest_even(v: Fraction, mags, is_even):
    """Brute force: nearest magnitude, ties to the even code, saturating."""
    best = None
    for code, m in enumerate(mags):
        d = abs(v - m)
        if best is None or d < best[0] or (d == best[0] and is_even(code)):
            best = (d, code)
    return best[1]


def _e2m1_brute(v: float) -> int:
    s = 8 if np.signbit(v) else 0
    return s | _nearest_even(abs(Fraction(float(v))), E2M1_MAGS, lambda c: c % 2 == 0)


E4M3_MAGS = None


def _e4m3_mags():
    global E4M3_MAGS
    if E4M3_MAGS is None:
        t = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
        E4M3_MAGS = [Fraction(float(v)) for v in t]
    return E4M3_MAGS


def _e4m3_brute(v: float) -> int:
    s = 0x80 if np.signbit(v) else 0
    return s | _nearest_even(abs(Fraction(float(v))), _e4m3_mags(), lambda c: c % 2 == 0)


def _interesting_f32(mags, rng, n_rand):
    """Every representable magnitude, every midpoint, and their fp32
    neighbours, plus random values over many binades, both signs."""
    pts = []
    ms = [float(m) for m in mags]
    for a, b in zip(ms[:-1], ms[1:]):
        mid = np.float32((a + b) / 2)
        pts += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))]
    for a in ms:
        a = np.float32(a)
        pts += [a, np.nextafter(a, np.float32(0)), np.nextafter(a, np.float32(np.inf))]
    top = np.float32(ms[-1])
    pts += [top * 1.01, top * 2, np.float32(3e38), np.float32(1e-45), np.float32(1e-40)]
    rnd = rng.uniform(-1, 1, n_rand) * 2.0 ** rng.integers(-20, 12, n_rand)
    pts = np.concatenate([np.array(pts, np.float32), rnd.astype(np.float32)])
    return np.concatenate([pts, -pts])


def test_e2m1_encode_bruteforce(orc):
    vals = _interesting_f32(E2M1_MAGS, np.random.default_rng(1), 4000)
    got = orc.e2m1_encode(vals)
    ref = np.array([_e2m1_brute(v) for v in vals], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_bruteforce(orc):
    vals = _interesting_f32(_e4m3_mags(), np.random.default_rng(2), 3000)
    got = orc.e4m3_encode(vals)
    ref = np.array([_e4m3_brute(v) for v in vals], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_vs_torch(orc):
    """torch's float8_e4m3fn cast (RNE) agrees below the saturation point."""
    rng = np.random.default_rng(3)
    v = (rng.uniform(-1, 1, 200000) * 2.0 ** rng.integers(-14, 9, 200000)).astype(np.float32)
    v = v[np.abs(v) < 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(v), ref)


def test_e4m3_hand_values(orc):
    for ln in golden_lines("e4m3_hand_values.txt"):
        v, b = ln.split()
        assert int(orc.e4m3_encode(np.array([float(v)], np.float32))[0]) == int(b, 16), ln


def test_e2m1_hand_table(orc):
    for ln in golden_lines("e2m1_rne_table.txt"):
        v, c = ln.split()
        x = np.array([float(v), -float(v)], np.float32)
        got = orc.e2m1_encode(x)
        assert got[0] == int(c), ln
        assert got[1] == int(c) | 8, ln  # sign kept, also on zero codes


@pytest.mark.parametrize("v", [np.inf, -np.inf])
def test_saturation_of_infinities(orc, v):
    x = np.array([v], np.float32)
    assert orc.e2m1_encode(x)[0] == (15 if v < 0 else 7)
    assert orc.e4m3_encode(x)[0] == (0xFE if v < 0 else 0x7E)
