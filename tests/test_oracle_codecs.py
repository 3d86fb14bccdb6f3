"""Pins of the oracle's codecs against the published formats and library routines.

- E4M3 decode: the OCP spec code points (tests/golden) and torch's float8_e4m3fn.
- E4M3 encode: torch's float32 -> float8_e4m3fn conversion (round to nearest even) on
  every finite bf16 value in [-448, 448], plus brute-force nearest-code search.
- bf16 rounding: torch's float32 -> bfloat16 on float32 inputs; an exact (Fraction)
  nearest/ties-even check on fp64 inputs.
- UE8M0 exponent: the defining inequality checked by brute force over e, and an
  independent closed form written from the mantissa.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore")
GOLD = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spec_points.txt")


def _torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_spec_points(orc):
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        got = orc.e4m3_decode(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_e4m3_decode_all_codes_match_torch(orc):
    ref = _torch_e4m3_table()
    for c in range(256):
        got = orc.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), hex(c)


def _finite_bf16_in_range():
    bits = np.arange(65536, dtype=np.uint32) << 16
    f = bits.view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) <= 448.0)
    return f[keep]


def test_e4m3_encode_matches_torch_on_all_bf16(orc):
    vals = _finite_bf16_in_range()
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in vals], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), int(got[i]), int(ref[i])) for i in bad[:5]]


def test_e4m3_encode_ties_to_even_and_brute_force(orc):
    table = _torch_e4m3_table()
    rng = np.random.default_rng(5)
    xs = list(rng.uniform(-448, 448, 3000)) + list(rng.uniform(-0.02, 0.02, 1500))
    for c in range(0, 0x7E):  # exact midpoints between neighbouring positive codes
        mid = 0.5 * (table[c] + table[c + 1])
        xs += [mid, -mid]
    for x in xs:
        got = orc.e4m3_encode(float(x))
        same_sign = range(0x80, 0xFF) if x < 0 else range(0x00, 0x7F)
        X = Fraction(float(x))
        dist = {c: abs(Fraction(float(table[c])) - X) for c in same_sign}
        best = min(dist.values())
        assert got in dist and dist[got] == best, (x, got)
        winners = [c for c in dist if dist[c] == best]
        if len(winners) == 2:
            assert got & 1 == 0, (x, got, winners)
    assert orc.e4m3_encode(-0.0) == 0x80 and orc.e4m3_encode(0.0) == 0x00


def test_bf16_rounding_matches_torch_on_float32(orc):
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_from_double(float(x)) for x in f], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_exact_on_float64(orc):
    rng = np.random.default_rng(2)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    for x in xs:
        b = orc.bf16_from_double(float(x))
        v = Fraction(orc.bf16_to_double(b))
        X = Fraction(float(x))
        lo = Fraction(orc.bf16_to_double(b - 1 if (b & 0x7FFF) else b))
        hi = Fraction(orc.bf16_to_double(b + 1))
        assert abs(X - v) <= abs(X - lo) and abs(X - v) <= abs(X - hi), x
        if abs(X - v) == abs(X - hi) or (abs(X - v) == abs(X - lo) and lo != v):
            assert b & 1 == 0, x


def test_ue8m0_exponent_definition(orc):
    rng = np.random.default_rng(3)
    amaxes = list(np.abs(rng.standard_normal(3000)) * 10.0 ** rng.integers(-20, 20, 3000))
    amaxes += [448.0 * 2.0 ** k for k in range(-30, 30)] + [math.nextafter(448.0 * 2.0 ** k, 0) for k in range(-5, 5)]
    for a in amaxes:
        e = orc.ue8m0_exponent(float(a))
        A = Fraction(float(a))
        assert A <= 448 * Fraction(2) ** e
        assert A > 448 * Fraction(2) ** (e - 1)
        # independent closed form: a = m * 2^k with m in [1, 2): e = k - 8 if m <= 1.75 else k - 7
        m, k = math.frexp(a)  # a = m * 2^k, m in [0.5, 1)
        m, k = 2 * m, k - 1
        assert e == (k - 8 if m <= 1.75 else k - 7)
        # the scaled block then lies in (224, 448]
        assert 224 < A / Fraction(2) ** e <= 448
    assert orc.ue8m0_exponent(0.0) == -127
