"""Pins of the oracle's element encodings against published tables and brute force.

The decoders are checked against the code tables of the OCP specifications
(tests/golden/e2m1_table.txt, e4m3_points.txt) and a bit-field derivation with
exact rationals; the rounding functions against brute force over the
enumerated code sets with exact rationals, plus a second, threshold-based
E2M1 rounding written independently.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if line:
            code, val = line.split()[:2]
            rows.append((int(code, 16), float(val)))
    return rows


def test_e2m1_table_matches_spec():
    rows = _read_table("e2m1_table.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = float(F.e2m1_decode(code))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)


def test_e4m3_named_points_match_spec():
    for code, val in _read_table("e4m3_points.txt"):
        got = float(F.e4m3_decode(code))
        if math.isnan(val):
            assert math.isnan(got), code
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (hex(code), got)


def _e4m3_fraction(code):
    """Value of an E4M3 code from its bit fields, as an exact rational (None for NaN)."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def test_e4m3_decode_all_256_codes():
    got = F.e4m3_decode(np.arange(256))
    for c in range(256):
        want = _e4m3_fraction(c)
        if want is None:
            assert math.isnan(got[c])
        else:
            assert Fraction(float(got[c])) == want, hex(c)
    finite = [_e4m3_fraction(c) for c in range(127)]
    assert finite == sorted(finite) and max(finite) == 448 and finite[1] == Fraction(1, 512)


# --------------------------------------------------------------------------- brute force rounding
def _brute_nearest(v, values):
    """Index of the nearest value to |v| (exact rationals); ties to the even index; saturate."""
    a = abs(Fraction(float(v)))
    if a >= values[-1]:
        return len(values) - 1
    best = None
    for i, c in enumerate(values):
        d = abs(a - c)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


E2M1_VALUES = [Fraction(v).limit_denominator(4) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
E4M3_VALUES = [_e4m3_fraction(c) for c in range(127)]


def _probe_values(values, rng, n_random, lo, hi):
    mids = [(a + b) / 2 for a, b in zip(values[:-1], values[1:])]
    pts = []
    for m in list(values) + mids:
        f = np.float32(float(m))
        pts += [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(0))]
    pts += list(np.exp(rng.uniform(np.log(lo), np.log(hi), n_random)).astype(np.float32))
    pts = np.array(pts, np.float32)
    return np.concatenate([pts, -pts])


def test_e2m1_quantize_brute_force():
    rng = np.random.default_rng(1)
    v = _probe_values(E2M1_VALUES, rng, 4000, 1e-3, 20.0)
    got = F.e2m1_quantize(v)
    for x, c in zip(v, got):
        want = _brute_nearest(x, E2M1_VALUES) | (8 if math.copysign(1, x) < 0 else 0)
        assert c == want, (x, c, want)


def _e2m1_thresholds(q):
    """Independent closed form: count the rounding thresholds passed (> at ties kept low)."""
    a = np.abs(q.astype(np.float64))
    mag = ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5)
           + (a >= 3.5) + (a > 5.0))
    return (mag | (np.signbit(q).astype(int) << 3)).astype(np.uint8)


def test_e2m1_quantize_matches_threshold_form():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 3,
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 1e30, -0.0, 0.0],
                                 np.float32)])
    assert np.array_equal(F.e2m1_quantize(v), _e2m1_thresholds(v))


def test_e2m1_quantize_special_values():
    v = np.array([np.nan, np.inf, -np.inf, -0.0, -1e-30], np.float32)
    assert list(F.e2m1_quantize(v)) == [0, 7, 15, 8, 8]


def test_e4m3_quantize_brute_force():
    rng = np.random.default_rng(3)
    v = _probe_values(E4M3_VALUES, rng, 3000, 2.0 ** -12, 2.0 ** 10)
    got = F.e4m3_quantize(v)
    for x, c in zip(v, got):
        want = _brute_nearest(x, E4M3_VALUES) | (0x80 if math.copysign(1, x) < 0 else 0)
        assert c == want, (float(x), hex(c), hex(want))


def test_e4m3_quantize_special_values():
    v = np.array([np.nan, np.inf, -np.inf, 448.0, 464.0, 1e9, 2.0 ** -10, 2.0 ** -10 * 1.0001, 0.0],
                 np.float32)
    assert [hex(c) for c in F.e4m3_quantize(v)] == [
        "0x0", "0x7e", "0xfe", "0x7e", "0x7e", "0x7e", "0x0", "0x1", "0x0"]


# --------------------------------------------------------------------------- bf16
def test_bf16_rounding_matches_torch_and_bit_form():
    rng = np.random.default_rng(4)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(10000) * 1e-38).astype(np.float32),      # bf16 subnormals
        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.3895314e38, -3.3895314e38],
                 np.float32),
    ])
    got = F.f64_to_bf16(x.astype(np.float64))
    via_torch = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, via_torch)
    u = x.view(np.uint32).astype(np.uint64)
    bit_form = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(got, bit_form)
    assert np.array_equal(F.bf16_to_f64(got).astype(np.float32).view(np.uint32) >> 16, got)


def test_bf16_rounding_from_double_is_single_rounding():
    # 1 + 2^-8 + 2^-30 is above the bf16 midpoint 1 + 2^-8; a detour through fp32
    # would land on the midpoint and round to even (1.0).
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    assert F.bf16_to_f64(F.f64_to_bf16(x))[0] == 1.0 + 2.0 ** -7


def test_nibble_order():
    codes = np.array([[1, 2, 3, 4]], np.uint8)
    packed = F.pack_nibbles(codes)
    assert list(packed[0]) == [0x21, 0x43]
    assert np.array_equal(F.unpack_nibbles(packed), codes)
