"""Pins of the oracle's NVFP4 and 8-bit block quantizers.

* hand-derived blocks (tests/golden/nvfp4_blocks.txt, fp8_blocks.txt);
* a second implementation of the same recipe in numpy float32 arithmetic
  (IEEE fp32 ops instead of the oracle's double-then-round emulation) with
  the threshold form of E2M1 rounding and brute-force E4M3 rounding;
* idempotence, exact dequantization, and the exact-integer property of FP4
  products (page "Infernix releases", release 2026.10.11, "Highlights": the
  4-bit products stay exact, their row sums integers in units of the scales).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cases(name):
    cases, cur = [], None
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "case":
            cur = {"name": rest[0]}
            cases.append(cur)
        else:
            cur[key] = rest
    return cases


@pytest.mark.parametrize("case", _cases("nvfp4_blocks.txt"), ids=lambda c: c["name"])
def test_nvfp4_hand_derived_blocks(case):
    x = np.array([[float(v) for v in case["x"]]], np.float32)
    g = np.float32(float(case["g"][0]))
    codes, scales = Q.nvfp4_quantize(x, g)
    assert scales[0, 0] == int(case["scale"][0], 16)
    want = np.array([int(c, 16) for c in case["codes"]], np.uint8)
    assert np.array_equal(F.unpack_nibbles(codes)[0], want), F.unpack_nibbles(codes)[0]


@pytest.mark.parametrize("case", _cases("fp8_blocks.txt"), ids=lambda c: c["name"])
def test_fp8_hand_derived_blocks(case):
    x = np.array([[float(v) for v in case["x"]]], np.float32)
    codes, scales = Q.fp8_block_quantize(x)
    assert scales[0, 0] == np.float32(float(case["scale"][0]))
    want = np.array([int(c, 16) for c in case["codes"]], np.uint8)
    assert np.array_equal(codes[0], want), [hex(c) for c in codes[0]]


# --------------------------------------------------------------------------- second implementation
E4M3_VALUES = [F.e4m3_decode(c) for c in range(127)]


def _e4m3_brute(v):
    a = abs(Fraction(float(v)))
    vals = [Fraction(float(x)) for x in E4M3_VALUES]
    if a >= vals[-1]:
        return 126
    best = min(range(127), key=lambda i: (abs(a - vals[i]), i % 2))
    return best


def _nvfp4_fp32(x, g):
    """The recipe in numpy float32 ops; E4M3 by brute force, E2M1 by thresholds."""
    x = x.astype(np.float32)
    R, K = x.shape
    b = x.reshape(R, K // 16, 16)
    g = np.float32(g)
    bamax = np.abs(b).max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (bamax / np.float32(6)) / g
    s = np.array([[_e4m3_brute(v) for v in row] for row in t], np.uint8)
    dec = np.array([[np.float32(float(E4M3_VALUES[c])) for c in row] for row in s], np.float32)
    d = dec * g
    with np.errstate(divide="ignore", invalid="ignore"):
        q = b / d[..., None]
    a = np.abs(q.astype(np.float64))
    mag = ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5)
           + (a >= 3.5) + (a > 5.0))
    codes = (mag | (np.signbit(q).astype(int) << 3)).astype(np.uint8)
    codes = np.where((d > 0)[..., None], codes, 0)
    return codes.reshape(R, K), s


@pytest.mark.parametrize("sigma,g", [(1.0, None), (0.02, None), (1.0, 1e-3), (1e-4, 1.0),
                                     (5.0, 2.0 ** -9)])
def test_nvfp4_matches_float32_implementation(sigma, g):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((24, 64)) * sigma).astype(np.float32)
    x[3, :16] = 0.0
    x[5, 5] = -0.0
    x[7, 16:32] *= 1e-6
    if g is None:
        g = Q.nvfp4_global_scale(np.abs(x).max())
    codes, scales = Q.nvfp4_quantize(x, g)
    want_codes, want_scales = _nvfp4_fp32(x, g)
    assert np.array_equal(scales, want_scales)
    assert np.array_equal(F.unpack_nibbles(codes), want_codes)


def test_global_scale_is_fp32_division():
    rng = np.random.default_rng(12)
    amax = np.abs(rng.standard_normal(10000)).astype(np.float32) * 10
    assert np.array_equal(Q.nvfp4_global_scale(amax), amax / np.float32(2688))


def test_per_row_global_scale():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    g = np.array([1e-3, 2e-3, 5e-4, 1.0], np.float32)
    codes, scales = Q.nvfp4_quantize(x, g)
    for r in range(4):
        c1, s1 = Q.nvfp4_quantize(x[r:r + 1], g[r])
        assert np.array_equal(codes[r], c1[0]) and np.array_equal(scales[r], s1[0])


def test_dequantize_is_exact_product():
    rng = np.random.default_rng(14)
    codes = rng.integers(0, 256, (3, 16), dtype=np.uint8)
    scales = rng.integers(0, 127, (3, 2), dtype=np.uint8)
    g = np.float32(0.00123)
    v = Q.nvfp4_dequantize(codes, scales, g)
    c = F.unpack_nibbles(codes)
    for r in range(3):
        for k in range(32):
            want = (Fraction(float(F.e2m1_decode(c[r, k]))) * Fraction(float(F.e4m3_decode(scales[r, k // 16])))
                    * Fraction(float(g)))
            assert Fraction(float(v[r, k])) == want


def test_nvfp4_idempotent_on_its_own_output():
    """Re-quantizing dequantized values under the same g reproduces codes and scales."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((64, 256)).astype(np.float32) * 0.02
    g = Q.nvfp4_global_scale(np.abs(x).max())
    codes, scales = Q.nvfp4_quantize(x, g)
    back = Q.nvfp4_dequantize(codes, scales, g).astype(np.float32)
    codes2, scales2 = Q.nvfp4_quantize(back, g)
    assert np.array_equal(scales, scales2)
    assert np.array_equal(codes, codes2)


def test_fp8_idempotent_on_its_own_output():
    rng = np.random.default_rng(16)
    x = rng.standard_normal((32, 128)).astype(np.float32)
    codes, s = Q.fp8_block_quantize(x)
    back = Q.fp8_block_dequantize(codes, s).astype(np.float32)
    codes2, s2 = Q.fp8_block_quantize(back)
    assert np.array_equal(s, s2) and np.array_equal(codes, codes2)


def test_quantization_error_bound():
    """|x - deq(x)| <= half an E2M1 step at the block's scale (or saturation)."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((128, 128)).astype(np.float32)
    g = Q.nvfp4_global_scale(np.abs(x).max())
    codes, scales = Q.nvfp4_quantize(x, g)
    err = np.abs(Q.nvfp4_dequantize(codes, scales, g) - x.astype(np.float64))
    d = (F.e4m3_decode(scales) * float(g)).repeat(16, axis=1)
    assert np.all(err <= d * 1.0 + 1e-30)   # largest E2M1 gap is 2 (4 -> 6): half of it is 1 * d


def test_exact_integer_row_sums():
    """Unit block scales and multipliers: 4-bit x 4-bit dot products are exact multiples of 1/4."""
    rng = np.random.default_rng(18)
    N, K = 8, 3072
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ac = rng.integers(0, 256, (2, K // 2), dtype=np.uint8)
    ones_w = np.full((N, K // 16), 0x38, np.uint8)
    ones_a = np.full((2, K // 16), 0x38, np.uint8)
    W = Q.nvfp4_dequantize(wc, ones_w, np.float32(1.0))
    A = Q.nvfp4_dequantize(ac, ones_a, np.float32(1.0))
    got = A @ W.T
    twice = {c: int(round(2 * float(F.e2m1_decode(c)))) for c in range(16)}   # E2M1 values are halves
    wi = np.vectorize(twice.get)(F.unpack_nibbles(wc))
    ai = np.vectorize(twice.get)(F.unpack_nibbles(ac))
    for t in range(2):
        for n in range(N):
            s4 = sum(int(a) * int(w) for a, w in zip(ai[t], wi[n]))    # 4 * sum, a Python integer
            assert Fraction(float(got[t, n])) == Fraction(s4, 4)
