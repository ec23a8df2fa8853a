"""Pins of the oracle's q4_g64_fp16 encoding (4-bit two's complement codes, one
fp16 scale per 64 values, the scale chosen by squared error over a fixed grid
of candidates) and of the fp16 activation mode its experts run in.

Each is checked against something other than its own code: the two's
complement table, IEEE binary16 rounding cases worked out by hand, brute force
over the candidate scales with exact rational arithmetic, groups whose values
are exactly representable, and a dense SwiGLU MLP in torch float64.
"""
from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F
from oracle import layer as L
from oracle import quant as Q


def test_int4_two_complement_table():
    assert F.int4_decode(np.arange(16)).tolist() == [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def test_fp16_rounding_cases():
    """IEEE binary16: 10 fraction bits, bias 15, ties to even, overflow to infinity."""
    cases = [(1.0 + 2.0 ** -11, 1.0),                   # tie between 1 and 1 + 2^-10 -> even (1)
             (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),   # tie -> even (1 + 2^-9)
             (65504.0, 65504.0), (65519.0, 65504.0), (65520.0, np.inf),
             (2.0 ** -24, 2.0 ** -24),                  # smallest subnormal
             (2.0 ** -25, 0.0),                         # tie between 0 and 2^-24 -> even (0)
             (3 * 2.0 ** -26, 2.0 ** -24),
             (-0.1, -0.0999755859375)]
    for v, want in cases:
        got = F.f16_to_f64(F.f64_to_f16(v))
        assert got == want, (v, got, want)
    assert F.f64_to_f16(1.0) == 0x3C00 and F.f64_to_f16(-2.0) == 0xC000


def _exact_choice(vals):
    """Brute force of the scale choice for one group with exact rationals: every
    candidate's fp16 scale, codes by nearest integer (ties to even) clamped to
    [-8, 7], and the exact squared error.  Returns [(d, q, err)] per candidate."""
    amax = max(abs(v) for v in vals)
    out = []
    for m in Q.Q4_DIVISORS:
        d = float(F.f16_to_f64(F.f64_to_f16(float(np.float32(amax / m)))))
        if not (d > 0 and np.isfinite(d)):
            out.append(None)
            continue
        q = []
        for v in vals:
            r = Fraction(float(np.float32(v / d)))
            n = int(np.floor(r))
            frac = r - n
            if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
                n += 1
            q.append(max(-8, min(7, n)))
        err = sum((Fraction(v) - Fraction(d) * qi) ** 2 for v, qi in zip(vals, q))
        out.append((d, q, err))
    return out


def test_q4_scale_is_the_least_squares_candidate():
    rng = np.random.default_rng(61)
    for trial in range(40):
        scale = 10.0 ** rng.uniform(-6, 2)
        w = (rng.standard_normal((1, 64)) * scale).astype(np.float32)
        if trial % 5 == 0:
            w[0, rng.integers(64)] *= 8                 # an outlier
        codes, sc = Q.q4g64_quantize(w)
        vals = [float(v) for v in w[0]]
        cands = _exact_choice(vals)
        best = min(c[2] for c in cands if c is not None)
        d = float(F.f16_to_f64(sc[0, 0]))
        chosen = [c for c in cands if c is not None and c[0] == d]
        assert chosen, (trial, d)
        assert chosen[0][2] <= best * (1 + 1e-9), (trial, float(chosen[0][2]), float(best))
        assert F.int4_decode(F.unpack_nibbles(codes))[0].tolist() == chosen[0][1]


def test_q4_exact_groups_and_zero_group():
    """A group of integers times an fp16 scale d with amax = 7 d is stored exactly
    (first candidate, zero error); an all-zero group stores d = 0 and zero codes."""
    rng = np.random.default_rng(62)
    d = float(F.f16_to_f64(F.f64_to_f16(0.0123)))
    q = rng.integers(-7, 8, size=(2, 64))
    q[:, 5] = 7
    w = (q * d).astype(np.float32)
    assert np.array_equal(w.astype(np.float64), q * d)
    w = np.concatenate([w, np.zeros((1, 64), np.float32)])
    codes, sc = Q.q4g64_quantize(w)
    assert np.array_equal(Q.q4g64_dequantize(codes, sc)[:2], q * d)
    assert sc[2, 0] == 0 and np.all(codes[2] == 0)


def test_q4_nibble_layout():
    w = np.zeros((1, 64), np.float32)
    w[0, 0], w[0, 1] = -7.0, 3.0
    codes, sc = Q.q4g64_quantize(w)
    assert F.f16_to_f64(sc[0, 0]) == 1.0
    assert codes[0, 0] == (0x9 | (0x3 << 4))           # element 0 (-7 = 0b1001) low, element 1 high


def test_q4_expert_in_fp16_mode_is_a_dense_swiglu_mlp():
    """One q4 expert in the "F16" mode: x rounded to fp16, fp16 intermediate;
    recomputed with torch float64 on the dequantized matrices."""
    rng = np.random.default_rng(63)
    H, I, T = 128, 64, 5
    ex = L.pack_expert_q4(*(rng.standard_normal(s).astype(np.float32) * 0.05 for s in ((I, H), (I, H), (H, I))))
    x = F.f64_to_bf16(rng.standard_normal((T, H)))
    res = L.expert_ffn(ex, x, "F16")
    xt = torch.from_numpy(F.bf16_to_f64(x)).to(torch.float16).to(torch.float64)
    g = xt @ torch.from_numpy(ex.gate()).T
    u = xt @ torch.from_numpy(ex.up()).T
    h = torch.nn.functional.silu(g) * u
    assert torch.allclose(torch.from_numpy(res.h), h, rtol=1e-12, atol=1e-300)
    hq = h.to(torch.float32).to(torch.float16).to(torch.float64)
    assert np.array_equal(res.hdq, hq.numpy())
    y = hq @ torch.from_numpy(ex.down()).T
    assert torch.allclose(torch.from_numpy(res.y), y, rtol=1e-12, atol=1e-300)
