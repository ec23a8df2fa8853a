"""Element encodings used by NVFP4 experts, written from their definitions.

* E2M1 (OCP Microscaling Formats (MX) v1.0, "FP4 (E2M1)" element type): one
  sign bit (bit 3) and three magnitude bits indexing {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E4M3 (OCP 8-bit Floating Point specification, "E4M3"): sign, 4 exponent bits
  (bias 7), 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the
  all-ones pattern S.1111.111 is NaN; there is no infinity; largest finite 448.
* bf16: the upper 16 bits of an IEEE fp32.
* fp16: IEEE binary16 (the scales and the 16-bit activations of the
  q4_g64_fp16 encoding); rounding to it is IEEE round-to-nearest-even with
  overflow to infinity (numpy's float16 conversion, pinned in the tests).
* int4: a 4-bit two's complement integer in a nibble (codes 0..7 are 0..7,
  codes 8..15 are -8..-1).

Rounding to these formats is round-to-nearest with ties to the even code (the
code whose lowest bit is 0, i.e. the even mantissa) and saturation at the
largest finite magnitude.  The sign bit is kept, so a negative value that
rounds to zero gets the negative-zero code.  NaN input maps to code 0 (the
layer never produces NaN from finite inputs; 0/0 in a scale quotient of an
all-zero block is the one place it could appear).

These are brute-force definitions: the nearest member of the enumerated value
set, compared with exact double arithmetic.
"""
from __future__ import annotations

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def f32(x):
    """Round double values to the nearest fp32 (ties to even): one emulated fp32 op."""
    return np.asarray(x, np.float64).astype(np.float32)


# ----------------------------------------------------------------------------- decoders
def e2m1_decode(codes):
    """Value of 4-bit E2M1 codes (0..15) as double."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e4m3_decode(codes):
    """Value of 8-bit E4M3 codes as double; 0x7F / 0xFF decode to NaN."""
    b = np.asarray(codes).astype(np.int64)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return np.where(((b >> 7) & 1) == 1, -mag, mag)


E4M3_FINITE = e4m3_decode(np.arange(0x7F))  # non-negative finite values, codes 0x00..0x7E, increasing


def bf16_to_f64(bits):
    """Value of bf16 bit patterns (uint16) as double (exact)."""
    u = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16(x):
    """Round double values to bf16 (8 significant bits, nearest, ties to even).

    Written from the definition: for |x| >= 2^-126 the value is rounded to
    8 significant bits; below, to a multiple of 2^-133 (bf16 subnormals).
    Magnitudes at or beyond the overflow midpoint become infinity.
    """
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return _f64_to_bf16(x)


def _f64_to_bf16(x):
    fin = np.isfinite(x)
    ax = np.abs(x)
    normal = fin & (ax >= 2.0 ** -126)
    m, e = np.frexp(np.where(normal, x, 1.0))             # x = m 2^e, 0.5 <= |m| < 1
    out_n = np.ldexp(np.rint(m * 256.0) / 256.0, e)        # 8 significant bits, rint ties to even
    out_s = np.rint(np.where(fin, x, 0.0) * 2.0 ** 133) * 2.0 ** -133
    out = np.where(normal, out_n, out_s)
    out = np.where(fin & (np.abs(out) >= 2.0 ** 128), np.copysign(np.inf, x), out)
    out = np.where(fin, out, x)
    bits = out.astype(np.float32).view(np.uint32) >> 16    # exact: out has <= 8 significant bits
    return bits.astype(np.uint16)


# ----------------------------------------------------------------------------- rounding
def _nearest_index(v, table):
    """Index of the member of increasing ``table`` nearest to v >= 0; ties to the even index;
    values above the last member saturate to it."""
    v = np.minimum(v, table[-1])
    hi = np.clip(np.searchsorted(table, v, side="left"), 0, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = v - table[lo]
    d_hi = table[hi] - v
    pick = np.where(d_hi < d_lo, hi, lo)
    tie = d_hi == d_lo
    pick = np.where(tie, np.where(hi % 2 == 0, hi, lo), pick)
    return pick


def e2m1_quantize(q):
    """E2M1 codes (0..15) of fp32 values: nearest, ties to even code, saturating at 6."""
    q = np.asarray(q, np.float32).astype(np.float64)
    nan = np.isnan(q)
    idx = _nearest_index(np.where(nan, 0.0, np.abs(q)), E2M1_MAGNITUDES)
    code = idx | (np.signbit(q).astype(np.int64) << 3)
    return np.where(nan, 0, code).astype(np.uint8)


def e4m3_quantize(v):
    """E4M3 codes of fp32 values: nearest, ties to even code, saturating at 448 (never NaN)."""
    v = np.asarray(v, np.float32).astype(np.float64)
    nan = np.isnan(v)
    idx = _nearest_index(np.where(nan, 0.0, np.abs(v)), E4M3_FINITE)
    code = idx | (np.signbit(v).astype(np.int64) << 7)
    return np.where(nan, 0, code).astype(np.uint8)


def f64_to_f16(x):
    """fp16 bit patterns (uint16) of values, rounded to nearest even (from double)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def f16_to_f64(bits):
    """Value of fp16 bit patterns (uint16) as double (exact)."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def int4_decode(codes):
    """Value of 4-bit two's complement codes (0..15) as integers -8..7."""
    c = np.asarray(codes).astype(np.int64) & 15
    return np.where(c >= 8, c - 16, c)


def pack_nibbles(codes):
    """Pack 4-bit codes [..., 2n] into bytes [..., n]: element 2i in the low nibble."""
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of pack_nibbles."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------- scale layout
# The engine's own arrangement of the NVFP4 block scales (the pages say the
# checkpoint is repacked into the engine's expert layout without changing a
# bit: page "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix (bit-exact)",
# section "What is bit-exact and what is quantized"; the arrangement itself is
# this library's, stated in its C header under moe_layout).  A scale row holds
# one pair of E4M3 bytes per chunk of 32 values.  The tiled order cuts the row
# into windows of 32 chunks; in a full window, chunk 4*i + g moves to position
# 8*g + i; a trailing partial window stays in place.

def tiled_scale_order(nc):
    """Tiled pair position of each canonical chunk pair 0 .. nc-1 of a row."""
    pos = list(range(nc))
    for w in range(nc // 32):
        for c in range(32):
            i, g = divmod(c, 4)
            pos[32 * w + c] = 32 * w + 8 * g + i
    return np.array(pos, dtype=np.int64)


def tiled_scales(scales):
    """Canonical scale bytes [..., K/16] (uint8) in the tiled order."""
    scales = np.asarray(scales, dtype=np.uint8)
    nc = scales.shape[-1] // 2
    pairs = scales.reshape(*scales.shape[:-1], nc, 2)
    out = np.empty_like(pairs)
    out[..., tiled_scale_order(nc), :] = pairs
    return out.reshape(scales.shape)
