"""NVFP4 and 8-bit block quantization, step by step.

NVFP4 (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix (bit-exact)",
section "What is bit-exact and what is quantized", routed experts): every
matrix holds E2M1 codes, one E4M3 scale per 16 consecutive values along the
reduction dimension K, and one fp32 multiplier for the whole matrix; for 4-bit
activations each matrix also carries an fp32 activation input scale.  The
pages name the parts but print no arithmetic; the recipe below is the
plainest one that produces them (the per-tensor scale is amax / (6 * 448),
the block scale is block amax / 6 / that, each value is divided by its
decoded block scale times the per-tensor scale and rounded to E2M1), every
operation one correctly rounded fp32 operation, in this order:

    g = f32(amax / 2688)                       per matrix (weights only)
    t = f32( f32(bamax / 6) / g )              per block of 16
    s = E4M3(t)                                 nearest-even, saturating at 448
    d = f32( dec(s) * g )
    c = E2M1( f32(v / d) )                      nearest-even, saturating at 6
    value = dec(c) * dec(s) * g                 (exact in double)

When d is not positive (an all-zero block, or g == 0) all 16 codes are +0.
Activations (4-bit mode) use the same steps with g the matrix's input scale.

The 8-bit mode (page "Infernix", section "Activation precision",
``--a8-activations``) is read as E4M3 codes with one fp32 scale per 16:

    s = f32(bamax / 448);  c = E4M3( f32(v / s) );  value = dec(c) * s

with all codes +0 when s is not positive.
"""
from __future__ import annotations

import numpy as np

from .formats import (E2M1_MAX, E4M3_MAX, e2m1_decode, e2m1_quantize, e4m3_decode,
                      e4m3_quantize, f16_to_f64, f32, f64_to_f16, int4_decode, pack_nibbles,
                      unpack_nibbles)

BLOCK = 16
NVFP4_AMAX_DIVISOR = E2M1_MAX * E4M3_MAX  # 2688


def _blocks(x):
    x = np.asarray(x, np.float32)
    assert x.ndim == 2 and x.shape[1] % BLOCK == 0, x.shape
    R, K = x.shape
    return x.astype(np.float64).reshape(R, K // BLOCK, BLOCK)


def _per_row(g, R):
    g = np.asarray(g, np.float32).astype(np.float64)
    return np.broadcast_to(g.reshape(-1, 1) if g.ndim else g, (R, 1))


def nvfp4_global_scale(amax):
    """Per-matrix fp32 multiplier: f32(amax / (6 * 448))."""
    return f32(np.asarray(amax, np.float64) / NVFP4_AMAX_DIVISOR)


def nvfp4_quantize(x, g):
    """Quantize fp32 rows x [R, K] under global scale g (scalar or per row [R]).

    Returns (codes [R, K/2] uint8, element 2i in the low nibble; scales [R, K/16] uint8 E4M3).
    """
    b = _blocks(x)
    R = b.shape[0]
    gg = _per_row(g, R)
    bamax = np.abs(b).max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = f32(f32(bamax / 6.0).astype(np.float64) / gg)
        s = e4m3_quantize(t)
        d = f32(e4m3_decode(s) * gg).astype(np.float64)
        q = f32(b / d[..., None])
    codes = e2m1_quantize(q)
    codes = np.where((d > 0)[..., None], codes, 0).astype(np.uint8)
    return pack_nibbles(codes.reshape(R, -1)), s


def nvfp4_dequantize(codes, scales, g):
    """Exact double value of packed NVFP4 rows: dec(code) * dec(scale) * g."""
    c = unpack_nibbles(codes)
    R, K = c.shape
    gg = _per_row(g, R)
    v = e2m1_decode(c).reshape(R, K // BLOCK, BLOCK) * e4m3_decode(scales)[..., None]
    return (v * gg[..., None]).reshape(R, K)


def fp8_block_quantize(x):
    """8-bit mode: E4M3 codes [R, K] uint8 and fp32 scales [R, K/16], s = f32(bamax / 448)."""
    b = _blocks(x)
    R = b.shape[0]
    bamax = np.abs(b).max(axis=2)
    s = f32(bamax / E4M3_MAX)
    sd = s.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = f32(b / sd[..., None])
    codes = e4m3_quantize(q)
    codes = np.where((sd > 0)[..., None], codes, 0).astype(np.uint8)
    return codes.reshape(R, -1), s


def fp8_block_dequantize(codes, scales):
    """Exact double value of 8-bit rows: dec(code) * s."""
    c = np.asarray(codes, np.uint8)
    R, K = c.shape
    v = e4m3_decode(c).reshape(R, K // BLOCK, BLOCK) * np.asarray(scales, np.float64)[..., None]
    return v.reshape(R, K)


# ----------------------------------------------------------------------------- q4_g64_fp16
Q4_GROUP = 64
# Candidate divisors of the group amax: 7, 7.125, ..., 8 (the codes reach -8 .. 7).
Q4_DIVISORS = 7.0 + np.arange(9) / 8.0


def q4g64_quantize(w):
    """q4_g64_fp16 packing of fp32 rows w [R, K] (K % 64 == 0).

    Page "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix (bit-exact)", section
    "Drafting only": the drafter's routed experts are 4-bit with one FP16 scale
    per 64 weights, the scales chosen by mean squared error from the exact
    weights.  The pages give no candidate set; the reading taken: per group of 64
    consecutive values along K, with amax = max |v|,

        d_j = fp16( f32(amax / m_j) ),  m_j = 7 + j/8, j = 0..8
        q_i = clamp( RNE( f32(v_i / d_j) ), -8, 7 )
        err_j = sum_i (v_i - d_j q_i)^2   in double, i ascending, each op rounded once

    the first j with the smallest err_j (candidates whose d_j is 0 or infinite
    are skipped; an all-zero group, or one with no candidate, stores d = +0 and
    q = 0).  Returns (codes [R, K/2] uint8, two's complement nibbles, element 2i
    in the low nibble; scales [R, K/64] fp16 bit patterns).
    """
    v = np.asarray(w, np.float32)
    R, K = v.shape
    assert K % Q4_GROUP == 0, K
    g = v.reshape(R, K // Q4_GROUP, Q4_GROUP).astype(np.float64)
    amax = np.abs(g).max(axis=2)
    best_err = np.full(amax.shape, np.inf)
    best_d = np.zeros(amax.shape, np.uint16)
    best_q = np.zeros(g.shape, np.int64)
    for m in Q4_DIVISORS:
        dbits = f64_to_f16(f32(amax / m).astype(np.float64))
        d = f16_to_f64(dbits)
        ok = (d > 0) & np.isfinite(d)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = f32(g / np.where(ok, d, 1.0)[..., None]).astype(np.float64)
        q = np.clip(np.rint(r), -8, 7).astype(np.int64)
        err = np.zeros(amax.shape)
        for i in range(Q4_GROUP):                      # index order, one rounding per op
            e = g[..., i] - d * q[..., i]
            err = err + e * e
        better = ok & (err < best_err)
        best_err = np.where(better, err, best_err)
        best_d = np.where(better, dbits, best_d)
        best_q = np.where(better[..., None], q, best_q)
    codes = (best_q & 15).astype(np.uint8).reshape(R, K)
    return pack_nibbles(codes), best_d.astype(np.uint16)


def q4g64_dequantize(codes, scales):
    """Exact double value of q4_g64_fp16 rows: int4(code) * fp16 scale of its group of 64."""
    q = int4_decode(unpack_nibbles(codes)).astype(np.float64)
    R, K = q.shape
    d = f16_to_f64(scales)
    return (q.reshape(R, K // Q4_GROUP, Q4_GROUP) * d[..., None]).reshape(R, K)
