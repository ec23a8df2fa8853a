"""Several correct answers: where a computed fp32 value decides a code.

The intermediate h = silu(g) * up is computed (fp32 sums on the GPU, double in
the oracle) and then rounded to bf16 (16-bit mode) or quantized per 16 (8- and
4-bit modes).  Where h lies within the accumulation error of a rounding
midpoint, both neighbouring codes are correct results of the method.  These
helpers compare "what is unique" exactly and check that "the rest is valid":

* every GPU code must lie in the range of codes the oracle's own rounding
  gives over [h - err, h + err] (err: a bound on the fp32 summation error of
  the gate/up dot products, propagated through SwiGLU);
* where the GPU's code is not the oracle's nominal one it must be such a
  candidate; the expected down-projection input is then the oracle's value of
  that candidate (dec(code) * dec(scale) * g), so the rest of the layer is
  checked against the oracle for the tie resolution the GPU made.

All arithmetic here uses the oracle's own rounding functions; GPU data only
selects among candidates the oracle produced and is validated first.

How many choices may differ.  The window is a worst-case bound on the fp32
sums' error, far wider than the error itself (the rounding errors of a
few-thousand-term sum of random-sign terms are about 2^-24 sqrt(depth)
||terms||_2, against 2^-17 ||terms||_1 here: a factor of about 10^3 at K =
3072).  So about half of all elements are "two-candidate" (their window holds
a rounding midpoint), yet an honest kernel flips only those whose midpoint lies
within its actual error: a fraction of order 10^-3 .. 10^-2 of them.  A
systematic bias or a dropped small term of the size of the window would flip
about half.  The tests therefore bound the flips: at most FLIP_FRACTION of the
two-candidate elements, plus FLIP_SLACK (counted in a TieReport, printed with
every check).
"""
from __future__ import annotations

import numpy as np

from oracle import formats as F
from oracle import quant as Q

# Bound on an fp32-accumulated dot product's error, as a fraction of the sum of
# the magnitudes of its terms (about 60x the typical error of a 3072-term sum).
SUM_WINDOW = 2.0 ** -17
# Relative error of the fp32 SwiGLU evaluation itself (a few ulps).
SWIGLU_WINDOW = 2.0 ** -20
# Flip budget: flipped choices <= FLIP_FRACTION * two-candidate elements + FLIP_SLACK.
FLIP_FRACTION = 0.1
FLIP_SLACK = 3


def h_error_bound(res):
    """Per-element bound on |h_gpu - h| for an oracle FfnResult."""
    g, u = res.g, res.u
    sig = 1.0 / (1.0 + np.exp(-g))
    dh_dg = np.abs(u * sig * (1.0 + g * (1.0 - sig)))
    dh_du = np.abs(g * sig)
    return (dh_dg * SUM_WINDOW * res.gate_abs + dh_du * SUM_WINDOW * res.up_abs
            + SWIGLU_WINDOW * np.abs(res.h) + 1e-30)


class TieReport:
    def __init__(self):
        self.elements = 0
        self.two_candidate = 0      # elements whose window admits a second code
        self.flipped = 0            # GPU code != the oracle's nominal code
        self.block_scale_flips = 0
        self.bad = []
        self.row_flips = None       # per row of the last call: any flipped element

    def budget(self):
        return FLIP_FRACTION * self.two_candidate + FLIP_SLACK

    def check(self):
        assert not self.bad, f"intermediate codes outside the tie windows: {self.bad[:5]}"
        assert self.flipped <= self.budget(), \
            f"{self.flipped} flipped intermediate codes exceed the budget {self.budget():.0f} ({self!r})"

    def __repr__(self):
        frac = self.flipped / self.two_candidate if self.two_candidate else 0.0
        return (f"TieReport(elements={self.elements}, two_candidate={self.two_candidate}, "
                f"flipped={self.flipped} ({frac:.2%} of two-candidate), "
                f"block_scale_flips={self.block_scale_flips}, bad={len(self.bad)})")


def _mag_range(lo, hi, d, table_fn):
    with np.errstate(divide="ignore", invalid="ignore"):
        qlo = F.f32(np.maximum(lo, 0.0) / d)
        qhi = F.f32(hi / d)
    return table_fn(qlo).astype(np.int64), table_fn(qhi).astype(np.int64)


def expected_intermediate(res, mode, gpu, dn_inscale=None, report=None):
    """The down product's input implied by the GPU's (validated) intermediate.

    ``gpu``: A16 -> bf16 bits [n, I]; A8 -> (codes [n, I], fp32 scales [n, I/16]);
    A4 -> (packed codes [n, I/2], E4M3 scales [n, I/16]).  Returns double [n, I].
    Invalid choices are appended to report.bad as (row, col, reason).
    """
    rep = report if report is not None else TieReport()
    h = res.h32.astype(np.float64)
    err = h_error_bound(res)
    n, I = h.shape
    rep.elements += n * I
    if mode in ("A16", "F16"):   # one rounding to bf16 / fp16
        to16, from16 = (F.f64_to_bf16, F.bf16_to_f64) if mode == "A16" else (F.f64_to_f16, F.f16_to_f64)
        g = np.asarray(gpu, np.uint16)
        lo = to16(F.f32(h - err).astype(np.float64))
        hi = to16(F.f32(h + err).astype(np.float64))
        gv, lv, hv = from16(g), from16(lo), from16(hi)
        ok = (gv >= lv) & (gv <= hv)
        nom = res.hq[0]
        rep.two_candidate += int(np.sum(lo != hi))
        rep.flipped += int(np.sum(g != nom))
        rep.row_flips = np.any(g != nom, axis=1)
        for r, c in zip(*np.nonzero(~ok)):
            rep.bad.append((int(r), int(c), f"{mode} h {gv[r, c]} outside [{lv[r, c]}, {hv[r, c]}]"))
        return gv
    blocks = h.reshape(n, I // 16, 16)
    eb = err.reshape(n, I // 16, 16)
    if mode == "A8":
        codes_g = np.asarray(gpu[0], np.uint8).reshape(n, I // 16, 16)
        s_g = np.asarray(gpu[1], np.float32).astype(np.float64)
        bamax = np.abs(blocks).max(axis=2)
        bam_err = eb.max(axis=2)
        s_lo = F.f32(np.maximum(bamax - bam_err, 0) / 448.0).astype(np.float64)
        s_hi = F.f32((bamax + bam_err) / 448.0).astype(np.float64)
        ok_s = (s_g >= s_lo) & (s_g <= s_hi)
        for r, b in zip(*np.nonzero(~ok_s)):
            rep.bad.append((int(r), int(b), f"fp8 block scale {s_g[r, b]} outside [{s_lo[r, b]}, {s_hi[r, b]}]"))
        d = s_g[..., None]
        mlo, mhi = _mag_range(np.abs(blocks) - eb, np.abs(blocks) + eb, d,
                              lambda q: F.e4m3_quantize(q) & 0x7F)
        mg = (codes_g & 0x7F).astype(np.int64)
        sign_ok = (np.signbit(blocks) == ((codes_g & 0x80) != 0)) | (np.abs(blocks) <= eb) | (mg == 0)
        zero_block = ~(s_g > 0)[..., None] & (codes_g == 0)
        ok = ((mg >= mlo) & (mg <= mhi) & sign_ok) | zero_block
        val = F.e4m3_decode(codes_g) * s_g[..., None]
        nom_c, nom_s = res.hq
        # the fp32 block scale is a continuous value (validated by its window
        # above; it differs from the oracle's in the last bits whenever the fp32
        # block amax does), so the choice that counts is each code under the
        # GPU's own scale: the oracle's rounding of its fp32 h by that scale
        with np.errstate(divide="ignore", invalid="ignore"):
            nom_g = F.e4m3_quantize(F.f32(res.h32.astype(np.float64).reshape(n, I // 16, 16) / d))
        nom_g = np.where((s_g > 0)[..., None], nom_g, 0).astype(np.uint8)
        rep.two_candidate += int(np.sum(mlo != mhi))
        fl = (codes_g != nom_g).reshape(n, I)
        rep.flipped += int(np.sum(fl))
        rep.block_scale_flips += int(np.sum(s_g != nom_s.astype(np.float64)))
        # rows whose stored codes differ from the oracle's own (also where only the
        # fp32 scale's last bit moved a code across a midpoint): no unique result
        rep.row_flips = np.any(fl | (codes_g.reshape(n, I) != nom_c), axis=1)
    else:
        g_in = np.float64(np.float32(dn_inscale))
        codes_g = F.unpack_nibbles(np.asarray(gpu[0], np.uint8)).reshape(n, I // 16, 16)
        s_g = np.asarray(gpu[1], np.uint8)
        bamax = np.abs(blocks).max(axis=2)
        bam_err = eb.max(axis=2)
        with np.errstate(divide="ignore", invalid="ignore"):
            t_lo = F.f32(F.f32(np.maximum(bamax - bam_err, 0) / 6.0).astype(np.float64) / g_in)
            t_hi = F.f32(F.f32((bamax + bam_err) / 6.0).astype(np.float64) / g_in)
        c_lo, c_hi = F.e4m3_quantize(t_lo).astype(int), F.e4m3_quantize(t_hi).astype(int)
        ok_s = (s_g.astype(int) >= c_lo) & (s_g.astype(int) <= c_hi)
        for r, b in zip(*np.nonzero(~ok_s)):
            rep.bad.append((int(r), int(b), f"nvfp4 block scale {s_g[r, b]:#x} outside [{c_lo[r, b]:#x}, {c_hi[r, b]:#x}]"))
        nom_c, nom_s = res.hq
        rep.block_scale_flips += int(np.sum(s_g != nom_s))
        d = F.f32(F.e4m3_decode(s_g) * g_in).astype(np.float64)[..., None]
        mlo, mhi = _mag_range(np.abs(blocks) - eb, np.abs(blocks) + eb, d,
                              lambda q: F.e2m1_quantize(q) & 7)
        mg = (codes_g & 7).astype(np.int64)
        sign_ok = (np.signbit(blocks) == ((codes_g & 8) != 0)) | (np.abs(blocks) <= eb) | (mg == 0)
        zero_block = ~(d > 0) & (codes_g == 0)
        ok = ((mg >= mlo) & (mg <= mhi) & sign_ok) | zero_block
        val = F.e2m1_decode(codes_g) * F.e4m3_decode(s_g)[..., None] * g_in
        scale_amb = np.repeat((c_lo != c_hi)[..., None], 16, axis=2)
        rep.two_candidate += int(np.sum((mlo != mhi) | scale_amb))
        fl = (F.unpack_nibbles(np.asarray(gpu[0], np.uint8)) != F.unpack_nibbles(nom_c)) | \
            np.repeat(s_g != nom_s, 16, axis=1)
        rep.flipped += int(np.sum(fl))
        rep.row_flips = np.any(fl, axis=1)
    for r, b, i in zip(*np.nonzero(~ok)):
        rep.bad.append((int(r), int(b * 16 + i), "code outside the candidate range"))
    return val.reshape(n, I)
