"""The routed-expert layer, step by step, in double precision.

Sources (cited by page title and section):

* Layer shape: 512 routed experts per layer, the top 10 chosen per token,
  48 layers (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix (bit-exact)",
  opening description); the router is stored BF16 (same page, section "What is
  bit-exact and what is quantized").
* Expert arithmetic modes (page "Infernix", section "Activation precision"):
  4-bit activations with the checkpoint's calibrated input scales (W4A4, the
  default), 8-bit activations, or 16-bit activations on the stored 4-bit
  weights.  Weight-only 4-bit experts with 16-bit activations are W4A16 (same
  page, the "Uncensored" conversion).
* Exactness of FP4 products (page "Infernix releases", release 2026.10.11,
  "Highlights"): products of 4-bit weights and activations are exact and their
  row sums are integers in units of the scales.

The pages print no router formula and no expert activation function.  The
plainest reading for a Qwen-style MoE decoder, taken here: softmax over all
expert logits, the k largest (ties to the lower expert index), weights
renormalised over the k chosen; SwiGLU experts h = silu(gate) * up with
silu(z) = z / (1 + exp(-z)); the output is the routing-weighted sum of the
chosen experts' down projections, rounded once to bf16.

Shared expert and its gate (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for
Infernix (bit-exact)", section "What is bit-exact and what is quantized": the
shared experts and the gates are among the BF16 dense projections, stored
BF16).  The pages print no formula; the Qwen-style reading taken here: one
SwiGLU expert that every token runs, with BF16 gate/up [2Is, H] and down
[H, Is] matrices, bf16 activations and a bf16 intermediate (the dense
projections' activation precision), scaled per token by sigmoid(x . g) with g
the BF16 gate vector [H], and added to the routed experts' weighted sum before
the output's single rounding to bf16.

Precision of the intermediate h (read from the activation modes, which
describe "activations" at every expert matmul input): 16-bit mode rounds h to
bf16, 8-bit mode quantizes it to E4M3 per 16, 4-bit mode to NVFP4 per 16 under
the down matrix's input scale.  The quantizers take their decisions on the
fp32 value of h (the precision the kernel holds h in).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .formats import bf16_to_f64, f16_to_f64, f32, f64_to_bf16, f64_to_f16
from .quant import (fp8_block_dequantize, fp8_block_quantize, nvfp4_dequantize,
                    nvfp4_global_scale, nvfp4_quantize, q4g64_dequantize, q4g64_quantize)

MODES = ("A16", "A8", "A4", "F16")


# ----------------------------------------------------------------------------- experts
@dataclasses.dataclass
class Expert:
    """One expert in canonical layout.

    gu_codes [2I, H/2] / gu_scales [2I, H/16]: gate rows 0..I-1, then up rows;
    dn_codes [H, I/2] / dn_scales [H, I/16]; element 2i of a row in the low
    nibble; fp32 multipliers gu_wscale [2] (gate, up) and dn_wscale; fp32
    activation input scales gu_inscale [2] and dn_inscale (4-bit mode only).
    """
    gu_codes: np.ndarray
    gu_scales: np.ndarray
    dn_codes: np.ndarray
    dn_scales: np.ndarray
    gu_wscale: np.ndarray
    dn_wscale: np.float32
    gu_inscale: np.ndarray | None = None
    dn_inscale: np.float32 | None = None

    @property
    def I(self):
        return self.gu_codes.shape[0] // 2

    @property
    def H(self):
        return self.dn_codes.shape[0]

    def gate(self):
        I = self.I
        return nvfp4_dequantize(self.gu_codes[:I], self.gu_scales[:I], self.gu_wscale[0])

    def up(self):
        I = self.I
        return nvfp4_dequantize(self.gu_codes[I:], self.gu_scales[I:], self.gu_wscale[1])

    def down(self):
        return nvfp4_dequantize(self.dn_codes, self.dn_scales, self.dn_wscale)


@dataclasses.dataclass
class Q4Expert:
    """One expert in the q4_g64_fp16 encoding (page "Qwen3.8-Flash-Next NVIDIA
    NVFP4 for Infernix (bit-exact)", section "Drafting only": the drafter's routed
    experts): the canonical layout of Expert with int4 codes and fp16 scales, one
    per 64 values along K: gu_scales [2I, H/64], dn_scales [H, I/64] (fp16 bits);
    no per-matrix multiplier.  It runs in the "F16" mode (16-bit float
    activations: the encoding's fp16 domain)."""
    gu_codes: np.ndarray
    gu_scales: np.ndarray
    dn_codes: np.ndarray
    dn_scales: np.ndarray
    gu_inscale = None
    dn_inscale = None

    @property
    def I(self):
        return self.gu_codes.shape[0] // 2

    @property
    def H(self):
        return self.dn_codes.shape[0]

    def gate(self):
        return q4g64_dequantize(self.gu_codes[:self.I], self.gu_scales[:self.I])

    def up(self):
        return q4g64_dequantize(self.gu_codes[self.I:], self.gu_scales[self.I:])

    def down(self):
        return q4g64_dequantize(self.dn_codes, self.dn_scales)


def pack_expert_q4(w_gate, w_up, w_down):
    """q4_g64_fp16-pack one expert's fp32 gate [I, H], up [I, H], down [H, I]."""
    cg, sg = q4g64_quantize(w_gate)
    cu, su = q4g64_quantize(w_up)
    cd, sd = q4g64_quantize(w_down)
    return Q4Expert(np.concatenate([cg, cu]), np.concatenate([sg, su]), cd, sd)


def pack_matrix(w):
    """NVFP4-pack one fp32 matrix [N, K]: its global multiplier from its own amax."""
    w = np.asarray(w, np.float32)
    g = nvfp4_global_scale(np.abs(w).max())
    codes, scales = nvfp4_quantize(w, g)
    return codes, scales, np.float32(g)


def pack_expert(w_gate, w_up, w_down):
    """Pack one expert's fp32 gate [I, H], up [I, H], down [H, I] matrices."""
    cg, sg, gg = pack_matrix(w_gate)
    cu, su, gu = pack_matrix(w_up)
    cd, sd, gd = pack_matrix(w_down)
    return Expert(np.concatenate([cg, cu]), np.concatenate([sg, su]), cd, sd,
                  np.array([gg, gu], np.float32), np.float32(gd))


# ----------------------------------------------------------------------------- router
@dataclasses.dataclass
class Route:
    ids: np.ndarray       # int32 [T, k], by descending logit
    w: np.ndarray         # double [T, k], renormalised weights
    logits: np.ndarray    # double [T, E] (bias included)
    probs: np.ndarray     # double [T, E] softmax over all experts


def route(x_bf16, wr_bf16, k, bias=None):
    """Router logits, softmax, top-k, renormalise (double precision).

    logits[t, e] = sum_h x[t, h] * Wr[e, h] (+ bias[e]); p = softmax over all E;
    the k largest logits in descending order, equal logits by lower index;
    w_j = p_j / sum of the chosen p.
    """
    x = bf16_to_f64(x_bf16)
    wr = bf16_to_f64(wr_bf16)
    logits = x @ wr.T
    if bias is not None:
        logits = logits + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k]
    psel = np.take_along_axis(p, ids, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True)
    return Route(ids.astype(np.int32), w, logits, p)


# ----------------------------------------------------------------------------- permute
@dataclasses.dataclass
class Permutation:
    offsets: np.ndarray       # int32 [E + 1]
    sorted_pairs: np.ndarray  # int32 [T*k]: pair ids p = t*k + j grouped by expert, ascending p
    pair_row: np.ndarray      # int32 [T*k]: inverse, pair_row[sorted_pairs[i]] = i


def permute(ids, E):
    """Stable counting sort of the pairs p = t*k + j by expert id."""
    flat = np.asarray(ids, np.int64).reshape(-1)
    cnt = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int32)
    pair_row = np.empty_like(sorted_pairs)
    pair_row[sorted_pairs] = np.arange(flat.size, dtype=np.int32)
    return Permutation(offsets, sorted_pairs, pair_row)


# ----------------------------------------------------------------------------- expert FFN
@dataclasses.dataclass
class FfnResult:
    a_gate: np.ndarray    # double [n, H]: activation as the gate product sees it
    a_up: np.ndarray
    g: np.ndarray         # double [n, I]
    u: np.ndarray
    h: np.ndarray         # double [n, I]: silu(g) * u
    h32: np.ndarray       # fp32 [n, I]
    hq: tuple             # intermediate as stored: (bf16,) | (codes, fp32 scales) | (codes, e4m3 scales)
    hdq: np.ndarray       # double [n, I]: the value the down product sees
    y: np.ndarray         # double [n, H]
    gate_abs: np.ndarray  # double [n, I]: sum_K |a_K * Wg[i, K]|  (size of the gate sum's terms)
    up_abs: np.ndarray


def quantize_activation(x32, mode, inscale=None):
    """Activation as an expert matrix sees it, per mode; returns (stored form, double value).
    "F16" (the q4_g64_fp16 experts): IEEE fp16, rounded to nearest even."""
    if mode == "A16":
        b = f64_to_bf16(x32)
        return (b,), bf16_to_f64(b)
    if mode == "F16":
        b = f64_to_f16(np.asarray(x32, np.float32).astype(np.float64))
        return (b,), f16_to_f64(b)
    if mode == "A8":
        c, s = fp8_block_quantize(x32)
        return (c, s), fp8_block_dequantize(c, s)
    if mode == "A4":
        c, s = nvfp4_quantize(x32, inscale)
        return (c, s), nvfp4_dequantize(c, s, inscale)
    raise ValueError(mode)


def expert_ffn(ex: Expert, x_bf16, mode):
    """One expert on rows x [n, H] (bf16 bits): gate/up, SwiGLU, intermediate, down."""
    x32 = bf16_to_f64(x_bf16).astype(np.float32)
    if mode == "A16":
        a_gate = a_up = x32.astype(np.float64)
    elif mode == "F16":
        a_gate = a_up = quantize_activation(x32, "F16")[1]
    elif mode == "A8":
        a_gate = a_up = quantize_activation(x32, "A8")[1]
    elif mode == "A4":
        a_gate = quantize_activation(x32, "A4", ex.gu_inscale[0])[1]
        a_up = quantize_activation(x32, "A4", ex.gu_inscale[1])[1]
    else:
        raise ValueError(mode)
    wg, wu = ex.gate(), ex.up()
    g = a_gate @ wg.T
    u = a_up @ wu.T
    h = u * (g / (1.0 + np.exp(-g)))
    h32 = f32(h)
    hq, hdq = quantize_activation(h32, mode, ex.dn_inscale)
    y = hdq @ ex.down().T
    return FfnResult(a_gate, a_up, g, u, h, h32, hq, hdq, y,
                     np.abs(a_gate) @ np.abs(wg).T, np.abs(a_up) @ np.abs(wu).T)


# ----------------------------------------------------------------------------- shared expert
@dataclasses.dataclass
class SharedExpert:
    """The shared expert in bf16 bits: gu [2Is, H] (gate rows, then up rows),
    dn [H, Is], gate [H] (the vector of its sigmoid gate)."""
    gu: np.ndarray
    dn: np.ndarray
    gate: np.ndarray

    @property
    def Is(self):
        return self.gu.shape[0] // 2


@dataclasses.dataclass
class SharedResult:
    g: np.ndarray         # double [T, Is]
    u: np.ndarray
    h: np.ndarray         # double silu(g) * u
    h32: np.ndarray       # fp32 [T, Is]
    hq: tuple             # (bf16 bits [T, Is],): the intermediate as stored
    hdq: np.ndarray       # double value of the stored intermediate
    y: np.ndarray         # double [T, H]: down projection, before the gate
    logit: np.ndarray     # double [T]: x . gate
    sig: np.ndarray       # double [T]: sigmoid(logit)
    gated: np.ndarray     # double [T, H]: sig * y, the term added to the output
    gate_abs: np.ndarray  # double [T, Is]: sum_K |x_K * Wg[i, K]|
    up_abs: np.ndarray


def shared_expert(sh: SharedExpert, x_bf16):
    """The shared expert on rows x [T, H] (bf16 bits), in double precision:
    g = x Wg^T, u = x Wu^T, h = silu(g) u, stored as bf16 of its fp32 value,
    y = h Wd^T, gated by sigmoid(x . gate)."""
    x = bf16_to_f64(x_bf16)
    Is = sh.Is
    wg = bf16_to_f64(sh.gu[:Is])
    wu = bf16_to_f64(sh.gu[Is:])
    wd = bf16_to_f64(sh.dn)
    g = x @ wg.T
    u = x @ wu.T
    h = u * (g / (1.0 + np.exp(-g)))
    h32 = f32(h)
    hb = f64_to_bf16(h32)
    hdq = bf16_to_f64(hb)
    y = hdq @ wd.T
    logit = x @ bf16_to_f64(sh.gate)
    sig = 1.0 / (1.0 + np.exp(-logit))
    return SharedResult(g, u, h, h32, (hb,), hdq, y, logit, sig, sig[:, None] * y,
                        np.abs(x) @ np.abs(wg).T, np.abs(x) @ np.abs(wu).T)


# ----------------------------------------------------------------------------- combine
def combine(y_sorted, pair_row, w):
    """out[t] = bf16( sum_j w[t, j] * y[pair_row[t*k + j]] ), j ascending, in double.

    Returns (the double sum before rounding [T, H], bf16 bits [T, H]).
    """
    w = np.asarray(w, np.float64)
    T, k = w.shape
    acc = np.zeros((T, y_sorted.shape[1]), np.float64)
    for j in range(k):
        acc += w[:, j:j + 1] * y_sorted[pair_row[np.arange(T) * k + j]]
    return acc, f64_to_bf16(acc)


def residual_add(x_bf16, out_bf16):
    """Next layer's input: bf16(x + out), both bf16; the sum is exact in double."""
    return f64_to_bf16(bf16_to_f64(x_bf16) + bf16_to_f64(out_bf16))


# ----------------------------------------------------------------------------- layer
@dataclasses.dataclass
class LayerResult:
    route: Route
    perm: Permutation
    ffn: dict             # expert id -> FfnResult over that expert's rows (sorted order)
    y_sorted: np.ndarray  # double [T*k, H]
    out_f64: np.ndarray   # double [T, H] before the bf16 rounding
    out: np.ndarray       # bf16 bits [T, H]
    shared: SharedResult | None = None


def moe_layer(x_bf16, wr_bf16, k, get_expert, mode, bias=None, shared=None):
    """The whole routed-expert layer for tokens x [T, H] (bf16 bits).

    get_expert(e) returns the Expert e (only the chosen experts are requested).
    With a SharedExpert, its gated output is added to the routed experts'
    weighted sum before the output's rounding to bf16.
    """
    x_bf16 = np.asarray(x_bf16, np.uint16)
    T, H = x_bf16.shape
    r = route(x_bf16, wr_bf16, k, bias)
    E = np.asarray(wr_bf16).shape[0]
    perm = permute(r.ids, E)
    y_sorted = np.zeros((T * k, H), np.float64)
    ffn = {}
    for e in np.nonzero(np.diff(perm.offsets))[0]:
        rows = slice(perm.offsets[e], perm.offsets[e + 1])
        tok = perm.sorted_pairs[rows] // k
        res = expert_ffn(get_expert(int(e)), x_bf16[tok], mode)
        ffn[int(e)] = res
        y_sorted[rows] = res.y
    acc, out = combine(y_sorted, perm.pair_row, r.w)
    sres = None
    if shared is not None:
        sres = shared_expert(shared, x_bf16)
        acc = acc + sres.gated
        out = f64_to_bf16(acc)
    return LayerResult(r, perm, ffn, y_sorted, acc, out, sres)


# ----------------------------------------------------------------------------- calibration
def calibrate_input_scales(x_calib_bf16, experts):
    """Activation input scales of 4-bit mode from a calibration batch.

    gate/up: f32(amax(x_calib) / 2688), the same for every expert and both
    matrices.  down: f32(amax(h_e) / 2688) with h_e = silu(g) * up over every
    calibration token through expert e, computed from bf16 x_calib and the
    dequantized weights without activation quantization.  ``experts`` is a
    sequence of Expert (all experts of the layer).
    Returns (gu_inscale [E, 2] fp32, dn_inscale [E] fp32).
    """
    x = bf16_to_f64(x_calib_bf16)
    gu = nvfp4_global_scale(np.abs(x).max())
    E = len(experts)
    gu_in = np.full((E, 2), gu, np.float32)
    dn_in = np.empty(E, np.float32)
    for e, ex in enumerate(experts):
        g = x @ ex.gate().T
        u = x @ ex.up().T
        h = u * (g / (1.0 + np.exp(-g)))
        dn_in[e] = nvfp4_global_scale(np.abs(h).max())
    return gu_in, dn_in
