"""Pins of the oracle's router, permutation, expert FFN, combine and calibration.

Each is checked against something other than its own formula: brute force in
pure Python (router ranking, stable sort), invariants (weights sum to one, the
inverse permutation, linearity), special cases that reduce to a textbook dense
SwiGLU MLP evaluated with torch's float64 CPU ops, and an independent torch
pipeline of the whole tiny layer.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import layer as L
from oracle import quant as Q


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------- router
def test_router_brute_force_tiny():
    rng = np.random.default_rng(21)
    for trial in range(20):
        T, E, H, k = 3, int(rng.integers(2, 9)), 16, None
        k = int(rng.integers(1, E + 1))
        x = _bf16(rng.standard_normal((T, H)))
        wr = _bf16(rng.standard_normal((E, H)) * 0.3)
        bias = (rng.standard_normal(E) * 0.1).astype(np.float32) if trial % 2 else None
        r = L.route(x, wr, k, bias)
        xv, wv = F.bf16_to_f64(x), F.bf16_to_f64(wr)
        for t in range(T):
            logits = [math.fsum(float(a) * float(b) for a, b in zip(xv[t], wv[e]))
                      + (float(bias[e]) if bias is not None else 0.0) for e in range(E)]
            order = sorted(range(E), key=lambda e: (-logits[e], e))[:k]
            assert list(r.ids[t]) == order
            m = max(logits)
            ex = [math.exp(l - m) for l in logits]
            sel = [ex[e] for e in order]
            for j in range(k):
                assert abs(r.w[t, j] - sel[j] / math.fsum(sel)) < 1e-14


def test_router_invariants():
    w = synth.CONFIGS[1]
    x = synth.tokens(w, T=4)
    wr = synth.router_weight(w)
    r = L.route(x, wr, w.k)
    assert np.allclose(r.w.sum(axis=1), 1.0, atol=1e-15)
    for t in range(4):
        assert len(set(r.ids[t])) == w.k
        assert np.all(np.diff(r.logits[t, r.ids[t]]) <= 0)
        assert r.logits[t, r.ids[t][-1]] >= np.delete(r.logits[t], r.ids[t]).max()


def test_router_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(22)
    x = _bf16(rng.standard_normal((2, 32)))
    wr = _bf16(rng.standard_normal((6, 32)) * 0.2)
    r = L.route(x, wr, 6)
    ref = torch.softmax(torch.from_numpy(F.bf16_to_f64(x) @ F.bf16_to_f64(wr).T), dim=1).numpy()
    assert np.allclose(np.take_along_axis(ref, r.ids.astype(np.int64), 1), r.w, rtol=1e-13)


def test_router_equal_logits_pick_lowest_ids():
    x = np.zeros((2, 16), np.uint16)
    wr = _bf16(np.ones((8, 16)))
    r = L.route(x, wr, 3)
    assert r.ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    assert np.allclose(r.w, 1 / 3)


# --------------------------------------------------------------------------- permute
def test_permute_brute_force():
    rng = np.random.default_rng(23)
    for _ in range(50):
        T, k, E = int(rng.integers(1, 12)), int(rng.integers(1, 4)), int(rng.integers(1, 9))
        k = min(k, E)
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        p = L.permute(ids, E)
        pairs = list(range(T * k))
        want = sorted(pairs, key=lambda q: ids.reshape(-1)[q])      # Python's sort is stable
        assert p.sorted_pairs.tolist() == want
        assert p.offsets[-1] == T * k and p.offsets[0] == 0
        for e in range(E):
            seg = p.sorted_pairs[p.offsets[e]:p.offsets[e + 1]]
            assert all(ids.reshape(-1)[q] == e for q in seg)
        assert np.array_equal(p.pair_row[p.sorted_pairs], np.arange(T * k))


# --------------------------------------------------------------------------- expert FFN
def _pow2_expert(rng, H, I, gscale=(2.0 ** -3, 2.0 ** -2), dscale=2.0 ** -1):
    """An expert whose weights are E2M1 values times powers of two, plus its dense matrices."""
    def mat(n, k, g):
        codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
        sc = rng.choice([0x30, 0x38, 0x40], (n, k // 16)).astype(np.uint8)   # 0.5, 1, 2
        dense = (F.e2m1_decode(codes) * F.e4m3_decode(sc).repeat(16, axis=1) * g)
        return F.pack_nibbles(codes), sc, dense
    cg, sg, dg = mat(I, H, gscale[0])
    cu, su, du = mat(I, H, gscale[1])
    cd, sd, dd = mat(H, I, dscale)
    ex = L.Expert(np.concatenate([cg, cu]), np.concatenate([sg, su]), cd, sd,
                  np.array(gscale, np.float32), np.float32(dscale),
                  np.array([0.01, 0.02], np.float32), np.float32(0.005))
    return ex, dg, du, dd


@pytest.mark.parametrize("mode", ["A16", "A8", "A4"])
def test_single_expert_is_dense_swiglu_mlp(mode):
    """E=1, k=1: the layer is a dense SwiGLU MLP; recompute it with torch float64."""
    rng = np.random.default_rng(24)
    H, I, T = 64, 32, 5
    ex, dg, du, dd = _pow2_expert(rng, H, I)
    x = _bf16(rng.standard_normal((T, H)))
    res = L.expert_ffn(ex, x, mode)
    xt = torch.from_numpy(F.bf16_to_f64(x))
    if mode == "A16":
        ag = au = xt
    elif mode == "A8":
        c, s = Q.fp8_block_quantize(F.bf16_to_f64(x).astype(np.float32))
        ag = au = torch.from_numpy(Q.fp8_block_dequantize(c, s))
    else:
        c0, s0 = Q.nvfp4_quantize(F.bf16_to_f64(x).astype(np.float32), ex.gu_inscale[0])
        c1, s1 = Q.nvfp4_quantize(F.bf16_to_f64(x).astype(np.float32), ex.gu_inscale[1])
        ag = torch.from_numpy(Q.nvfp4_dequantize(c0, s0, ex.gu_inscale[0]))
        au = torch.from_numpy(Q.nvfp4_dequantize(c1, s1, ex.gu_inscale[1]))
    g = ag @ torch.from_numpy(dg).T
    u = au @ torch.from_numpy(du).T
    h = torch.nn.functional.silu(g) * u
    assert torch.allclose(torch.from_numpy(res.h), h, rtol=1e-12, atol=1e-300)
    h32 = h.to(torch.float32)
    if mode == "A16":
        hq = h32.to(torch.bfloat16).to(torch.float64)
    elif mode == "A8":
        c, s = Q.fp8_block_quantize(h32.numpy())
        hq = torch.from_numpy(Q.fp8_block_dequantize(c, s))
    else:
        c, s = Q.nvfp4_quantize(h32.numpy(), ex.dn_inscale)
        hq = torch.from_numpy(Q.nvfp4_dequantize(c, s, ex.dn_inscale))
    y = hq @ torch.from_numpy(dd).T
    assert torch.allclose(torch.from_numpy(res.y), y, rtol=1e-12, atol=1e-300)


def test_zero_expert_gives_zero_and_down_is_linear():
    rng = np.random.default_rng(25)
    ex, *_ = _pow2_expert(rng, 32, 16)
    x = _bf16(rng.standard_normal((3, 32)))
    zero = L.Expert(np.zeros_like(ex.gu_codes), ex.gu_scales, ex.dn_codes, ex.dn_scales,
                    ex.gu_wscale, ex.dn_wscale)
    assert np.all(L.expert_ffn(zero, x, "A16").y == 0)
    y1 = L.expert_ffn(ex, x, "A16").y
    ex2 = L.Expert(ex.gu_codes, ex.gu_scales, ex.dn_codes, ex.dn_scales, ex.gu_wscale,
                   np.float32(ex.dn_wscale * 2))
    assert np.array_equal(L.expert_ffn(ex2, x, "A16").y, 2 * y1)


# --------------------------------------------------------------------------- combine
def test_combine_one_hot_and_order():
    rng = np.random.default_rng(26)
    T, k, H = 3, 2, 16
    y = rng.standard_normal((T * k, H))
    pair_row = rng.permutation(T * k).astype(np.int32)
    w = np.zeros((T, k))
    w[:, 1] = 1.0
    acc, out = L.combine(y, pair_row, w)
    for t in range(T):
        assert np.array_equal(acc[t], y[pair_row[t * k + 1]])
        assert np.array_equal(out[t], F.f64_to_bf16(y[pair_row[t * k + 1]]))


def test_residual_add_exact_then_round():
    a = _bf16(np.array([[1.0, 256.0, -3.0]]))
    b = _bf16(np.array([[2.0 ** -9, 1.0, 3.0]]))
    r = F.bf16_to_f64(L.residual_add(a, b))
    # 1 + 2^-9 is below half a bf16 ulp of 1; 257 is a tie between 256 and 258 -> even (256)
    assert r.tolist() == [[1.0, 256.0, 0.0]]


# --------------------------------------------------------------------------- whole tiny layer
@pytest.mark.parametrize("mode", ["A16", "A8", "A4"])
def test_tiny_layer_against_torch_pipeline(mode):
    """Configuration 0's layer through an independent torch pipeline (router, gather, MLP)."""
    w = synth.CONFIGS[0]
    x = synth.tokens(w, T=6)
    wr = synth.router_weight(w)
    experts = [L.pack_expert(*(synth.expert_matrix(w, 0, e, m) for m in range(3)))
               for e in range(w.E)]
    for ex in experts:
        ex.gu_inscale = np.array([0.002, 0.0021], np.float32)
        ex.dn_inscale = np.float32(0.0007)
    res = L.moe_layer(x, wr, w.k, lambda e: experts[e], mode)
    xt = torch.from_numpy(F.bf16_to_f64(x))
    logits = xt @ torch.from_numpy(F.bf16_to_f64(wr)).T
    p = torch.softmax(logits, dim=1)
    top = torch.topk(logits, w.k, dim=1)
    assert np.array_equal(top.indices.numpy(), res.route.ids)
    wts = torch.gather(p, 1, top.indices)
    wts = wts / wts.sum(dim=1, keepdim=True)
    assert torch.allclose(wts, torch.from_numpy(res.route.w), rtol=1e-13)
    out = torch.zeros(x.shape[0], w.H, dtype=torch.float64)
    for t in range(x.shape[0]):
        for j in range(w.k):
            e = int(top.indices[t, j])
            y = L.expert_ffn(experts[e], x[t:t + 1], mode).y[0]
            out[t] += wts[t, j] * torch.from_numpy(y)
    assert torch.allclose(out, torch.from_numpy(res.out_f64), rtol=1e-12, atol=1e-15)
    assert np.array_equal(res.out, F.f64_to_bf16(out.numpy()))


# --------------------------------------------------------------------------- shared expert
def test_shared_expert_equals_routed_expert_at_16_bits():
    """A shared expert whose bf16 matrices hold exactly the dequantized weights of an
    NVFP4 expert (E2M1 values times powers of two: bf16-exact) computes, before its
    gate, exactly what that routed expert computes in the 16-bit mode (a pinned
    function): same gate/up order, SwiGLU, bf16 intermediate and down orientation."""
    rng = np.random.default_rng(41)
    H, I, T = 64, 32, 5
    ex, dg, du, dd = _pow2_expert(rng, H, I)
    sh = L.SharedExpert(_bf16(np.concatenate([dg, du])), _bf16(dd), _bf16(np.zeros(H)))
    assert np.array_equal(F.bf16_to_f64(sh.gu), np.concatenate([dg, du]))   # exact in bf16
    x = _bf16(rng.standard_normal((T, H)))
    r = L.shared_expert(sh, x)
    e = L.expert_ffn(ex, x, "A16")
    assert np.array_equal(r.hq[0], e.hq[0])
    assert np.array_equal(r.y, e.y)
    assert np.all(r.sig == 0.5) and np.array_equal(r.gated, 0.5 * r.y)   # sigmoid(0)


def test_shared_expert_against_torch():
    """Random bf16 weights through an independent torch float64 pipeline: silu(g) * u,
    rounded to fp32 then bf16, the down projection, times torch.sigmoid of x . gate."""
    rng = np.random.default_rng(42)
    H, Is, T = 96, 48, 7
    sh = L.SharedExpert(_bf16(rng.standard_normal((2 * Is, H)) * 0.1), _bf16(rng.standard_normal((H, Is)) * 0.1),
                        _bf16(rng.standard_normal(H) * 0.2))
    x = _bf16(rng.standard_normal((T, H)))
    r = L.shared_expert(sh, x)
    xt = torch.from_numpy(F.bf16_to_f64(x))
    w = torch.from_numpy(F.bf16_to_f64(sh.gu))
    g, u = xt @ w[:Is].T, xt @ w[Is:].T
    h = torch.nn.functional.silu(g) * u
    hb = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    y = hb @ torch.from_numpy(F.bf16_to_f64(sh.dn)).T
    sg = torch.sigmoid(xt @ torch.from_numpy(F.bf16_to_f64(sh.gate)))
    assert torch.allclose(torch.from_numpy(r.h), h, rtol=1e-12, atol=1e-300)
    assert np.array_equal(F.bf16_to_f64(r.hq[0]), hb.numpy())
    assert torch.allclose(torch.from_numpy(r.gated), sg[:, None] * y, rtol=1e-12, atol=1e-300)
    # the gate: sigmoid(-z) = 1 - sigmoid(z), and a large logit saturates at 1
    r2 = L.shared_expert(L.SharedExpert(sh.gu, sh.dn, sh.gate ^ np.uint16(0x8000)), x)
    assert np.allclose(r.sig + r2.sig, 1.0, rtol=0, atol=1e-15)
    big = L.shared_expert(L.SharedExpert(sh.gu, sh.dn, _bf16(np.full(H, 64.0))), _bf16(np.ones((1, H))))
    assert big.sig[0] == 1.0


def test_layer_with_shared_expert_rounds_once():
    """The gated shared term joins the routed experts' weighted sum before the single
    bf16 rounding of the output."""
    w = synth.CONFIGS[0]
    x = synth.tokens(w, T=3)
    wr = synth.router_weight(w)
    experts = [L.pack_expert(*(synth.expert_matrix(w, 0, e, m) for m in range(3))) for e in range(w.E)]
    ws = synth.with_shared_expert(w, 64)
    sh = L.SharedExpert(*synth.shared_expert_weights(ws))
    assert sh.gu.shape == (128, w.H) and sh.dn.shape == (w.H, 64) and sh.gate.shape == (w.H,)
    base = L.moe_layer(x, wr, w.k, lambda e: experts[e], "A16")
    res = L.moe_layer(x, wr, w.k, lambda e: experts[e], "A16", shared=sh)
    gated = L.shared_expert(sh, x).gated
    assert np.array_equal(res.out_f64, base.out_f64 + gated)
    assert np.array_equal(res.out, F.f64_to_bf16(base.out_f64 + gated))
    assert not np.array_equal(res.out, L.residual_add(base.out, F.f64_to_bf16(gated)))   # not two roundings


# --------------------------------------------------------------------------- calibration
def test_calibration_scales():
    rng = np.random.default_rng(27)
    H, I = 32, 16
    experts = [_pow2_expert(rng, H, I)[0] for _ in range(3)]
    xc = _bf16(rng.standard_normal((8, H)))
    gu, dn = L.calibrate_input_scales(xc, experts)
    amax = np.abs(F.bf16_to_f64(xc)).max()
    assert np.all(gu == np.float32(amax) / np.float32(2688))
    xt = torch.from_numpy(F.bf16_to_f64(xc))
    for e, ex in enumerate(experts):
        h = torch.nn.functional.silu(xt @ torch.from_numpy(ex.gate()).T) * (xt @ torch.from_numpy(ex.up()).T)
        assert dn[e] == np.float32(h.abs().max().item() / 2688)
