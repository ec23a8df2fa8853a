"""GPU parity of each entry point against the oracle, through the C ABI.

Small and mid-size cases (seconds of oracle time) that span several tiles and
ragged tails; the full-size workloads are in test_gpu_workloads.py.
"""
import os
import sys

import numpy as np
import pytest
import torch

import synth
import nvfp4_block_scaled_softmax_amd as moe
from oracle import formats as F
from oracle import layer as OL
from oracle import quant as Q
from tests import oracle_cache, parity, ties

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_dev(u16, dev):
    return to_dev(np.asarray(u16, np.uint16).view(np.int16), dev).view(torch.bfloat16)


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def say(*a):
    print("[case]", *a, flush=True)


# --------------------------------------------------------------------------- generator
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_generator_gpu_matches_host(dev, dtype):
    cases = [(1001, synth.TAG_EXPERT, 5, 7, 3, 1, 0.02, 0, 100003),
             (1004, synth.TAG_X, 0, 0, 1, 0, 1.0, 13, 5000),
             (1003, synth.TAG_ROUTER, 47, 0, 1, 0, 0.02, 0, 512 * 3072),
             (1002, synth.TAG_EXPERT, 0, 500, 12, 2, 0.02, 1536 * 77, 1536 * 3)]
    for seed, tag, layer, e0, ne, m, sig, i0, n in cases:
        say("generator", dtype, seed, tag, layer, e0, ne, m, i0, n)
        t = torch.empty(ne, n, dtype=dtype, device=dev)
        synth.gpu_normal_(t, seed, tag, layer=layer, expert=e0, matrix=m, sigma=sig, i0=i0,
                          n_expert=ne)
        if dtype == torch.float32:
            want = synth.normal_f32(n, seed, tag, layer, e0, m, sig, i0, ne)
            got = host(t).reshape(want.shape)
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        else:
            want = synth.normal_bf16(n, seed, tag, layer, e0, m, sig, i0, ne)
            assert np.array_equal(host(t).reshape(want.shape), want)


# --------------------------------------------------------------------------- quantizers
def _golden_cases(name):
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


def test_nvfp4_quant_golden_blocks(dev):
    cases = _golden_cases("nvfp4_blocks.txt")
    x = np.zeros((len(cases), 32), np.float32)
    g = np.zeros(len(cases), np.float32)
    for i, c in enumerate(cases):
        x[i, :16] = [float(v) for v in c["x"]]
        g[i] = float(c["g"][0])
    say("golden nvfp4 blocks", len(cases))
    codes, scales = moe.act_quant_nvfp4(to_dev(x, dev), to_dev(g, dev),
                                        to_dev(np.arange(len(cases), dtype=np.int32), dev))
    codes, scales = host(codes), host(scales)
    for i, c in enumerate(cases):
        assert scales[i, 0] == int(c["scale"][0], 16), c["name"]
        want = [int(v, 16) for v in c["codes"]]
        assert F.unpack_nibbles(codes[i])[:16].tolist() == want, c["name"]


def _edge_rows(rng, cols):
    rows = [np.zeros(cols), -np.zeros(cols), np.full(cols, 1e-30), np.full(cols, 3e38),
            rng.standard_normal(cols) * 1e-6, rng.standard_normal(cols) * 1e4]
    mid = np.tile(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5, -0.25, -5.0, 0.1,
                            3.0, 4.0, 2.0, 1.0]), cols // 16)
    rows.append(mid)
    return np.array(rows, np.float32)


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_nvfp4_quant_matches_oracle(dev, xdt):
    rng = np.random.default_rng(101)
    cols = 3072
    x = np.concatenate([(rng.standard_normal((250, cols)) * s).astype(np.float32)
                        for s in (1.0, 0.02)] + [_edge_rows(rng, cols)])
    if xdt == "bf16":
        xb = F.f64_to_bf16(x.astype(np.float64))
        x = F.bf16_to_f64(xb).astype(np.float32)
        xin = bf16_dev(xb, dev)
    else:
        xin = to_dev(x, dev)
    R = x.shape[0]
    g = np.array([Q.nvfp4_global_scale(np.abs(x[r]).max()) if r % 3 else np.float32(1e-3 * (1 + r % 5))
                  for r in range(R)], np.float32)
    g[-7:] = [1.0, 1.0, 1.0, 1e30, 1e-3, 2.0, 1.0]
    say("nvfp4 quant vs oracle", xdt, R, cols)
    codes, scales = moe.act_quant_nvfp4(xin, to_dev(g, dev), to_dev(np.arange(R, dtype=np.int32), dev))
    wc, ws = Q.nvfp4_quantize(x, g)
    assert np.array_equal(host(scales), ws)
    assert np.array_equal(host(codes), wc)


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_fp8_quant_matches_oracle(dev, xdt):
    rng = np.random.default_rng(102)
    cols = 512
    x = np.concatenate([(rng.standard_normal((300, cols)) * s).astype(np.float32)
                        for s in (1.0, 1e-3, 300.0)] + [_edge_rows(rng, cols)[:2]])
    if xdt == "bf16":
        xb = F.f64_to_bf16(x.astype(np.float64))
        x = F.bf16_to_f64(xb).astype(np.float32)
        xin = bf16_dev(xb, dev)
    else:
        xin = to_dev(x, dev)
    say("fp8 quant vs oracle", xdt, x.shape)
    codes, scales = moe.act_quant_fp8(xin)
    wc, ws = Q.fp8_block_quantize(x)
    assert np.array_equal(host(scales).view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(host(codes), wc)
    for c in _golden_cases("fp8_blocks.txt"):
        xx = np.zeros((1, 32), np.float32)
        xx[0, :16] = [float(v) for v in c["x"]]
        cc, ss = moe.act_quant_fp8(to_dev(xx, dev))
        assert host(ss)[0, 0] == np.float32(float(c["scale"][0])), c["name"]
        assert [f"{v:02X}" for v in host(cc)[0, :16]] == [v.upper() for v in c["codes"]], c["name"]


def test_global_scale_matches_oracle(dev):
    rng = np.random.default_rng(103)
    x = (rng.standard_normal((7, 1000, 96)) * np.array([1, 0.02, 5, 1e-5, 1, 3, 0.5])[:, None, None]).astype(np.float32)
    x[3] = 0.0
    say("global scale", x.shape)
    g = host(moe.nvfp4_global_scale(to_dev(x, dev)))
    want = np.array([Q.nvfp4_global_scale(np.abs(x[m]).max()) for m in range(7)], np.float32)
    assert np.array_equal(g, want)


# --------------------------------------------------------------------------- router
@pytest.mark.parametrize("wi,T", [(0, 1), (0, 8), (1, 1), (1, 2), (1, 8), (1, 9), (1, 100), (4, 1024)])
def test_route_matches_oracle(dev, wi, T):
    w = synth.CONFIGS[wi]
    x = synth.tokens(w, batch=3, T=T)
    wr = synth.router_weight(w)
    bias = synth.zipf_bias(w)
    say("route", wi, T)
    ids, tw = moe.moe_route_topk(bf16_dev(x, dev), bf16_dev(wr, dev), w.k,
                                 None if bias is None else to_dev(bias, dev))
    r, flipped = parity.check_route(x, wr, bias, w.k, host(ids), host(tw))
    assert len(flipped) <= max(1, T // 100), flipped


@pytest.mark.parametrize("T,H,E,k", [(45, 32, 40, 3), (45, 64, 40, 3), (70, 96, 33, 5), (33, 4096, 97, 8)])
def test_route_wide_ragged(dev, T, H, E, k):
    """T > 8 takes the MFMA logits kernel: ragged token and expert tiles, K ranges
    shorter than the four-way split (H = 32, 64, 96), and the largest H."""
    rng = np.random.default_rng(T + H + E)
    x = F.f64_to_bf16(rng.standard_normal((T, H)))
    wr = F.f64_to_bf16(rng.standard_normal((E, H)) / np.sqrt(H))
    say("route wide", T, H, E, k)
    ids, tw = moe.moe_route_topk(bf16_dev(x, dev), bf16_dev(wr, dev), k)
    r, flipped = parity.check_route(x, wr, None, k, host(ids), host(tw))
    assert len(flipped) <= 1, flipped


def test_route_ties_and_small_k(dev):
    # equal logits: ids 0..k-1 in order, uniform weights
    x = np.zeros((3, 256), np.uint16)
    wr = F.f64_to_bf16(np.random.default_rng(5).standard_normal((40, 256)))
    ids, tw = moe.moe_route_topk(bf16_dev(x, dev), bf16_dev(wr, dev), 5)
    assert host(ids).tolist() == [[0, 1, 2, 3, 4]] * 3
    assert np.allclose(host(tw), 0.2, atol=1e-7)
    # k = E reproduces the full softmax ordering
    x = F.f64_to_bf16(np.random.default_rng(6).standard_normal((4, 256)))
    ids, tw = moe.moe_route_topk(bf16_dev(x, dev), bf16_dev(wr, dev), 40)
    parity.check_route(x, wr, None, 40, host(ids), host(tw))


# --------------------------------------------------------------------------- permute
@pytest.mark.parametrize("T,k,E", [(1, 10, 512), (8, 10, 512), (2, 10, 512), (1024, 10, 512),
                                   (33, 2, 8), (3000, 8, 1024), (7, 1, 1), (257, 8, 64), (1024, 10, 512)])
def test_permute_matches_oracle(dev, T, k, E):
    rng = np.random.default_rng(T * 1000 + k * 10 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if T >= 1024:   # skewed: a few popular experts, as with a Zipf router bias
        pop = rng.zipf(1.3, size=(T, k)) % E
        ids = np.array([list(dict.fromkeys(list(p) + list(rng.permutation(E))))[:k] for p in pop], np.int32)
    say("permute", T, k, E)
    off, sp, pr = moe.moe_permute(to_dev(ids, dev), E)
    p = OL.permute(ids, E)
    assert np.array_equal(host(off), p.offsets)
    assert np.array_equal(host(sp), p.sorted_pairs)
    assert np.array_equal(host(pr), p.pair_row)


def test_permute_drops_invalid_ids(dev):
    ids = np.array([[0, 5], [9, 1], [-1, 5], [3, 0]], np.int32)
    off, sp, pr = moe.moe_permute(to_dev(ids, dev), 6)
    assert host(off).tolist() == [0, 2, 3, 3, 4, 4, 6]
    assert host(sp)[:6].tolist() == [0, 7, 3, 6, 1, 5]
    assert host(pr).tolist() == [0, 4, -1, 2, -1, 5, 3, 1]


def test_permute_multiblock_invalid_ids(dev):
    """More than 2048 pairs (the several-workgroup path) with out-of-range ids
    scattered over the blocks, including a block boundary."""
    rng = np.random.default_rng(77)
    T, k, E = 700, 4, 96
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = rng.choice(T * k, 40, replace=False)
    ids.reshape(-1)[bad] = rng.choice([-1, E, E + 7, -5], 40)
    ids.reshape(-1)[1023:1026] = -1
    off, sp, pr = moe.moe_permute(to_dev(ids, dev), E)
    # expected: the stable sort of the valid pairs only; dropped pairs get row -1
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    want_off = np.concatenate([[0], np.cumsum(np.bincount(flat[valid], minlength=E))])
    order = np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")]
    want_pr = np.full(flat.size, -1)
    want_pr[order] = np.arange(order.size)
    assert np.array_equal(host(off), want_off)
    assert np.array_equal(host(sp)[:order.size], order)
    assert np.array_equal(host(pr), want_pr)


# --------------------------------------------------------------------------- combine
def test_combine_matches_oracle(dev):
    rng = np.random.default_rng(104)
    T, k, H = 37, 10, 3072
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    pr = rng.permutation(T * k).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    res = F.f64_to_bf16(rng.standard_normal((T, H)))
    say("combine", T, k, H)
    out = host(moe.moe_combine(to_dev(y, dev), to_dev(pr, dev), to_dev(w, dev)))
    acc, want = OL.combine(y.astype(np.float64), pr, w.astype(np.float64))
    # fp32 sums of ten terms: the bf16 result is the oracle's or one ulp away
    d = np.abs(F.bf16_to_f64(out) - F.bf16_to_f64(want))
    assert np.all(d <= np.abs(F.bf16_to_f64(want)) * 2.0 ** -7 + 1e-30)
    assert np.mean(out == want) > 0.99
    out2 = host(moe.moe_combine(to_dev(y, dev), to_dev(pr, dev), to_dev(w, dev), residual=bf16_dev(res, dev)))
    want2 = OL.residual_add(res, out)
    assert np.array_equal(out2, want2)


# --------------------------------------------------------------------------- expert FFN
def _small_workload(idx, E, k, H, I, T):
    return synth.Workload(100 + idx, f"small {idx}", E=E, k=k, H=H, I=I, T=T, modes=("A16",))


SMALL = [(0, 1, 1, 64, 64, 5), (1, 2, 2, 128, 64, 3), (2, 8, 2, 256, 128, 8),
         (3, 8, 1, 96, 160, 33), (4, 4, 2, 256, 256, 17), (5, 16, 4, 512, 96, 9)]


def _inscales_for(E, seed):
    rng = np.random.default_rng(seed)
    gu = (rng.uniform(0.5, 2.0, (E, 2)) * 4.0 / 2688).astype(np.float32)
    dn = (rng.uniform(0.5, 2.0, E) * 0.3 / 2688).astype(np.float32)
    return gu, dn


def _upload(ex_list, dev, inscales=None):
    st = lambda name: to_dev(np.stack([getattr(ex, name) for ex in ex_list]), dev)
    return moe.Experts(st("gu_codes"), st("gu_scales"), st("dn_codes"), st("dn_scales"),
                       st("gu_wscale"), to_dev(np.array([ex.dn_wscale for ex in ex_list], np.float32), dev),
                       None if inscales is None else to_dev(inscales[0], dev),
                       None if inscales is None else to_dev(inscales[1], dev))


@pytest.mark.parametrize("mode", ["A16", "A8", "A4"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"E{c[1]}k{c[2]}H{c[3]}I{c[4]}T{c[5]}")
def test_expert_ffn_small_shapes(dev, mode, case):
    idx, E, k, H, I, T = case
    w = _small_workload(idx, E, k, H, I, T)
    ins = _inscales_for(E, idx)
    cache = oracle_cache.ExpertCache(w, 0, ins)
    cache.prefetch(range(E))
    experts = _upload([cache(e) for e in range(E)], dev, ins)
    x = synth.tokens(w, batch=idx, T=T)
    rng = np.random.default_rng(idx)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    p = OL.permute(ids, E)
    say("ffn small", mode, case)
    y, wsb = moe.nvfp4_expert_ffn(experts, mode, bf16_dev(x, dev), k, to_dev(p.offsets, dev),
                                  to_dev(p.sorted_pairs, dev))
    views = {n: host(v) for n, v in moe.ffn_workspace_views(wsb, mode, T, k, H, I).items()}
    parity.check_experts(w, mode, x, cache, k, p.offsets, p.sorted_pairs, host(y), views)


# --------------------------------------------------------------------------- tiny layer
@pytest.mark.parametrize("mode", ["A16", "A8", "A4"])
def test_tiny_layer_matches_oracle(dev, mode):
    w = synth.CONFIGS[0]
    E, H, I, k = w.E, w.H, w.I, w.k
    ins = _inscales_for(E, 7) if mode == "A4" else None
    cache = oracle_cache.ExpertCache(w, 0, ins)
    cache.prefetch(range(E))
    experts = _upload([cache(e) for e in range(E)], dev, ins)
    wr = synth.router_weight(w)
    for T in (1, 4, 8, 19):
        x = synth.tokens(w, batch=T, T=T)
        say("tiny layer", mode, T)
        out, wsb = moe.moe_layer_forward(experts, mode, bf16_dev(x, dev), bf16_dev(wr, dev), k)
        v = {n: host(t) for n, t in moe.workspace_views(wsb, mode, T, k, E, H, I).items() if n != "ffn"}
        fv = {n: host(t) for n, t in moe.ffn_workspace_views(moe.workspace_views(wsb, mode, T, k, E, H, I)["ffn"], mode, T, k, H, I).items()}
        r, flipped = parity.check_route(x, wr, None, k, v["topk_ids"], v["topk_w"])
        parity.check_permutation(v["topk_ids"], E, v["expert_offsets"], v["sorted_pairs"], v["pair_row"], r.ids)
        y_exp, info = parity.check_experts(w, mode, x, cache, k, v["expert_offsets"], v["sorted_pairs"], v["y_pairs"], fv)
        parity.check_output(host(out), y_exp, v["pair_row"], r, v["topk_ids"], k, mode=mode,
                            y_nom=info["y_nominal"], row_flipped=info["row_flipped"], oracle_ids=r.ids)


def test_layer_is_deterministic(dev):
    w = synth.CONFIGS[0]
    cache = oracle_cache.ExpertCache(w)
    cache.prefetch(range(w.E))
    experts = _upload([cache(e) for e in range(w.E)], dev)
    x = bf16_dev(synth.tokens(w, batch=1, T=64), dev)
    wr = bf16_dev(synth.router_weight(w), dev)
    a, ws = moe.moe_layer_forward(experts, "A16", x, wr, w.k)
    b, _ = moe.moe_layer_forward(experts, "A16", x, wr, w.k)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # per-stage path (these sizes are not fused): the two halves equal the whole
    c = torch.empty_like(a)
    for stage in (0, 1):
        moe.moe_layer_forward_stage(experts, "A16", stage, x, wr, w.k, None, None, ws, c)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("mode", ["A4", "A16", "A8"])
@pytest.mark.parametrize("H,I", [(256, 128), (384, 256), (640, 384), (96, 160), (3072, 512)])
def test_expert_ffn_wide_hot_expert(dev, H, I, mode):
    """Calls wider than 8 tokens take the MFMA path when H and I are multiples of
    128 (K loops of 1-5 and 24 steps), the one-column kernels otherwise (96,
    160): one expert with more than 128 tokens (several passes), others with a
    few, one with none; in each activation mode."""
    E, k, T = 6, 2, 300
    w = _small_workload(20 + H % 7, E, k, H, I, T)
    ins = _inscales_for(E, 21)
    cache = oracle_cache.ExpertCache(w, 0, ins)
    cache.prefetch(range(E))
    experts = _upload([cache(e) for e in range(E)], dev, ins)
    x = synth.tokens(w, batch=5, T=T)
    rng = np.random.default_rng(22)
    ids = np.stack([[0, int(rng.choice([1, 2, 3, 5], p=[0.6, 0.3, 0.05, 0.05]))] for _ in range(T)]).astype(np.int32)
    p = OL.permute(ids, E)
    assert np.diff(p.offsets)[0] == T and np.diff(p.offsets)[4] == 0
    say("ffn wide", mode, H, I, np.diff(p.offsets))
    y, wsb = moe.nvfp4_expert_ffn(experts, mode, bf16_dev(x, dev), k, to_dev(p.offsets, dev),
                                  to_dev(p.sorted_pairs, dev))
    views = {n: host(v) for n, v in moe.ffn_workspace_views(wsb, mode, T, k, H, I).items()}
    _, info = parity.check_experts(w, mode, x, cache, k, p.offsets, p.sorted_pairs, host(y), views)
    say("ok", info["y_worst_rel"], info["ties"])
    if H % 128 == 0 and I % 128 == 0:
        # the work plan: each expert's rows in chunks of at most 32, experts in order
        want = [(e, r0, min(32, p.offsets[e + 1] - r0)) for e in range(E)
                for r0 in range(p.offsets[e], p.offsets[e + 1], 32)]
        plan = views["plan"]
        assert [tuple(int(v) for v in row[:3]) for row in plan[:len(want)]] == want
        n_used = min(T * k, E) + T * k // 32            # entries the kernels read
        assert np.all(plan[len(want):n_used, 0] == -1)
