"""Full-size workloads on the GPU, in the launch configuration bench.py times.

The layer is built as bench.py builds it: expert weights drawn on the GPU by
the seeded generator and NVFP4-packed by the library.  The oracle packs the
same experts from the host build of the generator; the packed bytes of every
expert a checked token touches must be identical (act_quant_nvfp4 on real
weight matrices), and the layer output is checked token by token: every token
of every call, the 1024-token prefill chunk included, and every layer of the
48-layer stack (each GPU layer fed the oracle chain's own input).
"""
import numpy as np
import pytest
import torch

import bench
import synth
import nvfp4_block_scaled_softmax_amd as moe
from oracle import formats as F
from oracle import layer as OL
from tests import oracle_cache, parity, ties

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def say(*a):
    print("[case]", *a, flush=True)


_LAYERS = {}


def gpu_layer_pair(w, layer, mode, dev):
    """Like gpu_layer, but several layers of one workload may be held at once."""
    key = ("pair", w.index, layer, mode)
    if key not in _LAYERS:
        say("building layer", key)
        _LAYERS[key] = bench.build_layer(w, layer, dev, mode)
    return _LAYERS[key]


def gpu_layer(w, layer, mode, dev):
    key = (w.index, layer, mode)
    if key not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        say("building layer", key)
        _LAYERS[key] = bench.build_layer(w, layer, dev, mode)
    return _LAYERS[key]


def check_packed_bytes(ex_gpu, cache, experts):
    """GPU-packed weights of these experts == the oracle's packing, byte for byte
    (tiled experts: the oracle's scales in the tiled order)."""
    tiled = getattr(ex_gpu, "layout", 0) == moe.LAYOUT_TILED
    for e in experts:
        o = cache(e)
        gs, ds = (F.tiled_scales(o.gu_scales), F.tiled_scales(o.dn_scales)) if tiled else (o.gu_scales, o.dn_scales)
        assert np.array_equal(host(ex_gpu.gu_codes[e]), o.gu_codes), e
        assert np.array_equal(host(ex_gpu.gu_scales[e]).view(gs.dtype), gs), e
        assert np.array_equal(host(ex_gpu.dn_codes[e]), o.dn_codes), e
        assert np.array_equal(host(ex_gpu.dn_scales[e]).view(ds.dtype), ds), e
        if cache.fmt == "q4":
            continue
        assert np.array_equal(host(ex_gpu.gu_wscale[e]).view(np.uint32), o.gu_wscale.view(np.uint32)), e
        assert host(ex_gpu.dn_wscale[e]).view(np.uint32) == np.float32(o.dn_wscale).view(np.uint32), e


def check_call(w, mode, layer, x, out, ws, sample=None, ex=None, cache=None, shared=None):
    """Full parity of one GPU layer call on tokens x (bf16 bits) against the oracle.
    ex: the GPU experts (default: the cached layer); cache: an oracle ExpertCache
    to reuse (default: a new one); shared: the oracle's SharedExpert of a block call
    (its intermediate and output are read from the block workspace)."""
    T = x.shape[0]
    wr = synth.router_weight(w, layer)
    bias_np = synth.zipf_bias(w)
    views = moe.workspace_views(ws, mode, T, w.k, w.E, w.H, w.I)
    v = {n: host(t) for n, t in views.items() if n != "ffn"}
    fv = {n: host(t) for n, t in moe.ffn_workspace_views(views["ffn"], mode, T, w.k, w.H, w.I).items()}
    r, flipped = parity.check_route(x, wr, bias_np, w.k, v["topk_ids"], v["topk_w"])
    parity.check_permutation(v["topk_ids"], w.E, v["expert_offsets"], v["sorted_pairs"], v["pair_row"], r.ids)
    if cache is None:
        ins = synth.load_input_scales(w) if mode == "A4" else None
        cache = oracle_cache.ExpertCache(w, layer, ins)
    toks = np.arange(T) if sample is None else np.asarray(sample)
    touched = np.unique(v["topk_ids"][toks])
    cache.prefetch(touched)
    if ex is None:
        ex = _LAYERS[(w.index, layer, mode)][0]
    check_packed_bytes(ex, cache, touched)
    rep = ties.TieReport()
    y_exp, info = parity.check_experts(w, mode, x, cache, w.k, v["expert_offsets"], v["sorted_pairs"],
                                       v["y_pairs"], fv, tokens=None if sample is None else toks, report=rep)
    y_nom, rflip = info.pop("y_nominal"), info.pop("row_flipped")
    sh_exp = sh_nom = None
    if shared is not None:
        bv = moe.block_workspace_views(ws, mode, T, w.k, w.E, w.H, w.I, shared.Is)
        sh_exp, sres, sinfo = parity.check_shared(shared, x, host(bv["shared_h"]), host(bv["shared_y"]))
        sh_nom = sres.gated
        # a token whose shared intermediate took another valid bf16 code: marked
        # with its pairs (only the 8/4-bit modes then skip its nominal comparison)
        rflip = rflip.copy()
        flipped_tokens = np.nonzero(sinfo.pop("shared_flipped_rows"))[0]
        for t in flipped_tokens:
            rflip[v["pair_row"][t * w.k:(t + 1) * w.k]] = True
        info.update(sinfo)
    info.update(parity.check_output(host(out), y_exp, v["pair_row"], r, v["topk_ids"], w.k, tokens=toks,
                                    mode=mode, y_nom=y_nom, row_flipped=rflip, oracle_ids=r.ids,
                                    shared_exp=sh_exp, shared_nom=sh_nom))
    info["router_flips"] = len(flipped)
    info["experts_touched"] = int(len(np.unique(v["topk_ids"])))
    say("ok", info)
    return info, v


def run_and_check(w, mode, layer, batch, dev, T=None, sample=None):
    T = w.T if T is None else T
    ex, router, bias = gpu_layer(w, layer, mode, dev)
    x = synth.tokens(w, batch=batch, T=T)
    say("layer", w.index, mode, "layer", layer, "batch", batch, "T", T)
    out, ws = moe.moe_layer_forward(ex, mode, bench.token_batch(w, batch, dev, T), router, w.k, bias=bias)
    torch.cuda.synchronize()
    moe.moe_layer_status(ws)           # no wait of the call gave up
    info, v = check_call(w, mode, layer, x, out, ws, sample)
    return info, v, host(out)


def test_decode_w4a16(dev):
    """One decode step, 512 experts top-10, H=3072, I=512, T=1, 16-bit activations."""
    w = synth.CONFIGS[1]
    for batch in (0, 1, 2, 63):
        run_and_check(w, "A16", 0, batch, dev)
    run_and_check(w, "A16", 5, 7, dev)        # another of the layer copies bench cycles through


def test_verify_w4a4(dev):
    """Speculative verification: 8 columns, 4-bit activations under calibrated input scales."""
    w = synth.CONFIGS[2]
    info, v, _ = run_and_check(w, "A4", 0, 0, dev)
    assert info["experts_touched"] >= 60          # about 75 expected for uniform routing
    run_and_check(w, "A4", 0, 1, dev)


@pytest.mark.timeout(900)
def test_prefill_w4a4_zipf(dev):
    """1024-token prefill chunk with a Zipf-biased router: every token's routing, the
    permutation, all 10,240 pairs' activation codes, intermediates and down outputs
    (all 512 experts), and every token's output."""
    w = synth.CONFIGS[4]
    info, v, out = run_and_check(w, "A4", 0, 0, dev)
    counts = np.diff(v["expert_offsets"])
    say("expert counts: max", counts.max(), "median", np.median(counts), "empty", int((counts == 0).sum()))
    assert counts.max() >= 64                     # the bias skews the load
    assert np.all(np.isfinite(F.bf16_to_f64(out)))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["A16", "A8"])
def test_prefill_zipf_16_and_8_bit(dev, mode):
    """The 1024-token Zipf-skewed prefill chunk with 16- and 8-bit activations (the
    matrix-core path of those modes): every token's routing, permutation, all
    10,240 pairs' intermediates and down outputs, and every token's output."""
    w = synth.CONFIGS[4]
    info, v, out = run_and_check(w, mode, 0, 0, dev)
    assert info["experts_touched"] == w.E
    assert np.all(np.isfinite(F.bf16_to_f64(out)))
    _LAYERS.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wi,mode", [(1, "A16"), (3, "A8"), (2, "A4")])
def test_decode_fused_equals_stages(dev, wi, mode):
    """Up to 8 tokens moe_layer_forward runs fused (two launches, counters in the
    workspace).  Its output and the routing it leaves in the workspace equal the
    per-stage entry points' bit for bit, over calls of changing token counts on
    one zero-initialised workspace (each call must leave its counters at zero)."""
    w = synth.CONFIGS[wi]
    ex, router, bias = gpu_layer(w, 0, mode, dev)
    ws = torch.zeros(moe.layer_workspace_bytes(mode, 8, w.k, w.E, w.H, w.I), dtype=torch.uint8, device=dev)
    for T, batch in ((w.T, 0), (1, 5), (8, 6), (2, 7), (w.T, 8), (w.T, 8)):
        xg = bench.token_batch(w, batch, dev, T)
        say("fused decode", wi, mode, "T", T, "batch", batch)
        ids, tw = moe.moe_route_topk(xg, router, w.k, bias)
        off, sp, pr = moe.moe_permute(ids, w.E)
        y, _ = moe.nvfp4_expert_ffn(ex, mode, xg, w.k, off, sp)
        ref = moe.moe_combine(y, pr, tw, residual=xg)
        out, _ = moe.moe_layer_forward(ex, mode, xg, router, w.k, bias=bias, residual=xg, ws=ws)
        torch.cuda.synchronize()
        v = moe.workspace_views(ws, mode, T, w.k, w.E, w.H, w.I)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(v["topk_ids"], ids) and torch.equal(v["topk_w"], tw)
        assert torch.equal(v["expert_offsets"], off)
        assert torch.equal(v["sorted_pairs"], sp) and torch.equal(v["pair_row"], pr)
        # the two halves run separately give the same result
        out2 = torch.empty_like(out)
        for stage in (0, 1):
            moe.moe_layer_forward_stage(ex, mode, stage, xg, router, w.k, bias, xg, ws, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert moe.layer_wait_timeouts(ws) == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["A16", "A8"])
def test_stack_layers(dev, mode):
    """48-layer decode stack, T=2, routing recomputed per layer.  Every layer gets the
    full parity check on the oracle chain's own input: the oracle runs
    x_{l+1} = bf16(x_l + out_l) from x_0, and GPU layer l is called on the oracle's
    x_l (its inputs never come from the GPU).  On the same input the fused residual
    call equals bf16(x + out) of the plain call.  Beside it the GPU runs its own
    chain from x_0; its drift from the oracle chain after 48 layers is reported."""
    w = synth.CONFIGS[3]
    xo = synth.tokens(w, batch=0)
    xg = bench.token_batch(w, 0, dev)
    worst, flips, two = 0.0, 0, 0
    for l in range(w.layers):
        ex, router, bias = gpu_layer(w, l, mode, dev)
        x_or = torch.from_numpy(xo.view(np.int16)).to(dev).view(torch.bfloat16)
        out, ws = moe.moe_layer_forward(ex, mode, x_or, router, w.k)
        nxt, _ = moe.moe_layer_forward(ex, mode, x_or, router, w.k, residual=x_or)
        xg, _ = moe.moe_layer_forward(ex, mode, xg, router, w.k, residual=xg)   # the GPU's own chain
        torch.cuda.synchronize()
        out_h, nxt_h = host(out), host(nxt)
        s_ = (torch.from_numpy(xo.astype(np.uint32) << 16).view(torch.float32)
              + torch.from_numpy(out_h.astype(np.uint32) << 16).view(torch.float32))
        assert np.array_equal(nxt_h, s_.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        assert moe.layer_wait_timeouts(ws) == 0
        cache = oracle_cache.ExpertCache(w, l)
        info, _ = check_call(w, mode, l, xo, out, ws, cache=cache)
        worst = max(worst, info["out_worst_rel_l2"])
        flips += info["tie_flipped"]
        two += info["tie_two_candidate"]
        res = OL.moe_layer(xo, synth.router_weight(w, l), w.k, cache, mode)
        xo = OL.residual_add(xo, res.out)
    got, want = F.bf16_to_f64(host(xg)), F.bf16_to_f64(xo)
    drift = np.linalg.norm(got - want, axis=1) / np.linalg.norm(want, axis=1)
    say("stack", mode, "48 layers checked; worst per-layer rel L2", worst, "flipped h codes", flips, "of", two,
        "two-candidate; GPU chain drift after 48 layers (reported, not gated):", drift)
    assert np.all(np.isfinite(got))
    _LAYERS.clear()
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ decode edges
# Shapes at the corners of the fused decode paths (single launch: 16- and 8-bit
# activations, up to 64 pairs; two launches otherwise): a router grid that does
# not fill its last workgroup, one pair, exactly 64 pairs with shared experts,
# 1024 experts (16 logits per top-k lane), the widest fused tiles (H=4096,
# I=1024), and 8-bit activations.  Seeds follow the workload index.
EDGES = [
    synth.Workload(20, "edge: E=33", E=33, k=4, H=1056, I=160, T=1, modes=("A16",)),
    synth.Workload(21, "edge: one pair", E=64, k=1, H=1056, I=160, T=1, modes=("A16",)),
    synth.Workload(22, "edge: 64 pairs", E=64, k=8, H=1056, I=160, T=8, modes=("A16",)),
    synth.Workload(23, "edge: E=1024", E=1024, k=6, H=1056, I=160, T=3, modes=("A16",)),
    synth.Workload(24, "edge: H=4096 I=1024", E=64, k=4, H=4096, I=1024, T=2, modes=("A16",)),
    synth.Workload(25, "edge: A8", E=40, k=5, H=1056, I=160, T=5, modes=("A8",)),
    synth.Workload(26, "edge: A8 two launches", E=40, k=9, H=1056, I=160, T=8, modes=("A8",)),
]


@pytest.mark.parametrize("w", EDGES, ids=[w.name for w in EDGES])
def test_decode_edges(dev, w):
    """Full oracle parity of the fused forward on edge shapes, its equality with the
    per-stage entry points bit for bit, over three token batches on one workspace."""
    mode = w.modes[0]
    single = mode in ("A16", "A8") and w.T * w.k <= 64
    assert moe.layer_launches(mode, w.T, w.k, w.H, w.I) == (1 if single else 2)
    ex, router, bias = gpu_layer(w, 0, mode, dev)
    ws = torch.zeros(moe.layer_workspace_bytes(mode, w.T, w.k, w.E, w.H, w.I), dtype=torch.uint8, device=dev)
    for batch in range(3):
        say("edge", w.name, "batch", batch)
        xg = bench.token_batch(w, batch, dev, w.T)
        out, _ = moe.moe_layer_forward(ex, mode, xg, router, w.k, bias=bias, residual=xg, ws=ws)
        ids, tw = moe.moe_route_topk(xg, router, w.k, bias)
        off, sp, pr = moe.moe_permute(ids, w.E)
        y, _ = moe.nvfp4_expert_ffn(ex, mode, xg, w.k, off, sp)
        ref = moe.moe_combine(y, pr, tw, residual=xg)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        if batch == 0:   # the oracle, on the call without residual
            out0, ws0 = moe.moe_layer_forward(ex, mode, xg, router, w.k, bias=bias)
            torch.cuda.synchronize()
            check_call(w, mode, 0, synth.tokens(w, batch=batch, T=w.T), out0, ws0)
    assert moe.layer_wait_timeouts(ws) == 0


# Tied router logits in the single-launch routing tail: an all-zero router
# (every logit 0: ids 0..k-1, weights 1/k) at E=512 (8 logits per top-k lane)
# and E=40 (one per lane, lanes past E empty), and router rows repeated in groups
# of 4, which puts equal logits within a lane and across lanes.
TIED = [
    (synth.Workload(26, "ties: zero router, E=512", E=512, k=10, H=1056, I=160, T=1, modes=("A16",)), 0),
    (synth.Workload(27, "ties: rows in groups of 4, E=512", E=512, k=10, H=1056, I=160, T=4, modes=("A16",)), 4),
    (synth.Workload(28, "ties: zero router, E=40", E=40, k=5, H=1056, I=160, T=3, modes=("A16",)), 0),
]


@pytest.mark.parametrize("w,group", TIED, ids=[w.name for w, _ in TIED])
def test_decode_tied_logits(dev, w, group):
    """Routing of the single-launch layer with exactly tied logits: the oracle's
    ids (ties to the lower expert), and the output equal to the per-stage entry
    points' bit for bit."""
    assert moe.layer_launches("A16", w.T, w.k, w.H, w.I) == 1
    ex, _, _ = gpu_layer(w, 0, "A16", dev)
    wr = synth.router_weight(w, 0)
    wr = np.zeros_like(wr) if group == 0 else np.ascontiguousarray(np.repeat(wr[::group], group, axis=0)[:w.E])
    router = torch.from_numpy(wr.view(np.int16)).to(dev).view(torch.bfloat16)
    ws = torch.zeros(moe.layer_workspace_bytes("A16", w.T, w.k, w.E, w.H, w.I), dtype=torch.uint8, device=dev)
    for batch in range(2):
        say("tied", w.name, "batch", batch)
        xg = bench.token_batch(w, batch, dev, w.T)
        out, _ = moe.moe_layer_forward(ex, "A16", xg, router, w.k, ws=ws)
        ids, tw = moe.moe_route_topk(xg, router, w.k)
        off, sp, pr = moe.moe_permute(ids, w.E)
        y, _ = moe.nvfp4_expert_ffn(ex, "A16", xg, w.k, off, sp)
        ref = moe.moe_combine(y, pr, tw)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        v = moe.workspace_views(ws, "A16", w.T, w.k, w.E, w.H, w.I)
        ids_h, w_h = host(v["topk_ids"]), host(v["topk_w"])
        r, flipped = parity.check_route(synth.tokens(w, batch=batch, T=w.T), wr, None, w.k, ids_h, w_h)
        assert np.array_equal(ids_h, r.ids) and not flipped
        if group == 0:
            assert np.array_equal(ids_h, np.tile(np.arange(w.k), (w.T, 1)))
            assert np.all(w_h == np.float32(1.0) / np.float32(w.k))
    assert moe.layer_wait_timeouts(ws) == 0


@pytest.mark.parametrize("wi,mode", [(1, "A16"), (3, "A8")])
def test_decode_graph_replay(dev, wi, mode):
    """Under stream capture the single-launch layer is recorded as one node that
    takes its epoch from the workspace and advances it itself (an epoch baked
    into the launch would repeat on replay).  Three replays, each with eager
    single-launch calls and a synchronisation before it, all equal the eager
    result bit for bit and pass the full oracle check; the graph holds one
    kernel node per layer call.  16-bit activations at T=1 and 8-bit at T=2
    (x quantized inside the launch)."""
    w = synth.CONFIGS[wi]
    ex, router, bias = gpu_layer(w, 0, mode, dev)
    nws = moe.layer_workspace_bytes(mode, w.T, w.k, w.E, w.H, w.I)
    ws_g = torch.zeros(nws, dtype=torch.uint8, device=dev)
    ws_e = torch.zeros(nws, dtype=torch.uint8, device=dev)
    x_g = bench.token_batch(w, 0, dev).clone()
    out_g = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    moe.moe_layer_forward(ex, mode, x_g, router, w.k, ws=ws_g, out=out_g)   # warm up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer_forward(ex, mode, x_g, router, w.k, ws=ws_g, out=out_g)
    assert moe.layer_launches(mode, w.T, w.k, w.H, w.I) == 1
    for rep, batch in enumerate((1, 2, 3)):
        say("graph replay", mode, rep, "batch", batch)
        x_new = bench.token_batch(w, batch, dev)
        ref, _ = moe.moe_layer_forward(ex, mode, x_new, router, w.k, ws=ws_e)   # eager, one launch
        x_g.copy_(x_new)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), ref.view(torch.int16)), rep
        check_call(w, mode, 0, synth.tokens(w, batch=batch), out_g, ws_g)   # the replay against the oracle
    assert moe.layer_wait_timeouts(ws_g) == 0 and moe.layer_wait_timeouts(ws_e) == 0


def test_decode_graph_chain(dev):
    """Six chained single-launch layers (each output plus its input feeds the
    next; two seeded layer copies alternate) captured as one graph of six nodes
    on one workspace: three replays on fresh inputs, each equal bit for bit to
    the same chain run eagerly on another workspace."""
    w = synth.CONFIGS[3]
    mode = "A16"
    layers = [gpu_layer_pair(w, l, mode, dev) for l in range(2)]
    nws = moe.layer_workspace_bytes(mode, w.T, w.k, w.E, w.H, w.I)
    ws_g = torch.zeros(nws, dtype=torch.uint8, device=dev)
    ws_e = torch.zeros(nws, dtype=torch.uint8, device=dev)
    x_g = bench.token_batch(w, 0, dev).clone()
    bufs = [torch.empty_like(x_g) for _ in range(2)]

    def chain(x_in, ws, outs):
        cur = x_in
        for l in range(6):
            ex, router, bias = layers[l % 2]
            moe.moe_layer_forward(ex, mode, cur, router, w.k, bias=bias, residual=cur, ws=ws, out=outs[l % 2])
            cur = outs[l % 2]
        return cur

    chain(x_g, ws_g, bufs)   # warm up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(x_g, ws_g, bufs)
    for rep, batch in enumerate((1, 2, 3)):
        say("graph chain replay", rep, "batch", batch)
        x_new = bench.token_batch(w, batch, dev)
        ref = chain(x_new, ws_e, [torch.empty_like(x_new) for _ in range(2)]).clone()
        x_g.copy_(x_new)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[1].view(torch.int16), ref.view(torch.int16)), rep
    assert moe.layer_wait_timeouts(ws_g) == 0 and moe.layer_wait_timeouts(ws_e) == 0
    _LAYERS.clear()
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_decode_graph_layers_oracle(dev):
    """Six single-launch layer calls of the 48-layer stack workload (layers 0-5, T=2)
    captured as one graph, each with its own input, workspace and output.  Before
    each of two replays the inputs are set to the oracle chain's x_0 .. x_5 (the
    oracle's inputs, never the GPU's); every replayed call then gets the full
    parity check against the oracle."""
    w = synth.CONFIGS[3]
    mode, n = "A16", 6
    layers = [gpu_layer_pair(w, l, mode, dev) for l in range(n)]
    nws = moe.layer_workspace_bytes(mode, w.T, w.k, w.E, w.H, w.I)
    wss = [torch.zeros(nws, dtype=torch.uint8, device=dev) for _ in range(n)]
    xins = [torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev) for _ in range(n)]
    outs = [torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev) for _ in range(n)]
    caches = [oracle_cache.ExpertCache(w, l) for l in range(n)]

    def calls():
        for l in range(n):
            ex, router, bias = layers[l]
            moe.moe_layer_forward(ex, mode, xins[l], router, w.k, bias=bias, ws=wss[l], out=outs[l])

    for xi in xins:
        xi.copy_(bench.token_batch(w, 0, dev))
    calls()   # warm up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep_, batch in enumerate((1, 2)):
        xo = synth.tokens(w, batch=batch)
        chain = []
        for l in range(n):
            chain.append(xo)
            res = OL.moe_layer(xo, synth.router_weight(w, l), w.k, caches[l], mode)
            xo = OL.residual_add(xo, res.out)
        for l in range(n):
            xins[l].copy_(torch.from_numpy(chain[l].view(np.int16)).to(dev).view(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(n):
            say("graph layers replay", rep_, "layer", l)
            check_call(w, mode, l, chain[l], outs[l], wss[l], ex=layers[l][0], cache=caches[l])
            assert moe.layer_wait_timeouts(wss[l]) == 0
    _LAYERS.clear()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wi,mode,T", [(1, "A16", None), (2, "A4", None), (4, "A4", None), (4, "A16", 96)],
                         ids=["decode-A16", "verify-A4", "prefill-A4", "wide-A16-T96"])
def test_tiled_layout(dev, wi, mode, T):
    """Experts repacked into the tiled scale layout (moe_nvfp4_repack): the
    repacked bytes are the oracle's in the tiled order, and the layer (the fused
    decode launch, the two-launch narrow path, the wide matrix-core path) gives
    the oracle's result and the canonical experts' output bit for bit."""
    w = synth.CONFIGS[wi]
    T = w.T if T is None else T
    ex, router, bias = gpu_layer(w, 0, mode, dev)
    tiled = moe.moe_nvfp4_repack(ex)
    torch.cuda.synchronize()
    assert tiled.layout == moe.LAYOUT_TILED and tiled.gu_codes.data_ptr() == ex.gu_codes.data_ptr()
    xb = bench.token_batch(w, 3, dev, T)
    say("tiled", w.index, mode, "T", T)
    out_c, _ = moe.moe_layer_forward(ex, mode, xb, router, w.k, bias=bias)
    out_t, ws = moe.moe_layer_forward(tiled, mode, xb, router, w.k, bias=bias)
    torch.cuda.synchronize()
    moe.moe_layer_status(ws)
    assert torch.equal(out_c.view(torch.int16), out_t.view(torch.int16))
    sample = None if T <= 8 else np.arange(0, T, max(1, T // 48))
    check_call(w, mode, 0, synth.tokens(w, batch=3, T=T), out_t, ws, sample=sample, ex=tiled)
    del tiled
