"""The shared expert and its gate on the GPU, against the oracle: the stand-alone
entry point (moe_shared_expert_forward) over ragged shapes, and whole blocks
(moe_block_forward: routed experts + shared expert, one output) in each launch
form of the layer -- the single-launch decode layer (T=1, 16-bit), the
two-launch decode form (T=8, 4-bit), and the per-stage kernels (the tiny layer
and a 24-token call)."""
import numpy as np
import pytest
import torch

import bench
import synth
import nvfp4_block_scaled_softmax_amd as moe
from oracle import layer as OL
from tests import parity, ties
from tests.test_gpu_workloads import _LAYERS, check_call, gpu_layer, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def shared_on_gpu(w, dev, layer=0):
    gu, dn, gate = synth.shared_expert_weights(w, layer)
    b = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return moe.SharedExpert(b(gu), b(dn), b(gate)), OL.SharedExpert(gu, dn, gate)


SHAPES = [(256, 64, 1), (256, 64, 19), (1056, 160, 3), (3072, 512, 1), (3072, 512, 8), (4096, 1024, 13),
          (3072, 512, 100)]


@pytest.mark.parametrize("H,Is,T", SHAPES, ids=[f"H{h}Is{i}T{t}" for h, i, t in SHAPES])
def test_shared_expert_matches_oracle(dev, H, Is, T):
    w = synth.Workload(30, "shared expert", E=8, k=2, H=H, I=128, T=T, modes=("A16",), Is=Is)
    sg, so = shared_on_gpu(w, dev)
    x = synth.tokens(w, batch=T)
    say("shared expert", H, Is, T)
    y, ws = moe.moe_shared_expert_forward(sg, torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16))
    torch.cuda.synchronize()
    h = host(ws[:T * Is * 2].view(torch.bfloat16).view(T, Is))
    rep = ties.TieReport()
    _, res, info = parity.check_shared(so, x, h, host(y), rep)
    assert np.all(res.sig > 0) and np.all(res.sig < 1)
    say("ok", info["shared_y_worst_rel"], info["shared_ties"])


BLOCKS = [(0, "A16", 4), (1, "A16", 1), (2, "A4", 8), (1, "A16", 24), (3, "A8", 2)]


@pytest.mark.parametrize("wi,mode,T", BLOCKS, ids=[f"w{wi}-{m}-T{t}" for wi, m, t in BLOCKS])
def test_block_forward_matches_oracle(dev, wi, mode, T):
    """Routed layer + shared expert through moe_block_forward; with a residual the
    output equals bf16(x + out) of the plain call, bit for bit."""
    w = synth.with_shared_expert(synth.CONFIGS[wi], 64 if wi == 0 else 512)
    ex, router, bias = gpu_layer(synth.CONFIGS[wi], 0, mode, dev)
    sg, so = shared_on_gpu(w, dev)
    ws = torch.zeros(moe.block_workspace_bytes(mode, T, w.k, w.E, w.H, w.I, w.Is), dtype=torch.uint8, device=dev)
    for batch in (0, 1):
        say("block", wi, mode, "T", T, "batch", batch)
        xg = bench.token_batch(w, batch, dev, T)
        out, _ = moe.moe_block_forward(ex, sg, mode, xg, router, w.k, bias=bias, ws=ws)
        torch.cuda.synchronize()
        moe.moe_layer_status(ws)
        check_call(synth.CONFIGS[wi], mode, 0, synth.tokens(w, batch=batch, T=T), out, ws, shared=so)
        nxt, _ = moe.moe_block_forward(ex, sg, mode, xg, router, w.k, bias=bias, residual=xg, ws=ws)
        torch.cuda.synchronize()
        ref = (xg.float() + out.float()).to(torch.bfloat16)
        assert torch.equal(nxt.view(torch.int16), ref.view(torch.int16))
    # the stand-alone calls give the same bits as the block
    xg = bench.token_batch(w, 1, dev, T)
    ids, tw = moe.moe_route_topk(xg, router, w.k, bias)
    off, sp, pr = moe.moe_permute(ids, w.E)
    y, _ = moe.nvfp4_expert_ffn(ex, mode, xg, w.k, off, sp)
    ys, _ = moe.moe_shared_expert_forward(sg, xg)
    ref = moe.moe_combine_shared(y, pr, tw, ys)
    out, _ = moe.moe_block_forward(ex, sg, mode, xg, router, w.k, bias=bias, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    _LAYERS.clear()
    torch.cuda.empty_cache()
