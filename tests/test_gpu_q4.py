"""q4_g64_fp16 experts on the GPU against the oracle: the packer bit for bit,
the narrow product core against exact integer sums, the expert FFN on ragged
shapes, and whole layers of 512 such experts at the decode shapes in each
launch form (two-launch decode at T=1 and T=8, per-stage kernels at T=24 and
on the tiny layer)."""
import numpy as np
import pytest
import torch

import bench
import synth
import nvfp4_block_scaled_softmax_amd as moe
from oracle import formats as F
from oracle import layer as OL
from oracle import quant as Q
from tests import oracle_cache, parity
from tests.test_gpu_workloads import _LAYERS, check_call, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def test_q4_packer_matches_oracle(dev):
    rng = np.random.default_rng(71)
    mats = [rng.standard_normal((64, 3072)).astype(np.float32) * 0.02,
            (rng.standard_normal((33, 512)) * 10.0 ** rng.uniform(-8, 3, (33, 1))).astype(np.float32),
            np.zeros((2, 128), np.float32),
            synth.expert_matrix(synth.CONFIGS[1], 0, 3, synth.MAT_GATE)]
    m = rng.standard_normal((16, 256)).astype(np.float32)
    m[:, ::17] *= 50.0                                    # outliers
    m[3, :64] = np.float32(1e-30)                         # subnormal-small group
    m[4, 64:128] = 0.0                                    # one zero group
    mats.append(m)
    for i, w in enumerate(mats):
        say("q4 packer", i, w.shape)
        c, s = moe.q4g64_quantize(to_dev(w, dev))
        torch.cuda.synchronize()
        oc, os_ = Q.q4g64_quantize(w)
        assert np.array_equal(host(c), oc), i
        assert np.array_equal(host(s).view(np.uint16), os_), i


@pytest.mark.parametrize("N,K,cols", [(256, 3072, 8), (200, 4096, 13), (70, 128, 1), (130, 512, 11)])
def test_q4_core_exact_integer_sums(dev, N, K, cols):
    """Unit fp16 scales and small-integer fp16 x: int4 x integer products and
    their sums are exact in fp32, so the core must return the exact sums."""
    rng = np.random.default_rng(N + K + cols)
    q = rng.integers(-8, 8, size=(N, K))
    codes = F.pack_nibbles((q & 15).astype(np.uint8))
    scales = np.full((N, K // 64), F.f64_to_f16(1.0), np.uint16)
    x = rng.integers(-16, 17, size=(cols, K))
    x16 = to_dev(F.f64_to_f16(x.astype(np.float64)), dev).view(torch.float16)
    got = moe.debug_q4g64_matmul(to_dev(codes, dev), to_dev(scales.view(np.int16), dev), x16)
    torch.cuda.synchronize()
    exact = (x @ q.T).astype(np.float64)
    assert np.array_equal(host(got).astype(np.float64), exact)


def _upload_q4(experts, dev):
    st = lambda n: to_dev(np.stack([getattr(ex, n) for ex in experts]), dev)
    return moe.Experts(st("gu_codes"), st("gu_scales").view(torch.int16), st("dn_codes"),
                       st("dn_scales").view(torch.int16), fmt=moe.FMT_Q4G64)


@pytest.mark.parametrize("E,k,H,I,T", [(4, 2, 256, 128, 5), (6, 3, 1088, 192, 3), (8, 2, 3072, 512, 8),
                                       (5, 2, 512, 256, 13)])
def test_q4_expert_ffn_matches_oracle(dev, E, k, H, I, T):
    w = synth.Workload(40, "q4 small", E=E, k=k, H=H, I=I, T=T, modes=("A16",))
    cache = oracle_cache.ExpertCache(w, 0, fmt="q4")
    cache.prefetch(range(E))
    ex = _upload_q4([cache(e) for e in range(E)], dev)
    x = synth.tokens(w, batch=1)
    wr = synth.router_weight(w)
    r = OL.route(x, wr, k)
    p = OL.permute(r.ids, E)
    xg = to_dev(x.view(np.int16), dev).view(torch.bfloat16)
    say("q4 ffn", E, k, H, I, T)
    y, ws = moe.nvfp4_expert_ffn(ex, "A16", xg, k, to_dev(p.offsets, dev), to_dev(p.sorted_pairs, dev))
    torch.cuda.synchronize()
    views = {n: host(t) for n, t in moe.ffn_workspace_views(ws, "A16", T, k, H, I).items()}
    _, info = parity.check_experts(w, "F16", x, cache, k, p.offsets, p.sorted_pairs, host(y), views)
    say("ok", info["y_worst_rel"], info["ties"])


@pytest.mark.parametrize("wi,T", [(1, 1), (1, 8), (1, 24), (0, 4)])
def test_q4_layer_matches_oracle(dev, wi, T):
    """A whole layer of q4_g64_fp16 experts, packed on the GPU from the seeded fp32
    weights (bytes checked against the oracle's packing), two token batches."""
    w = synth.CONFIGS[wi]
    ex, router, bias = bench.build_layer(w, 0, dev, "A16", fmt="q4")
    _LAYERS.clear()
    cache = oracle_cache.ExpertCache(w, 0, fmt="q4")
    assert moe.layer_launches("A16", T, w.k, w.H, w.I) in (0, 1, 2)
    for batch in (0, 1):
        say("q4 layer", wi, "T", T, "batch", batch)
        xg = bench.token_batch(w, batch, dev, T)
        out, ws = moe.moe_layer_forward(ex, "A16", xg, router, w.k, bias=bias)
        torch.cuda.synchronize()
        moe.moe_layer_status(ws)
        check_call(w, "F16", 0, synth.tokens(w, batch=batch, T=T), out, ws, ex=ex, cache=cache)
    del ex, router
    torch.cuda.empty_cache()
