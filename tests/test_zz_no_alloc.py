"""The allocation-free layer call (moe_layer_forward_noalloc) against the
workspace entry point (moe_layer_forward): same kernels, so the outputs must be
equal bit for bit, over consecutive calls that shrink (the device scratch keeps
the last call's contents).  Covers the single-launch decode layer, the
two-launch decode path (4-bit activations, 80 pairs) and the per-stage kernels
(24 tokens), and the host-side rejection of a call too large for the scratch."""
import numpy as np
import pytest
import torch

import bench
import synth
import nvfp4_block_scaled_softmax_amd as moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("wi,mode,Ts", [(1, "A16", (24, 8, 1)), (2, "A4", (8, 2)), (3, "A8", (8, 2))])
def test_noalloc_equals_workspace_call(dev, wi, mode, Ts):
    w = synth.CONFIGS[wi]
    ex, router, bias = bench.build_layer(w, 0, dev, mode)
    for i, T in enumerate(Ts):
        for residual in (False, True):
            say("noalloc", wi, mode, "T", T, "residual", residual)
            x = bench.token_batch(w, 10 + i, dev, T)
            res = x if residual else None
            ref, ws = moe.moe_layer_forward(ex, mode, x, router, w.k, bias=bias, residual=res)
            out = moe.moe_layer_forward_noalloc(ex, mode, x, router, w.k, bias=bias, residual=res)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (T, residual)
            assert torch.isfinite(out.float()).all()
            assert moe.layer_wait_timeouts(ws) == 0
    del ex, router
    torch.cuda.empty_cache()


def test_noalloc_rejects_oversized_call(dev):
    """A 1024-token call needs more than the scratch holds: MOE_E_WORKSPACE, nothing enqueued."""
    w = synth.CONFIGS[4]
    need = moe.layer_workspace_bytes("A4", w.T, w.k, w.E, w.H, w.I)
    assert need > moe.NOALLOC_SCRATCH_BYTES
    E, H, I = 4, w.H, w.I
    ex = moe.Experts(torch.zeros(E, 2 * I, H // 2, dtype=torch.uint8, device=dev),
                     torch.zeros(E, 2 * I, H // 16, dtype=torch.uint8, device=dev),
                     torch.zeros(E, H, I // 2, dtype=torch.uint8, device=dev),
                     torch.zeros(E, H, I // 16, dtype=torch.uint8, device=dev),
                     torch.ones(E, 2, device=dev), torch.ones(E, device=dev),
                     torch.ones(E, 2, device=dev), torch.ones(E, device=dev))
    x = torch.zeros(3000, H, dtype=torch.bfloat16, device=dev)
    router = torch.zeros(E, H, dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_noalloc(ex, "A4", x, router, 2)
    assert ei.value.code == -5 and "scratch" in str(ei.value)
