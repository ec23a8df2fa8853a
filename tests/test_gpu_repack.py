"""moe_nvfp4_repack and the tiled scale layout on shapes with full and partial
scale windows in both matrices (H = I = 1152: 36 chunks per row, one full
window of 32 and a partial one of 4).

The repacked bytes must be the oracle's tiled order of the canonical bytes
(seeded random bytes, not packed by the library), the codes unchanged; every
path (narrow tiles at 1 and 8 tokens, the wide matrix-core path at 64) must
give the same output from tiled experts as from canonical ones, bit for bit."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_softmax_amd as moe
from oracle import formats as F

pytestmark = pytest.mark.gpu

E, H, I, K_TOP = 16, 1152, 1152, 4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def _experts(dev, rng):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return moe.Experts(
        gu_codes=t(rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)),
        gu_scales=t(rng.integers(0x20, 0x48, size=(E, 2 * I, H // 16), dtype=np.uint8)),
        dn_codes=t(rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)),
        dn_scales=t(rng.integers(0x20, 0x48, size=(E, H, I // 16), dtype=np.uint8)),
        gu_wscale=t(np.full((E, 2), 0.02, np.float32)), dn_wscale=t(np.full(E, 0.02, np.float32)),
        gu_inscale=t(np.full((E, 2), 4.0 / 2688, np.float32)), dn_inscale=t(np.full(E, 1.0 / 2688, np.float32)))


def test_repack_bytes_match_the_oracle_order(dev):
    rng = np.random.default_rng(81)
    ex = _experts(dev, rng)
    tiled = moe.moe_nvfp4_repack(ex, share_codes=False)
    torch.cuda.synchronize()
    for n in ("gu", "dn"):
        canon = getattr(ex, n + "_scales").cpu().numpy()
        got = getattr(tiled, n + "_scales").cpu().numpy()
        assert np.array_equal(got, F.tiled_scales(canon)), n
        assert not np.array_equal(got, canon)                  # the full windows did move
        assert torch.equal(getattr(tiled, n + "_codes"), getattr(ex, n + "_codes"))


@pytest.mark.parametrize("mode,T", [("A16", 1), ("A4", 8), ("A8", 3), ("A16", 64), ("A8", 64), ("A4", 64)])
def test_tiled_equals_canonical(dev, mode, T):
    rng = np.random.default_rng(82 + T)
    ex = _experts(dev, rng)
    tiled = moe.moe_nvfp4_repack(ex)
    router = torch.from_numpy(F.f64_to_bf16(rng.standard_normal((E, H)) * 0.05).view(np.int16)).to(dev)
    x = torch.from_numpy(F.f64_to_bf16(rng.standard_normal((T, H))).view(np.int16)).to(dev)
    router, x = router.view(torch.bfloat16), x.view(torch.bfloat16)
    say("tiled vs canonical", mode, "T", T)
    out_c, ws_c = moe.moe_layer_forward(ex, mode, x, router, K_TOP)
    out_t, ws_t = moe.moe_layer_forward(tiled, mode, x, router, K_TOP)
    torch.cuda.synchronize()
    moe.moe_layer_status(ws_c)
    moe.moe_layer_status(ws_t)
    assert torch.isfinite(out_c.float()).all()
    assert torch.equal(out_c.view(torch.int16), out_t.view(torch.int16))
