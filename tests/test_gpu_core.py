"""The expert kernels' product core on its own (moe_debug_nvfp4_matmul), pinned
by exact integer sums.

Page "Infernix releases", release 2026.10.11, "Highlights": products of FP4
weights and activations are exact and their row sums stay exact.  With every
block scale 1 (E4M3 code 0x38) and unit multipliers, an E2M1 weight times an
E2M1 activation is a multiple of 1/4, and times a small-integer bf16 or E4M3
activation a multiple of 1/2; a K <= 4096 row sum is then below 2^20 units, so
every partial sum is exact in fp32 in any order and both cores (the narrow
tile and the wide matrix-core loop) must return the exact sum bit for bit.
The expected sums are integer arithmetic on the oracle's decoded values.
A second case with random block scales checks the same cores against the
oracle's dequantized product within the fp32 accumulation bound.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_softmax_amd as moe
from oracle import formats as F
from oracle import quant as Q

pytestmark = pytest.mark.gpu

E4M3_ONE = 0x38


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def f32_dev(v, dev):
    return torch.tensor([v], dtype=torch.float32, device=dev)


def _operands(rng, mode, N, K, cols, unit=True):
    """Random NVFP4 weights and x in the mode's stored form, plus their exact
    double values (the oracle's decoders)."""
    wc = rng.integers(0, 16, size=(N, K), dtype=np.uint8)             # every E2M1 code, -0 included
    if unit:
        ws = np.full((N, K // 16), E4M3_ONE, np.uint8)
    else:
        ws = rng.integers(0x20, 0x50, size=(N, K // 16), dtype=np.uint8)   # 2^-3 .. 2^2 ranges
    wv = F.e2m1_decode(wc) * np.repeat(F.e4m3_decode(ws), 16, axis=1)
    if mode == "A16":
        xi = rng.integers(-8, 9, size=(cols, K)).astype(np.float64)
        if not unit:
            xi = F.bf16_to_f64(F.f64_to_bf16(rng.standard_normal((cols, K))))
        x = F.f64_to_bf16(xi)
        return (F.pack_nibbles(wc), ws, wv), (x.view(np.int16), None, xi)
    if mode == "A8":
        xi = rng.integers(-16, 17, size=(cols, K)).astype(np.float64)   # exact in E4M3
        xc = F.e4m3_quantize(xi)
        assert np.array_equal(F.e4m3_decode(xc), xi)
        xs = np.ones((cols, K // 16), np.float32)
        if not unit:
            xs = (2.0 ** rng.integers(-4, 3, size=(cols, K // 16))).astype(np.float32)
        return (F.pack_nibbles(wc), ws, wv), (xc, xs, F.e4m3_decode(xc) * np.repeat(xs, 16, axis=1))
    xc = rng.integers(0, 16, size=(cols, K), dtype=np.uint8)
    xs = np.full((cols, K // 16), E4M3_ONE, np.uint8)
    if not unit:
        xs = rng.integers(0x20, 0x50, size=(cols, K // 16), dtype=np.uint8)
    xv = F.e2m1_decode(xc) * np.repeat(F.e4m3_decode(xs), 16, axis=1)
    return (F.pack_nibbles(wc), ws, wv), (F.pack_nibbles(xc), xs, xv)


def _run(dev, core, mode, w, x, wscale=1.0, inscale=1.0):
    codes, scales, _ = w
    xq, xs, _ = x
    xt = to_dev(xq, dev)
    if mode == "A16":
        xt = xt.view(torch.bfloat16)
    out = moe.debug_nvfp4_matmul(core, mode, to_dev(codes, dev), to_dev(scales, dev), f32_dev(wscale, dev), xt,
                                 None if xs is None else to_dev(xs, dev),
                                 f32_dev(inscale, dev) if mode == "A4" else None)
    torch.cuda.synchronize()
    return out.cpu().numpy()


NARROW = [("A16", 256, 3072, 8), ("A16", 200, 4096, 13), ("A16", 70, 160, 1),
          ("A8", 256, 3072, 8), ("A8", 130, 512, 11),
          ("A4", 256, 3072, 8), ("A4", 200, 4096, 9), ("A4", 64, 96, 3)]
WIDE = [("A4", 256, 3072, 40), ("A4", 128, 512, 1), ("A4", 3072, 512, 64), ("A4", 48, 4096, 33),
        ("A16", 256, 3072, 40), ("A16", 128, 512, 1), ("A16", 48, 4096, 33),
        ("A8", 256, 3072, 40), ("A8", 128, 512, 1), ("A8", 48, 4096, 33)]


@pytest.mark.parametrize("core,case", [(0, c) for c in NARROW] + [(1, c) for c in WIDE],
                         ids=[f"narrow-{c[0]}-N{c[1]}K{c[2]}c{c[3]}" for c in NARROW] +
                             [f"wide-{c[0]}-N{c[1]}K{c[2]}c{c[3]}" for c in WIDE])
def test_core_exact_integer_sums(dev, core, case):
    mode, N, K, cols = case
    say("exact core", core, case)
    rng = np.random.default_rng(N * 7 + K + cols + core)
    w, x = _operands(rng, mode, N, K, cols)
    unit = 4 if mode == "A4" else 2                  # the sums are integers in these units
    wi = np.rint(w[2] * 2).astype(np.int64)
    xi = np.rint(x[2] * (2 if mode == "A4" else 1)).astype(np.int64)
    assert np.array_equal(wi / 2.0, w[2])
    exact = (xi @ wi.T) / unit                       # int64 products and sums: exact
    assert np.abs(exact).max() < 2.0 ** 20
    got = _run(dev, core, mode, w, x)
    assert got.dtype == np.float32
    bad = np.nonzero(got.astype(np.float64) != exact)
    assert bad[0].size == 0, f"{bad[0].size} sums differ, first {got[bad][:4]} vs {exact[bad][:4]}"


@pytest.mark.parametrize("core,case", [(0, ("A16", 192, 3072, 8)), (0, ("A8", 192, 512, 5)),
                                       (0, ("A4", 192, 3072, 8)), (1, ("A4", 192, 3072, 40)),
                                       (1, ("A16", 192, 3072, 40)), (1, ("A8", 192, 512, 40))],
                         ids=["narrow-A16", "narrow-A8", "narrow-A4", "wide-A4", "wide-A16", "wide-A8"])
def test_core_scaled_matches_oracle(dev, core, case):
    """Random block scales and multipliers: the fp32 result within the fp32
    accumulation bound of the oracle's dequantized double product."""
    mode, N, K, cols = case
    say("scaled core", core, case)
    rng = np.random.default_rng(K + cols + 31 * core)
    w, x = _operands(rng, mode, N, K, cols, unit=False)
    wscale, inscale = np.float32(0.0173), np.float32(0.0041)
    want = x[2] @ (w[2] * np.float64(wscale)).T
    if mode == "A4":
        want = want * np.float64(inscale)
    absum = np.abs(x[2]) @ np.abs(w[2] * np.float64(wscale)).T * (np.float64(inscale) if mode == "A4" else 1.0)
    got = _run(dev, core, mode, w, x, wscale, inscale).astype(np.float64)
    err = np.abs(got - want)
    assert np.all(err <= 2.0 ** -17 * absum + 1e-30), float((err / np.maximum(absum, 1e-30)).max())


def test_core_oracle_quantized_x(dev):
    """4-bit x produced by the oracle's quantizer (a real activation row under an
    input scale) through both cores: the cores agree with each other within the
    fp32 bound and with the oracle's dequantized product."""
    rng = np.random.default_rng(5)
    N, K, cols = 256, 3072, 24
    w, _ = _operands(rng, "A4", N, K, cols, unit=False)
    x32 = rng.standard_normal((cols, K)).astype(np.float32)
    g = Q.nvfp4_global_scale(np.abs(x32).max())
    xc, xs = Q.nvfp4_quantize(x32, g)
    xv = Q.nvfp4_dequantize(xc, xs, g)
    x = (xc, xs, xv)
    want = xv @ w[2].T * 1.0
    absum = np.abs(xv) @ np.abs(w[2]).T
    # the cores apply the input scale as a multiplier of the E2M1 x values
    xv_unit = Q.nvfp4_dequantize(xc, xs, np.float32(1.0))
    outs = [_run(dev, core, "A4", w, (xc, xs, xv_unit), 1.0, float(g)).astype(np.float64) for core in (0, 1)]
    for got in outs:
        assert np.all(np.abs(got - want) <= 2.0 ** -17 * absum + 1e-30)
    assert np.all(np.abs(outs[0] - outs[1]) <= 2.0 ** -16 * absum + 1e-30)
