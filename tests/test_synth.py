"""The seeded input generator: published Philox answers, determinism, random access,
and the distributions the workloads ask for.  (Its GPU build is checked against
this host build bit for bit in test_gpu_synth.py.)"""
import os

import numpy as np
import torch

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    n = 0
    for line in open(os.path.join(GOLD, "philox4x32_10_kat.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        inp, out = line.split(":")
        words = [int(v, 16) for v in inp.split()]
        want = [int(v, 16) for v in out.split()]
        assert list(synth.philox4x32_10(words[:4], words[4:])) == want
        n += 1
    assert n == 3


def test_random_access_and_determinism():
    a = synth.normal_f32(1000, 7, synth.TAG_EXPERT, layer=3, expert=9, matrix=1, sigma=0.02)
    b = synth.normal_f32(1000, 7, synth.TAG_EXPERT, layer=3, expert=9, matrix=1, sigma=0.02)
    assert np.array_equal(a, b)
    part = synth.normal_f32(37, 7, synth.TAG_EXPERT, layer=3, expert=9, matrix=1, sigma=0.02, i0=501)
    assert np.array_equal(part, a[501:538])
    multi = synth.normal_f32(1000, 7, synth.TAG_EXPERT, layer=3, expert=8, matrix=1, sigma=0.02,
                             n_expert=3)
    assert np.array_equal(multi[1], a)
    other = synth.normal_f32(1000, 7, synth.TAG_EXPERT, layer=3, expert=9, matrix=2, sigma=0.02)
    assert not np.array_equal(other, a)


def test_bf16_is_nearest_even_of_f32():
    f = synth.normal_f32(100000, 3, synth.TAG_X)
    b = synth.normal_bf16(100000, 3, synth.TAG_X)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_normal_moments():
    v = synth.normal_f32(1 << 20, 11, synth.TAG_EXPERT, sigma=0.02).astype(np.float64)
    assert abs(v.mean()) < 1e-4 and abs(v.std() - 0.02) < 1e-4
    z = v / 0.02
    assert abs(np.mean(z ** 4) - 3.0) < 0.05          # Gaussian kurtosis
    assert abs(np.mean(np.abs(z) > 1.96) - 0.05) < 0.002


def test_zipf_bias():
    w = synth.CONFIGS[4]
    b = synth.zipf_bias(w).astype(np.float64)
    assert abs(np.exp(b / w.zipf_beta).sum() - 1.0) < 1e-5
    ranks = np.argsort(-b, kind="stable")
    assert len(set(ranks.tolist())) == w.E
    r = np.arange(1, w.E + 1)
    assert np.allclose(np.sort(b)[::-1] - b.max(), -w.zipf_beta * w.zipf_s * np.log(r), atol=1e-5)
    assert synth.zipf_bias(synth.CONFIGS[2]) is None


def test_workload_shapes():
    c = synth.CONFIGS
    assert [w.T for w in c] == [1, 1, 8, 2, 1024]
    assert c[1].expert_bytes == 2654208 and c[0].expert_bytes == 55296
