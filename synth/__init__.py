"""Seeded synthetic inputs for the NVFP4 routed-expert layer.

This module only draws numbers.  It holds none of the layer's arithmetic: no
quantizer, no router, no expert product.  Both sides of every parity check
(the CPU oracle and the HIP library) take their inputs from here:

* ``libsynth_cpu.so`` (built from ``synth_cpu.c``) fills host arrays;
* ``libsynth_gpu.so`` (built from ``synth_gpu.hip``) fills device memory with
  the same bits, for workloads too large to generate on the host (a 48-layer
  stack is 1.2e11 normals).

Both are compiled from ``synth_core.h`` (Philox4x32-10 + Box-Muller in plain
IEEE double arithmetic); the GPU tests check that they agree bit for bit.

Workloads (``CONFIGS``) restate the five layer shapes this library is measured
on.  Their value recipe: token activations bf16 ~N(0, 1); router weights bf16
~N(0, 0.02); expert weights fp32 ~N(0, 0.02) before NVFP4 packing; a 64-token
calibration batch bf16 ~N(0, 1); seeds 1000 + workload index.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

TAG_X = 1
TAG_ROUTER = 2
TAG_EXPERT = 3
TAG_CALIB = 4
TAG_ZIPF = 5
TAG_SHARED = 6

MAT_GATE = 0
MAT_UP = 1
MAT_DOWN = 2
MAT_SHARED_GATE_VEC = 3

SIGMA_X = 1.0
SIGMA_W = 0.02
CALIB_TOKENS = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    """One layer-call shape.  ``mode`` is the expert activation precision."""
    index: int
    name: str
    E: int
    k: int
    H: int
    I: int
    T: int
    modes: tuple
    layers: int = 1
    zipf_s: float | None = None
    zipf_beta: float = 0.25
    Is: int = 0          # shared expert intermediate size (0: no shared expert)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def expert_bytes(self) -> int:
        """Packed bytes of one expert: E2M1 codes + E4M3 scales of gate, up, down."""
        gu = 2 * self.I * self.H
        dn = self.H * self.I
        return (gu + dn) // 2 + (gu + dn) // 16


CONFIGS = (
    Workload(0, "tiny W4A16", E=8, k=2, H=256, I=128, T=1, modes=("A16",)),
    Workload(1, "decode W4A16", E=512, k=10, H=3072, I=512, T=1, modes=("A16",)),
    Workload(2, "verify W4A4", E=512, k=10, H=3072, I=512, T=8, modes=("A4",)),
    Workload(3, "48-layer decode stack W4A16/W4A8", E=512, k=10, H=3072, I=512, T=2,
             modes=("A16", "A8"), layers=48),
    Workload(4, "prefill chunk W4A4 Zipf-skewed", E=512, k=10, H=3072, I=512, T=1024,
             modes=("A4",), zipf_s=1.1),
)


def with_shared_expert(w: Workload, Is: int = 512) -> Workload:
    """The same workload with a BF16 shared expert of intermediate size Is beside the
    routed experts (its weights have their own stream tag, so every other input is
    unchanged)."""
    return dataclasses.replace(w, Is=Is, name=f"{w.name} + shared expert Is={Is}")


# --------------------------------------------------------------------------- CPU generator
_cpu = None


def _cpu_lib():
    global _cpu
    if _cpu is None:
        # SYNTH_CPU_LIB: another build of synth_cpu.c (the host-sanitizer build)
        path = os.environ.get("SYNTH_CPU_LIB") or os.path.join(_HERE, "libsynth_cpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        fill_args = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64] + [ctypes.c_uint32] * 6 + [
            ctypes.c_double]
        lib.synth_normal_f32.argtypes = fill_args
        lib.synth_normal_f32.restype = None
        lib.synth_normal_bf16.argtypes = fill_args
        lib.synth_normal_bf16.restype = None
        lib.synth_u32.argtypes = [ctypes.c_void_p, ctypes.c_uint64] + [ctypes.c_uint32] * 5
        lib.synth_u32.restype = None
        lib.synth_philox.argtypes = [ctypes.c_uint32] * 6 + [ctypes.c_void_p]
        lib.synth_philox.restype = None
        _cpu = lib
    return _cpu


def philox4x32_10(counter, key):
    """One Philox4x32-10 block: four uint32 words for a 4-word counter and 2-word key."""
    out = np.zeros(4, np.uint32)
    _cpu_lib().synth_philox(*[int(v) & 0xFFFFFFFF for v in tuple(counter) + tuple(key)],
                            out.ctypes.data)
    return out


def normal_f32(n, seed, tag, layer=0, expert=0, matrix=0, sigma=1.0, i0=0, n_expert=1):
    """fp32 values i0..i0+n-1 of streams (seed, tag, layer, expert+e, matrix), e < n_expert."""
    out = np.empty((n_expert, n), np.float32)
    _cpu_lib().synth_normal_f32(out.ctypes.data, i0, n, seed, tag, layer, expert, n_expert,
                                matrix, sigma)
    return out if n_expert > 1 else out[0]


def normal_bf16(n, seed, tag, layer=0, expert=0, matrix=0, sigma=1.0, i0=0, n_expert=1):
    """As normal_f32, rounded to bf16 (nearest-even); returned as uint16 bit patterns."""
    out = np.empty((n_expert, n), np.uint16)
    _cpu_lib().synth_normal_bf16(out.ctypes.data, i0, n, seed, tag, layer, expert, n_expert,
                                 matrix, sigma)
    return out if n_expert > 1 else out[0]


def raw_u32(n, seed, tag, layer=0, expert=0, matrix=0):
    """The first n raw 32-bit Philox words of stream (seed, tag, layer, expert, matrix)."""
    n4 = (n + 3) // 4
    out = np.empty(4 * n4, np.uint32)
    _cpu_lib().synth_u32(out.ctypes.data, n4, seed, tag, layer, expert, matrix)
    return out[:n]


def bf16_bits_to_f32(u16):
    """Widen bf16 bit patterns to the fp32 values they encode (exact)."""
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- workload inputs
def tokens(w: Workload, batch: int = 0, T: int | None = None):
    """Token activations [T, H] bf16 bits; ``batch`` selects one of many seeded batches."""
    T = w.T if T is None else T
    return normal_bf16(T * w.H, w.seed, TAG_X, layer=batch, sigma=SIGMA_X).reshape(T, w.H)


def calibration_tokens(w: Workload):
    """The 64-token calibration batch [64, H] bf16 bits."""
    return normal_bf16(CALIB_TOKENS * w.H, w.seed, TAG_CALIB, sigma=SIGMA_X).reshape(
        CALIB_TOKENS, w.H)


def router_weight(w: Workload, layer: int = 0):
    """Router weight [E, H] bf16 bits."""
    return normal_bf16(w.E * w.H, w.seed, TAG_ROUTER, layer=layer, sigma=SIGMA_W).reshape(w.E, w.H)


def expert_matrix(w: Workload, layer: int, expert: int, matrix: int, rows=None):
    """fp32 weights of one expert matrix before packing: gate/up [I, H], down [H, I].

    ``rows`` (a range) restricts the result to those rows.
    """
    R, K = (w.I, w.H) if matrix in (MAT_GATE, MAT_UP) else (w.H, w.I)
    if rows is None:
        rows = range(R)
    i0 = rows.start * K
    n = (rows.stop - rows.start) * K
    return normal_f32(n, w.seed, TAG_EXPERT, layer=layer, expert=expert, matrix=matrix,
                      sigma=SIGMA_W, i0=i0).reshape(-1, K)


def shared_expert_weights(w: Workload, layer: int = 0):
    """The shared expert's bf16 weights (bits): gate/up [2Is, H] (gate rows first),
    down [H, Is] and its gate vector [H], all ~N(0, 0.02)."""
    H, Is = w.H, w.Is
    g = normal_bf16(Is * H, w.seed, TAG_SHARED, layer=layer, matrix=MAT_GATE, sigma=SIGMA_W)
    u = normal_bf16(Is * H, w.seed, TAG_SHARED, layer=layer, matrix=MAT_UP, sigma=SIGMA_W)
    d = normal_bf16(H * Is, w.seed, TAG_SHARED, layer=layer, matrix=MAT_DOWN, sigma=SIGMA_W)
    v = normal_bf16(H, w.seed, TAG_SHARED, layer=layer, matrix=MAT_SHARED_GATE_VEC, sigma=SIGMA_W)
    return np.concatenate([g, u]).reshape(2 * Is, H), d.reshape(H, Is), v


def zipf_bias(w: Workload):
    """Router bias [E] fp32: beta * ln p(rank(e)), p(r) proportional to r^-s.

    ranks come from a seeded permutation of the experts (sort by a Philox word,
    ties by index); the log-normaliser is included, so exp(bias / beta) sums to 1.
    """
    if w.zipf_s is None:
        return None
    keys = raw_u32(w.E, w.seed, TAG_ZIPF)
    order = np.argsort(keys, kind="stable")          # order[r] = expert holding rank r + 1
    r = np.arange(1, w.E + 1, dtype=np.float64)
    logp = -w.zipf_s * np.log(r)
    logp -= math.log(np.exp(logp).sum())
    bias = np.empty(w.E, np.float64)
    bias[order] = w.zipf_beta * logp
    return bias.astype(np.float32)


# --------------------------------------------------------------------------- GPU generator
_gpu = None


def _gpu_lib():
    global _gpu
    if _gpu is None:
        path = os.path.join(_HERE, "libsynth_gpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        args = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64] + [ctypes.c_uint32] * 6 + [
            ctypes.c_double, ctypes.c_void_p]
        lib.synth_gpu_normal_f32.argtypes = args
        lib.synth_gpu_normal_f32.restype = ctypes.c_int
        lib.synth_gpu_normal_bf16.argtypes = args
        lib.synth_gpu_normal_bf16.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def gpu_normal_(out, seed, tag, layer=0, expert=0, matrix=0, sigma=1.0, i0=0, n_expert=1,
                stream=None):
    """Fill a contiguous CUDA tensor (float32 or bfloat16, n_expert * n elements) in place."""
    import torch
    assert out.is_cuda and out.is_contiguous()
    n = out.numel() // n_expert
    assert n * n_expert == out.numel()
    if out.dtype == torch.float32:
        fn = _gpu_lib().synth_gpu_normal_f32
    elif out.dtype == torch.bfloat16:
        fn = _gpu_lib().synth_gpu_normal_bf16
    else:
        raise TypeError(out.dtype)
    rc = fn(ctypes.c_void_p(out.data_ptr()), i0, n, seed, tag, layer, expert, n_expert, matrix,
            sigma, _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"synth_gpu fill failed ({rc})")
    return out


# --------------------------------------------------------------------------- stored input scales
def load_input_scales(w: Workload):
    """Calibrated 4-bit-mode activation input scales of a workload's experts.

    Read from tests/golden/inscale_w<index>.txt (written once by
    tests/golden/make_inscales.py).  Returns (gu_inscale [E, 2] fp32,
    dn_inscale [E] fp32).
    """
    path = os.path.join(os.path.dirname(_HERE), "tests", "golden", f"inscale_w{w.index}.txt")
    gu = np.empty((w.E, 2), np.float32)
    dn = np.empty(w.E, np.float32)
    seen = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        e, a, b, c = line.split()
        e = int(e)
        gu[e] = [float.fromhex(a), float.fromhex(b)]
        dn[e] = float.fromhex(c)
        seen += 1
    if seen != w.E:
        raise ValueError(f"{path}: {seen} experts, expected {w.E}")
    return gu, dn
