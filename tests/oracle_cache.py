"""Oracle-packed experts for the parity tests, built in a process pool.

Packing one full-size expert in the oracle takes ~0.7 s of numpy; the GPU
tests need tens of them.  The pool is started (spawned) by conftest before any
test initialises the GPU; its workers only run numpy and the host generator.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import synth
from oracle import layer as OL

_POOL = None


def start_pool():
    global _POOL
    if _POOL is None:
        n = max(1, min(8, (os.cpu_count() or 2) - 1))
        _POOL = mp.get_context("spawn").Pool(n)


def stop_pool():
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL = None


def _pack(args):
    w, layer, e, fmt = args
    pack = OL.pack_expert_q4 if fmt == "q4" else OL.pack_expert
    return e, pack(*(synth.expert_matrix(w, layer, e, m) for m in range(3)))


class ExpertCache:
    """Lazily packed oracle experts of one (workload, layer); fmt "nvfp4" or "q4"
    (q4_g64_fp16)."""

    def __init__(self, w, layer=0, inscales=None, fmt="nvfp4"):
        self.w, self.layer, self.inscales, self.fmt = w, layer, inscales, fmt
        self.cache = {}

    def prefetch(self, experts):
        todo = sorted(set(int(e) for e in experts) - set(self.cache))
        if not todo:
            return
        args = [(self.w, self.layer, e, self.fmt) for e in todo]
        results = _POOL.map(_pack, args) if _POOL is not None and len(todo) > 1 else map(_pack, args)
        for e, ex in results:
            self._store(e, ex)

    def _store(self, e, ex):
        if self.inscales is not None:
            ex.gu_inscale = np.array(self.inscales[0][e], np.float32)
            ex.dn_inscale = np.float32(self.inscales[1][e])
        self.cache[e] = ex

    def __call__(self, e):
        e = int(e)
        if e not in self.cache:
            self._store(*_pack((self.w, self.layer, e, self.fmt)))
        return self.cache[e]
