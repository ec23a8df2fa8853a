"""Write the 4-bit-mode activation input scales of the W4A4 workloads.

The checkpoint the pages describe carries calibrated fp32 activation input
scales per expert matrix (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix
(bit-exact)", section "What is bit-exact and what is quantized"; used by the
default 4-bit mode, page "Infernix", section "Activation precision").  The
synthetic checkpoints get theirs from a 64-token seeded calibration batch run
densely through every expert by the oracle (oracle.layer.calibrate_input_scales).

This script calls only ``oracle`` (and ``synth`` for the inputs).  Output:
tests/golden/inscale_w<index>.txt, one line per expert, exact hex floats:
    expert gate_inscale up_inscale down_inscale

Usage: python tests/golden/make_inscales.py [workload index ...]   (default 2 4)
"""
import multiprocessing as mp
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import layer as L  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def _one(args):
    wi, e = args
    w = synth.CONFIGS[wi]
    ex = L.pack_expert(*(synth.expert_matrix(w, 0, e, m) for m in range(3)))
    gu, dn = L.calibrate_input_scales(synth.calibration_tokens(w), [ex])
    return e, gu[0], dn[0]


def path_for(wi):
    return os.path.join(HERE, f"inscale_w{wi}.txt")


def main(indices):
    for wi in indices:
        w = synth.CONFIGS[wi]
        with mp.Pool(min(8, os.cpu_count() or 1)) as pool:
            rows = sorted(pool.map(_one, [(wi, e) for e in range(w.E)]))
        with open(path_for(wi), "w") as f:
            f.write(f"# activation input scales of workload {wi} ({w.name}), seed {w.seed}\n")
            f.write("# written by tests/golden/make_inscales.py from oracle.layer.calibrate_input_scales\n")
            f.write("# expert gate_inscale up_inscale down_inscale (exact fp32 as hex floats)\n")
            for e, gu, dn in rows:
                f.write(f"{e} {float(gu[0]).hex()} {float(gu[1]).hex()} {float(dn).hex()}\n")
        print("wrote", path_for(wi))


if __name__ == "__main__":
    main([int(a) for a in sys.argv[1:]] or [2, 4])
