"""CPU oracle of the NVFP4 routed-expert (mixture-of-experts) layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, table or helper with the HIP
library (``nvfp4_block_scaled_softmax_amd``); its inputs come from ``synth``
(seeded generators that hold none of the layer's arithmetic) or from the
tests' own fixtures.

It is plain and slow on purpose: every dot product, exponential and sum is in
IEEE double; the fp32 steps that the format fixes (the quantizers' scale
arithmetic) are emulated exactly, each fp32 +, -, *, / computed in double and
rounded to fp32 once (exact, since 53 >= 2 * 24 + 2).

What each part follows:

* ``formats`` -- the element encodings: E2M1 (OCP Microscaling Formats v1.0,
  "FP4 (E2M1)" element type) and E4M3 (OCP 8-bit Floating Point
  specification, "E4M3" encoding); bf16 as the upper half of an fp32.
* ``quant`` -- NVFP4 block quantization: E2M1 codes, one E4M3 scale per 16
  values, one fp32 multiplier per matrix (page "Qwen3.8-Flash-Next NVIDIA
  NVFP4 for Infernix (bit-exact)", section "What is bit-exact and what is
  quantized", routed experts); the 8-bit activation mode (page "Infernix",
  section "Activation precision").
* ``layer`` -- the routed-expert layer: router softmax / top-k / renormalise,
  the token-to-expert permutation, the SwiGLU expert FFN in the three
  activation modes, the weighted combine and the residual across layers.

Parity pins (tests/test_oracle_*.py): every function here is pinned to
something other than itself -- the published code tables, brute force over
the enumerated code sets with exact rationals, closed forms, the exact-integer
property of FP4 products, permutation invariants and brute-force sorting, and
special cases that reduce to a textbook dense SwiGLU MLP.  No function is
parity unpinned.  The pages print no worked numeric example, so no pin comes
from a value printed on them.
"""
from . import formats, quant, layer  # noqa: F401
