"""Reference oracle for the sparse MoE expert layer — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation (numpy, float64) of what the layer
computes.  It exists to check the HIP library, and only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it.  It shares no code with the HIP path
(``mxfp4_expert_layer_amd``): it imports nothing from that package, and that package imports
nothing from here.  Inputs come from the seeded generators, which hold no layer arithmetic.

Modules
  fp4     E2M1 / E8M0 / E4M3 element and scale values; MXFP4 / NVFP4 dequantisation; bf16.
  moe     top-k softmax routing, SwiGLU expert FFN, routing-weighted combine, the exact
          (bf16-activation) layer and the MXFP4-activation variant (S1).
  policy  q* split rule, miss ordering and the LRU slot-pool simulator.
  perm    prefill permutation by expert (counts, offsets, positions).
  mxq     the OCP MX quantiser used by the S1 variant.

Pins: every function is checked in tests/test_oracle_*.py against values fixed by the
format definitions, the pages (the q* table of the smzdm explainer a825qpgl, section 二),
closed forms, invariants and brute force on tiny inputs.  No function is "parity unpinned".
"""
