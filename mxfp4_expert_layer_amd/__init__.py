"""MI355X-native sparse MoE expert layer with block-scaled FP4 (MXFP4 / NVFP4) experts.

The compute path lives in the HIP library ``libft.so`` (built from ``csrc/``); the Python
module ``mxfp4_expert_layer_amd.ft`` is a thin ctypes binding over its C ABI.  Importing
this package does not load the library, so the seeded input generators in ``synth`` stay
usable on machines without a GPU.
"""
