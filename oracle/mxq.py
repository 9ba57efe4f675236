"""OCP MX quantiser to MXFP4 in float64 — oracle (test infrastructure only).

Used only by the scaled-FP4 prefill variant (S1), where activations and h are quantised to
MXFP4 so that both MFMA operands are FP4.  The pages name MXFP4 but give no quantiser; this
is the OCP Microscaling v1.0 conversion rule:

  per 32-element block along K:  X = 2^(floor(log2(max|v|)) - 2)   (2 = E2M1's max exponent)
  with the exponent clamped to [-127, 127] (E8M0 code = exponent + 127);
  code_i = v_i / X rounded to the nearest E2M1 value, ties to the even mantissa, saturating
  at +-6; the code's sign bit is v_i's sign bit (so -0.0 and negatives that round to zero
  give the -0 code 0x8).  An all-zero block gets scale code 0.
"""
from __future__ import annotations

import numpy as np

from . import fp4

_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def quantize(v: np.ndarray):
    """v float64 [R][K] (K % 32 == 0) -> (codes int64 [R][K] in 0..15, scales int64 [R][K/32])."""
    v = np.asarray(v, dtype=np.float64)
    R, K = v.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    b = v.reshape(R, K // 32, 32)
    amax = np.abs(b).max(axis=2)
    nz = amax > 0
    _, ex = np.frexp(np.where(nz, amax, 1.0))        # amax = f * 2^ex, f in [0.5, 1)
    sexp = np.clip(ex - 1 - 2, -127, 127)
    scale_code = np.where(nz, sexp + 127, 0)
    r = np.abs(b) / np.ldexp(1.0, sexp)[..., None]
    # nearest grid point, the lowest index among equally near ones (one pass per point)
    best = np.zeros(r.shape, dtype=np.int64)
    bestd = np.abs(r - _GRID[0])
    for i in range(1, len(_GRID)):
        di = np.abs(r - _GRID[i])
        closer = di < bestd
        best = np.where(closer, i, best)
        bestd = np.where(closer, di, bestd)
    nxt = np.minimum(best + 1, 7)
    tie = (np.abs(r - _GRID[nxt]) == bestd) & (nxt != best)
    best = np.where(tie & (best % 2 == 1), nxt, best)  # ties go to the even mantissa
    codes = best | np.where(np.signbit(b), 8, 0)
    return codes.reshape(R, K).astype(np.int64), scale_code.astype(np.int64)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    v = fp4.e2m1_value(codes)
    return v * np.repeat(fp4.e8m0_value(scales), 32, axis=1)


def quantize_dequant(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    shp = v.shape
    v2 = v.reshape(-1, shp[-1])
    c, s = quantize(v2)
    return dequantize(c, s).reshape(shp)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """int [R][K] codes -> uint8 [R][K/2], element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
