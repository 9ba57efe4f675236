"""FP4 element and scale codecs in float64 — oracle (test infrastructure only).

Definitions (OCP Microscaling Formats v1.0 for E2M1, E8M0 and E4M3; NVFP4 as E2M1 values
with an E4M3 scale per 16 elements and one fp32 scale per tensor).  The FreeToken pages only
name the formats: MXFP4 expert weights for DeepSeek-V4-Flash and NVFP4 for Qwen3.6-35B
(smzdm explainer a825qpgl, section 一; the same page's section 五 lists NVFP4/MXFP4 as the
supported quantisation formats).

Layout reading (the pages are silent): two codes per byte, element 2i in bits 0-3 and
element 2i+1 in bits 4-7; scale blocks run along each matrix's contraction axis and scales
are stored [rows][K / block].
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code):
    """E2M1: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0; no inf or NaN.

    exponent 0 is subnormal: m * 2^-1; otherwise 2^(e-1) * (1 + m/2)."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int32)))
    return np.where(s == 1, -mag, mag)


def e8m0_value(code):
    """E8M0 scale: 2^(code - 127); code 255 is NaN; there is no zero."""
    c = np.asarray(code, dtype=np.int64)
    v = np.ldexp(np.ones(c.shape, dtype=np.float64), (c - 127).astype(np.int32))
    return np.where(c == 255, np.nan, v)


def e4m3_value(code):
    """E4M3 (the 'FN' variant, no infinities): sign bit 7, exponent bits 6-3 (bias 7),
    mantissa bits 2-0.  exponent 0 is subnormal: 2^-6 * m/8; S.1111.111 is NaN."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    sub = np.ldexp(m / 8.0, -6)
    nrm = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 [R][K/2] -> int [R][K]; element 2i is the low nibble of byte i."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, half = codes.shape
    out = np.empty((R, 2 * half), dtype=np.int64)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def _element_values(codes: np.ndarray) -> np.ndarray:
    """E2M1 values [R][K] of packed codes [R][K/2]: the closed form above evaluated once per
    code (16 values) and indexed, low nibble = even element."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = e2m1_value(np.arange(16))
    R, half = codes.shape
    out = np.empty((R, 2 * half), dtype=np.float64)
    out[:, 0::2] = table[codes & 0xF]
    out[:, 1::2] = table[codes >> 4]
    return out


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 matrix: value[r][k] = E2M1(code[r][k]) * E8M0(scale[r][k // 32])."""
    v = _element_values(codes)
    R, K = v.shape
    s = e8m0_value(np.asarray(scales, dtype=np.int64))
    return (v.reshape(R, K // 32, 32) * s[:, :, None]).reshape(R, K)


def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray, tensor_scale: float) -> np.ndarray:
    """NVFP4 matrix: value[r][k] = E2M1(code[r][k]) * E4M3(scale[r][k // 16]) * tensor_scale."""
    v = _element_values(codes)
    R, K = v.shape
    s = e4m3_value(np.asarray(scales, dtype=np.int64))
    return (v.reshape(R, K // 16, 16) * s[:, :, None]).reshape(R, K) * np.float64(tensor_scale)


def dequant(fmt: str, codes, scales, tensor_scale=1.0) -> np.ndarray:
    if fmt == "mxfp4":
        return dequant_mxfp4(codes, scales)
    if fmt == "nvfp4":
        return dequant_nvfp4(codes, scales, tensor_scale)
    raise ValueError(f"unknown format {fmt!r}")


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


_BF16_MAX = np.ldexp(2.0 - 2.0 ** -7, 127)


def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    bf16 has 8 significant bits and fp32's exponent range (normal down to 2^-126,
    subnormal quantum 2^-133); results beyond the largest finite bf16 become +-inf."""
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    fin = np.isfinite(v) & (v != 0)
    _, ex = np.frexp(v[fin])                 # |v| = f * 2^ex, f in [0.5, 1)
    q_exp = np.maximum(ex - 8, -133)         # quantum 2^(ex-8), floored at the subnormal step
    r = np.ldexp(np.rint(np.ldexp(v[fin], -q_exp)), q_exp)
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out
