"""Pins for the oracle's FP4 codecs and bf16 rounding (CPU only).

Each codec is checked over every code against an independent source: the value table that
the OCP Microscaling v1.0 specification lists for E2M1, and PyTorch's own float8_e8m0fnu and
float8_e4m3fn conversions for the two scale formats."""
import math

import numpy as np
import pytest
import torch

from oracle import fp4

# OCP MX v1.0, FP4 E2M1 value table (positive half; the sign bit mirrors it).
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_all_codes_match_spec_table():
    v = fp4.e2m1_value(np.arange(16))
    assert list(v[:8]) == E2M1_SPEC
    assert list(v[8:]) == [-a for a in E2M1_SPEC]
    assert math.copysign(1.0, v[8]) == -1.0          # code 0x8 is -0
    assert np.all(np.isfinite(v))


def test_e8m0_all_codes_match_torch():
    c = np.arange(256)
    ours = fp4.e8m0_value(c)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(ours), ~fin)
    assert np.array_equal(ours[fin], ref[fin])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_e4m3_all_codes_match_torch():
    c = np.arange(256)
    ours = fp4.e4m3_value(c)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0
    # the NVFP4 scale range used by the prefill workload: 49 codes with values in [2^-6, 1]
    pos = ours[:0x80]
    sel = np.nonzero((pos >= 2.0 ** -6) & (pos <= 1.0))[0]
    assert list(sel) == list(range(0x08, 0x39))


def test_nibble_order_and_block_assignment_mx():
    R, K = 2, 64
    codes = np.zeros((R, K // 2), np.uint8)
    codes[0, 0] = 0x21          # element 0 -> code 1 (0.5), element 1 -> code 2 (1.0)
    codes[1, 16] = 0xF7         # element 32 -> code 7 (6.0), element 33 -> code 15 (-6.0)
    scales = np.array([[127, 128], [125, 130]], np.uint8)
    v = fp4.dequant_mxfp4(codes, scales)
    assert v[0, 0] == 0.5 and v[0, 1] == 1.0 and np.count_nonzero(v[0]) == 2
    assert v[1, 32] == 6.0 * 8 and v[1, 33] == -6.0 * 8 and np.count_nonzero(v[1]) == 2


def test_nibble_order_and_block_assignment_nv():
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 7] = 0x50          # element 14 -> 0 , element 15 -> code 5 (3.0)
    codes[0, 8] = 0x03          # element 16 -> code 3 (1.5)
    scales = np.array([[0x38, 0x30, 0x40, 0x38]], np.uint8)   # 1.0, 0.5, 2.0, 1.0
    v = fp4.dequant_nvfp4(codes, scales, 0.25)
    assert v[0, 15] == 3.0 * 1.0 * 0.25
    assert v[0, 16] == 1.5 * 0.5 * 0.25
    assert np.count_nonzero(v) == 2


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 65536, 97, dtype=np.uint16)
    ours = fp4.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(5)
    z = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
    ])
    # exact halfway points between neighbouring bf16 values (ties to even)
    base = rng.integers(0x3000, 0x5000, size=2000).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    z = np.concatenate([z, ties])
    ours = fp4.round_bf16(z.astype(np.float64))
    ref = torch.from_numpy(z).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_round_bf16_specials():
    v = fp4.round_bf16(np.array([0.0, -0.0, np.inf, -np.inf, 3.5e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]))
    assert v[0] == 0 and math.copysign(1, v[1]) == -1
    assert v[2] == np.inf and v[3] == -np.inf and v[4] == np.inf
    assert v[5] == 1.0                   # tie -> even (1.0)
    assert v[6] == 1.0 + 2 ** -6         # tie -> even (1 + 4*2^-8)
