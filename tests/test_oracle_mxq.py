"""Pins for the oracle's OCP MX quantiser (used by the scaled-FP4 prefill variant), CPU."""
import numpy as np

from oracle import fp4, mxq


def _block(vals, fill=0.0):
    b = np.full((1, 32), fill)
    b[0, :len(vals)] = vals
    return b


def test_scale_from_amax():
    for n in (-5, 0, 3):
        c, s = mxq.quantize(_block([2.0 ** n]))
        assert s[0, 0] == 127 + n - 2                   # X = 2^(n - 2)
        assert fp4.e2m1_value(c[0, 0]) == 4.0
        c, s = mxq.quantize(_block([2.0 ** n * (1 - 2 ** -20)]))
        assert s[0, 0] == 127 + n - 3
        assert fp4.e2m1_value(c[0, 0]) == 6.0           # 7.99.. saturates to 6


def test_tie_points_go_to_even_mantissa():
    X = 2.0 ** -3
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    vals = [4.0 * X] + [t * X for t in ties] + [-t * X for t in ties]
    c, s = mxq.quantize(_block(vals))
    assert s[0, 0] == 127 - 3
    got = fp4.e2m1_value(c[0, :len(vals)])
    assert list(got[1:8]) == expect
    assert list(got[8:15]) == [-e for e in expect]


def test_saturation_and_zero_block():
    c, s = mxq.quantize(_block([7.0, -7.9, 1.0]))
    assert s[0, 0] == 127 and list(fp4.e2m1_value(c[0, :3])) == [6.0, -6.0, 1.0]
    c, s = mxq.quantize(np.zeros((2, 64)))
    assert np.all(c == 0) and np.all(s == 0)
    c, s = mxq.quantize(_block([-0.0, 0.0, -1e-30, 1.0]))
    assert list(c[0, :4]) == [8, 0, 8, 6]               # the sign bit survives rounding to 0


def test_idempotent_and_nearest_by_exhaustive_search():
    rng = np.random.default_rng(9)
    v = rng.standard_normal((16, 128)) * np.exp(rng.uniform(-8, 8, size=(16, 1)))
    c, s = mxq.quantize(v)
    d = mxq.dequantize(c, s)
    c2, s2 = mxq.quantize(d)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    # brute force: every element's code is a nearest code among all 16, ties to even mantissa
    allv = fp4.e2m1_value(np.arange(16))
    X = fp4.e8m0_value(np.repeat(s, 32, axis=1))
    for r in range(v.shape[0]):
        for kk in range(v.shape[1]):
            err = np.abs(allv * X[r, kk] - v[r, kk])
            best = err.min()
            assert err[c[r, kk]] == best
            cands = [cc for cc in range(16) if err[cc] == best]
            if len(set(allv[cands])) > 1:                 # a genuine tie between two values
                assert c[r, kk] % 2 == 0


def test_pack_codes_low_nibble_first():
    c = np.array([[1, 2, 15, 8]])
    assert list(mxq.pack_codes(c)[0]) == [0x21, 0x8F]


def test_requantising_an_mxfp4_block_keeps_its_values():
    """An MXFP4 block (E2M1 codes times 2^(s-127)) is a fixed point of the quantiser's
    values for every scale code 0..254 and every largest code magnitude: scaling its codes
    by 2^(2 - floor(log2 max|code|)) stays on the E2M1 grid.  The codes themselves may change
    (a block whose largest code is 1 is re-expressed with a 4x smaller scale)."""
    rng = np.random.default_rng(11)
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rows = []
    for s in range(0, 255):
        for top in range(8):                      # largest code magnitude index in the block
            c = rng.integers(0, top + 1, 32) | (rng.integers(0, 2, 32) << 3)
            c[rng.integers(0, 32)] = top
            rows.append((c, s))
    codes = np.stack([r[0] for r in rows])
    scales = np.array([[r[1]] for r in rows])
    v = fp4.dequant_mxfp4(mxq.pack_codes(codes), scales)
    assert v.shape == (len(rows), 32)
    assert np.array_equal(mxq.quantize_dequant(v), v)
    # a block whose largest magnitude is 4 or 6 keeps its scale and, bar the sign of zeros,
    # its codes
    keep = np.array([max(grid[c & 7] for c in r[0]) >= 4.0 for r in rows])
    c2, s2 = mxq.quantize(v[keep])
    assert np.array_equal(s2[:, 0], scales[keep, 0])
    nz = (codes[keep] & 7) != 0
    assert np.array_equal(c2[nz], codes[keep][nz])
