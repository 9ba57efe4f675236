"""Helpers shared by the GPU parity tests (imports torch/libft lazily)."""
import numpy as np

from oracle import moe

REL_L2 = 1e-3          # layer-output bounds of the contract
MAX_ABS_FRAC = 1e-2
TIE_GAP = 1e-6         # near-tie rule for top-k indices
# Routing weights: the GPU's logits are fp32 dot products over H <= 6144 terms whose rounding
# error reaches a few 1e-6 (3e-6 measured at H = 6144); softmax turns a logit error eps into
# at most 2 eps w_j in w_j, so w is compared with rtol 1e-5 (eps <= 5e-6) plus atol 1e-6.
W_RTOL, W_ATOL = 1e-5, 1e-6


def to_dev(x_bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to("cuda")


def check_routing(idx_gpu, w_gpu, ref):
    """Indices bit-exact except for tokens whose k-th/(k+1)-th oracle logits are within
    TIE_GAP (then the GPU set must still be the top-k up to that tie); weights within
    W_RTOL, W_ATOL."""
    ties = []
    for t in range(idx_gpu.shape[0]):
        if np.array_equal(idx_gpu[t], ref["idx"][t]):
            np.testing.assert_allclose(w_gpu[t], ref["w"][t], atol=W_ATOL, rtol=W_RTOL)
            continue
        assert ref["gap"][t] < TIE_GAP, f"token {t}: {idx_gpu[t]} vs {ref['idx'][t]}"
        lg = ref["logits"][t]
        kth = np.sort(lg)[::-1][len(idx_gpu[t]) - 1]
        assert np.all(lg[idx_gpu[t]] >= kth - TIE_GAP)
        ties.append(t)
    return ties


def check_output(y, ref, what=""):
    err = moe.rel_l2(y, ref)
    mx = float(np.max(np.abs(y - ref)))
    bound = MAX_ABS_FRAC * float(np.max(np.abs(ref)))
    assert err <= REL_L2, f"{what}: rel-L2 {err:.3e}"
    assert mx <= bound, f"{what}: max abs {mx:.3e} > {bound:.3e}"
    return err


# Quantiser decisions taken on values the GPU computed in fp32 (h) may differ from the
# oracle's fp64 ones only this close to a decision boundary (relative).
NEAR = 1e-5
_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])   # E2M1 rounding midpoints


def unpack_nibbles(codes):
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty((c.shape[0], 2 * c.shape[1]), dtype=np.int64)
    out[:, 0::2] = c & 15
    out[:, 1::2] = c >> 4
    return out


def check_mx_quant(codes, scales, ref, what, exact=False):
    """GPU MXFP4 rows (codes packed [R][K/2] low nibble first, E8M0 scales [R][K/32]) against
    the oracle's quantisation of ref (float64 [R][K]).

    exact=True: bit-exact (the GPU quantised the same values the oracle did).  Otherwise a
    decision may differ only within NEAR of its boundary: a block scale when max|v| is that
    close to a power of two (the block's codes are then not compared), a code when v/scale is
    that close to a rounding midpoint (one step apart, same sign), or the sign of a zero code
    when v/scale is that close to 0.  Returns the number of differing decisions."""
    from oracle import mxq
    rc, rs = mxq.quantize(ref)
    gc = unpack_nibbles(codes)
    gs = np.asarray(scales).astype(np.int64)
    if exact:
        assert np.array_equal(gs, rs), f"{what}: scales differ"
        assert np.array_equal(gc, rc), f"{what}: codes differ"
        return 0
    R, K = ref.shape
    b = np.asarray(ref).reshape(R, K // 32, 32)
    bad_s = gs != rs
    if bad_s.any():
        l2 = np.log2(np.abs(b).max(axis=2)[bad_s])
        assert np.all(np.abs(l2 - np.round(l2)) < NEAR), f"{what}: a scale differs away from a power of two"
    r = np.abs(b) / np.ldexp(1.0, rs - 127)[..., None]
    g3, o3 = gc.reshape(R, K // 32, 32), rc.reshape(R, K // 32, 32)
    diff = (g3 != o3) & ~bad_s[..., None]
    if diff.any():
        rd, g, o = r[diff], g3[diff], o3[diff]
        near_mid = np.min(np.abs(rd[:, None] - _MIDS), axis=1) <= NEAR * np.maximum(rd, 0.25)
        one_step = np.abs((g & 7) - (o & 7)) == 1
        same_sign = (g & 8) == (o & 8)
        zero_sign = ((g & 7) == 0) & ((o & 7) == 0) & (rd <= NEAR)
        ok = (near_mid & one_step & same_sign) | zero_sign
        assert np.all(ok), f"{what}: {int((~ok).sum())} codes differ away from a boundary"
    return int(diff.sum() + bad_s.sum())
