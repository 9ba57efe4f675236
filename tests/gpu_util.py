"""Helpers shared by the GPU parity tests (imports torch/libft lazily)."""
import numpy as np

from oracle import moe

REL_L2 = 1e-3          # layer-output bounds of the contract
MAX_ABS_FRAC = 1e-2
TIE_GAP = 1e-6         # near-tie rule for top-k indices


def to_dev(x_bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to("cuda")


def check_routing(idx_gpu, w_gpu, ref):
    """Indices bit-exact except for tokens whose k-th/(k+1)-th oracle logits are within
    TIE_GAP (then the GPU set must still be the top-k up to that tie); weights within 1e-6."""
    ties = []
    for t in range(idx_gpu.shape[0]):
        if np.array_equal(idx_gpu[t], ref["idx"][t]):
            np.testing.assert_allclose(w_gpu[t], ref["w"][t], atol=1e-6, rtol=0)
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
