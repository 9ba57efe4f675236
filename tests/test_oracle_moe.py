"""Pins for the oracle's routing, expert FFN and combine (CPU only).

Checks: routing invariants and the full-softmax identity; dense all-experts evaluation
masked to the chosen k on the tiny workload and 50 seeded tiny layers; special cases with
closed forms (k = E with identical experts is one dense SwiGLU FFN evaluated with torch;
k = 1 gives weight 1; all-zero codes give 0; an E8M0 shift scales y by a power of two;
relabelling experts together with their router rows changes nothing)."""
import copy

import numpy as np
import pytest
import scipy.special
import torch

from mxfp4_expert_layer_amd import synth
from oracle import fp4, moe


def _tiny(seed, **kw):
    cfg = synth.small_config(seed=seed, **kw)
    return synth.gen_layer(cfg, threads=1)


def test_routing_invariants_and_softmax_identity():
    rng = np.random.default_rng(0)
    for trial in range(20):
        E, H, k, T = int(rng.integers(2, 40)), 64, None, 8
        k = int(rng.integers(1, E + 1))
        x = rng.standard_normal((T, H))
        wr = rng.standard_normal((E, H)) * 0.3
        b = rng.standard_normal(E) if trial % 2 else None
        idx, w, logits, gap = moe.route(x, wr, b, k)
        for t in range(T):
            assert len(set(idx[t])) == k
            assert abs(w[t].sum() - 1.0) <= 1e-12
            full = np.sort(logits[t])[::-1]
            assert np.array_equal(np.sort(logits[t, idx[t]])[::-1], full[:k])
            assert np.all(np.diff(logits[t, idx[t]]) <= 0)          # rank order
            p = scipy.special.softmax(logits[t])                       # softmax over all E
            np.testing.assert_allclose(w[t], p[idx[t]] / p[idx[t]].sum(), rtol=1e-13)


def test_routing_ties_go_to_lower_index():
    x = np.ones((1, 4))
    wr = np.array([[1, 0, 0, 0], [0, 0, 0, 1], [1, 0, 0, 0], [0, 0, 2, 0]], float)
    idx, w, _, gap = moe.route(x, wr, None, 3)
    assert list(idx[0]) == [3, 0, 1]
    assert gap[0] == 0.0


def test_k1_weight_is_one():
    L = _tiny(3, k=1, E=5)
    x = synth.gen_tokens(L.cfg, 6)
    r = moe.moe_forward(L, x)
    assert np.all(r["w"] == 1.0)


@pytest.mark.parametrize("seed", range(50))
def test_dense_masked_equality_tiny(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 9))
    k = int(rng.integers(1, E + 1))
    H = int(rng.choice([32, 64]))
    I = int(rng.choice([32, 64]))
    fmt = synth.MXFP4 if seed % 3 else synth.NVFP4
    L = _tiny(100 + seed, E=E, k=k, H=H, I=I, fmt=fmt, n_shared=seed % 2,
              nv_tensor_scale=0.5 if fmt == synth.NVFP4 else 1.0)
    x = synth.gen_tokens(L.cfg, 5, batch=seed)
    ys = moe.moe_forward(L, x)["y"]
    yd = moe.dense_masked_forward(L, x)
    assert np.max(np.abs(ys - yd)) <= 1e-12 * max(1.0, np.max(np.abs(yd)))


def test_dense_masked_equality_tiny_workload():
    L = synth.gen_layer(synth.CONFIGS["cfg1"], threads=1)
    x = synth.gen_tokens(L.cfg, 4)
    ys = moe.moe_forward(L, x)["y"]
    yd = moe.dense_masked_forward(L, x)
    assert np.max(np.abs(ys - yd)) <= 1e-12 * np.max(np.abs(yd))
    assert np.max(np.abs(yd)) > 0


def _torch_swiglu(x64, wg, wu, wd):
    xt = torch.from_numpy(x64)
    g = torch.nn.functional.linear(xt, torch.from_numpy(wg))
    u = torch.nn.functional.linear(xt, torch.from_numpy(wu))
    h = (torch.nn.functional.silu(g) * u).float().to(torch.bfloat16).double()
    return torch.nn.functional.linear(h, torch.from_numpy(wd)).numpy()


@pytest.mark.parametrize("fmt", [synth.MXFP4, synth.NVFP4])
def test_all_experts_identical_k_eq_E_is_dense_ffn(fmt):
    cfg = synth.small_config(seed=11, E=4, k=4, H=64, I=64, fmt=fmt, nv_tensor_scale=0.75,
                             code_dist="normal")
    L = synth.gen_layer(cfg, threads=1)
    for e in range(1, 4):
        L.experts[e] = L.experts[0]
    x = synth.gen_tokens(cfg, 7)
    y = moe.moe_forward(L, x)["y"]
    wg, wu, wd = moe.expert_weights(L, L.expert(0))
    ref = _torch_swiglu(fp4.bf16_bits_to_f64(x), wg, wu, wd)
    # torch rounds h via fp32 (double rounding is possible but rare), hence not bit-exact
    assert moe.rel_l2(y, ref) < 1e-5
    # swapping gate and up, or dropping the bf16 rounding of h, would fail this
    alt = _torch_swiglu(fp4.bf16_bits_to_f64(x), wu, wg, wd)
    assert moe.rel_l2(alt, ref) > 1e-2


def test_zero_codes_give_zero_or_shared_only():
    L = _tiny(21, E=4, k=2, n_shared=1)
    for e in range(4):
        ex = copy.deepcopy(L.expert(e))
        for f in ("gate_codes", "up_codes", "down_codes"):
            getattr(ex, f)[:] = 0
        L.experts[e] = ex
    x = synth.gen_tokens(L.cfg, 3)
    r = moe.moe_forward(L, x)
    np.testing.assert_array_equal(r["y"], r["shared"][:, 0])
    assert np.all(r["ys"] == 0)


def test_e8m0_shift_of_down_scales_scales_output_exactly():
    L = _tiny(22, E=4, k=2)
    x = synth.gen_tokens(L.cfg, 3)
    y0 = moe.moe_forward(L, x)["y"]
    L2 = copy.deepcopy(L)
    for e in range(4):
        L2.experts[e].down_scales = (L2.experts[e].down_scales + 3).astype(np.uint8)
    y1 = moe.moe_forward(L2, x)["y"]
    assert np.array_equal(y1, y0 * 8.0)


def test_expert_relabelling_invariance():
    L = _tiny(23, E=6, k=3)
    x = synth.gen_tokens(L.cfg, 5)
    y0 = moe.moe_forward(L, x)["y"]
    perm = np.array([3, 5, 0, 1, 4, 2])
    L2 = copy.deepcopy(L)
    L2.router_w = L.router_w[perm]
    L2.experts = {i: L.expert(int(perm[i])) for i in range(6)}
    y1 = moe.moe_forward(L2, x)["y"]
    np.testing.assert_allclose(y1, y0, rtol=0, atol=1e-12 * np.max(np.abs(y0)))


def test_gate_not_applied_to_up():
    """silu acts on the gate projection only: with W_u = 0 the output must vanish, with W_g
    = 0 it must vanish as well (silu(0) = 0), but scaling W_g must not scale y linearly."""
    L = _tiny(24, E=2, k=1)
    x = synth.gen_tokens(L.cfg, 2)
    y0 = moe.moe_forward(L, x)["y"]
    L2 = copy.deepcopy(L)
    for e in range(2):
        L2.experts[e].gate_scales = (L2.experts[e].gate_scales + 1).astype(np.uint8)
    y1 = moe.moe_forward(L2, x)["y"]
    assert moe.rel_l2(y1, 2 * y0) > 1e-3
