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
    L = synth.gen_layer(synth.CONFIGS["tiny"], threads=1)
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


# ---- the routing override (idx=) ----------------------------------------------------------
# moe_forward(layer, x, idx=...) evaluates a given index set with the weights of that set's own
# logits (the near-tie rule: either of two tied sets is valid, and the output check reruns the
# oracle with the set the GPU chose).  Pinned against the default path, which is pinned above.

def _override_layer():
    cfg = synth.small_config(seed=31, H=64, I=32, E=6, k=2, router_sigma=0.5)
    L = synth.gen_layer(cfg, threads=1)
    L.router_b = np.zeros(cfg.E, np.float32)
    return L


def test_idx_override_with_own_selection_is_identity():
    L = _override_layer()
    x = synth.gen_tokens(L.cfg, 5, batch=3)
    own = moe.moe_forward(L, x)
    again = moe.moe_forward(L, x, idx=own["idx"])
    assert np.array_equal(again["idx"], own["idx"])
    assert np.array_equal(again["w"], own["w"])
    assert np.array_equal(again["y"], own["y"])


def test_idx_override_rank_order_does_not_change_y():
    L = _override_layer()
    x = synth.gen_tokens(L.cfg, 5, batch=4)
    own = moe.moe_forward(L, x)
    rev = moe.moe_forward(L, x, idx=own["idx"][:, ::-1])
    assert np.array_equal(rev["w"], own["w"][:, ::-1])
    np.testing.assert_allclose(rev["y"], own["y"], rtol=1e-13,
                               atol=1e-13 * np.max(np.abs(own["y"])))


def test_idx_override_other_set_gets_its_own_softmax():
    """An index set that is not the oracle's choice: the override must weight it by the softmax
    of its own logits.  Layer B is layer A with +100 added to the bias of those two experts, so
    that B's own routing picks exactly that set with the same logit difference (a common shift
    leaves the softmax unchanged); A evaluated with the set as override must equal B evaluated
    normally.  Taking the weights of A's own selection instead fails this."""
    A = _override_layer()
    x = synth.gen_tokens(A.cfg, 4, batch=5)
    own = moe.moe_forward(A, x)
    alt = [4, 1]
    assert not any(set(own["idx"][t]) == set(alt) for t in range(4))
    B = copy.copy(A)
    B.router_b = A.router_b.copy()
    B.router_b[alt] += 100.0
    rb = moe.moe_forward(B, x)
    assert all(set(rb["idx"][t]) == set(alt) for t in range(4))
    ra = moe.moe_forward(A, x, idx=rb["idx"])
    np.testing.assert_allclose(ra["w"], rb["w"], rtol=1e-12)
    assert np.max(np.abs(ra["w"] - own["w"])) > 1e-3
    np.testing.assert_allclose(ra["y"], rb["y"], rtol=1e-12,
                               atol=1e-12 * np.max(np.abs(rb["y"])))


# ---- the scaled-FP4 composition (mode="mxfp4") ---------------------------------------------

def _hand_layer():
    """One NVFP4 expert, H = I = 32, k = 1 (weight 1), tensor scales 1/64, with few nonzeros.

    gate row 0: block 0 (E4M3 1.25 = code 0x3A): elements 0, 1 = E2M1 1.5, 1.0
                -> exact values 1.875/64, 1.25/64
    gate row 1: block 0 (1.25): element 0 = E2M1 6.0 -> 7.5/64 (unused by y: up row 1 is 0)
    gate row 2: block 0 (E4M3 2.0 = code 0x40): element 1 = E2M1 6.0 -> 12/64
    up row 0:   block 0 (E4M3 1.0 = code 0x38): elements 0, 1 = E2M1 2.0, 0.5 -> 2/64, 0.5/64
    up row 2:   block 0 (2.0): element 1 = E2M1 4.0 -> 8/64
    down row 0: block 0 (1.0): element 0 (I index 0) = E2M1 1.0 -> 1/64
    down row 1: block 0 (1.0): element 2 (I index 2) = E2M1 1.0 -> 1/64
    x:          x_0 = 3.0, x_1 = 0.3125 (both exact in bf16), the rest 0."""
    cfg = synth.small_config("hand", seed=1, H=32, I=32, E=1, k=1, fmt=synth.NVFP4,
                             nv_tensor_scale=1.0 / 64.0)
    z = lambda r, k: np.zeros((r, k // 2), np.uint8)
    s = lambda r, k: np.full((r, k // 16), 0x38, np.uint8)
    gc, gs, uc, us, dc, ds = z(32, 32), s(32, 32), z(32, 32), s(32, 32), z(32, 32), s(32, 32)
    gc[0, 0] = 0x3 | (0x2 << 4)
    gs[0, 0] = 0x3A
    gc[1, 0] = 0x7
    gs[1, 0] = 0x3A
    gc[2, 0] = 0x7 << 4
    gs[2, 0] = 0x40
    uc[0, 0] = 0x4 | (0x1 << 4)
    uc[2, 0] = 0x6 << 4
    us[2, 0] = 0x40
    dc[0, 0] = 0x2
    dc[1, 1] = 0x2
    ex = synth.Expert(gc, gs, uc, us, dc, ds, np.full(3, 1.0 / 64.0, np.float32))
    L = synth.Layer(cfg, np.zeros((1, 32), np.float32), None, {0: ex}, [])
    x = np.zeros((1, 32), np.uint16)
    x[0, :2] = synth.f32_to_bf16_bits(np.array([3.0, 0.3125], np.float32))
    return L, x


def test_mxfp4_mode_hand_worked_layer():
    """S1 on the hand layer, every quantiser step worked by hand (OCP MX rule, 32 along K):

    x block: amax 3 -> scale 2^(1-2) = 1/2; 3/(1/2) = 6 -> 6; 0.3125/(1/2) = 0.625 -> 0.5
      (nearest) -> xq = (3.0, 0.25).
    gate row 0 (the whole row is one block along H): amax 1.875/64 -> scale 2^(-6-2) = 2^-8;
      1.875/64 * 256 = 7.5 -> 6 (saturates); 1.25/64 * 256 = 5 -> tie of 4 and 6, ties to
      the even code (4 = code 6) -> Wg = (6, 4) * 2^-8.
    gate row 2: amax 12/64 -> scale 2^-5: 6 -> unchanged.
    up row 0: amax 2/64 -> scale 2^-7: 4 and 1 are on the grid -> unchanged.
    up row 2: amax 8/64 -> scale 2^-5: 4 -> unchanged.  down rows: 1/64 -> unchanged.
    g_0 = 6/256 * 3 + 4/256 * 0.25 = 0.07421875; u_0 = 2/64 * 3 + 0.5/64 * 0.25 = 0.095703125;
    a_0 = silu(g_0) u_0 = 0.0036832.  g_2 = 12/64 * 0.25 = 0.046875; u_2 = 8/64 * 0.25 =
    0.03125; a_2 = silu(g_2) u_2 = 0.00074958.  Every other a_i is 0 (its up row is 0).
    h block (I = 32 is one block): amax a_0 -> scale 2^(-9-2) = 2^-11; a_0 / 2^-11 = 7.54 -> 6
      (saturates); a_2 / 2^-11 = 1.535 -> 1.5.
    y_0 = (1/64) * 6 * 2^-11 = 6 * 2^-17 and y_1 = (1/64) * 1.5 * 2^-11 = 1.5 * 2^-17, exactly;
    every other output is 0."""
    L, x = _hand_layer()
    y = moe.moe_forward(L, x, mode="mxfp4")["y"]
    exp = np.zeros((1, 32))
    exp[0, 0] = 6.0 * 2.0 ** -17
    exp[0, 1] = 1.5 * 2.0 ** -17
    assert np.array_equal(y, exp)


def test_mxfp4_mode_hand_layer_catches_plausible_mistakes(monkeypatch):
    """The hand-worked values above must fail when the composition is wrong: weights quantised
    along the other axis (gate column 0 then holds 7.5/64 from row 1, whose scale 2^-6 sends
    1.875/64 to 2/64), the weight quantisation skipped, h left unquantised, or x left
    unquantised (then a_2 / 2^-11 = 2.41 and h_2 = 2 * 2^-11)."""
    L, x = _hand_layer()
    good = np.array([6.0 * 2.0 ** -17, 1.5 * 2.0 ** -17])
    ident = lambda a: a
    from oracle import mxq

    def wrong_axis(ws):
        return tuple(mxq.quantize_dequant(w.T).T for w in ws)

    variants = {
        "wrong axis": (mxq.quantize_dequant, mxq.quantize_dequant, wrong_axis),
        "no weight quantisation": (mxq.quantize_dequant, mxq.quantize_dequant, ident),
        "no h quantisation": (mxq.quantize_dequant, fp4.round_bf16,
                              lambda ws: tuple(mxq.quantize_dequant(w) for w in ws)),
        "no x quantisation": (ident, mxq.quantize_dequant,
                              lambda ws: tuple(mxq.quantize_dequant(w) for w in ws)),
    }
    for name, ops in variants.items():
        monkeypatch.setattr(moe, "mode_ops", lambda mode, ops=ops: ops)
        y = moe.moe_forward(L, x, mode="mxfp4")["y"]
        assert not np.array_equal(y[0, :2], good), name


@pytest.mark.parametrize("mode", ["exact", "mxfp4"])
def test_weights_fn_with_the_modes_own_weights_changes_nothing(mode):
    """moe_forward's weights_fn hook (a caller supplying each expert's transformed weights)
    gives the same y as the default path when it supplies what the mode computes, and is
    called once per routed expert; supplying other weights changes y."""
    from oracle import mxq
    L = _tiny(41, E=5, k=2, H=64, I=32, fmt=synth.NVFP4, nv_tensor_scale=0.25)
    x = synth.gen_tokens(L.cfg, 6, batch=2)
    ref = moe.moe_forward(L, x, mode=mode)
    _, _, wq = moe.mode_ops(mode)
    calls = []

    def fn(e):
        calls.append(e)
        return wq(moe.expert_weights(L, L.expert(e)))
    got = moe.moe_forward(L, x, mode=mode, weights_fn=fn)
    assert np.array_equal(got["y"], ref["y"])
    assert sorted(calls) == sorted(set(int(e) for e in np.unique(ref["idx"])))
    other = moe.moe_forward(L, x, mode=mode, weights_fn=lambda e: tuple(
        2.0 * w for w in wq(moe.expert_weights(L, L.expert(e)))))
    assert not np.array_equal(other["y"], ref["y"])
