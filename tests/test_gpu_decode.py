"""GPU parity of the decode path (libft through its C ABI) against the float64 oracle."""
import sys

import numpy as np
import pytest

from mxfp4_expert_layer_amd import synth
from oracle import fp4, moe, policy

from gpu_util import check_output, check_routing, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ft = pytest.importorskip("mxfp4_expert_layer_amd.ft")
from mxfp4_expert_layer_amd.layer import GpuLayer, stream_ptr  # noqa: E402


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = ft.Context(0)
    yield c
    c.close()


_layers = {}


def layer_for(ctx, name, **kw):
    """One GpuLayer per name for the whole module (building the big layers takes seconds)."""
    if name not in _layers:
        cfg = kw.pop("cfg") if "cfg" in kw else synth.CONFIGS[name]
        log(f"[gpu] building layer {name} {cfg.H}x{cfg.I} E={cfg.E}")
        _layers[name] = GpuLayer(ctx, cfg, **kw)
    return _layers[name]


def run_decode(ctx, L, x_bits, stats=None):
    T = x_bits.shape[0]
    xd = to_dev(x_bits)
    y = torch.empty((T, L.cfg.H), dtype=torch.float32, device="cuda")
    ft.moe_decode(ctx, L.handle, xd, T, y, stream_ptr(), stats)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def run_route(ctx, L, x_bits):
    T = x_bits.shape[0]
    xd = to_dev(x_bits)
    idx = torch.empty((T, L.cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, L.cfg.k), dtype=torch.float32, device="cuda")
    ft.route(ctx, L.handle, xd, T, idx, w, stream_ptr())
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


# ---- A3: dequantisation, bit-exact ----------------------------------------------------------

def _dequant(L, slot, matrix):
    cfg = L.cfg
    R, K = (cfg.H, cfg.I) if matrix == 2 else (cfg.I, cfg.H)
    out = torch.empty((R, K), dtype=torch.float32, device="cuda")
    ft.debug_dequant(L.handle, slot, matrix, out, stream_ptr())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _expected(L, ex, matrix, fmt):
    names = [("gate_codes", "gate_scales"), ("up_codes", "up_scales"), ("down_codes", "down_scales")]
    c, s = names[matrix]
    v = fp4.dequant(fmt, getattr(ex, c), getattr(ex, s), float(ex.tensor_scales[matrix]))
    with np.errstate(over="ignore"):
        return v.astype(np.float32)


def _same(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        a[~np.isnan(a)].view(np.uint32), b[~np.isnan(b)].view(np.uint32))


def test_dequant_bit_exact_tiny_workload(ctx):
    L = layer_for(ctx, "tiny", max_tokens=16)
    OL = L.oracle_layer()
    for slot in range(L.cfg.E):
        for m in range(3):
            assert _same(_dequant(L, slot, m), _expected(L, OL.expert(slot), m, "mxfp4")), (slot, m)


def _allcodes_layer(ctx):
    cfg = synth.small_config("allcodes", seed=3, H=256, I=256, E=2, k=1)
    ex = synth.gen_expert(cfg, 0)
    rows, nb = cfg.I, cfg.H // 2
    ex.gate_codes = ((np.arange(rows)[:, None] * nb + np.arange(nb)[None, :]) % 256).astype(np.uint8)
    ex.gate_scales = (np.arange(rows * cfg.H // 32) % 256).astype(np.uint8).reshape(rows, -1)
    return layer_for(ctx, "allcodes", cfg=cfg, max_tokens=1, experts={0: ex}), ex


def test_dequant_every_code_normal_scales(ctx):
    """Every byte of E2M1 code pairs under E8M0 scale codes 2..253.  Up to 252 every product
    is a normal fp32 number; at 253 the products of +-4 and +-6 (2^128 and 1.5 * 2^128)
    exceed the fp32 range and must be +-inf on both sides."""
    L, ex = _allcodes_layer(ctx)
    got = _dequant(L, 0, 0)
    exp = _expected(L, ex, 0, "mxfp4")
    sc = np.repeat(ex.gate_scales.astype(np.int64), 32, axis=1)
    sel = (sc >= 2) & (sc <= 253)
    assert _same(got[sel], exp[sel])


def test_dequant_extreme_scales(ctx):
    """E8M0 codes 0, 1, 254 and 255: subnormal, overflowing and NaN products."""
    L, ex = _allcodes_layer(ctx)
    got = _dequant(L, 0, 0)
    exp = _expected(L, ex, 0, "mxfp4")
    sc = np.repeat(ex.gate_scales.astype(np.int64), 32, axis=1)
    for code in (0, 1, 254, 255):
        sel = sc == code
        g, e = got[sel], exp[sel]
        bad = ~((g == e) | (np.isnan(g) & np.isnan(e)))
        assert not bad.any(), (code, list(zip(g[bad][:6], e[bad][:6])))


def test_dequant_nvfp4_bit_exact(ctx):
    cfg = synth.small_config("nvsmall", seed=5, H=256, I=128, E=3, k=2, fmt=synth.NVFP4,
                             code_dist="uniform", nv_tensor_scale=1 / 64)
    L = layer_for(ctx, "nvsmall", cfg=cfg, max_tokens=2)
    OL = L.oracle_layer()
    for slot in range(3):
        for m in range(3):
            assert _same(_dequant(L, slot, m), _expected(L, OL.expert(slot), m, "nvfp4"))


def test_dequant_nvfp4_every_scale_code(ctx):
    """Every E4M3 scale code, subnormals (0x01..0x07), negative codes and the NaN codes 0x7f
    and 0xff included, under every E2M1 code pair: the kernels' scale decode is bit-exact."""
    cfg = synth.small_config("nvallscales", seed=9, H=256, I=256, E=2, k=1, fmt=synth.NVFP4,
                             nv_tensor_scale=1 / 64)
    ex = synth.gen_expert(cfg, 0)
    rows, nb = cfg.I, cfg.H // 2
    ex.gate_codes = ((np.arange(rows)[:, None] * nb + np.arange(nb)[None, :]) % 256).astype(np.uint8)
    ex.gate_scales = (np.arange(rows * cfg.H // 16) % 256).astype(np.uint8).reshape(rows, -1)
    L = layer_for(ctx, "nvallscales", cfg=cfg, max_tokens=1, experts={0: ex})
    assert _same(_dequant(L, 0, 0), _expected(L, ex, 0, "nvfp4"))


# ---- A1: routing ------------------------------------------------------------------------------

@pytest.mark.parametrize("name,T", [("tiny", 4), ("35b-a3b", 1), ("35b-a3b", 8), ("284b", 1),
                                    ("284b", 16)])
def test_route_matches_oracle(ctx, name, T):
    L = layer_for(ctx, name, max_tokens=16)
    OL = L.oracle_layer()
    x = synth.gen_tokens(L.cfg, T, batch=7)
    idx, w = run_route(ctx, L, x)
    xr = fp4.bf16_bits_to_f64(x)
    r_idx, r_w, logits, gap = moe.route(xr, OL.router_w, OL.router_b, L.cfg.k)
    check_routing(idx, w, dict(idx=r_idx, w=r_w, logits=logits, gap=gap))
    assert np.all(np.abs(w.sum(1) - 1) <= 1e-6)


def test_route_exact_ties_go_to_lower_index(ctx):
    """Duplicated router rows give bit-identical logits; the lower expert id must win."""
    cfg = synth.small_config("ties", seed=31, H=256, I=128, E=64, k=6, router_sigma=1 / 16)
    w, _ = synth.gen_router(cfg)
    w = w.copy()
    for a, b in [(3, 40), (7, 8), (21, 63), (50, 2), (11, 12), (12, 13)]:
        w[b] = w[a]
    L = layer_for(ctx, "ties", cfg=cfg, max_tokens=16, router=(w, None))
    OL = L.oracle_layer()
    x = synth.gen_tokens(cfg, 16, batch=4)
    idx, wt = run_route(ctx, L, x)
    r_idx, r_w, logits, gap = moe.route(fp4.bf16_bits_to_f64(x), OL.router_w, OL.router_b, cfg.k)
    # ties inside the kept set are exact on both sides; only the kept/dropped boundary may
    # legitimately differ under the near-tie rule
    check_routing(idx, wt, dict(idx=r_idx, w=r_w, logits=logits, gap=gap))
    assert (idx == r_idx).mean() > 0.9


# ---- A4-A6: decode layer outputs ------------------------------------------------------------

def _decode_and_check(ctx, L, T, batch):
    x = synth.gen_tokens(L.cfg, T, batch=batch)
    log(f"[gpu] decode {L.cfg.name} T={T} batch={batch}")
    y = run_decode(ctx, L, x)
    idx, w = run_route(ctx, L, x)
    OL = L.oracle_layer()
    ref = moe.moe_forward(OL, x)
    ties = check_routing(idx, w, ref)
    if ties:
        ref = moe.moe_forward(OL, x, idx=idx)
    return check_output(y, ref["y"], f"{L.cfg.name} T={T}")


@pytest.mark.parametrize("name,T", [("tiny", 4), ("35b-a3b", 1), ("35b-a3b", 8),
                                    ("284b", 1), ("284b", 4), ("284b", 16),
                                    ("35b-a3b-nvfp4", 1), ("35b-a3b-nvfp4", 8)])
def test_decode_matches_oracle(ctx, name, T):
    L = layer_for(ctx, name, max_tokens=16)
    err = _decode_and_check(ctx, L, T, batch=100 + T)
    log(f"[gpu] {name} T={T} rel-L2 {err:.2e}")


@pytest.mark.parametrize("H,I,E,k,ns,T", [(128, 128, 4, 2, 0, 3), (384, 256, 5, 3, 1, 7),
                                          (640, 384, 9, 4, 2, 16), (1152, 640, 17, 5, 1, 11),
                                          (256, 1152, 6, 1, 0, 2), (512, 2176, 3, 3, 1, 5),
                                          (256, 128, 40, 16, 1, 16), (128, 128, 16, 16, 0, 1),
                                          (256, 1152, 6, 2, 1, 1), (384, 1664, 12, 9, 1, 1)])
def test_decode_ragged_shapes(ctx, H, I, E, k, ns, T):
    """K chunk counts that do not divide the wave split, odd row-tile counts, shared experts;
    the largest k (16), with sixteen tokens, and with k = E (every expert selected); one token
    with 9 and 13 down-projection K chunks (two load batches, the second partly filled) and
    ten list entries (two per wave of the down kernel)."""
    cfg = synth.small_config(f"rag{H}_{I}", seed=H + I, H=H, I=I, E=E, k=k, n_shared=ns,
                             code_dist="normal", router_sigma=1 / np.sqrt(H))
    L = layer_for(ctx, cfg.name, cfg=cfg, max_tokens=16)
    _decode_and_check(ctx, L, T, batch=1)


@pytest.mark.parametrize("H,I,E,k,ns,T,ts", [(256, 128, 5, 2, 1, 1, 0.7), (384, 640, 7, 3, 1, 5, 1 / 64),
                                             (1152, 256, 9, 4, 0, 16, 3.0),
                                             (256, 1408, 9, 4, 1, 1, 0.7)])
def test_decode_nvfp4_shapes(ctx, H, I, E, k, ns, T, ts):
    """NVFP4 experts (E4M3 scales per 16 over all 256 codes' normal range, a tensor scale that
    is not a power of two in two of the cases), shared experts, ragged chunk counts."""
    cfg = synth.small_config(f"nv{H}_{I}", seed=H + 3 * I, H=H, I=I, E=E, k=k, n_shared=ns,
                             fmt=synth.NVFP4, code_dist="normal", router_sigma=1 / np.sqrt(H),
                             scale_lo=0x01, scale_hi=0x7e, nv_tensor_scale=ts)
    L = layer_for(ctx, cfg.name, cfg=cfg, max_tokens=16)
    _decode_and_check(ctx, L, T, batch=2)


def test_decode_is_deterministic(ctx):
    L = layer_for(ctx, "35b-a3b", max_tokens=16)
    x = synth.gen_tokens(L.cfg, 8, batch=3)
    a = run_decode(ctx, L, x)
    b = run_decode(ctx, L, x)
    assert np.array_equal(a, b)


def test_decode_rejects_bad_token_count(ctx):
    L = layer_for(ctx, "tiny_T4", cfg=synth.CONFIGS["tiny"], max_tokens=4)
    x = synth.gen_tokens(L.cfg, 5)
    with pytest.raises(ft.FtError) as e:
        run_decode(ctx, L, x)
    assert e.value.code == ft.FT_EINVAL


# ---- A2/A7: slot pool and miss path ---------------------------------------------------------

def _miss_sequence(ctx, L, steps, bp, bh, check_every, T=1, q_force=None, batch0=0):
    cfg = L.cfg
    OL = L.oracle_layer()
    pool = policy.LruPool(cfg.E, L.n_slots)
    ft.set_bandwidth(L.handle, bp, bh)
    ft.force_q(L.handle, -1 if q_force is None else q_force)
    hits = total = 0
    for s in range(steps):
        x = synth.gen_tokens(cfg, T, batch=batch0 + s)
        st = ft.DecodeStats()
        y = run_decode(ctx, L, x, st)
        xr = fp4.bf16_bits_to_f64(x)
        r_idx, r_w, logits, gap = moe.route(xr, OL.router_w, OL.router_b, cfg.k)
        assert np.all(gap >= 1e-6), "near-tie in a miss-path step; choose another seed"
        res = pool.step(r_idx, r_w, bp, bh, q_override=q_force)
        e2s, s2e = ft.debug_tables(L.handle, cfg.E, L.n_slots)
        assert np.array_equal(e2s, res.e2s), f"step {s}: e2s differs"
        assert np.array_equal(s2e, res.s2e), f"step {s}: s2e differs"
        assert (st.n_hits, st.n_miss, st.q, st.n_streamed, st.n_host) == (
            len(res.hits), len(res.misses), res.q, len(res.streamed), len(res.host)), s
        hits += len(res.hits)
        total += len(res.selected)
        if s % check_every == 0 or s == steps - 1:
            ref = moe.moe_forward(OL, x)
            check_output(y, ref["y"], f"miss step {s}")
    return hits / max(1, total)


def test_miss_path_small_pool(ctx):
    cfg = synth.small_config("misssmall", seed=77, H=256, I=128, E=16, k=3, n_shared=1,
                             code_dist="normal", router_sigma=1 / 16, zipf_c=0.7)
    L = layer_for(ctx, "misssmall", cfg=cfg, resident=False, n_slots=5, max_tokens=4)
    _miss_sequence(ctx, L, steps=30, bp=1.0, bh=2.5, check_every=3, T=2)


def test_miss_path_nvfp4_small_pool(ctx):
    """NVFP4 experts through the slot pool: streamed misses, host-computed misses (the host
    FFN decodes E4M3 scales and the tensor scale) and hits in one sequence."""
    cfg = synth.small_config("missnv", seed=79, H=384, I=256, E=14, k=3, n_shared=1,
                             fmt=synth.NVFP4, code_dist="normal", router_sigma=1 / 20,
                             zipf_c=0.7, nv_tensor_scale=1 / 64)
    L = layer_for(ctx, "missnv", cfg=cfg, resident=False, n_slots=5, max_tokens=2)
    _miss_sequence(ctx, L, steps=24, bp=1.0, bh=2.5, check_every=2, T=2)


@pytest.mark.parametrize("q_force", [0, 2, 99])
def test_miss_path_forced_split_gives_same_outputs(ctx, q_force):
    cfg = synth.small_config("missforce", seed=78, H=384, I=256, E=12, k=4, n_shared=0,
                             code_dist="normal", router_sigma=1 / 20)
    L = layer_for(ctx, f"missforce{q_force}", cfg=cfg, resident=False, n_slots=4, max_tokens=2)
    _miss_sequence(ctx, L, steps=8, bp=1.0, bh=3.0, check_every=1, T=1, q_force=q_force)


@pytest.mark.parametrize("rule", [0, 1])
def test_miss_path_adaptive_bandwidths(ctx, rule):
    """Bp and Bh re-measured during decode (running average, alpha = 1/2) under both split
    rules: the oracle's pool replays each call's split with the Bp, Bh that call reports, so
    the slot tables stay bit-exact; each estimate moves toward its observation by alpha."""
    cfg = synth.small_config("missadapt", seed=81, H=384, I=256, E=14, k=3, n_shared=1,
                             code_dist="normal", router_sigma=1 / 20, zipf_c=0.7)
    L = layer_for(ctx, f"missadapt{rule}", cfg=cfg, resident=False, n_slots=5, max_tokens=2)
    with pytest.raises(ft.FtError) as e:
        ft.set_miss_policy(L.handle, 7, 0.5)
    assert e.value.code == ft.FT_EINVAL
    with pytest.raises(ft.FtError) as e:
        ft.set_miss_policy(L.handle, rule, 1.5)
    assert e.value.code == ft.FT_EINVAL
    ft.set_bandwidth(L.handle, 1.0e9, 3.0e9)
    ft.force_q(L.handle, -1)
    ft.set_miss_policy(L.handle, rule, 0.5)
    OL = L.oracle_layer()
    pool = policy.LruPool(cfg.E, L.n_slots)
    prev, seen_bp, seen_bh = None, 0, 0
    try:
        for s in range(24):
            x = synth.gen_tokens(cfg, 2, batch=300 + s)
            st = ft.DecodeStats()
            y = run_decode(ctx, L, x, st)
            r_idx, r_w, logits, gap = moe.route(fp4.bf16_bits_to_f64(x), OL.router_w, OL.router_b, cfg.k)
            assert np.all(gap >= 1e-6), "near-tie in a miss-path step; choose another seed"
            res = pool.step(r_idx, r_w, st.bp, st.bh, rule="makespan" if rule else "round")
            e2s, s2e = ft.debug_tables(L.handle, cfg.E, L.n_slots)
            assert np.array_equal(e2s, res.e2s) and np.array_equal(s2e, res.s2e), f"step {s}"
            assert (st.q, st.n_streamed, st.n_host) == (res.q, len(res.streamed), len(res.host)), s
            if prev is not None:
                bp = prev.bp + 0.5 * (st.bp_obs - prev.bp) if st.bp_obs > 0 else prev.bp
                bh = prev.bh + 0.5 * (prev.bh_obs - prev.bh) if prev.bh_obs > 0 else prev.bh
                assert st.bp == pytest.approx(bp, rel=1e-12) and st.bh == pytest.approx(bh, rel=1e-12), s
            seen_bp += st.bp_obs > 0
            seen_bh += prev is not None and prev.bh_obs > 0
            if s % 4 == 0:
                check_output(y, moe.moe_forward(OL, x)["y"], f"adaptive step {s}")
            prev = st
    finally:
        ft.set_miss_policy(L.handle, ft.FT_SPLIT_ROUND, 0.0)
    assert seen_bp > 0 and seen_bh > 0, (seen_bp, seen_bh)
    log(f"[gpu] adaptive rule {rule}: final Bp {prev.bp / 1e9:.2f} GB/s, Bh {prev.bh / 1e9:.2f} GB/s")


def test_miss_path_load_rule(ctx):
    """The split's load variant: every call times its hit experts' kernels, the next call
    reports that GPU time and the per-expert estimate it split with, and its q is the load
    rule's for the call's m, hits (+ shared), Bp, Bh and that estimate; the oracle's pool,
    given each call's q, keeps the slot tables bit-exact, and outputs match the oracle."""
    cfg = synth.small_config("missload", seed=85, H=512, I=256, E=16, k=3, n_shared=1,
                             code_dist="normal", router_sigma=1 / 22, zipf_c=0.7)
    L = layer_for(ctx, "missload", cfg=cfg, resident=False, n_slots=6, max_tokens=2)
    # bandwidths in a ratio where a GPU term of a few microseconds per expert moves q
    bp, bh = 2.0e9, 5.0e9
    ft.set_bandwidth(L.handle, bp, bh)
    ft.force_q(L.handle, -1)
    ft.set_miss_policy(L.handle, ft.FT_SPLIT_LOAD, 0.0)
    OL = L.oracle_layer()
    pool = policy.LruPool(cfg.E, L.n_slots)
    seen, prev_hits = 0, None
    try:
        for s in range(20):
            x = synth.gen_tokens(cfg, 2, batch=700 + s)
            st = ft.DecodeStats()
            y = run_decode(ctx, L, x, st)
            if prev_hits:
                assert st.gpu_us_obs > 0, s
                assert st.t_gpu == pytest.approx(st.gpu_us_obs * 1e-6 / prev_hits, rel=1e-6), s
                seen += 1
            g0 = st.n_hits + cfg.n_shared
            assert st.q == ft.qstar_split_load(st.n_miss, g0, st.bp, st.bh, float(L.stride),
                                               st.t_gpu)
            assert st.q == policy.qstar_load(st.n_miss, g0, st.bp, st.bh, float(L.stride),
                                             st.t_gpu)
            r_idx, r_w, _, gap = moe.route(fp4.bf16_bits_to_f64(x), OL.router_w, OL.router_b, cfg.k)
            assert np.all(gap >= 1e-6)
            res = pool.step(r_idx, r_w, bp, bh, q_override=st.q)
            e2s, s2e = ft.debug_tables(L.handle, cfg.E, L.n_slots)
            assert np.array_equal(e2s, res.e2s) and np.array_equal(s2e, res.s2e), s
            if s % 3 == 0:
                check_output(y, moe.moe_forward(OL, x)["y"], f"load rule step {s}")
            prev_hits = st.n_hits + cfg.n_shared
        log(f"[gpu] load rule: t_gpu {st.t_gpu * 1e6:.2f} us per expert")
    finally:
        ft.set_miss_policy(L.handle, ft.FT_SPLIT_ROUND, 0.0)
    assert seen > 0


def test_measure_bandwidth_feeds_the_split(ctx):
    """The startup probes: Bp (pinned H2D copies of expert blobs) and Bh (the host expert FFN
    over blobs) come back finite and positive, the next decode calls report exactly those
    values and split their misses by them (q = round(m Bp / Bh)), and the slot tables follow
    the oracle's pool driven by the measured pair."""
    cfg = synth.small_config("missmeas", seed=83, H=512, I=256, E=16, k=3, n_shared=1,
                             code_dist="normal", router_sigma=1 / 22, zipf_c=0.7)
    L = layer_for(ctx, "missmeas", cfg=cfg, resident=False, n_slots=5, max_tokens=2)
    bp, bh = ft.measure_bandwidth(ctx, L.handle)
    log(f"[gpu] measured Bp {bp / 1e9:.2f} GB/s, Bh {bh / 1e9:.2f} GB/s")
    assert np.isfinite(bp) and np.isfinite(bh) and bp > 0 and bh > 0
    assert 1e8 < bp < 1e12 and 1e8 < bh < 1e13
    ft.force_q(L.handle, -1)
    OL = L.oracle_layer()
    pool = policy.LruPool(cfg.E, L.n_slots)
    for s in range(6):
        x = synth.gen_tokens(cfg, 2, batch=500 + s)
        st = ft.DecodeStats()
        y = run_decode(ctx, L, x, st)
        assert (st.bp, st.bh) == (bp, bh)
        q, qstar = ft.qstar_split(st.n_miss, bp, bh)
        assert st.q == q and st.qstar == pytest.approx(qstar, rel=1e-12)
        r_idx, r_w, _, gap = moe.route(fp4.bf16_bits_to_f64(x), OL.router_w, OL.router_b, cfg.k)
        assert np.all(gap >= 1e-6)
        res = pool.step(r_idx, r_w, bp, bh)
        e2s, s2e = ft.debug_tables(L.handle, cfg.E, L.n_slots)
        assert np.array_equal(e2s, res.e2s) and np.array_equal(s2e, res.s2e), s
        if s % 2 == 0:
            check_output(y, moe.moe_forward(OL, x)["y"], f"measured split step {s}")


def test_context_binds_host_threads_to_the_gpu_node(ctx):
    """ft_ctx_create binds the host pool's workers to the CPUs of the GPU's NUMA node: when it
    reports a binding, that many workers run with exactly that node's CPU list."""
    import os
    from mxfp4_expert_layer_amd.layer import node_cpus
    node, pinned = ft.ctx_numa(ctx)
    log(f"[gpu] GPU NUMA node {node}, host threads bound to {pinned} CPUs")
    assert node >= -1 and pinned >= 0
    if pinned == 0:
        assert not node_cpus(node) or os.environ.get("FT_HOST_AFFINITY") == "0"
        return
    cpus = node_cpus(node)
    assert len(cpus) == pinned
    bound = 0
    for tid in os.listdir("/proc/self/task"):
        try:
            with open(f"/proc/self/task/{tid}/status") as fh:
                line = [ln for ln in fh if ln.startswith("Cpus_allowed_list")][0]
        except (OSError, IndexError):
            continue
        if set(ft.debug_parse_cpulist(line.split(":", 1)[1].strip())) == cpus:
            bound += 1
    assert bound >= 1


def test_miss_path_284b_layer(ctx):
    """The 284B-class layer with a 48-slot pool: 64 warm-up and 64 timed single tokens with the
    slot tables checked after every step and the outputs every 8th step."""
    L = layer_for(ctx, "284b-miss-path", resident=False, n_slots=48, max_tokens=1)
    rate = _miss_sequence(ctx, L, steps=128, bp=50e9, bh=120e9, check_every=16, T=1)
    log(f"[gpu] 284b-miss-path hit rate over 128 steps: {rate:.3f}")


def _bf16_rne_bits(f32):
    """float32 array -> bf16 bits, round to nearest even (the definition, NaNs made quiet)."""
    u = f32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f32)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


@pytest.mark.parametrize("n,offset,scale", [(0, 0, 1.0), (1, 0, 1.0), (7, 0, 0.25),
                                            (8, 0, 1.0), (4096 * 3 + 5, 0, 1.0),
                                            (4096 * 3 + 5, 0, 0.1), (1000, 1, 0.3)])
def test_residual_bf16_exact(ctx, n, offset, scale):
    """x + scale*y rounded to bf16: bit-exact against the fp32 product and sum (numpy float32
    arithmetic) rounded to nearest even, on ragged sizes, a misaligned view (scalar path) and
    in place (out aliasing x)."""
    rng = np.random.default_rng(n + 17 * offset)
    xf = (rng.standard_normal(n + offset) * 4).astype(np.float32)
    xb = _bf16_rne_bits(xf)
    y = (rng.standard_normal(n + offset) * rng.choice([1e-3, 1.0, 300.0], n + offset)).astype(np.float32)
    if n > 10:
        xb[:4] = [0x7F80, 0xFF80, 0x7F7F, 0x0001]     # +inf, -inf, max finite, subnormal
        y[2] = 3.0e38                                  # overflows to inf
        y[5] = np.nan
    xs = (xb.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = _bf16_rne_bits((xs + np.float32(scale) * y)[offset:])
    xd = torch.from_numpy(xb.view(np.int16).copy()).to("cuda")
    yd = torch.from_numpy(y).to("cuda")
    out = torch.empty_like(xd)
    ft.residual_bf16(ctx, xd[offset:], yd[offset:], n, out[offset:], stream_ptr(), scale)
    ft.residual_bf16(ctx, xd[offset:], yd[offset:], n, xd[offset:], stream_ptr(), scale)
    torch.cuda.synchronize()
    for got in (out[offset:], xd[offset:]):
        g = got.cpu().numpy().view(np.uint16)
        nan_ref = np.isnan((ref.astype(np.uint32) << 16).view(np.float32))
        assert np.array_equal(g[~nan_ref], ref[~nan_ref])
        assert np.all(np.isnan((g[nan_ref].astype(np.uint32) << 16).view(np.float32)))


def _stack(ctx, tag, n_layers, **kw):
    layers = []
    for li in range(n_layers):
        cfg = synth.small_config(f"{tag}{li}", seed=91 + 7 * li, **kw)
        layers.append(layer_for(ctx, f"{tag}{li}", cfg=cfg, resident=False, n_slots=5,
                                max_tokens=2))
    return layers


def test_prefetch_layer_stack_matches_oracle(ctx):
    """Three chained miss-path layers (input of layer l+1 = bf16(x_l + g y_l), g = 2^-14 so
    that |g y| is about a third of |x| for these random weights), layer 0 prefetching for
    layer 1 (depth 2) and layer 1 for layer 2 (depth 3): after every call the slot tables
    equal the oracle's pools replaying the same steps and prefetches, the prefetch counts
    agree, and the outputs match the oracle.  The pools order experts by routing weight, an
    ordering the library takes on fp32 weights, so the oracle's weights enter the pools
    rounded to fp32 (a weight that underflows in fp32 ties at zero on both sides)."""
    Ls = _stack(ctx, "pfstack", 3, H=384, I=256, E=14, k=3, n_shared=1, code_dist="normal",
                router_sigma=1 / 20, zipf_c=0.7)
    depths = [2, 3]
    OLs = [L.oracle_layer() for L in Ls]
    pools = [policy.LruPool(L.cfg.E, L.n_slots) for L in Ls]
    for L in Ls:
        ft.set_bandwidth(L.handle, 1.0, 2.5)
        ft.force_q(L.handle, -1)
    ft.set_prefetch(Ls[0].handle, Ls[1].handle, depths[0])
    ft.set_prefetch(Ls[1].handle, Ls[2].handle, depths[1])
    n_pf = n_pf_hits = 0
    try:
        for s in range(20):
            T = 1 + s % 2
            xb = synth.gen_tokens(Ls[0].cfg, T, batch=500 + s)
            for li, L in enumerate(Ls):
                cfg = L.cfg
                st = ft.DecodeStats()
                y = run_decode(ctx, L, xb, st)
                xr = fp4.bf16_bits_to_f64(xb)
                r_idx, r_w, _, gap = moe.route(xr, OLs[li].router_w, OLs[li].router_b, cfg.k)
                assert np.all(gap >= 1e-6), "near-tie; choose another seed"
                res = pools[li].step(r_idx, r_w.astype(np.float32), 1.0, 2.5)
                e2s, s2e = ft.debug_tables(L.handle, cfg.E, L.n_slots)
                assert np.array_equal(e2s, res.e2s) and np.array_equal(s2e, res.s2e), (s, li)
                assert st.n_prefetch_hits == res.prefetch_hits, (s, li)
                assert (st.n_hits, st.n_streamed, st.n_host) == (
                    len(res.hits), len(res.streamed), len(res.host)), (s, li)
                if li + 1 < len(Ls):
                    nO = OLs[li + 1]
                    p_idx, p_w, _, pgap = moe.route(xr, nO.router_w, nO.router_b, Ls[li + 1].cfg.k)
                    assert np.all(pgap >= 1e-6), "near-tie in the prediction; choose another seed"
                    f = pools[li + 1].prefetch(p_idx, p_w.astype(np.float32), depths[li])
                    assert st.n_prefetched == len(f.admitted), (s, li)
                    n_pf += len(f.admitted)
                else:
                    assert st.n_prefetched == 0
                n_pf_hits += st.n_prefetch_hits
                if s % 3 == 0 or s == 19:
                    check_output(y, moe.moe_forward(OLs[li], xb)["y"], f"stack step {s} layer {li}")
                # the next layer's input: bf16(x + g y) on the device
                g = 2.0 ** -14
                xd = to_dev(xb)
                yd = torch.from_numpy(y).to("cuda")
                ft.residual_bf16(ctx, xd, yd, xd.numel(), xd, stream_ptr(), g)
                torch.cuda.synchronize()
                xn = xd.cpu().numpy().view(np.uint16).reshape(xb.shape)
                xs = (xb.astype(np.uint32) << 16).view(np.float32)
                assert np.array_equal(xn, _bf16_rne_bits(xs + np.float32(g) * y)), (s, li)
                xb = xn
    finally:
        ft.set_prefetch(Ls[0].handle, None, 0)
        ft.set_prefetch(Ls[1].handle, None, 0)
    assert n_pf > 0 and n_pf_hits > 0, (n_pf, n_pf_hits)
    log(f"[gpu] prefetch stack: {n_pf} prefetched, {n_pf_hits} prefetch hits")


def test_set_prefetch_rejects_bad_links(ctx):
    a, b = _stack(ctx, "pflink", 2, H=256, I=128, E=12, k=2, n_shared=0, code_dist="normal",
                  router_sigma=1 / 16)
    res = layer_for(ctx, "pfres", cfg=synth.small_config("pfres", seed=5, H=256, I=128, E=6,
                                                        k=2), resident=True, max_tokens=2)
    c = GpuLayer(ctx, synth.small_config("pflink_c", seed=6, H=256, I=128, E=12, k=2),
                 resident=False, n_slots=4, max_tokens=2)
    odd = GpuLayer(ctx, synth.small_config("pflink_h", seed=8, H=384, I=128, E=12, k=2),
                   resident=False, n_slots=4, max_tokens=2)
    try:
        for args in [(a.handle, a.handle, 1), (a.handle, b.handle, -1),
                     (a.handle, b.handle, b.n_slots + 1), (a.handle, res.handle, 1),
                     (res.handle, a.handle, 1), (a.handle, odd.handle, 1)]:
            with pytest.raises(ft.FtError) as e:
                ft.set_prefetch(*args)
            assert e.value.code == ft.FT_EINVAL, args
        ft.set_prefetch(a.handle, b.handle, 2)
        with pytest.raises(ft.FtError) as e:      # b already has a predecessor
            ft.set_prefetch(c.handle, b.handle, 1)
        assert e.value.code == ft.FT_EINVAL
        ft.set_prefetch(a.handle, c.handle, 1)    # relinking a moves its target
        ft.set_prefetch(b.handle, a.handle, 1)
        ft.set_prefetch(c.handle, b.handle, 1)    # b is free again
        c.close()                                  # destroying c unlinks a -> c and c -> b
        ft.set_bandwidth(a.handle, 1.0, 1.0)
        ft.force_q(a.handle, -1)
        st = ft.DecodeStats()
        run_decode(ctx, a, synth.gen_tokens(a.cfg, 1, batch=3), st)
        assert st.n_prefetched == 0
        ft.set_prefetch(b.handle, None, 0)
    finally:
        c.close()
        odd.close()


def _pinned_aligned(nbytes):
    raw = torch.empty(nbytes + 4096, dtype=torch.uint8, pin_memory=True)
    off = (-raw.data_ptr()) % 4096
    return raw, raw[off:off + nbytes]


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_disk_tier_matches_oracle(ctx, tmp_path, fmt):
    """Three tiers: the layer's blobs in an FTW file, 7 host-memory slots over it, 5 VRAM
    slots.  After every call the VRAM tables and the host-memory tier's tables equal the
    oracle's two pools replaying the same calls, the disk reads are the oracle's loads, and
    the outputs match the oracle."""
    extra = dict(fmt=synth.NVFP4, nv_tensor_scale=1 / 64) if fmt == "nvfp4" else {}
    cfg = synth.small_config(f"disk{fmt}", seed=83, H=384, I=256, E=14, k=3, n_shared=1,
                             code_dist="normal", router_sigma=1 / 20, zipf_c=0.5, **extra)
    L = layer_for(ctx, f"disk{fmt}", cfg=cfg, resident=False, n_slots=5, max_tokens=2)
    path = str(tmp_path / "layer.ftw")
    # the file holds the routed experts and the shared one (packed like the layer's)
    store = np.zeros((cfg.E + 1) * L.stride, dtype=np.uint8)
    store[:cfg.E * L.stride] = L.host_blobs.numpy()
    ft.pack_expert_into(cfg.fmt, cfg.H, cfg.I, synth.gen_expert(cfg, 0, shared=True),
                        store[cfg.E * L.stride:])
    ft.ftw_write(path, cfg.fmt, cfg.H, cfg.I, cfg.E, 1, store, L.stride)
    f = ft.Ftw(path)
    n_ram = 7
    keep, ram = _pinned_aligned(n_ram * L.stride)
    with pytest.raises(ft.FtError) as e:
        ft.set_disk_tier(L.handle, f, ram, 5)          # below max_tokens * k
    assert e.value.code == ft.FT_EINVAL
    ft.set_disk_tier(L.handle, f, ram, n_ram)
    OL = L.oracle_layer()
    vram, host = policy.LruPool(cfg.E, L.n_slots), policy.LruPool(cfg.E, n_ram)
    ft.set_bandwidth(L.handle, 1.0, 2.5)
    ft.force_q(L.handle, -1)
    reads = 0
    try:
        for s in range(24):
            T = 1 + s % 2
            x = synth.gen_tokens(cfg, T, batch=700 + s)
            st = ft.DecodeStats()
            y = run_decode(ctx, L, x, st)
            r_idx, r_w, _, gap = moe.route(fp4.bf16_bits_to_f64(x), OL.router_w, OL.router_b, cfg.k)
            assert np.all(gap >= 1e-6), "near-tie; choose another seed"
            res = vram.step(r_idx, r_w.astype(np.float32), 1.0, 2.5)
            tr = policy.tier_step(host, res.misses)
            e2s, s2e = ft.debug_tables(L.handle, cfg.E, L.n_slots)
            assert np.array_equal(e2s, res.e2s) and np.array_equal(s2e, res.s2e), s
            e2r, r2e = ft.debug_host_tier(L.handle, cfg.E, n_ram)
            assert np.array_equal(e2r, tr.e2s) and np.array_equal(r2e, tr.s2e), s
            assert (st.n_disk, st.n_streamed, st.n_host) == (
                len(tr.loaded), len(res.streamed), len(res.host)), s
            reads += st.n_disk
            if s % 3 == 0 or s == 23:
                check_output(y, moe.moe_forward(OL, x)["y"], f"disk tier step {s}")
    finally:
        ft.set_disk_tier(L.handle, None, None, 0)
        f.close()
    assert reads > n_ram, reads          # the tier was refilled from disk
    log(f"[gpu] disk tier {fmt}: {reads} blob reads over 24 calls")


@pytest.mark.parametrize("T", [1, 3, 8])
def test_decode_more_than_256_experts(ctx, T):
    """E = 300 (> 256): the top-k paths for wide expert sets (16 logits per lane), resident
    decode at T = 1, 3 and 8 and ft_route against the oracle."""
    cfg = synth.small_config("wide300", seed=301, H=256, I=128, E=300, k=8, n_shared=1,
                             code_dist="normal", router_sigma=1 / 16)
    L = layer_for(ctx, "wide300", cfg=cfg, max_tokens=16)
    OL = L.oracle_layer()
    x = synth.gen_tokens(cfg, T, batch=31 + T)
    idx, w = run_route(ctx, L, x)
    ref = moe.moe_forward(OL, x)
    check_routing(idx, w, ref)
    check_output(run_decode(ctx, L, x), ref["y"], f"E=300 T={T}")


def test_miss_path_more_than_256_experts(ctx):
    """The one-launch miss-path routing with 16 logits per lane (E = 300), tables bit-exact."""
    cfg = synth.small_config("wide300m", seed=302, H=256, I=128, E=300, k=8, n_shared=1,
                             code_dist="normal", router_sigma=1 / 16, zipf_c=0.9)
    L = layer_for(ctx, "wide300m", cfg=cfg, resident=False, n_slots=20, max_tokens=2)
    _miss_sequence(ctx, L, steps=12, bp=1.0, bh=2.5, check_every=3, T=2)


def test_miss_path_sixteen_tokens(ctx):
    """The miss path at its largest call (T = 16): the one-launch routing with 16 token rows,
    long work lists, host experts with up to 16 token columns; tables bit-exact each call."""
    cfg = synth.small_config("miss16", seed=87, H=384, I=256, E=24, k=4, n_shared=1,
                             code_dist="normal", router_sigma=1 / 20, zipf_c=0.6)
    L = layer_for(ctx, "miss16", cfg=cfg, resident=False, n_slots=10, max_tokens=16)
    _miss_sequence(ctx, L, steps=10, bp=1.0, bh=2.0, check_every=2, T=16)


@pytest.mark.parametrize("nbytes", [(1 << 20), (1 << 20) + 16, (3 << 20) + 1008])
def test_hbm_read_probe(ctx, nbytes):
    """The read probe over buffers that are and are not whole 1 KB blocks (the LDS form reads
    the tail with register loads): a finite positive rate, and bad sizes are refused."""
    log(f"[gpu] read probe over {nbytes} bytes")
    buf = torch.ones((nbytes + 15) // 16 * 4, dtype=torch.int32, device="cuda")
    v = ft.probe_hbm_read(ctx, buf, nbytes, reps=2)
    torch.cuda.synchronize()
    assert np.isfinite(v) and v > 0
    with pytest.raises(ft.FtError):
        ft.probe_hbm_read(ctx, buf, nbytes - 8, reps=1)


def test_miss_path_alternating_streams(ctx):
    """Miss-path calls on one layer alternate between two streams with no host wait between
    them: each call orders its device work after the previous call's (which still reads the
    layer's pinned staging), so every output matches the oracle."""
    cfg = synth.small_config("missstreams", seed=91, H=384, I=256, E=16, k=3, n_shared=1,
                             code_dist="normal", router_sigma=1 / 20, zipf_c=0.7)
    L = layer_for(ctx, "missstreams", cfg=cfg, resident=False, n_slots=5, max_tokens=2)
    OL = L.oracle_layer()
    ft.set_bandwidth(L.handle, 1.0, 2.5)
    ft.force_q(L.handle, -1)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    xs = [synth.gen_tokens(cfg, 2, batch=300 + s) for s in range(12)]
    xd = [to_dev(x) for x in xs]
    ys = [torch.empty((2, cfg.H), dtype=torch.float32, device="cuda") for _ in xs]
    torch.cuda.synchronize()
    for s in range(len(xs)):
        ft.moe_decode(ctx, L.handle, xd[s], 2, ys[s], streams[s % 2].cuda_stream, None)
    torch.cuda.synchronize()
    for s, x in enumerate(xs):
        _, _, _, gap = moe.route(fp4.bf16_bits_to_f64(x), OL.router_w, OL.router_b, cfg.k)
        assert np.all(gap >= 1e-6), "near-tie; choose another seed"
        check_output(ys[s].cpu().numpy(), moe.moe_forward(OL, x)["y"], f"alternating step {s}")
