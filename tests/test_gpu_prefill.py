"""GPU parity of the prefill path (routing, permutation, grouped GEMMs, unpermute-combine)."""
import sys

import numpy as np
import pytest

from mxfp4_expert_layer_amd import synth
from oracle import fp4, moe, mxq, perm

import tiled
from gpu_util import check_mx_quant, check_output, check_routing, to_dev

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


def layer_for(ctx, name, cfg, **kw):
    if name not in _layers:
        log(f"[gpu] building layer {name} {cfg.H}x{cfg.I} E={cfg.E} {cfg.fmt}")
        # every prefill layer also carries the weights of the scaled-FP4 mode
        _layers[name] = GpuLayer(ctx, cfg, max_tokens=1, prefill_mxfp4=True, **kw)
    return _layers[name]


def run_prefill(ctx, L, x_bits, mode=ft.FT_PREFILL_EXACT):
    T = x_bits.shape[0]
    nbytes = ft.moe_prefill_workspace_size(L.handle, T, mode)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((T, L.cfg.H), dtype=torch.float32, device="cuda")
    ft.moe_prefill(ctx, L.handle, to_dev(x_bits), T, y, mode, ws, nbytes, stream_ptr())
    torch.cuda.synchronize()
    return y.cpu().numpy(), ws


def prefill_state(L, ws, T):
    k, E = L.cfg.k, L.cfg.E
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty((T, k), dtype=torch.int32, device="cuda")
    s = stream_ptr()
    ft.debug_prefill_route(L.handle, ws, T, idx, w, s)
    ft.debug_prefill_perm(L.handle, ws, T, counts, offsets, pos, s)
    torch.cuda.synchronize()
    return (idx.cpu().numpy(), w.cpu().numpy(), counts.cpu().numpy(), offsets.cpu().numpy(),
            pos.cpu().numpy())


def prefill_quant(L, ws, T, which):
    """The MXFP4 operands of the last scaled-FP4 call: which 0 tokens, 1 permuted h."""
    rows = T if which == 0 else T * L.cfg.k
    K = L.cfg.H if which == 0 else L.cfg.I
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
    ft.debug_prefill_quant(L.handle, ws, T, which, codes, scales, stream_ptr())
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def prefill_weights(L, e):
    """(codes, scales) of gate, up, down in the MXFP4 blob the scaled-FP4 mode uses for e."""
    cfg = L.cfg
    nb = ft.blob_bytes("mxfp4", cfg.H, cfg.I)
    out = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ft.debug_prefill_weights(L.handle, e, out, stream_ptr())
    torch.cuda.synchronize()
    blob = out.cpu().numpy()
    hdr = blob[:16].view(np.int32)
    assert hdr[0] == 0x31425446 and hdr[1] == ft.FT_MXFP4 and hdr[2] == cfg.H and hdr[3] == cfg.I
    return tiled.matrices(blob, "mxfp4", cfg.H, cfg.I)


def check_s1_weights(L, OL, e, threads=1, got=None):
    """The expert's MXFP4 weights against the oracle's requantisation of its exact weights:
    codes and scales bit-exact for a transcoded NVFP4 expert, values for an MXFP4 pool blob
    (requantising keeps an MXFP4 block's values but may re-express its codes).  Returns the
    oracle's requantised weights (gate, up, down) as float64."""
    from concurrent.futures import ThreadPoolExecutor
    ws = moe.expert_weights(OL, OL.expert(e))
    with ThreadPoolExecutor(max_workers=max(1, threads)) as pool:
        qs = list(pool.map(mxq.quantize, ws))
    if got is None:
        got = prefill_weights(L, e)
    out = []
    for m, ((c, s), (gc, gs)) in enumerate(zip(qs, got)):
        if L.cfg.fmt == synth.NVFP4:
            assert np.array_equal(gs, s.astype(np.uint8)), f"expert {e} matrix {m}: scales"
            assert np.array_equal(gc, mxq.pack_codes(c)), f"expert {e} matrix {m}: codes"
        deq = mxq.dequantize(c, s)
        assert np.array_equal(fp4.dequant_mxfp4(gc, gs), deq), f"expert {e} matrix {m}: values"
        out.append(deq)
    return out


def _check_perm(idx, counts, offsets, pos, E):
    """Permutation bit-exact against the oracle's, applied to the GPU's own routing."""
    r_counts, r_off, r_pos, _ = perm.permutation(idx, E)
    assert np.array_equal(counts, r_counts)
    assert np.array_equal(offsets, r_off)
    assert np.array_equal(pos, r_pos)


SMALL = [
    # name, fmt, H, I, E, k, T
    ("pf_nv_a", synth.NVFP4, 512, 256, 12, 3, 300),
    ("pf_nv_b", synth.NVFP4, 1024, 384, 37, 5, 777),
    ("pf_mx_a", synth.MXFP4, 768, 512, 20, 4, 513),
    ("pf_nv_one", synth.NVFP4, 256, 128, 6, 2, 1),
    ("pf_mx_wide", synth.MXFP4, 256, 128, 300, 8, 200),   # E > 256: two router expert groups
    # about 370 rows per expert: every expert spans two 256-row blocks, the second partial
    ("pf_nv_deep", synth.NVFP4, 256, 128, 6, 2, 1100),
    # twelve 128-K chunks: three passes of the scaled-FP4 gate/up GEMM's four-step loop
    ("pf_nv_k12", synth.NVFP4, 1536, 256, 10, 3, 600),
    # one expert takes every token: three row blocks of 256, 256 and 1 rows
    ("pf_mx_e1", synth.MXFP4, 256, 128, 1, 1, 513),
    # sixteen choices per token (the largest k), 303 tokens: a partial last top-k workgroup
    # and permutation block
    ("pf_mx_k16", synth.MXFP4, 256, 128, 40, 16, 303),
]


@pytest.mark.parametrize("name,fmt,H,I,E,k,T", SMALL)
def test_prefill_matches_oracle(ctx, name, fmt, H, I, E, k, T):
    cfg = synth.small_config(name, seed=H + E, H=H, I=I, E=E, k=k, fmt=fmt, code_dist="normal",
                             router_sigma=0.5 / np.sqrt(H), nv_tensor_scale=1 / 64)
    L = layer_for(ctx, name, cfg)
    x = synth.gen_tokens(cfg, T, batch=5)
    log(f"[gpu] prefill {name} T={T}")
    y, ws = run_prefill(ctx, L, x)
    idx, w, counts, offsets, pos = prefill_state(L, ws, T)
    OL = L.oracle_layer()
    ref = moe.moe_forward(OL, x)
    ties = check_routing(idx, w, ref)
    _check_perm(idx, counts, offsets, pos, E)
    if name == "pf_nv_deep":
        assert int(np.asarray(counts).min()) > 256, counts   # every expert has a second block
    if ties:
        ref = moe.moe_forward(OL, x, idx=idx)
    check_output(y, ref["y"], name)


def test_prefill_repeat_agrees(ctx):
    """The exact mode combines the k expert outputs of a token by fp32 atomic adds into y, so
    the summation order (and only that) may differ between calls: two calls agree to a few
    fp32 roundings of k = 5 terms (2^-24 each, relative to the largest output), and every
    intermediate (routing, permutation) is identical."""
    name, fmt, H, I, E, k, T = SMALL[1]
    cfg = synth.small_config(name, seed=H + E, H=H, I=I, E=E, k=k, fmt=fmt, code_dist="normal",
                             router_sigma=0.5 / np.sqrt(H), nv_tensor_scale=1 / 64)
    L = layer_for(ctx, name, cfg)
    x = synth.gen_tokens(cfg, T, batch=9)
    a, wsa = run_prefill(ctx, L, x)
    sa = prefill_state(L, wsa, T)
    b, wsb = run_prefill(ctx, L, x)
    sb = prefill_state(L, wsb, T)
    for u, v in zip(sa, sb):
        assert np.array_equal(u, v)
    assert np.max(np.abs(a - b)) <= k * 2.0 ** -22 * np.max(np.abs(a))


def test_prefill_rejects_bad_calls(ctx):
    name, fmt, H, I, E, k, T = SMALL[0]
    cfg = synth.small_config(name, seed=H + E, H=H, I=I, E=E, k=k, fmt=fmt, code_dist="normal",
                             router_sigma=0.5 / np.sqrt(H), nv_tensor_scale=1 / 64)
    L = layer_for(ctx, name, cfg)
    with pytest.raises(ft.FtError) as e:
        ft.moe_prefill_workspace_size(L.handle, 0, ft.FT_PREFILL_EXACT)
    assert e.value.code == ft.FT_EINVAL
    nbytes = ft.moe_prefill_workspace_size(L.handle, 8, ft.FT_PREFILL_EXACT)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((8, H), dtype=torch.float32, device="cuda")
    x = to_dev(synth.gen_tokens(cfg, 8))
    with pytest.raises(ft.FtError) as e:
        ft.moe_prefill(ctx, L.handle, x, 8, y, ft.FT_PREFILL_EXACT, ws, nbytes - 256, stream_ptr())
    assert e.value.code == ft.FT_EINVAL
    with pytest.raises(ft.FtError) as e:
        ft.moe_prefill_workspace_size(L.handle, 8, 7)
    assert e.value.code == ft.FT_EINVAL
    # an NVFP4 layer created without FT_LAYER_PREFILL_MXFP4 has no MXFP4 weights
    bare = GpuLayer(ctx, cfg, max_tokens=1)
    try:
        with pytest.raises(ft.FtError) as e:
            ft.moe_prefill_workspace_size(bare.handle, 8, ft.FT_PREFILL_MXFP4)
        assert e.value.code == ft.FT_ESTATE
        with pytest.raises(ft.FtError) as e:
            ft.debug_prefill_weights(bare.handle, 0, ws, stream_ptr())
        assert e.value.code == ft.FT_ESTATE
    finally:
        bare.close()


def expert_cover_sample(idx, E, n=256, seed=0):
    """A seeded sample of n tokens that routes to every expert: for each expert the last token
    routed to it (its row is the last row of the expert's last row block, in every block size
    the grouped GEMMs use), then first tokens of experts, then random tokens."""
    rng = np.random.default_rng(seed)
    T = idx.shape[0]
    last, first = [], []
    for e in range(E):
        tt = np.nonzero((idx == e).any(axis=1))[0]
        if len(tt):
            last.append(int(tt[-1]))
            first.append(int(tt[0]))
    pick = set(last)
    for t in rng.permutation(first):
        if len(pick) >= n:
            break
        pick.add(int(t))
    while len(pick) < n:
        pick.add(int(rng.integers(0, T)))
    sample = np.array(sorted(pick))
    assert set(np.unique(idx[sample])) == set(np.unique(idx))
    return sample


def test_prefill_753b_layer(ctx):
    """The 753B-class NVFP4 layer at T = 4096: routing and the full permutation checked
    exactly; outputs checked on a seeded sample of 256 tokens that routes to all 160 experts,
    including each expert's last row (the oracle evaluates those tokens only)."""
    cfg = synth.CONFIGS["753b"]
    L = layer_for(ctx, "753b", cfg, threads=16)
    T = 4096
    x = synth.gen_tokens(cfg, T, batch=0)
    log("[gpu] prefill 753b-class T=4096")
    y, ws = run_prefill(ctx, L, x)
    idx, w, counts, offsets, pos = prefill_state(L, ws, T)
    OL = L.oracle_layer()
    xr = fp4.bf16_bits_to_f64(x)
    r_idx, r_w, logits, gap = moe.route(xr, OL.router_w, OL.router_b, cfg.k)
    check_routing(idx, w, dict(idx=r_idx, w=r_w, logits=logits, gap=gap))
    _check_perm(idx, counts, offsets, pos, cfg.E)
    assert counts.sum() == T * cfg.k and np.all(counts > 0)
    sample = expert_cover_sample(idx, cfg.E)
    log(f"[gpu] oracle on {len(sample)} sampled tokens ({len(np.unique(idx[sample]))} experts)")
    ref = moe.moe_forward(OL, x[sample], idx=idx[sample], threads=16)
    check_output(y[sample], ref["y"], "753b-class sampled tokens")
    assert np.all(np.isfinite(y))


# ---- scaled-FP4 mode (both MFMA operands MXFP4) ----------------------------------------------

def _small_layer(ctx, name, fmt, H, I, E, k):
    cfg = synth.small_config(name, seed=H + E, H=H, I=I, E=E, k=k, fmt=fmt, code_dist="normal",
                             router_sigma=0.5 / np.sqrt(H), nv_tensor_scale=1 / 64)
    return cfg, layer_for(ctx, name, cfg)


@pytest.mark.parametrize("name,fmt,H,I,E,k,T", SMALL)
def test_prefill_mxfp4_matches_oracle(ctx, name, fmt, H, I, E, k, T):
    """Routing and permutation exact, quantised tokens and weights bit-exact, quantised h
    equal up to fp32-vs-fp64 boundary cases, y within the output bounds of the oracle's
    "mxfp4" mode."""
    cfg, L = _small_layer(ctx, name, fmt, H, I, E, k)
    x = synth.gen_tokens(cfg, T, batch=5)
    log(f"[gpu] prefill mxfp4 {name} T={T}")
    y, ws = run_prefill(ctx, L, x, mode=ft.FT_PREFILL_MXFP4)
    idx, w, counts, offsets, pos = prefill_state(L, ws, T)
    OL = L.oracle_layer()
    ref = moe.moe_forward(OL, x, mode="mxfp4")
    ties = check_routing(idx, w, ref)
    _check_perm(idx, counts, offsets, pos, E)
    xr = fp4.bf16_bits_to_f64(x)
    xc, xs = prefill_quant(L, ws, T, 0)
    check_mx_quant(xc, xs, xr, "tokens", exact=True)
    hc, hs = prefill_quant(L, ws, T, 1)
    xq = mxq.quantize_dequant(xr)
    ndiff = 0
    for e in np.unique(idx):
        wg, wu, _ = check_s1_weights(L, OL, int(e))
        tt, jj = np.nonzero(idx == e)
        rows = pos[tt, jj]
        ndiff += check_mx_quant(hc[rows], hs[rows], moe.swiglu_hidden(xq[tt], wg, wu), f"h of {e}")
    log(f"[gpu] {name}: {ndiff} h decisions at fp32/fp64 boundaries")
    if ties:
        ref = moe.moe_forward(OL, x, idx=idx, mode="mxfp4")
    check_output(y, ref["y"], name)


def test_prefill_mxfp4_down_blocks_per_workgroup(ctx):
    """More down-GEMM blocks than resident workgroups (H = 6016: 24 feature blocks, the last
    one half outside the matrix), so workgroups take a second block and the first chunks of
    that block load during the first block's epilogue; the whole output is checked."""
    name, fmt, H, I, E, k, T = "pf_persist", synth.MXFP4, 6016, 256, 6, 2, 1200
    cfg, L = _small_layer(ctx, name, fmt, H, I, E, k)
    x = synth.gen_tokens(cfg, T, batch=11)
    log(f"[gpu] prefill mxfp4 {name} T={T}")
    y, ws = run_prefill(ctx, L, x, mode=ft.FT_PREFILL_MXFP4)
    idx, w, counts, offsets, pos = prefill_state(L, ws, T)
    assert ((counts + 255) // 256).sum() * ((H + 255) // 256) > 256
    OL = L.oracle_layer()
    ref = moe.moe_forward(OL, x, mode="mxfp4", threads=16)
    ties = check_routing(idx, w, ref)
    _check_perm(idx, counts, offsets, pos, E)
    if ties:
        ref = moe.moe_forward(OL, x, idx=idx, mode="mxfp4", threads=16)
    check_output(y, ref["y"], name)


def test_prefill_mxfp4_token_quantiser_edge_cases(ctx):
    """Blocks of zeros, -0, bf16 subnormals, values at every rounding midpoint, and very
    large and very small magnitudes are quantised exactly as the oracle does."""
    name, fmt, H, I, E, k, T = SMALL[2]
    cfg, L = _small_layer(ctx, name, fmt, H, I, E, k)
    x = synth.gen_tokens(cfg, 8, batch=3).copy()
    xr = fp4.bf16_bits_to_f64(x)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 4.0])
    xr[0, :] = 0.0
    xr[1, :32] = -0.0
    xr[2, :32] = np.ldexp(np.arange(1, 33), -133)           # subnormal in bf16 and fp32
    xr[2, 32:64] = np.ldexp(np.arange(-16, 16), -126)      # around the smallest normal
    xr[3, :len(ties)] = ties * 2.0 ** -5
    xr[3, 32:32 + len(ties)] = -ties * 2.0 ** 7
    xr[4, :] = xr[4, :] * 2.0 ** 100
    xr[5, :] = xr[5, :] * 2.0 ** -100
    xr[6, 0] = 2.0 ** 127
    xb = synth.f32_to_bf16_bits(xr.astype(np.float32))
    assert np.array_equal(fp4.bf16_bits_to_f64(xb), xr.astype(np.float32).astype(np.float64))
    _, ws = run_prefill(ctx, L, xb, mode=ft.FT_PREFILL_MXFP4)
    xc, xs = prefill_quant(L, ws, 8, 0)
    check_mx_quant(xc, xs, fp4.bf16_bits_to_f64(xb), "edge-case tokens", exact=True)


def test_prefill_mxfp4_is_deterministic(ctx):
    name, fmt, H, I, E, k, T = SMALL[1]
    cfg, L = _small_layer(ctx, name, fmt, H, I, E, k)
    x = synth.gen_tokens(cfg, T, batch=9)
    a, _ = run_prefill(ctx, L, x, mode=ft.FT_PREFILL_MXFP4)
    b, _ = run_prefill(ctx, L, x, mode=ft.FT_PREFILL_MXFP4)
    assert np.array_equal(a, b)


def test_prefill_mxfp4_753b_layer(ctx):
    """The 753B-class NVFP4 layer at T = 4096 in the scaled-FP4 mode: routing, permutation and
    all quantised tokens exact; all 160 transcoded experts bit-exact (codes and scales); the
    quantised h rows and the outputs of a seeded 256-token sample that routes to every expert
    (each expert's last row included) against the oracle's "mxfp4" mode.  Each expert's
    weights are requantised by the oracle once: the transcode check and the oracle's forward
    pass use the same values."""
    import threading

    cfg = synth.CONFIGS["753b"]
    L = layer_for(ctx, "753b", cfg, threads=16)
    T = 4096
    x = synth.gen_tokens(cfg, T, batch=1)
    log("[gpu] prefill mxfp4 753b-class T=4096")
    y, ws = run_prefill(ctx, L, x, mode=ft.FT_PREFILL_MXFP4)
    idx, w, counts, offsets, pos = prefill_state(L, ws, T)
    OL = L.oracle_layer()
    xr = fp4.bf16_bits_to_f64(x)
    r_idx, r_w, logits, gap = moe.route(xr, OL.router_w, OL.router_b, cfg.k)
    check_routing(idx, w, dict(idx=r_idx, w=r_w, logits=logits, gap=gap))
    _check_perm(idx, counts, offsets, pos, cfg.E)
    xc, xs = prefill_quant(L, ws, T, 0)
    check_mx_quant(xc, xs, xr, "tokens", exact=True)
    hc, hs = prefill_quant(L, ws, T, 1)
    sample = expert_cover_sample(idx, cfg.E, seed=1)
    xq = mxq.quantize_dequant(xr[sample])
    # the GPU's MXFP4 blobs of all experts, read before the oracle's worker threads start
    blobs = {e: prefill_weights(L, e) for e in range(cfg.E)}
    lock = threading.Lock()
    done, ndiff = [], [0]

    def weights_fn(e):
        deq = check_s1_weights(L, OL, e, got=blobs.pop(e))
        # h of the sampled rows routed to e, from the oracle's own quantised operands
        tt, jj = np.nonzero(idx[sample] == e)
        nd = check_mx_quant(hc[pos[sample[tt], jj]], hs[pos[sample[tt], jj]],
                            moe.swiglu_hidden(xq[tt], deq[0], deq[1]), f"h of {e}")
        with lock:
            done.append(e)
            ndiff[0] += nd
            if len(done) % 32 == 0:
                log(f"[gpu] 753b mxfp4: {len(done)} experts checked")
        return tuple(deq)

    log(f"[gpu] oracle on {len(sample)} sampled tokens, all {cfg.E} experts requantised")
    ref = moe.moe_forward(OL, x[sample], idx=idx[sample], mode="mxfp4", threads=16,
                          weights_fn=weights_fn)
    assert sorted(done) == list(range(cfg.E))
    log(f"[gpu] 753b mxfp4: {ndiff[0]} h decisions at fp32/fp64 boundaries")
    check_output(y[sample], ref["y"], "753b-class mxfp4 sampled tokens")
    assert np.all(np.isfinite(y))
