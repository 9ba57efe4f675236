"""GPU parity of the prefill path (routing, permutation, grouped GEMMs, unpermute-combine)."""
import sys

import numpy as np
import pytest

from mxfp4_expert_layer_amd import synth
from oracle import fp4, moe, perm

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


def layer_for(ctx, name, cfg, **kw):
    if name not in _layers:
        log(f"[gpu] building layer {name} {cfg.H}x{cfg.I} E={cfg.E} {cfg.fmt}")
        _layers[name] = GpuLayer(ctx, cfg, max_tokens=1, **kw)
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
    if ties:
        ref = moe.moe_forward(OL, x, idx=idx)
    check_output(y, ref["y"], name)


def test_prefill_is_deterministic(ctx):
    name, fmt, H, I, E, k, T = SMALL[1]
    cfg = synth.small_config(name, seed=H + E, H=H, I=I, E=E, k=k, fmt=fmt, code_dist="normal",
                             router_sigma=0.5 / np.sqrt(H), nv_tensor_scale=1 / 64)
    L = layer_for(ctx, name, cfg)
    x = synth.gen_tokens(cfg, T, batch=9)
    a, _ = run_prefill(ctx, L, x)
    b, _ = run_prefill(ctx, L, x)
    assert np.array_equal(a, b)


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


def test_prefill_753b_layer(ctx):
    """The 753B-class NVFP4 layer at T = 4096: routing and the full permutation checked
    exactly, outputs checked on sampled tokens (the oracle evaluates those tokens only)."""
    cfg = synth.CONFIGS["cfg5"]
    L = layer_for(ctx, "cfg5", cfg, threads=16)
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
    assert counts.sum() == T * cfg.k
    sample = np.array([0, 1377, 2900, T - 1])
    ref = moe.moe_forward(OL, x[sample], idx=idx[sample])
    check_output(y[sample], ref["y"], "753b-class sampled tokens")
    assert np.all(np.isfinite(y))
