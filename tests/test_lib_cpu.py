"""libft on the CPU: symbols, blob layout, split rule and the host expert FFN (no GPU calls)."""
import os
import re

import numpy as np
import pytest

from mxfp4_expert_layer_amd import synth
from oracle import fp4, moe, policy

import tiled

ft = pytest.importorskip("mxfp4_expert_layer_amd.ft", reason="libft.so not built")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ft.h")).read()
    return set(re.findall(r"FT_API\s+(?:const\s+char\s*\*|int)\s+(ft_\w+)\s*\(", src))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 19
    for n in names:
        assert hasattr(ft.lib, n), n
    assert names == set(ft.DECLARED)


def test_qstar_split_matches_oracle():
    for m in range(0, 13):
        for bp, bh in [(49.0, 53.8), (52.7, 77.3), (25.1, 63.2), (11.8, 47.5), (60, 50), (1, 2)]:
            assert ft.qstar_split(m, bp, bh) == pytest.approx(policy.qstar_split(m, bp, bh))
    with pytest.raises(ft.FtError) as e:
        ft.qstar_split(-1, 1.0, 1.0)
    assert e.value.code == ft.FT_EINVAL
    with pytest.raises(ft.FtError):
        ft.qstar_split(1, 0.0, 1.0)


def test_blob_bytes_and_alignment():
    assert ft.blob_bytes("mxfp4", 4096, 2048) == 4096 + 13_369_344
    assert ft.blob_bytes("mxfp4", 2048, 512) % 4096 == 0
    with pytest.raises(ft.FtError):
        ft.blob_bytes("mxfp4", 100, 128)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_pack_roundtrip(fmt):
    cfg = synth.small_config(seed=4, H=256, I=128, fmt=fmt)
    ex = synth.gen_expert(cfg, 0)
    blob = ft.pack_expert(fmt, cfg.H, cfg.I, ex)
    assert blob.size % 4096 == 0
    hdr = blob[:16].view(np.int32)
    assert hdr[0] == 0x31425446 and hdr[2] == 256 and hdr[3] == 128
    # sub-tensors start on 4096-byte boundaries in the order g codes, g scales, u..., d...
    sb = 64 if fmt == "mxfp4" else 128
    sizes = [128 * 256 // 2, (128 // 16) * 2 * sb] * 2 + [256 * 128 // 2, 16 * 1 * sb]
    offs, o = [], 4096
    for s in sizes:
        offs.append(o)
        o = (o + s + 4095) // 4096 * 4096
    assert o == blob.size
    assert (offs, o) == tiled.blob_offsets(fmt, cfg.H, cfg.I)
    mats = tiled.matrices(blob, fmt, cfg.H, cfg.I)
    for (c, s), (cn, sn) in zip(mats, [("gate_codes", "gate_scales"), ("up_codes", "up_scales"),
                                       ("down_codes", "down_scales")]):
        assert np.array_equal(c, getattr(ex, cn))
        assert np.array_equal(s, getattr(ex, sn))


@pytest.mark.parametrize("scalar", [False, True])
@pytest.mark.parametrize("fmt,T", [("mxfp4", 1), ("mxfp4", 3), ("nvfp4", 2)])
def test_host_expert_ffn_matches_oracle(fmt, T, scalar, monkeypatch):
    """Both host paths (AVX-512 BF16 where the CPU has it, and the scalar one)."""
    monkeypatch.setenv("FT_HOST_SCALAR", "1" if scalar else "0")
    cfg = synth.small_config(seed=8, H=256, I=128, fmt=fmt, code_dist="normal",
                             nv_tensor_scale=1 / 64)
    ex = synth.gen_expert(cfg, 1)
    blob = ft.pack_expert(fmt, cfg.H, cfg.I, ex)
    x = synth.gen_tokens(cfg, T)
    y = ft.host_expert_ffn(fmt, cfg.H, cfg.I, blob, x)

    class _L:  # duck-typed layer for the oracle's expert_weights
        pass
    L = _L()
    L.cfg = cfg
    wg, wu, wd = moe.expert_weights(L, ex)
    ref = moe.swiglu_ffn(fp4.bf16_bits_to_f64(x), wg, wu, wd)
    assert moe.rel_l2(y, ref) <= 1e-3
    assert np.max(np.abs(y - ref)) <= 1e-2 * np.max(np.abs(ref))


def test_bad_arguments_return_einval():
    with pytest.raises(ft.FtError) as e:
        ft.host_expert_ffn("mxfp4", 256, 128, np.zeros(16, np.uint8), np.zeros((1, 256), np.uint16))
    assert e.value.code == ft.FT_EINVAL          # blob header mismatch
    with pytest.raises(ft.FtError) as e:
        ft.pack_expert("mxfp4", 250, 128, synth.gen_expert(synth.small_config(H=256, I=128), 0))
    assert e.value.code == ft.FT_EINVAL


def test_host_expert_ffn_nan_scale_propagates():
    """E8M0 code 255 is NaN: the outputs that depend on it are NaN (scalar path taken)."""
    cfg = synth.small_config(seed=8, H=256, I=128, code_dist="normal")
    ex = synth.gen_expert(cfg, 2)
    ex.down_scales = ex.down_scales.copy()
    ex.down_scales[5, 1] = 255
    blob = ft.pack_expert("mxfp4", cfg.H, cfg.I, ex)
    y = ft.host_expert_ffn("mxfp4", cfg.H, cfg.I, blob, synth.gen_tokens(cfg, 1))

    class _L:
        pass
    L = _L()
    L.cfg = cfg
    wg, wu, wd = moe.expert_weights(L, ex)
    ref = moe.swiglu_ffn(fp4.bf16_bits_to_f64(synth.gen_tokens(cfg, 1)), wg, wu, wd)
    assert np.array_equal(np.isnan(y), np.isnan(ref)) and np.isnan(y[0, 5])
    fin = ~np.isnan(ref)
    assert moe.rel_l2(y[fin], ref[fin]) <= 1e-3


def test_makespan_split_matches_oracle():
    """The library's makespan variant against the oracle's on a grid that includes the
    pages' four measured bandwidth pairs, and its argument checks."""
    pairs = [(49.0, 53.8), (52.7, 77.3), (25.1, 63.2), (11.8, 47.5), (60.0, 50.0), (1.0, 2.0)]
    rng = np.random.default_rng(3)
    pairs += [(float(a), float(b)) for a, b in rng.uniform(1.0, 100.0, size=(200, 2))]
    for Bp, Bh in pairs:
        for m in range(0, 17):
            assert ft.qstar_split_makespan(m, Bp, Bh) == policy.qstar_makespan(m, Bp, Bh), (m, Bp, Bh)
    for bad in ((-1, 1.0, 1.0), (1, 0.0, 1.0), (1, 1.0, 0.0), (1, float("nan"), 1.0)):
        with pytest.raises(ft.FtError) as e:
            ft.qstar_split_makespan(*bad)
        assert e.value.code == ft.FT_EINVAL
