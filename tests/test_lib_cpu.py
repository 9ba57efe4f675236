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
    # the largest square NVFP4 expert under 2 GiB, and the next size up
    # (3 matrices x 9/16 B per weight: 35584^2 is 2,136,752,128 B, 35712^2 is 2,152,161,280 B)
    assert ft.blob_bytes("nvfp4", 35584, 35584) == 2_136_752_128
    with pytest.raises(ft.FtError):
        ft.blob_bytes("nvfp4", 35712, 35712)


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
        ft.host_expert_ffn("mxfp4", 256, 128, np.zeros(ft.blob_bytes("mxfp4", 256, 128), np.uint8),
                           np.zeros((1, 256), np.uint16))
    assert e.value.code == ft.FT_EINVAL          # a whole blob whose header is not one
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


def test_load_split_matches_oracle():
    """The library's load variant against the oracle's over random (m, g0, Bp, Bh, t_gpu),
    including no GPU term and a busy GPU, and its argument checks."""
    rng = np.random.default_rng(4)
    blob = 13369344.0
    for i in range(600):
        m, g0 = int(rng.integers(0, 17)), int(rng.integers(0, 12))
        Bp, Bh = float(rng.uniform(1e9, 60e9)), float(rng.uniform(1e9, 250e9))
        t = 0.0 if i % 5 == 0 else float(rng.uniform(0, 5e-4))
        assert ft.qstar_split_load(m, g0, Bp, Bh, blob, t) == policy.qstar_load(m, g0, Bp, Bh, blob, t), \
            (m, g0, Bp, Bh, t)
    for bad in ((-1, 0, 1.0, 1.0, 1.0, 0.0), (1, -1, 1.0, 1.0, 1.0, 0.0), (1, 0, 0.0, 1.0, 1.0, 0.0),
                (1, 0, 1.0, 1.0, 0.0, 0.0), (1, 0, 1.0, 1.0, 1.0, -1.0),
                (1, 0, 1.0, 1.0, 1.0, float("inf"))):
        with pytest.raises(ft.FtError) as e:
            ft.qstar_split_load(*bad)
        assert e.value.code == ft.FT_EINVAL


def _aligned(nbytes):
    """A 4096-aligned uint8 view of nbytes (O_DIRECT destinations)."""
    raw = np.zeros(nbytes + 4096, dtype=np.uint8)
    off = (-raw.ctypes.data) % 4096
    return raw[off:off + nbytes]


def _packed_store(fmt, E, n_shared, seed=12):
    cfg = synth.small_config(seed=seed, H=256, I=128, E=E, fmt=fmt, n_shared=n_shared)
    stride = ft.blob_bytes(fmt, cfg.H, cfg.I)
    store = np.zeros((E + n_shared) * stride, dtype=np.uint8)
    for e in range(E):
        ft.pack_expert_into(fmt, cfg.H, cfg.I, synth.gen_expert(cfg, e),
                            store[e * stride:(e + 1) * stride])
    for s in range(n_shared):
        ft.pack_expert_into(fmt, cfg.H, cfg.I, synth.gen_expert(cfg, s, shared=True),
                            store[(E + s) * stride:(E + s + 1) * stride])
    return cfg, stride, store


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("direct,staged", [(True, False), (False, False), (True, True)])
def test_ftw_roundtrip_and_layout(tmp_path, fmt, direct, staged):
    """An FTW file holds the packed blobs unchanged, with its header page first and every
    tensor on a 4096-byte boundary of the file; reads in whole blobs or in 4 KiB requests,
    on one thread, return the same bytes."""
    cfg, stride, store = _packed_store(fmt, E=5, n_shared=1)
    path = str(tmp_path / "layer.ftw")
    ft.ftw_write(path, fmt, cfg.H, cfg.I, 5, 1, store, stride)
    raw = np.fromfile(path, dtype=np.uint8)
    hdr = raw[:4096]
    assert hdr[:8].view(np.uint32).tolist() == [0x31575446, 1]
    assert hdr[8:28].view(np.int32).tolist() == [ft.FORMATS[fmt], 256, 128, 5, 1]
    blob_bytes, blob_stride, data_off, file_bytes = hdr[32:64].view(np.uint64).tolist()
    assert (blob_bytes, blob_stride, data_off) == (stride, stride, 4096)
    assert file_bytes == raw.size == 4096 + 6 * stride
    offs, _ = tiled.blob_offsets(fmt, cfg.H, cfg.I)
    for i in range(6):
        base = data_off + i * blob_stride
        assert all((base + o) % 4096 == 0 for o in [0] + offs)
        assert np.array_equal(raw[base:base + stride], store[i * stride:(i + 1) * stride])
    f = ft.Ftw(path, direct=direct, staged=staged)
    try:
        inf = f.info()
        assert (inf.E, inf.n_shared, inf.blob_bytes, inf.file_bytes) == (5, 1, stride, raw.size)
        assert direct or inf.direct == 0
        assert inf.staged == (inf.direct and staged)
        ids = [5, 0, 3, 3]
        for chunk in (0, 4096, 3 * 4096):
            dst = _aligned(len(ids) * stride)
            f.read(ids, dst, stride, chunk=chunk)
            for j, e in enumerate(ids):
                assert np.array_equal(dst[j * stride:(j + 1) * stride],
                                      store[e * stride:(e + 1) * stride]), (chunk, j)
        with pytest.raises(ft.FtError) as e:
            f.read([6], _aligned(stride), stride)
        assert e.value.code == ft.FT_EINVAL
        if inf.direct:
            with pytest.raises(ft.FtError) as e:     # O_DIRECT needs aligned destinations
                f.read([0], _aligned(stride + 8)[8:], stride)
            assert e.value.code == ft.FT_EINVAL
    finally:
        f.close()


def test_ftw_rejects_bad_files(tmp_path):
    cfg, stride, store = _packed_store("mxfp4", E=3, n_shared=0)
    good = str(tmp_path / "good.ftw")
    ft.ftw_write(good, "mxfp4", cfg.H, cfg.I, 3, 0, store, stride)
    raw = np.fromfile(good, dtype=np.uint8)

    def expect(code, data=None, path=None):
        p = path or str(tmp_path / "bad.ftw")
        if data is not None:
            data.tofile(p)
        with pytest.raises(ft.FtError) as e:
            ft.Ftw(p)
        assert e.value.code == code

    bad = raw.copy(); bad[0] ^= 1
    expect(ft.FT_EINVAL, bad)                       # magic
    bad = raw.copy(); bad[4] = 9
    expect(ft.FT_EINVAL, bad)                       # version
    expect(ft.FT_EINVAL, raw[:-4096].copy())        # truncated
    bad = raw.copy(); bad[32:40] = np.array([stride + 16], dtype=np.uint64).view(np.uint8)
    expect(ft.FT_EINVAL, bad)                       # blob size of other dimensions
    expect(ft.FT_EIO, path=str(tmp_path / "missing.ftw"))
    # the writer checks each blob's header against the dimensions it is given
    with pytest.raises(ft.FtError) as e:
        ft.ftw_write(str(tmp_path / "x.ftw"), "mxfp4", 384, cfg.I, 3, 0, store, stride)
    assert e.value.code == ft.FT_EINVAL
    with pytest.raises(ft.FtError) as e:
        ft.ftw_write(str(tmp_path / "x.ftw"), "mxfp4", cfg.H, cfg.I, 3, 0, store, stride - 4096)
    assert e.value.code == ft.FT_EINVAL


def test_host_expert_ffn_mixed_scale_ranges():
    """A gate row tile holding E8M0 codes 0 and 1 (outside the range the AVX-512 table path
    takes exactly) next to ordinary tiles: that tile goes to the scalar path, the rest stay
    vectorised, and the whole FFN still matches the oracle."""
    cfg = synth.small_config(seed=9, H=256, I=128, code_dist="normal")
    ex = synth.gen_expert(cfg, 4)
    ex.gate_scales = ex.gate_scales.copy()
    ex.gate_scales[3, :] = 1          # row 3 of the gate: every block scale 2^-126
    ex.gate_scales[20, 2] = 0         # one block of row 20 (another row tile): 2^-127
    blob = ft.pack_expert("mxfp4", cfg.H, cfg.I, ex)
    x = synth.gen_tokens(cfg, 2)
    y = ft.host_expert_ffn("mxfp4", cfg.H, cfg.I, blob, x)

    class _L:
        pass
    L = _L()
    L.cfg = cfg
    wg, wu, wd = moe.expert_weights(L, ex)
    ref = moe.swiglu_ffn(fp4.bf16_bits_to_f64(x), wg, wu, wd)
    assert moe.rel_l2(y, ref) <= 1e-3


def test_host_expert_ffn_scale_code_253(monkeypatch):
    """E8M0 code 253 (2^126) with codes 6 and -4 in the block: 6 * 2^126 and 4 * 2^126 are past
    the bf16 and fp32 range, so the AVX-512 table path must not take that row tile.  One gate
    block of row 7 holds +6 and -4 at the two elements where x is 2^-126 (a normal bf16), so
    the block adds exactly 6 - 4 = 2 to that row's dot product; the vectorised path (on CPUs
    with AVX-512 BF16), the scalar path and the oracle must agree, with every output finite."""
    cfg = synth.small_config(seed=10, H=256, I=128, code_dist="normal")
    ex = synth.gen_expert(cfg, 5)
    ex.gate_codes = ex.gate_codes.copy()
    ex.gate_scales = ex.gate_scales.copy()
    ex.gate_codes[7, 32:48] = 0
    ex.gate_codes[7, 32] = 0x7 | (0xE << 4)       # elements 64, 65: +6, -4
    ex.gate_scales[7, 2] = 253                     # block 2 = elements 64..95
    blob = ft.pack_expert("mxfp4", cfg.H, cfg.I, ex)
    x = synth.gen_tokens(cfg, 2)
    x[:, 64:66] = synth.f32_to_bf16_bits(np.full(2, 2.0 ** -126, np.float32))
    ys = []
    for scalar in ("0", "1"):
        monkeypatch.setenv("FT_HOST_SCALAR", scalar)
        ys.append(ft.host_expert_ffn("mxfp4", cfg.H, cfg.I, blob, x))

    class _L:
        pass
    L = _L()
    L.cfg = cfg
    wg, wu, wd = moe.expert_weights(L, ex)
    ref = moe.swiglu_ffn(fp4.bf16_bits_to_f64(x), wg, wu, wd)
    for y in ys:
        assert np.all(np.isfinite(y))
        assert moe.rel_l2(y, ref) <= 1e-3
    assert moe.rel_l2(ys[0], ys[1]) <= 1e-5


@pytest.mark.parametrize("threads,jobs,pause_us", [(8, 400, 0), (8, 40, 1500), (1, 10, 0),
                                                   (16, 25, 700)])
def test_host_thread_pool_runs_every_job_once(threads, jobs, pause_us):
    """The spin-then-sleep pool: back-to-back jobs (workers spinning) and jobs after pauses
    longer than the spin (workers asleep, woken by the next job) each run every index once;
    a lost wake-up would hang here (the test has a timeout)."""
    ft.check(ft.lib.ft_debug_pool_stress(threads, jobs, pause_us))


def test_null_arguments_return_einval():
    """Every entry point that takes an object rejects a null one with FT_EINVAL (and touches
    no GPU doing so)."""
    L = ft.lib
    calls = [
        lambda: L.ft_set_prefetch(None, None, 0),
        lambda: L.ft_set_miss_policy(None, 0, 0.0),
        lambda: L.ft_set_bandwidth(None, 1.0, 1.0),
        lambda: L.ft_force_q(None, 0),
        lambda: L.ft_layer_set_disk_tier(None, None, None, 0),
        lambda: L.ft_debug_host_tier(None, None, None),
        lambda: L.ft_debug_tables(None, None, None),
        lambda: L.ft_residual_bf16(None, None, None, 1.0, 1, None, None),
        lambda: L.ft_probe_hbm_read(None, None, 1 << 20, 1, None),
        lambda: L.ft_ftw_open(None, 0, None),
        lambda: L.ft_ftw_get_info(None, None),
        lambda: L.ft_ftw_read(None, None, None, 1, None, 0, 0, None),
        lambda: L.ft_ftw_write(None, 0, 256, 128, 1, 0, None, 0),
        lambda: L.ft_moe_decode(None, None, None, 1, None, None, None),
        lambda: L.ft_route(None, None, None, 1, None, None, None),
        lambda: L.ft_layer_create(None, None, None),
        lambda: L.ft_measure_bandwidth(None, None, None, None),
        lambda: L.ft_debug_pool_stress(0, 1, 0),
    ]
    for i, c in enumerate(calls):
        assert c() == ft.FT_EINVAL, i
    # destroying nothing is a no-op
    assert L.ft_layer_destroy(None) == ft.FT_OK and L.ft_ctx_destroy(None) == ft.FT_OK
    assert L.ft_ftw_close(None) == ft.FT_OK


@pytest.mark.parametrize("kind,code,text", [(0, "FT_OK", None), (1, "FT_ENOMEM", "out of host memory"),
                                            (2, "FT_ESTATE", "planted exception"),
                                            (3, "FT_ENOMEM", None), (7, "FT_EINVAL", "kind must be")])
def test_exceptions_do_not_cross_the_abi(kind, code, text):
    """An exception thrown inside an entry point comes back as a status code with a message
    naming the entry point (bad_alloc and system_error: FT_ENOMEM; others: FT_ESTATE)."""
    code = getattr(ft, code)
    rc = ft.lib.ft_debug_throw(kind)
    assert rc == code
    if code:
        msg = ft.lib.ft_last_error().decode()
        assert msg.startswith("ft_debug_throw"), msg
        if text:
            assert text in msg, msg


def test_cpulist_parser():
    """The Linux cpulist format the context reads a NUMA node's CPUs in: ranges and single
    CPUs, in order; a malformed list gives no CPUs."""
    assert ft.debug_parse_cpulist("0-3,8,10-11") == [0, 1, 2, 3, 8, 10, 11]
    assert ft.debug_parse_cpulist("5\n") == [5]
    assert ft.debug_parse_cpulist("0-1, 4") == [0, 1, 4]
    for bad in ("", "a-b", "4-2", "1-", "3x"):
        assert ft.debug_parse_cpulist(bad) == []
