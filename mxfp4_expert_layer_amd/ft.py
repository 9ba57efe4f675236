"""ctypes binding of libft's C ABI (include/ft.h): argument marshalling only.

Every compute step runs in libft's HIP kernels or its native host runtime; this module only
converts Python values to C arguments and C status codes to exceptions.  Importing it
raises if libft.so has not been built, so no code path can silently fall back to Python.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FT_LIB", os.path.join(_HERE, "libft.so"))

FT_OK, FT_EINVAL, FT_ENOMEM, FT_EHIP, FT_EUNSUPPORTED, FT_ESTATE, FT_EIO = 0, -1, -2, -3, -4, -5, -6
FT_FTW_DIRECT, FT_FTW_STAGED = 1, 2
FT_MXFP4, FT_NVFP4 = 0, 1
FT_PREFILL_EXACT, FT_PREFILL_MXFP4 = 0, 1
FT_LAYER_PREFILL_MXFP4 = 1
FT_SPLIT_ROUND, FT_SPLIT_MAKESPAN, FT_SPLIT_LOAD = 0, 1, 2
MAX_DECODE_TOKENS = 16
FORMATS = {"mxfp4": FT_MXFP4, "nvfp4": FT_NVFP4}


class FtError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libft error {code}: {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libft.so not found at {LIB_PATH}: build it with "
                      "`python -m mxfp4_expert_layer_amd.build` (no fallback path exists)")
# torch carries its own HIP runtime under the same soname (libamdhip64.so.7) as the ROCm one
# libft is linked against, and a process holds one copy of a soname: whichever loads first
# serves both.  torch's own HIP libraries need the runtime they were built with, so torch is
# loaded first and libft binds to that same runtime (the buffers and streams it is handed
# come from it).
try:
    import torch  # noqa: F401
except ImportError:   # a process without torch uses the ROCm runtime libft is linked against
    pass
lib = C.CDLL(LIB_PATH)


class LayerDesc(C.Structure):
    _fields_ = [("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("n_shared", C.c_int32), ("format", C.c_int32), ("n_slots", C.c_int32),
                ("max_tokens", C.c_int32), ("router_w", C.c_void_p), ("router_b", C.c_void_p),
                ("pool", C.c_void_p), ("shared_blobs", C.c_void_p),
                ("host_blobs", C.c_void_p), ("blob_stride", C.c_uint64),
                ("resident", C.c_int32), ("flags", C.c_int32)]


class DecodeStats(C.Structure):
    _fields_ = [("n_selected", C.c_int32), ("n_hits", C.c_int32), ("n_miss", C.c_int32),
                ("q", C.c_int32), ("n_streamed", C.c_int32), ("n_host", C.c_int32),
                ("n_evicted", C.c_int32), ("step", C.c_int32), ("qstar", C.c_double),
                ("bp", C.c_double), ("bh", C.c_double), ("host_us", C.c_double),
                ("wait_us", C.c_double), ("bp_obs", C.c_double), ("bh_obs", C.c_double),
                ("n_prefetched", C.c_int32), ("n_prefetch_hits", C.c_int32),
                ("n_disk", C.c_int32), ("disk_us", C.c_double),
                ("gpu_us_obs", C.c_double), ("t_gpu", C.c_double)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class FtwInfo(C.Structure):
    _fields_ = [("format", C.c_int32), ("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32),
                ("n_shared", C.c_int32), ("direct", C.c_int32), ("staged", C.c_int32),
                ("reserved", C.c_int32), ("blob_bytes", C.c_uint64), ("file_bytes", C.c_uint64)]


_vp, _i, _u64, _d = C.c_void_p, C.c_int, C.c_uint64, C.c_double
_sig = {
    "ft_blob_bytes": [_i, _i, _i, C.POINTER(_u64)],
    "ft_pack_expert": [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "ft_ctx_create": [_i, C.POINTER(_vp)],
    "ft_ctx_destroy": [_vp],
    "ft_ctx_numa": [_vp, C.POINTER(_i), C.POINTER(_i)],
    "ft_debug_parse_cpulist": [C.c_char_p, _vp, _i, C.POINTER(_i)],
    "ft_layer_create": [_vp, C.POINTER(LayerDesc), C.POINTER(_vp)],
    "ft_layer_destroy": [_vp],
    "ft_route": [_vp, _vp, _vp, _i, _vp, _vp, _vp],
    "ft_moe_decode": [_vp, _vp, _vp, _i, _vp, C.POINTER(DecodeStats), _vp],
    "ft_moe_prefill_workspace_size": [_vp, _i, _i, C.POINTER(C.c_size_t)],
    "ft_moe_prefill": [_vp, _vp, _vp, _i, _vp, _i, _vp, C.c_size_t, _vp],
    "ft_moe_prefill_noalloc": [_vp, _vp, _vp, _i, _vp, _i, _vp],
    "ft_qstar_split": [_i, _d, _d, C.POINTER(_i), C.POINTER(_d)],
    "ft_measure_bandwidth": [_vp, _vp, C.POINTER(_d), C.POINTER(_d)],
    "ft_set_bandwidth": [_vp, _d, _d],
    "ft_force_q": [_vp, _i],
    "ft_qstar_split_makespan": [_i, _d, _d, C.POINTER(_i)],
    "ft_qstar_split_load": [_i, _i, _d, _d, _d, _d, C.POINTER(_i)],
    "ft_set_miss_policy": [_vp, _i, _d],
    "ft_set_prefetch": [_vp, _vp, _i],
    "ft_debug_pool_stress": [_i, _i, _i],
    "ft_debug_throw": [_i],
    "ft_probe_hbm_read": [_vp, _vp, _u64, _i, C.POINTER(_d)],
    "ft_ftw_write": [C.c_char_p, _i, _i, _i, _i, _i, _vp, _u64],
    "ft_ftw_open": [C.c_char_p, _i, C.POINTER(_vp)],
    "ft_ftw_get_info": [_vp, C.POINTER(FtwInfo)],
    "ft_ftw_close": [_vp],
    "ft_ftw_read": [_vp, _vp, _vp, _i, _vp, _u64, _u64, C.POINTER(_d)],
    "ft_layer_set_disk_tier": [_vp, _vp, _vp, _i],
    "ft_debug_host_tier": [_vp, _vp, _vp],
    "ft_residual_bf16": [_vp, _vp, _vp, C.c_float, C.c_int64, _vp, _vp],
    "ft_debug_dequant": [_vp, _i, _i, _vp, _vp],
    "ft_debug_tables": [_vp, _vp, _vp],
    "ft_host_expert_ffn": [_vp, _i, _i, _i, _vp, _vp, _i, _vp],
    "ft_debug_prefill_perm": [_vp, _vp, _i, _vp, _vp, _vp, _vp],
    "ft_debug_prefill_route": [_vp, _vp, _i, _vp, _vp, _vp],
    "ft_debug_prefill_quant": [_vp, _vp, _i, _i, _vp, _vp, _vp],
    "ft_debug_prefill_weights": [_vp, _i, _vp, _vp],
    "ft_profile_begin": [_vp, _i],
    "ft_profile_end": [_vp, C.POINTER(_d), C.POINTER(_d), C.POINTER(_i)],
}
for _name, _args in _sig.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = C.c_int
lib.ft_last_error.argtypes = []
lib.ft_last_error.restype = C.c_char_p

DECLARED = tuple(_sig) + ("ft_last_error",)


def check(rc: int):
    if rc != FT_OK:
        raise FtError(rc, lib.ft_last_error().decode(errors="replace"))


def _ptr(a) -> int:
    """Address of a numpy array or torch tensor (or an int address)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


def blob_bytes(fmt: str, H: int, I: int) -> int:
    v = C.c_uint64()
    check(lib.ft_blob_bytes(FORMATS[fmt], H, I, C.byref(v)))
    return v.value


def pack_expert_into(fmt: str, H: int, I: int, ex, dst) -> None:
    """Pack an expert (synth.Expert-like) into host memory at dst (array, tensor or address)."""
    arrs = [np.ascontiguousarray(getattr(ex, f)) for f in
            ("gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales")]
    ts = np.ascontiguousarray(ex.tensor_scales, dtype=np.float32)
    check(lib.ft_pack_expert(FORMATS[fmt], H, I, *[_ptr(a) for a in arrs], _ptr(ts), _ptr(dst)))


def pack_expert(fmt: str, H: int, I: int, ex) -> np.ndarray:
    out = np.empty(blob_bytes(fmt, H, I), dtype=np.uint8)
    pack_expert_into(fmt, H, I, ex, out)
    return out


def qstar_split(m: int, Bp: float, Bh: float):
    q, qs = C.c_int(), C.c_double()
    check(lib.ft_qstar_split(m, Bp, Bh, C.byref(q), C.byref(qs)))
    return q.value, qs.value


def host_expert_ffn(fmt: str, H: int, I: int, blob: np.ndarray, x_bits: np.ndarray,
                    ctx=None) -> np.ndarray:
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T = x.shape[0]
    y = np.empty((T, H), dtype=np.float32)
    check(lib.ft_host_expert_ffn(ctx.handle if ctx else None, FORMATS[fmt], H, I, _ptr(blob),
                                 _ptr(x), T, _ptr(y)))
    return y


class Context:
    def __init__(self, device: int = 0):
        h = C.c_void_p()
        check(lib.ft_ctx_create(device, C.byref(h)))
        self.handle = h.value
        self.device = device

    def close(self):
        if self.handle:
            check(lib.ft_ctx_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def layer_create(ctx: Context, desc: LayerDesc) -> int:
    h = C.c_void_p()
    check(lib.ft_layer_create(ctx.handle, C.byref(desc), C.byref(h)))
    return h.value


def layer_destroy(handle: int) -> None:
    check(lib.ft_layer_destroy(handle))


def route(ctx, layer_h, x, T, idx, w, stream=None):
    check(lib.ft_route(ctx.handle, layer_h, _ptr(x), T, _ptr(idx), _ptr(w), stream))


def moe_decode(ctx, layer_h, x, T, y, stream=None, stats: DecodeStats = None):
    check(lib.ft_moe_decode(ctx.handle, layer_h, _ptr(x), T, _ptr(y),
                            C.byref(stats) if stats is not None else None, stream))


def moe_prefill_workspace_size(layer_h, T, mode) -> int:
    v = C.c_size_t()
    check(lib.ft_moe_prefill_workspace_size(layer_h, T, mode, C.byref(v)))
    return v.value


def moe_prefill(ctx, layer_h, x, T, y, mode, ws, ws_bytes, stream=None):
    check(lib.ft_moe_prefill(ctx.handle, layer_h, _ptr(x), T, _ptr(y), mode, _ptr(ws), ws_bytes,
                             stream))


# bytes of the library's static device scratch behind ft_moe_prefill_noalloc
PREFILL_STATIC_SCRATCH_BYTES = 64 << 20


def moe_prefill_noalloc(ctx, layer_h, x, T, y, mode, stream=None):
    check(lib.ft_moe_prefill_noalloc(ctx.handle, layer_h, _ptr(x), T, _ptr(y), mode, stream))


def ctx_numa(ctx):
    """(NUMA node of the context's GPU or -1, CPUs its host threads are bound to or 0)."""
    node, n = C.c_int(), C.c_int()
    check(lib.ft_ctx_numa(ctx.handle, C.byref(node), C.byref(n)))
    return node.value, n.value


def debug_parse_cpulist(text: str):
    n = C.c_int()
    buf = (C.c_int32 * 4096)()
    check(lib.ft_debug_parse_cpulist(text.encode(), buf, 4096, C.byref(n)))
    return list(buf[:min(n.value, 4096)])


def measure_bandwidth(ctx, layer_h):
    bp, bh = C.c_double(), C.c_double()
    check(lib.ft_measure_bandwidth(ctx.handle, layer_h, C.byref(bp), C.byref(bh)))
    return bp.value, bh.value


def set_bandwidth(layer_h, Bp, Bh):
    check(lib.ft_set_bandwidth(layer_h, Bp, Bh))


def force_q(layer_h, q):
    check(lib.ft_force_q(layer_h, q))


def qstar_split_load(m: int, g0: int, Bp: float, Bh: float, blob: float, t_gpu: float) -> int:
    q = C.c_int()
    check(lib.ft_qstar_split_load(m, g0, Bp, Bh, blob, t_gpu, C.byref(q)))
    return q.value


def qstar_split_makespan(m: int, Bp: float, Bh: float) -> int:
    q = C.c_int()
    check(lib.ft_qstar_split_makespan(m, Bp, Bh, C.byref(q)))
    return q.value


def set_miss_policy(layer_h, rule=FT_SPLIT_ROUND, alpha=0.0):
    check(lib.ft_set_miss_policy(layer_h, rule, alpha))


def set_prefetch(layer_h, next_h, depth):
    """Link layer_h's decode calls to prefetch next_h's predicted experts (None/0 unlinks)."""
    check(lib.ft_set_prefetch(layer_h, next_h, depth))


def residual_bf16(ctx, x, y, n, out, stream=None, scale=1.0):
    """out = bf16(x + scale * y) on the device (x, out bf16 bits; y fp32)."""
    check(lib.ft_residual_bf16(ctx.handle, _ptr(x), _ptr(y), scale, n, _ptr(out), stream))


def debug_dequant(layer_h, slot, matrix, out, stream=None):
    check(lib.ft_debug_dequant(layer_h, slot, matrix, _ptr(out), stream))


def debug_tables(layer_h, E, S):
    e2s = np.empty(E, np.int32)
    s2e = np.empty(S, np.int32)
    check(lib.ft_debug_tables(layer_h, _ptr(e2s), _ptr(s2e)))
    return e2s, s2e


def debug_prefill_perm(layer_h, ws, T, counts, offsets, pos, stream=None):
    check(lib.ft_debug_prefill_perm(layer_h, _ptr(ws), T, _ptr(counts), _ptr(offsets), _ptr(pos),
                                    stream))


def profile_begin(layer_h, n):
    check(lib.ft_profile_begin(layer_h, n))


def profile_end(layer_h):
    """(mean gate/up kernel us, mean down kernel us, calls recorded)."""
    a, b, n = C.c_double(), C.c_double(), C.c_int()
    check(lib.ft_profile_end(layer_h, C.byref(a), C.byref(b), C.byref(n)))
    return a.value, b.value, n.value


def debug_prefill_route(layer_h, ws, T, idx, w, stream=None):
    check(lib.ft_debug_prefill_route(layer_h, _ptr(ws), T, _ptr(idx), _ptr(w), stream))


def debug_prefill_quant(layer_h, ws, T, which, codes, scales, stream=None):
    """which 0: quantised tokens; 1: quantised h (permuted rows) of the last MXFP4 prefill."""
    check(lib.ft_debug_prefill_quant(layer_h, _ptr(ws), T, which, _ptr(codes), _ptr(scales),
                                     stream))


def debug_prefill_weights(layer_h, e, out, stream=None):
    check(lib.ft_debug_prefill_weights(layer_h, e, _ptr(out), stream))


def ftw_write(path, fmt, H, I, E, n_shared, blobs, src_stride):
    """Write an FTW file from packed blobs (a host buffer: numpy array or CPU tensor)."""
    check(lib.ft_ftw_write(os.fsencode(path), FORMATS[fmt] if isinstance(fmt, str) else fmt,
                           H, I, E, n_shared, _ptr(blobs), src_stride))


class Ftw:
    """An open FTW file (closed by close() or when collected)."""

    def __init__(self, path, direct=True, staged=False):
        h = C.c_void_p()
        flags = (FT_FTW_DIRECT if direct else 0) | (FT_FTW_STAGED if staged else 0)
        check(lib.ft_ftw_open(os.fsencode(path), flags, C.byref(h)))
        self.handle = h.value

    def info(self) -> FtwInfo:
        inf = FtwInfo()
        check(lib.ft_ftw_get_info(self.handle, C.byref(inf)))
        return inf

    def read(self, ids, dst, dst_stride, chunk=0, ctx=None) -> float:
        """Read blobs ids into dst (host buffer) at dst_stride; returns the seconds taken."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        sec = C.c_double()
        check(lib.ft_ftw_read(ctx.handle if ctx is not None else None, self.handle,
                              ids.ctypes.data, len(ids), _ptr(dst), dst_stride, chunk,
                              C.byref(sec)))
        return sec.value

    def close(self):
        if self.handle:
            lib.ft_ftw_close(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def set_disk_tier(layer_h, ftw, ram, n_ram):
    """Attach a host-memory tier of n_ram pinned slots over an open FTW file (None detaches)."""
    check(lib.ft_layer_set_disk_tier(layer_h, ftw.handle if ftw is not None else None,
                                     _ptr(ram) if ram is not None else None, n_ram))


def debug_host_tier(layer_h, E, n_ram):
    e2r = np.empty(E, dtype=np.int32)
    r2e = np.empty(n_ram, dtype=np.int32)
    check(lib.ft_debug_host_tier(layer_h, e2r.ctypes.data, r2e.ctypes.data))
    return e2r, r2e


def probe_hbm_read(ctx, buf, nbytes, reps=10) -> float:
    """GB/s of a plain streaming read of nbytes of device memory at buf."""
    v = C.c_double()
    check(lib.ft_probe_hbm_read(ctx.handle, _ptr(buf), nbytes, reps, C.byref(v)))
    return v.value
