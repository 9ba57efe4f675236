"""Seeded synthetic inputs for the MoE expert layer (shared by the oracle and the GPU path).

This module only draws random bits and lays them out as the layer's input tensors:
bf16 activations, fp32 router weights and bias, FP4 code bytes and 8-bit scale codes.
It performs none of the layer's arithmetic (no decoding, routing, FFN or combine), so the
oracle and the HIP path can both consume its output without sharing any method code.

Shapes follow the workloads the FreeToken pages describe: a DeepSeek-V4-Flash-like layer of
256 experts with 6 active (smzdm explainer a825qpgl, section 二), MXFP4 and NVFP4 expert
weights (same page, section 一), and the 35B-A3B / 753B classes named there.  The pages
publish no dataset or weights, so every tensor is drawn here from numpy's PCG64 generator
with a documented seed and draw order.

Tensor layout conventions (logical, row-major):
  x            uint16 [T][H]          bf16 bit patterns
  router_w     float32 [E][H]
  router_b     float32 [E] or None
  gate/up      codes uint8 [I][H/2], scales uint8 [I][H/B]
  down         codes uint8 [H][I/2], scales uint8 [H][I/B]
Two E2M1 codes per byte, element 2i in the low nibble; scale blocks run along the
contraction axis (B = 32 for MXFP4 with E8M0 scales, B = 16 for NVFP4 with E4M3 scales).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MXFP4 = "mxfp4"
NVFP4 = "nvfp4"

# Seed-sequence stream tags (the first entropy word is the config seed).
_STREAM_ROUTER = 0
_STREAM_EXPERT = 1
_STREAM_SHARED = 2
_STREAM_TOKENS = 3


@dataclass(frozen=True)
class LayerConfig:
    name: str
    seed: int
    H: int
    I: int
    E: int
    k: int
    n_shared: int
    fmt: str
    n_slots: int                 # device slot-pool size (== E when all experts are resident)
    router_sigma: float          # std-dev of router weights
    zipf_c: float = 0.0          # router bias b_e = -c * ln(rank_e); 0 disables the bias
    code_dist: str = "normal"    # "uniform" (all 16 codes) or "normal" (rounded N(0,1))
    scale_lo: int = 0            # E8M0 code range (MXFP4) or E4M3 code range (NVFP4)
    scale_hi: int = 0
    nv_tensor_scale: float = 1.0
    batches: tuple = (1,)        # decode token counts (or prefill T)

    @property
    def block(self) -> int:
        return 32 if self.fmt == MXFP4 else 16


# The five workloads (sizes from the pages' model classes; distributions are this build's
# synthetic stand-ins).  E8M0 exponent e maps to code e + 127.
CONFIGS = {
    "tiny": LayerConfig(
        "tiny-decode", 1001, H=256, I=128, E=8, k=2, n_shared=0, fmt=MXFP4, n_slots=8,
        router_sigma=0.02, code_dist="uniform", scale_lo=127 - 8, scale_hi=127 - 4,
        batches=(4,)),
    "35b-a3b": LayerConfig(
        "35b-a3b-decode", 1002, H=2048, I=512, E=256, k=8, n_shared=0, fmt=MXFP4, n_slots=256,
        router_sigma=1.0 / math.sqrt(2048), scale_lo=127 - 7, scale_hi=127 - 3,
        batches=(1, 8)),
    "284b": LayerConfig(
        "284b-decode", 1003, H=4096, I=2048, E=256, k=6, n_shared=1, fmt=MXFP4, n_slots=256,
        router_sigma=1.0 / math.sqrt(4096), zipf_c=1.1, scale_lo=127 - 8, scale_hi=127 - 3,
        batches=(1, 4, 16)),
    "284b-miss-path": LayerConfig(
        "284b-miss-path", 1004, H=4096, I=2048, E=256, k=6, n_shared=1, fmt=MXFP4, n_slots=48,
        router_sigma=1.0 / math.sqrt(4096), zipf_c=1.1, scale_lo=127 - 8, scale_hi=127 - 3,
        batches=(1,)),
    # NVFP4 scales: the 49 E4M3 codes 0x08..0x38 (values 2^-6 .. 2^0), tensor scale 1/64.
    # The 35B-A3B class with NVFP4 experts (the format of the pages' laptop decode result).
    "35b-a3b-nvfp4": LayerConfig(
        "35b-a3b-decode-nvfp4", 1006, H=2048, I=512, E=256, k=8, n_shared=0, fmt=NVFP4,
        n_slots=256, router_sigma=1.0 / math.sqrt(2048), scale_lo=0x08, scale_hi=0x38,
        nv_tensor_scale=1.0 / 64.0, batches=(1, 8)),
    "753b": LayerConfig(
        "753b-prefill", 1005, H=6144, I=2048, E=160, k=8, n_shared=0, fmt=NVFP4, n_slots=160,
        router_sigma=0.5 / math.sqrt(6144), scale_lo=0x08, scale_hi=0x38,
        nv_tensor_scale=1.0 / 64.0, batches=(4096,)),
}


def small_config(name="tiny", seed=7, H=64, I=32, E=4, k=2, n_shared=0, fmt=MXFP4,
                 n_slots=None, code_dist="uniform", router_sigma=0.5, zipf_c=0.0,
                 scale_lo=None, scale_hi=None, nv_tensor_scale=1.0) -> LayerConfig:
    """A small layer for tests (H and I multiples of 32)."""
    if scale_lo is None:
        scale_lo, scale_hi = ((127 - 4, 127 + 1) if fmt == MXFP4 else (0x08, 0x38))
    return LayerConfig(name, seed, H=H, I=I, E=E, k=k, n_shared=n_shared, fmt=fmt,
                       n_slots=E if n_slots is None else n_slots, router_sigma=router_sigma,
                       zipf_c=zipf_c, code_dist=code_dist, scale_lo=scale_lo,
                       scale_hi=scale_hi, nv_tensor_scale=nv_tensor_scale)


def _rng(*words) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(words)))


# --- E2M1 code distribution ------------------------------------------------------------
# "Codes drawn from a rounded N(0,1)": the probability that z ~ N(0,1) lands in each cell
# of the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} under round-to-nearest (cell edges at the
# midpoints), with the sign taken from z.  Draws use one uint16 per code through a
# 65536-entry table, i.e. the distribution is quantised to 1/65536 (the +-6 cells, mass
# 5.7e-7, do not occur).
_E2M1_CELL_EDGES = (0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, math.inf)


def _normal_code_table() -> np.ndarray:
    def phi(a):
        return 0.5 * (1.0 + math.erf(a / math.sqrt(2.0))) if a != math.inf else 1.0
    mag_p = [phi(_E2M1_CELL_EDGES[i + 1]) - phi(_E2M1_CELL_EDGES[i]) for i in range(8)]
    # codes 0..7 positive magnitudes, 8..15 the same magnitudes with the sign bit
    p = np.array([0.5 * q for q in mag_p] * 2, dtype=np.float64)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return np.searchsorted(cdf, u, side="right").astype(np.uint8)


_NORMAL_TABLE = _normal_code_table()


def _draw_codes(rng: np.random.Generator, rows: int, K: int, dist: str) -> np.ndarray:
    """uint8 [rows][K/2] of packed E2M1 codes (low nibble = even element)."""
    nbytes = rows * (K // 2)
    if dist == "uniform":
        out = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    else:
        u = rng.integers(0, 65536, size=2 * nbytes, dtype=np.uint16)
        c = np.take(_NORMAL_TABLE, u)
        out = c[0::2] | (c[1::2] << 4)
    return out.reshape(rows, K // 2)


def _draw_scales(rng: np.random.Generator, rows: int, K: int, cfg: LayerConfig) -> np.ndarray:
    return rng.integers(cfg.scale_lo, cfg.scale_hi + 1, size=(rows, K // cfg.block),
                        dtype=np.uint8)


@dataclass
class Expert:
    gate_codes: np.ndarray
    gate_scales: np.ndarray
    up_codes: np.ndarray
    up_scales: np.ndarray
    down_codes: np.ndarray
    down_scales: np.ndarray
    tensor_scales: np.ndarray = field(default_factory=lambda: np.ones(3, np.float32))


def gen_expert(cfg: LayerConfig, e: int, shared: bool = False) -> Expert:
    """Expert e (or shared expert e) of the layer; independent of every other expert."""
    rng = _rng(cfg.seed, _STREAM_SHARED if shared else _STREAM_EXPERT, e)
    H, I, d = cfg.H, cfg.I, cfg.code_dist
    gc = _draw_codes(rng, I, H, d)
    gs = _draw_scales(rng, I, H, cfg)
    uc = _draw_codes(rng, I, H, d)
    us = _draw_scales(rng, I, H, cfg)
    dc = _draw_codes(rng, H, I, d)
    ds = _draw_scales(rng, H, I, cfg)
    ts = np.full(3, cfg.nv_tensor_scale if cfg.fmt == NVFP4 else 1.0, dtype=np.float32)
    return Expert(gc, gs, uc, us, dc, ds, ts)


def gen_router(cfg: LayerConfig, copy: int = 0):
    """(router_w float32 [E][H], router_b float32 [E] or None).

    copy > 0 redraws the Zipf rank permutation only (router weights stay the same), so that
    replicated layer copies have different hot experts."""
    rng = _rng(cfg.seed, _STREAM_ROUTER, 0)
    w = (rng.standard_normal((cfg.E, cfg.H)) * cfg.router_sigma).astype(np.float32)
    if cfg.zipf_c == 0.0:
        return w, None
    prng = rng if copy == 0 else _rng(cfg.seed, _STREAM_ROUTER, copy)
    rank = prng.permutation(cfg.E).astype(np.float64) + 1.0
    b = (-cfg.zipf_c * np.log(rank)).astype(np.float32)
    return w, b


def f32_to_bf16_bits(z: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    bits = np.ascontiguousarray(z, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bits = bits + 0x7FFF + ((bits >> 16) & 1)
    return (bits >> 16).astype(np.uint16)


def gen_tokens(cfg: LayerConfig, T: int, batch: int = 0) -> np.ndarray:
    """bf16 bits uint16 [T][H] with values N(0,1) rounded to bf16; batch selects the draw."""
    rng = _rng(cfg.seed, _STREAM_TOKENS, batch)
    z = rng.standard_normal((T, cfg.H), dtype=np.float32)
    return f32_to_bf16_bits(z)


@dataclass
class Layer:
    cfg: LayerConfig
    router_w: np.ndarray
    router_b: Optional[np.ndarray]
    experts: dict            # e -> Expert (possibly only a subset, generated lazily)
    shared: list             # list of Expert (n_shared entries)

    def expert(self, e: int) -> Expert:
        if e not in self.experts:
            self.experts[e] = gen_expert(self.cfg, e)
        return self.experts[e]


def gen_layer(cfg: LayerConfig, experts="all", threads: int = 8, copy: int = 0) -> Layer:
    """Generate a layer.  experts="all" draws all E experts (in parallel threads), a list draws
    only those ids, None draws none (they are generated on first access)."""
    w, b = gen_router(cfg, copy)
    if experts == "all":
        ids = list(range(cfg.E))
    elif experts is None:
        ids = []
    else:
        ids = sorted(set(int(e) for e in experts))
    exp = {}
    if ids:
        with ThreadPoolExecutor(max_workers=max(1, threads)) as pool:
            for e, ex in zip(ids, pool.map(lambda i: gen_expert(cfg, i), ids)):
                exp[e] = ex
    shared = [gen_expert(cfg, s, shared=True) for s in range(cfg.n_shared)]
    return Layer(cfg, w, b, exp, shared)
