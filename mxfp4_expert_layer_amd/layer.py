"""Device-side set-up of a layer for libft: torch allocates the buffers, libft packs the blobs.

``GpuLayer`` draws a synthetic layer (``synth``), packs every expert into libft's blob layout
with ``ft_pack_expert`` (host threads; ctypes releases the GIL), and hands the device pool,
router tensors, shared-expert blobs and (for a partial pool) the pinned host blob store to
``ft_layer_create``.  torch is used only to own device and pinned memory and streams.
"""
from __future__ import annotations

import contextlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import ft, synth


def node_cpus(node: int):
    """CPUs of a NUMA node that this process may run on (empty when unknown)."""
    if node < 0:
        return set()
    try:
        with open(f"/sys/devices/system/node/node{node}/cpulist") as fh:
            cpus = set(ft.debug_parse_cpulist(fh.read().strip()))
    except OSError:
        return set()
    return cpus & os.sched_getaffinity(0)


@contextlib.contextmanager
def on_gpu_node(ctx):
    """Run the block on the CPUs of the GPU's NUMA node, so that host memory allocated in it
    (pinned pages land on the allocating thread's node) sits next to the GPU and to the
    library's host threads, which the context binds there."""
    node, _ = ft.ctx_numa(ctx)
    cpus = node_cpus(node)
    old = os.sched_getaffinity(0)
    if not cpus or cpus == old:
        yield
        return
    os.sched_setaffinity(0, cpus)
    try:
        yield
    finally:
        os.sched_setaffinity(0, old)


def _pack_all(cfg, ids, dst: np.ndarray, stride: int, threads: int, shared=False,
              override=None):
    def one(pair):
        slot, e = pair
        ex = override[e] if override and e in override else synth.gen_expert(cfg, e, shared=shared)
        ft.pack_expert_into(cfg.fmt, cfg.H, cfg.I, ex, dst[slot * stride:(slot + 1) * stride])
    with ThreadPoolExecutor(max_workers=max(1, threads)) as pool:
        list(pool.map(one, list(enumerate(ids))))


class GpuLayer:
    """A libft layer over torch-owned memory.

    resident=True: the pool holds all E experts (slot e = expert e).  resident=False: the
    pool has n_slots empty slots and all E blobs live in pinned host memory (miss path);
    host_store reuses another miss-path layer's pinned blobs instead of packing new ones.
    copies > 1 packs the pool once and replicates it to further device buffers (separate
    addresses with the same bytes) that ``select_copy`` switches between; each copy has its
    own router bias draw so hot experts differ between copies."""

    def __init__(self, ctx: ft.Context, cfg: synth.LayerConfig, *, resident=True,
                 n_slots=None, max_tokens=16, threads=8, copies=1, device="cuda",
                 experts=None, router=None, prefill_mxfp4=False, host_store=None):
        self.ctx, self.cfg = ctx, cfg
        self.device = device
        self.stride = ft.blob_bytes(cfg.fmt, cfg.H, cfg.I)
        E = cfg.E
        self.n_slots = E if resident else (n_slots or cfg.n_slots)
        self.max_tokens = max_tokens
        self.resident = resident
        self.override = experts or {}
        if host_store is not None:
            # share another layer's pinned blob store (same expert bytes, e.g. for timing)
            assert not resident and host_store.numel() == E * self.stride and host_store.is_pinned()
            host = host_store
        elif resident:
            host = torch.empty(E * self.stride, dtype=torch.uint8)
            _pack_all(cfg, list(range(E)), host.numpy(), self.stride, threads,
                      override=self.override)
        else:
            # the pinned blob store the miss path streams and computes from: on the GPU's node
            with on_gpu_node(ctx):
                host = torch.empty(E * self.stride, dtype=torch.uint8, pin_memory=True)
                _pack_all(cfg, list(range(E)), host.numpy(), self.stride, threads,
                          override=self.override)
        if resident:
            self.pools = [host.to(device)]
            for _ in range(1, copies):
                self.pools.append(self.pools[0].clone())
            self.host_blobs = None
            del host
        else:
            self.pools = [torch.zeros(self.n_slots * self.stride, dtype=torch.uint8, device=device)]
            self.host_blobs = host
        if cfg.n_shared:
            sh = np.empty(cfg.n_shared * self.stride, dtype=np.uint8)
            _pack_all(cfg, list(range(cfg.n_shared)), sh, self.stride, 1, shared=True)
            self.shared = torch.from_numpy(sh).to(device)
        else:
            self.shared = None
        self.routers = []
        self.router_override = router
        for c in range(max(1, copies)):
            w, b = router if router is not None else synth.gen_router(cfg, c)
            self.routers.append((torch.from_numpy(w).to(device),
                                 torch.from_numpy(b).to(device) if b is not None else None))
        self.handles = []
        for c in range(len(self.pools)):
            wr, br = self.routers[c]
            desc = ft.LayerDesc(
                H=cfg.H, I=cfg.I, E=E, k=cfg.k, n_shared=cfg.n_shared,
                format=ft.FORMATS[cfg.fmt], n_slots=self.n_slots, max_tokens=max_tokens,
                router_w=wr.data_ptr(), router_b=br.data_ptr() if br is not None else None,
                pool=self.pools[c].data_ptr(),
                shared_blobs=self.shared.data_ptr() if self.shared is not None else None,
                host_blobs=self.host_blobs.data_ptr() if self.host_blobs is not None else None,
                blob_stride=self.stride, resident=1 if resident else 0,
                flags=ft.FT_LAYER_PREFILL_MXFP4 if prefill_mxfp4 else 0)
            self.handles.append(ft.layer_create(ctx, desc))
        self.handle = self.handles[0]

    def select_copy(self, c: int):
        self.handle = self.handles[c]

    def oracle_layer(self, copy: int = 0):
        """The synth.Layer the oracle evaluates (experts drawn lazily on access)."""
        L = synth.gen_layer(self.cfg, experts=None, copy=copy)
        L.experts.update(self.override)
        if self.router_override is not None:
            L.router_w, L.router_b = self.router_override
        return L

    def close(self):
        for h in self.handles:
            ft.layer_destroy(h)
        self.handles = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stream_ptr(stream=None):
    s = stream or torch.cuda.current_stream()
    return s.cuda_stream
