#!/usr/bin/env python3
"""Benchmark of the FP4 MoE expert layer on one MI355X (prints one JSON line).

Workloads (seeded synthetic layers, no trained weights exist for these shapes):
  decode-35b-a3b   hidden 2048, 256 experts, top-8, intermediate 512, MXFP4
  decode-35b-a3b-nvfp4  the same layer with NVFP4 experts (E4M3 per 16, tensor scale 1/64)
  decode-284b      hidden 4096, 256 experts + 1 shared, top-6, intermediate 2048, MXFP4
  miss-path-284b   the 284B-class layer with a 48-slot pool, q* split of misses
                   (--layers N chains N such layers, --prefetch D adds cross-layer prefetch)
  prefill-753b     4096 tokens through hidden 6144, 160 experts, top-8, intermediate 2048,
                   NVFP4 (exact bf16-MFMA grouped GEMMs)
  headline         (default) prefill-753b as the line's value and roofline, plus the same
                   layer in the scaled-FP4 mode and decode-284b at 1, 4 and 16 tokens per
                   step as extra keys
A decode step is one ft_moe_decode call of T tokens (routing, gate/up + SwiGLU, down,
combine); a prefill step is one ft_moe_prefill call of 4096 tokens.
Decode steps are captured in a HIP graph and replayed; inputs are resident in HBM; the
layer is replicated to several device copies (different addresses) so repeated steps are
not served from the 256 MB Infinity Cache.

roofline (the dominant kernel, its duration from start/stop events that its own dispatches
record on the call's stream):
  prefill, exact mode: the gate/up grouped GEMM, bound by the bf16 MFMA; achieved =
    2 * (T*k) * 2*I*H flop per launch / its mean duration, peak 2.5 PFLOP/s;
  prefill, scaled-FP4 mode: the gate/up grouped GEMM, bound by HBM (its arithmetic intensity
    is below the FP4 ridge); achieved = its algorithmic bytes per launch / duration, peak
    8 TB/s, with its FP4 MFMA rate against 10.1 PFLOP/s alongside;
  decode: the gate/up kernel, which reads two thirds of the expert bytes; achieved =
    distinct experts of the call x 2*I*H*(1/2 + 1/B) bytes (codes + one scale byte per block
    of B = 32 (MXFP4) or 16 (NVFP4)) / duration, peak 8 TB/s (MI355X HBM3E).
cpu_baseline: the float64 oracle on a bounded sample of the same steps (host cores).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode tok/s + HBM GB/s % peak; prefill tok/s + FP4 MFMA %"
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    "decode-35b-a3b": dict(cfg="35b-a3b", T=1, copies=8, steps=2048, warmup=128),
    "decode-35b-a3b-nvfp4": dict(cfg="35b-a3b-nvfp4", T=1, copies=8, steps=2048, warmup=128),
    "decode-284b": dict(cfg="284b", T=1, copies=4, steps=2048, warmup=128),
    "miss-path-284b": dict(cfg="284b-miss-path", T=1, copies=1, steps=64, warmup=64),
    "prefill-753b": dict(cfg="753b", T=4096, copies=1, steps=20, warmup=3),
    "prefill-753b-mxfp4": dict(cfg="753b", T=4096, copies=1, steps=20, warmup=3, mode="mxfp4"),
}
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP4_PEAK_TFLOPS = 10100.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


KERNEL_SOURCES = {
    "decode": ["ft_internal.h", "ft_device.h", "ft_decode.hip"],
    "prefill": ["ft_internal.h", "ft_device.h", "ft_prefill.hip"],
}


def kernel_sources_sha(kind):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "mxfp4_expert_layer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(key, kind):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy) from
    profiles/hbm_traffic.json, or None when the kernel sources changed since the counters
    were taken (or no counters were recorded)."""
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as fh:
            rec = json.load(fh)["kernels"][key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_sha(kind):
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def read_reference(ctx, achieved):
    """This machine's plain HBM read bandwidth (2 GiB streamed, far above the 256 MB Infinity
    Cache; the faster of the library probe's register-load and LDS-copy forms) and the
    kernel's achieved bandwidth as a fraction of it."""
    import torch

    from mxfp4_expert_layer_amd import ft

    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    v = ft.probe_hbm_read(ctx, buf, nbytes, reps=10)
    del buf
    return {"measured_read_GBps": v, "frac_of_measured_read": achieved / v if v > 0 else None}


def host_info():
    """nproc (CPUs this process may run on), the machine's logical CPU count and its model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"nproc": nproc, "logical_cpus": os.cpu_count(), "cpu_model": model}


def cpu_baseline(cfg, x_batches, seconds):
    """Time the float64 oracle (as it stands) on decode steps of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from mxfp4_expert_layer_amd import synth
    from oracle import fp4, moe

    OL = synth.gen_layer(cfg, experts=None)
    # draw the experts the sample touches beforehand: drawing inputs is not oracle work
    n = 0
    todo = []
    for xb in x_batches:
        idx, _, _, _ = moe.route(fp4.bf16_bits_to_f64(xb), OL.router_w, OL.router_b, cfg.k)
        for e in np.unique(idx):
            OL.expert(int(e))
        todo.append(xb)
    from threadpoolctl import threadpool_limits

    def timed(budget):
        t0 = time.perf_counter()
        tokens = steps = 0
        while True:
            xb = todo[steps % len(todo)]
            moe.moe_forward(OL, xb)
            tokens += xb.shape[0]
            steps += 1
            if time.perf_counter() - t0 >= budget or steps >= 4096:
                break
        return tokens, steps, time.perf_counter() - t0

    tokens, n, dt = timed(seconds)
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    # the same oracle on one thread (a third of the time budget)
    with threadpool_limits(limits=1, user_api="blas"):
        t1, n1, dt1 = timed(seconds / 3)
    return {"value": tokens / dt, "unit": "tokens/s", "cores": max(blas) if blas else 1,
            "kind": "oracle", **host_info(),
            "sample": f"{n} steps of {x_batches[0].shape[0]} token(s) ({tokens} tokens) of the "
                      f"same workload, float64 numpy oracle, {dt:.1f} s",
            "single_thread": {"value": t1 / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{n1} steps ({t1} tokens), {dt1:.1f} s"}}


def decode_layer(ctx, cfg, copies, max_tokens):
    from mxfp4_expert_layer_amd.layer import GpuLayer

    log(f"[bench] building {copies} device copies of {cfg.name} (E={cfg.E}, H={cfg.H}, I={cfg.I})")
    return GpuLayer(ctx, cfg, resident=True, max_tokens=max_tokens, copies=copies, threads=16)


def decode_run(ctx, L, cfg, T, K, W, copies, tag):
    """K timed decode steps of T tokens (graph replay, after W eager warm-up steps and one
    untimed replay of every captured graph), the gate/up and down kernels' event-timed
    durations over an eager pass of 64 steps, and the algorithmic bytes behind them."""
    import numpy as np
    import torch

    from mxfp4_expert_layer_amd import ft, synth

    NB = 16
    xh = [synth.gen_tokens(cfg, T, batch=1000 + b) for b in range(NB)]
    xs = [torch.from_numpy(x.view(np.int16)).to("cuda") for x in xh]
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def step(i, s):
        ft.moe_decode(ctx, L.handles[i % copies], xs[i % NB], T, y, s.cuda_stream)

    with torch.cuda.stream(stream):
        for i in range(W):
            step(i, stream)
    torch.cuda.synchronize()

    G = 64

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                step(i, stream)
        return g

    full = capture(G) if K >= G else None
    rest = capture(K % G) if K % G else None
    # one untimed replay of each graph: its first launch uploads it
    for g in (full, rest):
        if g is not None:
            g.replay()
    torch.cuda.synchronize()
    reps = K // G
    t0 = time.perf_counter()
    for _ in range(reps):
        full.replay()
    if rest is not None:
        rest.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"[bench] {tag}: timed {K} steps in {dt * 1e3:.2f} ms")

    # dominant kernel: start/stop events recorded by the gate/up dispatches themselves, over
    # an eager pass of the same steps (events cannot be timed inside a captured graph).  The
    # stream first runs a 250 ms spin kernel, so every step is queued before the GPU reaches
    # it and the steps run back to back as in a replay, whatever the host's launch speed.
    for h in L.handles:
        ft.profile_begin(h, G // copies + 1)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(2.4e9 * 0.25))
        for i in range(G):
            step(i, stream)
    torch.cuda.synchronize()
    gu, dn, nrec = [], [], 0
    for h in L.handles:
        a, b, n = ft.profile_end(h)
        if n:
            gu.append(a * n)
            dn.append(b * n)
            nrec += n
    gate_us = sum(gu) / nrec
    down_us = sum(dn) / nrec

    # distinct experts per step from the library's routing of the same batches
    uniq = []
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    for b in range(NB):
        ft.route(ctx, L.handles[0], xs[b], T, idx, wts, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        uniq.append(len(np.unique(idx.cpu().numpy())) + cfg.n_shared)
    n_exp = float(np.mean(uniq))
    per_weight = 0.5 + 1 / cfg.block          # E2M1 code + one scale byte per block
    gu_bytes_expert = 2 * cfg.I * cfg.H * per_weight
    dn_bytes_expert = cfg.H * cfg.I * per_weight
    router_bytes = cfg.E * cfg.H * 4
    achieved = n_exp * gu_bytes_expert / (gate_us * 1e-6) / 1e9
    step_bytes = n_exp * (gu_bytes_expert + dn_bytes_expert) + router_bytes
    step_s = dt / K
    return dict(tokens_per_s=T * K / dt, steps=K, ms_per_step=step_s * 1e3, xh=xh,
                gate_us=gate_us, down_us=down_us, n_exp=n_exp, achieved=achieved,
                gu_bytes=n_exp * gu_bytes_expert, step_bytes=step_bytes,
                layer_GBps=step_bytes / step_s / 1e9)


def bench_decode(args, wl):
    from mxfp4_expert_layer_amd import ft, synth

    cfg = synth.CONFIGS[wl["cfg"]]
    T = args.tokens or wl["T"]
    copies = args.copies or wl["copies"]
    K = args.steps if args.steps is not None else wl["steps"]
    W = args.warmup if args.warmup is not None else wl["warmup"]
    ctx = ft.Context(0)
    L = decode_layer(ctx, cfg, copies, max(T, 1))
    r = decode_run(ctx, L, cfg, T, K, W, copies, f"{args.workload}-T{T}")
    achieved = r["achieved"]
    res = {
        "metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}-T{T}", "hidden": cfg.H, "intermediate": cfg.I,
                   "experts": cfg.E, "top_k": cfg.k, "shared_experts": cfg.n_shared,
                   "tokens_per_step": T, "weights": cfg.fmt, "layer_copies": copies,
                   "graph_replay": True},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(f"k_gateup@{args.workload}-T{T}", "decode"),
                     "kernel": "k_gateup", "kernel_us": r["gate_us"], "timing": "dispatch-events",
                     "bytes_per_launch": r["gu_bytes"], **read_reference(ctx, achieved)},
        "layer": {"algorithmic_bytes_per_step": r["step_bytes"],
                  "GBps_per_step": r["layer_GBps"],
                  "hbm_frac_per_step": r["layer_GBps"] / HBM_PEAK_GBS,
                  "down_kernel_us": r["down_us"], "distinct_experts_per_step": r["n_exp"]},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(cfg, r["xh"], args.cpu_seconds)
    L.close()
    ctx.close()
    return res


def decode_sweep(ctx, cfg_name, Ts, copies, K=1024, W=64):
    """The decode layer of one class at several token counts: tokens/s and the gate/up
    kernel's and the whole step's fraction of the 8 TB/s HBM peak, per T."""
    from mxfp4_expert_layer_amd import synth

    cfg = synth.CONFIGS[cfg_name]
    L = decode_layer(ctx, cfg, copies, max(Ts))
    out = {}
    for T in Ts:
        r = decode_run(ctx, L, cfg, T, K, W, copies, f"{cfg.name}-T{T}")
        out[f"T{T}"] = {"tokens_per_s": r["tokens_per_s"], "us_per_step": r["ms_per_step"] * 1e3,
                        "gateup_us": r["gate_us"], "down_us": r["down_us"],
                        "gateup_GBps": r["achieved"],
                        "gateup_hbm_frac": r["achieved"] / HBM_PEAK_GBS,
                        "layer_hbm_frac": r["layer_GBps"] / HBM_PEAK_GBS,
                        "distinct_experts": r["n_exp"], "steps": K}
    L.close()
    return out


def bench_miss_path(args, wl):
    """Miss-path decode of single tokens through `--layers` chained layers of the 284B class
    (48-slot pools over one shared pinned store; each layer has its own router draw and pool;
    layer l+1's input is bf16(x_l + y_l)); `--prefetch D` links every layer to the next for
    cross-layer prefetch of up to D predicted experts.  A step is one token through all
    layers; value = tokens/s.  `--residual-scale g` makes layer l+1's input bf16(x_l + g y_l):
    with random weights an expert output is several times its input, so g sets how far the
    input drifts per layer (reported as residual_ratio = |g y| / |x|, measured in warm-up),
    and with it how well the next router on x_l predicts its routing on x_{l+1}."""
    import dataclasses

    import numpy as np
    import torch

    from mxfp4_expert_layer_amd import ft, synth
    from mxfp4_expert_layer_amd.layer import GpuLayer

    cfg = synth.CONFIGS[wl["cfg"]]
    if args.zipf_c is not None:
        cfg = dataclasses.replace(cfg, zipf_c=args.zipf_c)
    K = args.steps if args.steps is not None else wl["steps"]
    W = args.warmup if args.warmup is not None else wl["warmup"]
    NL = max(1, args.layers)
    ctx = ft.Context(0)
    log(f"[bench] building {NL} miss-path layer(s) ({cfg.n_slots} of {cfg.E} slots, pinned store)")
    Ls = [GpuLayer(ctx, cfg, resident=False, n_slots=cfg.n_slots, max_tokens=1, threads=16)]
    for li in range(1, NL):
        router = synth.gen_router(dataclasses.replace(cfg, seed=cfg.seed + 100 * li))
        Ls.append(GpuLayer(ctx, cfg, resident=False, n_slots=cfg.n_slots, max_tokens=1,
                           router=router, host_store=Ls[0].host_blobs))
    bp, bh = ft.measure_bandwidth(ctx, Ls[0].handle)
    log(f"[bench] measured Bp {bp / 1e9:.1f} GB/s, Bh {bh / 1e9:.1f} GB/s")
    disk = None
    if args.disk_dir is not None:
        disk = disk_tier_setup(args, ctx, Ls, cfg)
    rule = {"round": ft.FT_SPLIT_ROUND, "makespan": ft.FT_SPLIT_MAKESPAN,
            "load": ft.FT_SPLIT_LOAD}[args.split]
    for li, L in enumerate(Ls):
        ft.set_bandwidth(L.handle, bp, bh)
        ft.set_miss_policy(L.handle, rule, args.adaptive)
        if args.prefetch > 0 and li + 1 < NL:
            ft.set_prefetch(L.handle, Ls[li + 1].handle, args.prefetch)
    xs = [torch.from_numpy(synth.gen_tokens(cfg, 1, batch=2000 + b).view(np.int16)).to("cuda")
          for b in range(W + K)]
    xl = torch.empty((1, cfg.H), dtype=torch.int16, device="cuda")
    y = torch.empty((1, cfg.H), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    st = ft.DecodeStats()
    tot = dict(hits=0, sel=0, m=0, q=0, streamed=0, host=0, pf=0, pf_hits=0, disk=0)
    disk_us = 0.0
    host_us = wait_us = 0.0
    bp_obs, bh_obs = [], []

    def token(x, count):
        nonlocal host_us, wait_us, disk_us
        for li, L in enumerate(Ls):
            ft.moe_decode(ctx, L.handle, x if li == 0 else xl, 1, y, s, st)
            if li + 1 < NL:
                if ratios is not None:
                    xin = (x if li == 0 else xl).view(torch.bfloat16).float()
                    ratios.append(float(args.residual_scale * y.norm() / xin.norm()))
                ft.residual_bf16(ctx, x if li == 0 else xl, y, cfg.H, xl, s, args.residual_scale)
            if not count:
                continue
            for key, v in (("hits", st.n_hits), ("sel", st.n_selected), ("m", st.n_miss),
                           ("q", st.q), ("streamed", st.n_streamed), ("host", st.n_host),
                           ("pf", st.n_prefetched), ("pf_hits", st.n_prefetch_hits),
                           ("disk", st.n_disk)):
                tot[key] += v
            disk_us += st.disk_us
            host_us += st.host_us
            wait_us += st.wait_us
            if st.bp_obs > 0:
                bp_obs.append(st.bp_obs)
            if st.bh_obs > 0:
                bh_obs.append(st.bh_obs)

    ratios = []     # |g y| / |x| of the first warm-up tokens (syncs; not timed)
    for i in range(W):
        token(xs[i], False)
        if i == 7:
            ratios_w, ratios = ratios, None
    if ratios is not None:
        ratios_w, ratios = ratios, None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        token(xs[W + i], True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    blob = Ls[0].stride
    calls = K * NL
    res = {
        "metric": METRIC, "value": K / dt, "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": dt / K * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "hidden": cfg.H, "intermediate": cfg.I,
                   "experts": cfg.E, "top_k": cfg.k, "shared_experts": cfg.n_shared,
                   "slots": cfg.n_slots, "zipf_c": cfg.zipf_c, "weights": cfg.fmt,
                   "layers": NL, "prefetch_depth": args.prefetch,
                   "residual_scale": args.residual_scale},
        "miss_path": {"Bp_GBps": bp / 1e9, "Bh_GBps": bh / 1e9,
                      "hit_rate": tot["hits"] / max(1, tot["sel"]),
                      "mean_m": tot["m"] / calls, "mean_q": tot["q"] / calls,
                      "streamed": tot["streamed"], "host_computed": tot["host"],
                      "prefetched": tot["pf"], "prefetch_hits": tot["pf_hits"],
                      "residual_ratio": float(np.mean(ratios_w)) if ratios_w else None,
                      "pcie_GBps": (tot["streamed"] + tot["pf"]) * blob / dt / 1e9,
                      "host_GBps": tot["host"] * blob / max(host_us * 1e-6, 1e-9) / 1e9,
                      "mean_host_us": host_us / calls, "mean_wait_us": wait_us / calls,
                      "split_rule": args.split, "adaptive_alpha": args.adaptive,
                      "final_Bp_GBps": st.bp / 1e9, "final_Bh_GBps": st.bh / 1e9,
                      "final_t_gpu_us": st.t_gpu * 1e6 if args.split == "load" else None,
                      "median_Bp_obs_GBps": float(np.median(bp_obs)) / 1e9 if bp_obs else None,
                      "median_Bh_obs_GBps": float(np.median(bh_obs)) / 1e9 if bh_obs else None},
        "roofline": None,
    }
    if disk is not None:
        disk.update({"reads": tot["disk"], "reads_per_token": tot["disk"] / K,
                     "read_GBps": tot["disk"] * blob / max(disk_us * 1e-6, 1e-9) / 1e9,
                     "mean_read_ms": disk_us / max(1, tot["disk"]) / 1e3})
        res["config"]["ram_slots"] = args.ram_slots
        res["miss_path"]["disk_tier"] = disk
        disk["staged"] = disk["_ftw"].info().staged
        ft.set_disk_tier(Ls[0].handle, None, None, 0)
        disk["_ftw"].close()
        del disk["_ftw"], disk["_ram"]
        os.remove(disk.pop("_path"))
    for L in Ls:
        L.close()
    ctx.close()
    return res


def disk_tier_setup(args, ctx, Ls, cfg):
    """Write layer 0's blobs to an FTW file, time direct reads of random blobs at several
    request sizes, and attach a host-memory tier of --ram-slots pinned slots over the file."""
    import tempfile

    import numpy as np
    import torch

    from mxfp4_expert_layer_amd import ft

    if len(Ls) != 1 or args.prefetch:
        raise SystemExit("--disk-dir runs one layer without prefetch")
    L = Ls[0]
    d = tempfile.mkdtemp(prefix="ftw_", dir=args.disk_dir)
    path = os.path.join(d, "layer.ftw")
    store = L.host_blobs.numpy()
    shared = np.zeros(cfg.n_shared * L.stride, dtype=np.uint8)
    from mxfp4_expert_layer_amd import synth
    for s_ in range(cfg.n_shared):
        ft.pack_expert_into(cfg.fmt, cfg.H, cfg.I, synth.gen_expert(cfg, s_, shared=True),
                            shared[s_ * L.stride:(s_ + 1) * L.stride])
    both = np.concatenate([store, shared]) if cfg.n_shared else store
    t0 = time.perf_counter()
    ft.ftw_write(path, cfg.fmt, cfg.H, cfg.I, cfg.E, cfg.n_shared, both, L.stride)
    write_s = time.perf_counter() - t0
    del both
    f = ft.Ftw(path, direct=True)
    inf = f.info()
    log(f"[bench] FTW file {inf.file_bytes / 1e9:.2f} GB written in {write_s:.1f} s; "
        f"direct={inf.direct}")
    # request-size sweep: 24 random blobs into plain aligned memory, per request size
    rng = np.random.default_rng(5)
    n = 24
    raw = np.empty(n * L.stride + 4096, dtype=np.uint8)
    dst = raw[(-raw.ctypes.data) % 4096:][:n * L.stride]
    sweep = {}
    for chunk in (0, 1 << 20, 1 << 16, 1 << 12):
        ids = rng.choice(cfg.E, n, replace=False)
        sec = f.read(ids, dst, L.stride, chunk=chunk, ctx=ctx)
        sweep["whole_blob" if chunk == 0 else f"{chunk // 1024}KiB"] = n * L.stride / sec / 1e9
    log(f"[bench] direct reads GB/s by request size: {sweep}")
    del raw
    keep = torch.empty(args.ram_slots * L.stride + 4096, dtype=torch.uint8, pin_memory=True)
    off = (-keep.data_ptr()) % 4096
    ram = keep[off:off + args.ram_slots * L.stride]
    ft.set_disk_tier(L.handle, f, ram, args.ram_slots)
    return {"file_GB": inf.file_bytes / 1e9, "direct": inf.direct, "write_s": write_s,
            "read_GBps_by_request": sweep, "_ftw": f, "_ram": (keep, ram), "_path": path}


def cpu_baseline_prefill(cfg, x, seconds, mode="exact"):
    """The float64 oracle on a sample of the prefill tokens (experts drawn beforehand): the
    sample's distinct experts are evaluated on `threads` host threads (one per expert at a
    time, numpy's BLAS held to one thread each, so `cores` is the threads used).  The "mxfp4"
    mode requantises every selected expert's weights, so its sample is one token."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from mxfp4_expert_layer_amd import synth
    from oracle import fp4, moe

    info = host_info()
    threads = max(1, min(16, info["nproc"] or 1))
    OL = synth.gen_layer(cfg, experts=None)
    n_tok = 4 if mode == "exact" else 1
    xs = x[:n_tok]
    idx, _, _, _ = moe.route(fp4.bf16_bits_to_f64(xs), OL.router_w, OL.router_b, cfg.k)
    for e in np.unique(idx):
        OL.expert(int(e))
    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        reps = 0
        while True:
            moe.moe_forward(OL, xs, mode=mode, threads=threads)
            reps += 1
            if time.perf_counter() - t0 >= seconds or reps >= 64:
                break
        dt = time.perf_counter() - t0
    return {"value": reps * n_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            **info,
            "sample": f"{reps} x {n_tok} of the 4096 prefill tokens ({len(np.unique(idx))} "
                      f"experts; float64 numpy oracle, mode {mode}, {dt:.1f} s)"}


def prefill_run(ctx, L, cfg, T, K, W, s1, workload):
    """K timed ft_moe_prefill calls of T tokens (after W untimed ones) in one mode, then the
    two grouped GEMMs' event-timed durations over K more calls."""
    import numpy as np
    import torch

    from mxfp4_expert_layer_amd import ft, synth

    xh = [synth.gen_tokens(cfg, T, batch=b) for b in range(2)]
    xs = [torch.from_numpy(x.view(np.int16)).to("cuda") for x in xh]
    y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    mode = ft.FT_PREFILL_MXFP4 if s1 else ft.FT_PREFILL_EXACT
    nbytes = ft.moe_prefill_workspace_size(L.handle, T, mode)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for i in range(W):
        ft.moe_prefill(ctx, L.handle, xs[i % 2], T, y, mode, ws, nbytes, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ft.moe_prefill(ctx, L.handle, xs[i % 2], T, y, mode, ws, nbytes, s)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"[bench] {workload}: timed {K} prefill steps in {dt * 1e3:.1f} ms")
    ft.profile_begin(L.handle, K)
    for i in range(K):
        ft.moe_prefill(ctx, L.handle, xs[i % 2], T, y, mode, ws, nbytes, s)
    torch.cuda.synchronize()
    gu_us, dn_us, nrec = ft.profile_end(L.handle)
    del ws
    pairs = T * cfg.k
    fl_gu = 2.0 * pairs * 2 * cfg.I * cfg.H
    fl_dn = 2.0 * pairs * cfg.H * cfg.I
    step_s = dt / K
    gu_tf = fl_gu / (gu_us * 1e-6) / 1e12
    peak = FP4_PEAK_TFLOPS if s1 else BF16_PEAK_TFLOPS
    if s1:
        # algorithmic bytes of k_s1_gemm<0>: the gate and up MXFP4 weights of every expert
        # (17/32 byte per weight: code nibble + E8M0 byte per 32), the quantised tokens once,
        # the quantised h written once
        mx = 17.0 / 32.0
        by_gu = cfg.E * 2 * cfg.I * cfg.H * mx + T * cfg.H * mx + pairs * cfg.I * mx
        gbs = by_gu / (gu_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS,
                "traffic": measured_traffic(f"k_s1_gemm<0>@{workload}", "prefill"),
                "kernel": "k_s1_gemm<0> (gate/up + SwiGLU + MXFP4 quantise of h)",
                "kernel_us": gu_us, "bytes_per_launch": by_gu, "flops_per_launch": fl_gu,
                "fp4_mfma_tflops": gu_tf, "fp4_mfma_frac": gu_tf / FP4_PEAK_TFLOPS,
                "timing": "dispatch-events"}
    else:
        roof = {"bound": "mfma", "achieved": gu_tf, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": gu_tf / BF16_PEAK_TFLOPS,
                "traffic": measured_traffic(f"k_xgemm<0>@{workload}", "prefill"),
                "kernel": "k_xgemm<0> (gate/up + SwiGLU)", "kernel_us": gu_us,
                "flops_per_launch": fl_gu, "timing": "dispatch-events"}
    layer = {"flops_per_step": fl_gu + fl_dn,
             "TFLOPs_per_step": (fl_gu + fl_dn) / step_s / 1e12,
             "fp4_peak_frac": (fl_gu + fl_dn) / step_s / 1e12 / FP4_PEAK_TFLOPS,
             "bf16_peak_frac": (fl_gu + fl_dn) / step_s / 1e12 / BF16_PEAK_TFLOPS,
             "down_kernel_us": dn_us,
             "down_TFLOPs": fl_dn / (dn_us * 1e-6) / 1e12,
             # algorithmic FLOPs over the two grouped GEMMs' summed kernel time
             "grouped_gemm_TFLOPs": (fl_gu + fl_dn) / ((gu_us + dn_us) * 1e-6) / 1e12,
             "grouped_gemm_peak_frac": (fl_gu + fl_dn) / ((gu_us + dn_us) * 1e-6) / 1e12 / peak,
             "peak_TFLOPs": peak}
    return dict(tokens_per_s=T * K / dt, ms_per_step=step_s * 1e3, roofline=roof, layer=layer,
                xh=xh)


def prefill_config(cfg, T, workload, s1):
    return {"workload": workload, "tokens": T, "hidden": cfg.H, "intermediate": cfg.I,
            "experts": cfg.E, "top_k": cfg.k, "weights": cfg.fmt,
            "mode": "mxfp4-scaled-fp4-mfma" if s1 else "exact-bf16-mfma"}


def bench_prefill(args, wl):
    from mxfp4_expert_layer_amd import ft, synth
    from mxfp4_expert_layer_amd.layer import GpuLayer

    cfg = synth.CONFIGS[wl["cfg"]]
    T = args.tokens or wl["T"]
    K = args.steps if args.steps is not None else wl["steps"]
    W = args.warmup if args.warmup is not None else wl["warmup"]
    ctx = ft.Context(0)
    s1 = wl.get("mode") == "mxfp4"
    log(f"[bench] building {cfg.name} (E={cfg.E}, H={cfg.H}, I={cfg.I}, {cfg.fmt})")
    L = GpuLayer(ctx, cfg, resident=True, max_tokens=1, threads=16, prefill_mxfp4=s1)
    r = prefill_run(ctx, L, cfg, T, K, W, s1, args.workload)
    roof = r["roofline"]
    if s1:
        roof.update(read_reference(ctx, roof["achieved"]))
    res = {
        "metric": METRIC, "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4" if s1 else "bf16", "data": "synthetic",
        "config": prefill_config(cfg, T, args.workload, s1),
        "roofline": roof, "layer": r["layer"],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline_prefill(cfg, r["xh"][0], args.cpu_seconds,
                                                   "mxfp4" if s1 else "exact")
    L.close()
    ctx.close()
    return res


def bench_headline(args):
    """The default line: the 753B-class prefill of 4096 tokens in the exact mode (bf16
    activations, bf16 MFMA) is `value`, with its gate/up grouped GEMM as the roofline kernel.
    The same run adds the scaled-FP4 mode of that layer (tokens/s, its gate/up kernel's HBM
    and FP4 MFMA fractions, both grouped GEMMs' FP4 fraction), the 284B-class decode at 1,
    4 and 16 tokens per step (tokens/s and HBM fractions), the 35B-A3B-class decode at 1 and
    8 tokens per step in both weight formats, and the 284B-class miss path (48 of
    256 experts in the pool, Zipf c = 0.7 so that the hit rate falls in 60-90%; tokens/s, hit
    rate, m, q, Bp, Bh), as extra keys."""
    from mxfp4_expert_layer_amd import ft, synth
    from mxfp4_expert_layer_amd.layer import GpuLayer

    wl = WORKLOADS["prefill-753b"]
    cfg = synth.CONFIGS[wl["cfg"]]
    T = wl["T"]
    K = args.steps if args.steps is not None else wl["steps"]
    W = args.warmup if args.warmup is not None else wl["warmup"]
    ctx = ft.Context(0)
    log(f"[bench] building {cfg.name} (E={cfg.E}, H={cfg.H}, I={cfg.I}, {cfg.fmt}) with its "
        f"MXFP4 transcode")
    L = GpuLayer(ctx, cfg, resident=True, max_tokens=1, threads=16, prefill_mxfp4=True)
    r0 = prefill_run(ctx, L, cfg, T, K, W, False, "prefill-753b")
    r1 = prefill_run(ctx, L, cfg, T, K, W, True, "prefill-753b-mxfp4")
    L.close()
    del L
    ref = read_reference(ctx, r1["roofline"]["achieved"])
    r1["roofline"].update(ref)
    Ts = (1, 4, 16)
    dec = decode_sweep(ctx, "284b", Ts, copies=4)
    for v in dec.values():
        v["gateup_frac_of_measured_read"] = v["gateup_GBps"] / ref["measured_read_GBps"]
    res = {
        "metric": METRIC, "value": r0["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": r0["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": prefill_config(cfg, T, "prefill-753b-T4096", False),
        "roofline": r0["roofline"], "layer": r0["layer"],
        "prefill_mxfp4": {"tokens_per_s": r1["tokens_per_s"], "ms_per_step": r1["ms_per_step"],
                          "dtype": "mxfp4", "roofline": r1["roofline"], "layer": r1["layer"]},
        "decode_284b": {"config": {"hidden": 4096, "intermediate": 2048, "experts": 256,
                                   "top_k": 6, "shared_experts": 1, "weights": "mxfp4",
                                   "layer_copies": 4, "graph_replay": True},
                        "measured_read_GBps": ref["measured_read_GBps"], **dec},
    }
    for name, key in (("35b-a3b", "decode_35b_a3b"), ("35b-a3b-nvfp4", "decode_35b_a3b_nvfp4")):
        c35 = synth.CONFIGS[name]
        d35 = decode_sweep(ctx, name, (1, 8), copies=8)
        for v in d35.values():
            v["gateup_frac_of_measured_read"] = v["gateup_GBps"] / ref["measured_read_GBps"]
        res[key] = {"config": {"hidden": c35.H, "intermediate": c35.I, "experts": c35.E,
                               "top_k": c35.k, "shared_experts": c35.n_shared,
                               "weights": c35.fmt, "layer_copies": 8, "graph_replay": True},
                    **d35}
    # the miss path on its own protocol (64 untimed then 64 timed single tokens), in a
    # context of its own
    margs = argparse.Namespace(**vars(args))
    margs.workload, margs.zipf_c, margs.steps, margs.warmup = "miss-path-284b", 0.7, None, None
    mp = bench_miss_path(margs, WORKLOADS["miss-path-284b"])
    res["miss_path_284b"] = {"tokens_per_s": mp["value"], "ms_per_step": mp["ms_per_step"],
                             "steps": mp["steps"], "warmup": mp["warmup"],
                             "config": mp["config"], **mp["miss_path"]}
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline_prefill(cfg, r0["xh"][0], args.cpu_seconds, "exact")
    ctx.close()
    return res


def copy_probe(args):
    """A plain 256 MiB device-to-device copy, repeated: the reference kernel whose FETCH_SIZE
    and WRITE_SIZE counters calibrate the HBM-traffic figures (known bytes per dispatch)."""
    import torch

    nbytes = 256 << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    reps = 8
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return {"metric": "copy probe", "value": 2 * nbytes * reps / dt / 1e9, "unit": "GB/s",
            "bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes, "copies": reps}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="headline", choices=["headline"] + sorted(WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None, help="decode tokens per step")
    ap.add_argument("--copies", type=int, default=None, help="device copies of the layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--zipf-c", type=float, default=None,
                    help="miss path: router bias strength c of b_e = -c ln(rank_e)")
    ap.add_argument("--split", choices=["round", "makespan", "load"], default="round",
                    help="miss path: split rule (round(q*), the makespan variant, or the "
                         "variant that also balances the GPU's measured load)")
    ap.add_argument("--adaptive", type=float, default=0.0,
                    help="miss path: running-average weight for re-measuring Bp, Bh (0: fixed)")
    ap.add_argument("--layers", type=int, default=1,
                    help="miss path: chained layers per token (input of l+1 = bf16(x_l + y_l))")
    ap.add_argument("--prefetch", type=int, default=0,
                    help="miss path: cross-layer prefetch depth (0: off)")
    ap.add_argument("--residual-scale", type=float, default=1.0,
                    help="miss path: input of layer l+1 = bf16(x_l + g * y_l)")
    ap.add_argument("--disk-dir", default=None,
                    help="miss path: put the experts in an FTW file under this directory, with "
                         "a host-memory tier of --ram-slots over it")
    ap.add_argument("--ram-slots", type=int, default=96,
                    help="miss path: host-memory slots over the FTW file")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this layer is built and timed on a single MI355X; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        print(json.dumps(copy_probe(args)), flush=True)
        return
    if args.workload == "headline":
        print(json.dumps(bench_headline(args)), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if args.workload == "miss-path-284b":
        res = bench_miss_path(args, wl)
    elif args.workload.startswith("prefill-"):
        res = bench_prefill(args, wl)
    else:
        res = bench_decode(args, wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
