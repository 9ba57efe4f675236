"""The sparse MoE expert layer in float64 — oracle (test infrastructure only).

What the layer computes (FreeToken pages: a gate picks a few experts per token — mubeitech
explainer, the MoE paragraph; 6 of 256 experts are active per token and the outputs of all
selected experts are merged by routing weight — smzdm explainer a825qpgl, section 二):

  logits  l_t = x_t . W_r^T + b                      (fp64 here; fp32 on the GPU)
  select  S_t = the k largest logits, ties to the lower expert index, in rank order
  weights w_tj = exp(l_j - l_max) / sum_{i in S_t} exp(l_i - l_max)
          (softmax over all E then renormalised over the kept k is the same number)
  expert  g = W_g x, u = W_u x, h = bf16(silu(g) * u), y_e = W_d h,  silu(z) = z/(1+e^-z)
  combine y_t = sum_j w_tj y_{e_j}(x_t) + sum_shared y_s(x_t)   (shared experts weight 1)

Readings where the pages are silent: SwiGLU with separate gate and up matrices and no
biases; h rounded to bf16 (round-to-nearest-even) before the down projection, on both
sides, so every contraction takes bf16-valued inputs; shared experts added with weight 1.

The layer object is duck-typed: ``layer.cfg`` has H, I, E, k, n_shared and fmt ("mxfp4" or
"nvfp4"); ``layer.router_w`` [E][H] and ``layer.router_b`` ([E] or None) are float32;
``layer.expert(e)`` and ``layer.shared[s]`` expose gate/up/down codes and scales (uint8) and
``tensor_scales`` (3 floats, gate/up/down, used by NVFP4).
"""
from __future__ import annotations

import numpy as np

from . import fp4, mxq


def expert_weights(layer, ex):
    """Dequantised (W_g [I][H], W_u [I][H], W_d [H][I]) of one expert, exact in float64."""
    fmt = layer.cfg.fmt
    ts = np.asarray(ex.tensor_scales, dtype=np.float64)
    wg = fp4.dequant(fmt, ex.gate_codes, ex.gate_scales, ts[0])
    wu = fp4.dequant(fmt, ex.up_codes, ex.up_scales, ts[1])
    wd = fp4.dequant(fmt, ex.down_codes, ex.down_scales, ts[2])
    return wg, wu, wd


def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def route(x: np.ndarray, router_w, router_b, k: int):
    """Top-k softmax routing of float64 tokens x [T][H].

    Returns (idx int64 [T][k], w float64 [T][k], logits float64 [T][E], gap float64 [T]);
    gap is l_(k) - l_(k+1), the margin between the last kept and first dropped logit
    (inf when k == E)."""
    wr = np.asarray(router_w, dtype=np.float64)
    logits = x @ wr.T
    if router_b is not None:
        logits = logits + np.asarray(router_b, dtype=np.float64)[None, :]
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int64)
    w = np.empty((T, k), dtype=np.float64)
    gap = np.full(T, np.inf)
    ids = np.arange(E)
    for t in range(T):
        order = np.lexsort((ids, -logits[t]))      # logit descending, then index ascending
        sel = order[:k]
        idx[t] = sel
        lmax = logits[t, sel[0]]
        p = np.exp(logits[t, sel] - lmax)
        w[t] = p / p.sum()
        if k < E:
            gap[t] = logits[t, order[k - 1]] - logits[t, order[k]]
    return idx, w, logits, gap


def swiglu_hidden(xs: np.ndarray, wg, wu) -> np.ndarray:
    """silu(W_g x) * (W_u x) on float64 rows xs [n][H], before any rounding of h."""
    g = xs @ wg.T
    u = xs @ wu.T
    return silu(g) * u


def swiglu_ffn(xs: np.ndarray, wg, wu, wd, h_quant=None) -> np.ndarray:
    """SwiGLU expert FFN on float64 rows xs [n][H]; h is rounded to bf16 unless ``h_quant``
    (a function on [n][I] float64 arrays) replaces that rounding."""
    a = swiglu_hidden(xs, wg, wu)
    h = fp4.round_bf16(a) if h_quant is None else h_quant(a)
    return h @ wd.T


def expert_outputs(layer, x: np.ndarray, idx: np.ndarray, mode: str = "exact",
                   threads: int = 1, weights_fn=None):
    """Per-(t, j) expert outputs y_{t,j} [T][k][H] and shared outputs [T][n_shared][H].

    Each selected (token, expert) pair is evaluated by the definition above; tokens sharing
    an expert are evaluated together with one matmul (a library primitive), which changes
    nothing but the order of independent rows.  threads > 1 evaluates distinct experts
    concurrently (each writes only its own rows).  weights_fn(e), when given, supplies routed
    expert e's weights after the mode's weight transform (the caller computes the same values,
    e.g. to check them against another implementation on the way); it is called once per
    expert, from the worker threads."""
    cfg = layer.cfg
    T, k = idx.shape
    ys = np.zeros((T, k, cfg.H))
    x_in, hq, wq = mode_ops(mode)
    xq = x_in(x)

    def one(e):
        tt, jj = np.nonzero(idx == e)
        if weights_fn is not None:
            wg, wu, wd = weights_fn(int(e))
        else:
            wg, wu, wd = wq(expert_weights(layer, layer.expert(int(e))))
        ys[tt, jj] = swiglu_ffn(xq[tt], wg, wu, wd, hq)

    experts = [int(e) for e in np.unique(idx)]
    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as pool:
            list(pool.map(one, experts))
    else:
        for e in experts:
            one(e)
    sh = np.zeros((T, cfg.n_shared, cfg.H))
    for s in range(cfg.n_shared):
        wg, wu, wd = wq(expert_weights(layer, layer.shared[s]))
        sh[:, s] = swiglu_ffn(xq, wg, wu, wd, hq)
    return ys, sh


def combine(w: np.ndarray, ys: np.ndarray, sh: np.ndarray) -> np.ndarray:
    """y_t = sum_j w_tj y_tj + sum_s shared_ts."""
    return np.einsum("tj,tjh->th", w, ys) + sh.sum(axis=1)


def moe_forward(layer, x_bits: np.ndarray, idx=None, mode: str = "exact", threads: int = 1,
                weights_fn=None):
    """The whole layer on bf16 tokens x_bits (uint16 [T][H]).

    ``idx`` overrides the routing choice (its weights are then recomputed from the oracle's
    own logits), which the tests use when a near-tie makes two index sets valid.
    mode "exact" is the bf16-activation layer; "mxfp4" is the S1 variant (see ``mxq``).
    ``weights_fn``: see ``expert_outputs``.
    Returns dict(y, idx, w, logits, gap)."""
    cfg = layer.cfg
    x = fp4.bf16_bits_to_f64(x_bits)
    r_idx, r_w, logits, gap = route(x, layer.router_w, layer.router_b, cfg.k)
    if idx is not None:
        idx = np.asarray(idx, dtype=np.int64)
        sel = np.take_along_axis(logits, idx, axis=1)
        p = np.exp(sel - sel.max(axis=1, keepdims=True))
        r_w = p / p.sum(axis=1, keepdims=True)
        r_idx = idx
    ys, sh = expert_outputs(layer, x, r_idx, mode, threads, weights_fn)
    y = combine(r_w, ys, sh)
    return dict(y=y, idx=r_idx, w=r_w, logits=logits, gap=gap, ys=ys, shared=sh)


def dense_masked_forward(layer, x_bits: np.ndarray):
    """The same layer evaluated densely: every expert on every token, multiplied by a mask
    m_te that is the renormalised routing weight when e is selected and 0 otherwise."""
    cfg = layer.cfg
    x = fp4.bf16_bits_to_f64(x_bits)
    idx, w, _, _ = route(x, layer.router_w, layer.router_b, cfg.k)
    T = x.shape[0]
    mask = np.zeros((T, cfg.E))
    for t in range(T):
        mask[t, idx[t]] = w[t]
    y = np.zeros((T, cfg.H))
    for e in range(cfg.E):
        wg, wu, wd = expert_weights(layer, layer.expert(e))
        y += mask[:, e:e + 1] * swiglu_ffn(x, wg, wu, wd)
    for s in range(cfg.n_shared):
        wg, wu, wd = expert_weights(layer, layer.shared[s])
        y += swiglu_ffn(x, wg, wu, wd)
    return y


def mode_ops(mode):
    """(token transform, h transform or None for bf16 rounding, weight transform) of a mode:
    "exact" is the bf16-activation layer; "mxfp4" quantises x, h and the weights by the OCP
    MX rule (``mxq``)."""
    ident = lambda a: a
    if mode == "exact":
        return ident, None, ident
    if mode == "mxfp4":
        def wq(ws):
            return tuple(mxq.quantize_dequant(w) for w in ws)
        return mxq.quantize_dequant, mxq.quantize_dequant, wq
    raise ValueError(f"unknown mode {mode!r}")


def rel_l2(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (den if den > 0 else 1.0))
