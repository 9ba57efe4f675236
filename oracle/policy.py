"""Miss-path policy: q* split, miss ordering and the LRU slot pool — oracle (test only).

Sources.  The bandwidth-adaptive split sends q* = m * Bp / Bh of a token's m missed experts
over PCIe into GPU slots and computes the rest on host cores in host RAM at the same time,
Bp being the measured PCIe transfer bandwidth and Bh the measured effective host memory
bandwidth (smzdm explainer a825qpgl, section 二, formula and table).  The source-reading
article (lowalt.boxinlu2.cn, section 二) states the same rule as pull : compute =
pcie_bw : (cpu_bw - pcie_bw), because the DMA itself consumes Bp of host memory bandwidth;
solving q / (m - q) = Bp / (Bh - Bp) gives q = m * Bp / Bh.  Experts enter VRAM through a
global LRU slot pool: recently used experts are brought in, cold ones evicted (smzdm
explainer aomxznrn, "FreeToken干的事", item 2).

Readings where the pages are silent:
  * q is the nearest integer to q*, halves rounded up, clamped to [0, m]; Bh <= Bp gives m.
  * misses are ordered by descending routing weight summed over the call's tokens, ties to
    the lower expert id; the first q are streamed, the rest computed on the host.
  * streamed misses are admitted to the pool; host-computed misses are not; hits refresh
    their slot's last-use step.  Admission takes the lowest-index empty slot, else evicts
    the occupied slot with the smallest last-use step among slots not used in this step,
    ties to the lower slot index.  When no slot can be taken the expert is computed on the
    host instead (so at most the number of takeable slots are streamed).

Cross-layer prefetch.  While the GPU computes one layer, the experts the next layer will
probably use are streamed into VRAM in the background, with double buffering (mubeitech
article, closing section; lpnh.cn article, section 2.3, predictive prefetch).  The pages give
no predictor; the reading taken here:
  * the prediction for layer l+1 is layer l+1's own routing (top-k softmax) applied to layer
    l's input;
  * at the next layer's upcoming step n (its call counter), every predicted expert already
    resident has its slot's last use set to n, so no prefetch of that batch evicts it;
  * the predicted experts not resident, in descending summed predicted weight (ties to the
    lower id), are admitted one by one through the same slot rule at step n, at most `depth`
    of them; a prefetched slot's last use is n, so the step-n call cannot evict it either;
  * a step-n hit on a slot filled by a prefetch and not used since counts as a prefetch hit.

Three tiers.  Weights sit on disk, in system memory and in VRAM; the hot ones are in system
memory and the recently used ones in VRAM slots (smzdm explainer aomxznrn, "FreeToken干的事",
items 1 and 2).  The reading for the host-memory tier when it holds fewer than E experts:
  * it is a second pool of the same kind (R slots, its own call counter);
  * every miss of a call's VRAM step needs its blob in host memory (a streamed miss is
    copied from there, a host-computed one is computed there): in miss order, the ones
    already there have their last use set to the call's counter first, then the others are
    read from disk into slots taken by the same slot rule at that counter.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def qstar_split(m: int, Bp: float, Bh: float):
    """(q, q*) for m misses at PCIe bandwidth Bp and host bandwidth Bh."""
    if m < 0 or not (Bp > 0) or not (Bh > 0):
        raise ValueError("need m >= 0, Bp > 0, Bh > 0")
    qstar = m * Bp / Bh
    q = int(math.floor(qstar + 0.5))
    return max(0, min(m, q)), qstar


def qstar_makespan(m: int, Bp: float, Bh: float) -> int:
    """Variant (reported, not the contract): the integer q minimising the finishing time
    max(q / Bp, (m - q) / (Bh - Bp)) of the two concurrent sides; lowest q on ties."""
    if m < 0 or not (Bp > 0) or not (Bh > 0):
        raise ValueError("need m >= 0, Bp > 0, Bh > 0")
    if Bh <= Bp:
        return m
    cost = [max(q / Bp, (m - q) / (Bh - Bp)) for q in range(m + 1)]
    return int(np.argmin(cost))


def qstar_load(m: int, g0: int, Bp: float, Bh: float, blob: float, t_gpu: float) -> int:
    """Variant with the GPU's load (mubeitech explainer: the balancing watches the PCIe
    bandwidth, the CPU's compute and the GPU's load, so that the two sides finish at the same
    moment).  The integer q in [0, m] minimising max(T_gpu(q), T_host(q)), lowest q on ties:
      T_gpu(q)  = max(g0 t_gpu, q blob / Bp) + q t_gpu: the GPU runs the g0 experts it holds
                  while the q copies stream, then the q streamed experts, t_gpu seconds each;
      T_host(q) = (m - q) blob / (Bh - Bp): the host experts, the copies taking Bp of the
                  host's memory bandwidth.
    Bh <= Bp gives m; t_gpu = 0 is the makespan variant."""
    if m < 0 or g0 < 0 or not (Bp > 0) or not (Bh > 0) or not (blob > 0) or not (t_gpu >= 0):
        raise ValueError("need m, g0 >= 0, Bp, Bh, blob > 0, t_gpu >= 0")
    if Bh <= Bp:
        return m
    cost = [max(max(g0 * t_gpu, q * blob / Bp) + q * t_gpu, (m - q) * blob / (Bh - Bp))
            for q in range(m + 1)]
    return int(np.argmin(cost))


def order_misses(misses, weight):
    """Misses sorted by descending total routing weight, ties to the lower expert id."""
    return sorted(misses, key=lambda e: (-weight[e], e))


@dataclass
class StepResult:
    step: int
    selected: list
    hits: list
    misses: list
    q: int               # q from the split rule
    streamed: list       # experts copied into slots this step (admitted), in order
    host: list           # experts computed on the host this step
    evicted: list        # (slot, expert) pairs evicted this step
    e2s: np.ndarray = field(repr=False, default=None)
    s2e: np.ndarray = field(repr=False, default=None)
    prefetch_hits: int = 0   # hits on slots a prefetch filled and nothing used since


@dataclass
class PrefetchResult:
    step: int            # the pool's upcoming step the prefetch is for
    predicted: list      # distinct predicted experts, in admission order
    admitted: list       # experts copied into slots, in order
    evicted: list        # (slot, expert) pairs evicted
    e2s: np.ndarray = field(repr=False, default=None)
    s2e: np.ndarray = field(repr=False, default=None)


class LruPool:
    """Expert-slot pool with E experts and S slots (the pool starts empty)."""

    def __init__(self, E: int, S: int):
        self.E, self.S = E, S
        self.e2s = np.full(E, -1, dtype=np.int64)
        self.s2e = np.full(S, -1, dtype=np.int64)
        self.last_use = np.full(S, -1, dtype=np.int64)
        self.pref = np.zeros(S, dtype=bool)   # filled by a prefetch, not used since
        self.step_no = 0

    def _take_slot(self, step: int):
        empty = np.nonzero(self.s2e < 0)[0]
        if empty.size:
            return int(empty[0]), None
        cand = [s for s in range(self.S) if self.last_use[s] < step]
        if not cand:
            return None, None
        s = min(cand, key=lambda s: (self.last_use[s], s))
        return s, int(self.s2e[s])

    def step(self, idx: np.ndarray, w: np.ndarray, Bp: float, Bh: float, q_override=None,
             rule: str = "round"):
        """One decode call: idx/w [T][k] routing of its tokens; rule "round" (the contract's
        q = round(q*)) or "makespan" (the variant)."""
        step = self.step_no
        weight = {}
        for t in range(idx.shape[0]):
            for j in range(idx.shape[1]):
                e = int(idx[t, j])
                weight[e] = weight.get(e, 0.0) + float(w[t, j])
        selected = sorted(weight)
        hits = [e for e in selected if self.e2s[e] >= 0]
        prefetch_hits = 0
        for e in hits:
            s = self.e2s[e]
            self.last_use[s] = step
            prefetch_hits += int(self.pref[s])
            self.pref[s] = False
        misses = order_misses([e for e in selected if self.e2s[e] < 0], weight)
        m = len(misses)
        if q_override is not None:
            q = max(0, min(m, q_override))
        elif rule == "makespan":
            q = qstar_makespan(m, Bp, Bh)
        elif rule == "load":
            raise ValueError("the load rule needs g0, blob and t_gpu: pass q_override")
        else:
            q = qstar_split(m, Bp, Bh)[0]
        streamed, host, evicted = [], [], []
        for n, e in enumerate(misses):
            if n >= q:
                host.append(e)
                continue
            s, old = self._take_slot(step)
            if s is None:
                host.append(e)
                continue
            if old is not None:
                self.e2s[old] = -1
                evicted.append((s, old))
            self.s2e[s] = e
            self.e2s[e] = s
            self.last_use[s] = step
            self.pref[s] = False
            streamed.append(e)
        self.step_no += 1
        return StepResult(step, selected, hits, misses, q, streamed, host, evicted,
                          self.e2s.copy(), self.s2e.copy(), prefetch_hits)

    def prefetch(self, idx: np.ndarray, w: np.ndarray, depth: int):
        """Prefetch before this pool's next step: idx/w [T][k] the predicted routing."""
        step = self.step_no
        weight = {}
        for t in range(idx.shape[0]):
            for j in range(idx.shape[1]):
                e = int(idx[t, j])
                weight[e] = weight.get(e, 0.0) + float(w[t, j])
        order = order_misses(list(weight), weight)
        for e in order:
            if self.e2s[e] >= 0:
                self.last_use[self.e2s[e]] = step
        admitted, evicted = [], []
        for e in order:
            if len(admitted) >= depth:
                break
            if self.e2s[e] >= 0:
                continue
            s, old = self._take_slot(step)
            if s is None:
                break
            if old is not None:
                self.e2s[old] = -1
                evicted.append((s, old))
            self.s2e[s] = e
            self.e2s[e] = s
            self.last_use[s] = step
            self.pref[s] = True
            admitted.append(e)
        return PrefetchResult(step, order, admitted, evicted, self.e2s.copy(), self.s2e.copy())


@dataclass
class TierResult:
    needed: list         # experts the call needed from this tier, in order
    loaded: list         # of those, read from the tier below (disk), in order
    evicted: list        # (slot, expert) pairs evicted
    e2s: np.ndarray = field(repr=False, default=None)
    s2e: np.ndarray = field(repr=False, default=None)


def tier_step(pool: LruPool, needed):
    """One call's use of a lower tier (host memory over disk): `needed` in order."""
    step = pool.step_no
    for e in needed:
        if pool.e2s[e] >= 0:
            pool.last_use[pool.e2s[e]] = step
    loaded, evicted = [], []
    for e in needed:
        if pool.e2s[e] >= 0:
            continue
        s, old = pool._take_slot(step)
        if s is None:
            raise ValueError("host-memory tier smaller than one call's misses")
        if old is not None:
            pool.e2s[old] = -1
            evicted.append((s, old))
        pool.s2e[s] = e
        pool.e2s[e] = s
        pool.last_use[s] = step
        loaded.append(e)
    pool.step_no += 1
    return TierResult(list(needed), loaded, evicted, pool.e2s.copy(), pool.s2e.copy())
