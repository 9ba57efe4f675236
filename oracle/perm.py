"""Prefill permutation by expert — oracle (test infrastructure only).

Prefill and decode get separate strategies, prefill being compute-bound (smzdm explainer
aomxznrn, "FreeToken干的事", item 4); for prefill the (token, expert) pairs are sorted by
expert so each expert's tokens form one contiguous group for a grouped GEMM.  Reading (the
pages are silent on the order): expert ascending, then token ascending (stable).
"""
from __future__ import annotations

import numpy as np


def permutation(idx: np.ndarray, E: int):
    """idx [T][k] -> (counts [E], offsets [E+1], pos [T][k], rows [T*k] of (t, j)).

    counts[e] = number of pairs routed to e; offsets = exclusive prefix sum of counts;
    pos[t][j] = offsets[e] + (number of tokens t' < t routed to e), e = idx[t][j];
    rows[p] = the (t, j) pair placed at position p."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for e in idx.ravel():
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    pos = np.empty((T, k), dtype=np.int64)
    rows = np.empty((T * k, 2), dtype=np.int64)
    fill = offsets[:-1].copy()
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            pos[t, j] = fill[e]
            rows[fill[e]] = (t, j)
            fill[e] += 1
    return counts, offsets, pos, rows
