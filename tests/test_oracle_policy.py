"""Pins for the oracle's q* split, miss ordering, LRU pool and prefill permutation (CPU)."""
import os

import math

import numpy as np
import pytest

from oracle import perm, policy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qstar_table.txt")


def _qstar_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, bp, bh, pct = line.split()
        rows.append((name, float(bp), float(bh), float(pct)))
    return rows


def test_qstar_reproduces_the_pages_table():
    rows = _qstar_rows()
    assert len(rows) == 4
    for name, bp, bh, pct in rows:
        m = 1000
        _, qstar = policy.qstar_split(m, bp, bh)
        assert round(100.0 * qstar / m, 1) == pct, name


def test_qstar_matches_pull_to_compute_ratio_form():
    """pull : compute = Bp : (Bh - Bp) is the same rule as q* = m Bp / Bh."""
    for _, bp, bh, _ in _qstar_rows():
        for m in (1, 2, 3, 6, 7, 12):
            _, q = policy.qstar_split(m, bp, bh)
            assert q / (m - q) == pytest.approx(bp / (bh - bp), rel=1e-12)


def test_qstar_integer_rule():
    assert policy.qstar_split(0, 50.0, 60.0) == (0, 0.0)
    assert policy.qstar_split(1, 1.0, 2.0)[0] == 1          # 0.5 rounds up
    assert policy.qstar_split(3, 1.0, 2.0)[0] == 2          # 1.5 rounds up
    assert policy.qstar_split(6, 49.0, 53.8)[0] == 5        # 5.465
    assert policy.qstar_split(6, 60.0, 50.0)[0] == 6        # Bh <= Bp: everything streams
    assert policy.qstar_split(6, 1.0, 1e9)[0] == 0
    for bad in ((-1, 1.0, 1.0), (1, 0.0, 1.0), (1, 1.0, 0.0), (1, float("nan"), 1.0)):
        with pytest.raises(ValueError):
            policy.qstar_split(*bad)


def test_makespan_variant_differs_where_expected():
    # the finishing-time variant of the split picks 6 on the 5090 desktop at m = 6
    assert policy.qstar_makespan(6, 49.0, 53.8) == 6
    assert policy.qstar_split(6, 49.0, 53.8)[0] == 5
    assert policy.qstar_makespan(2, 52.7, 77.3) == 2
    assert policy.qstar_makespan(3, 11.8, 47.5) == 0
    assert policy.qstar_split(3, 11.8, 47.5)[0] == 1


def test_makespan_variant_brackets_qstar():
    """Both sides finish together at the continuous optimum of max(q/Bp, (m-q)/(Bh-Bp)):
    q/Bp = (m-q)/(Bh-Bp) solves to q = m Bp / Bh = q*, and the cost falls then rises in q, so
    the best integer is floor(q*) or ceil(q*) (m when Bh <= Bp)."""
    rng = np.random.default_rng(5)
    for _ in range(2000):
        m = int(rng.integers(0, 17))
        Bp = float(rng.uniform(1.0, 100.0))
        Bh = float(rng.uniform(1.0, 120.0))
        q = policy.qstar_makespan(m, Bp, Bh)
        if Bh <= Bp:
            assert q == m
            continue
        qs = m * Bp / Bh
        assert q in (math.floor(qs), math.ceil(qs)), (m, Bp, Bh, q, qs)
    # an exact tie between the two candidates goes to the lower q: m = 1, Bh = 2 Bp
    assert policy.qstar_makespan(1, 1.0, 2.0) == 0


def test_lru_makespan_rule_uses_the_variant():
    P = policy.LruPool(E=8, S=8)
    # 5090 desktop bandwidths, six misses: round gives 5, the makespan variant 6
    r = P.step(np.array([[0, 1, 2, 3, 4, 5]]), np.full((1, 6), 1 / 6), 49.0, 53.8, rule="makespan")
    assert r.q == 6 and len(r.streamed) == 6
    P2 = policy.LruPool(E=8, S=8)
    r2 = P2.step(np.array([[0, 1, 2, 3, 4, 5]]), np.full((1, 6), 1 / 6), 49.0, 53.8)
    assert r2.q == 5 and len(r2.host) == 1


def test_miss_order():
    w = {4: 0.2, 1: 0.5, 9: 0.2, 2: 0.1}
    assert policy.order_misses([4, 1, 9, 2], w) == [1, 4, 9, 2]


def test_lru_scripted_sequence():
    P = policy.LruPool(E=8, S=2)
    r = P.step(np.array([[3, 5]]), np.array([[0.6, 0.4]]), 1.0, 1.0)
    assert r.streamed == [3, 5] and list(r.s2e) == [3, 5] and r.evicted == []
    r = P.step(np.array([[5, 1]]), np.array([[0.7, 0.3]]), 1.0, 1.0)
    assert r.hits == [5] and r.streamed == [1] and r.evicted == [(0, 3)]
    assert list(r.s2e) == [1, 5] and r.e2s[3] == -1
    r = P.step(np.array([[2, 4]]), np.array([[0.5, 0.5]]), 1.0, 1.0)
    assert r.misses == [2, 4] and r.evicted == [(0, 1), (1, 5)] and list(r.s2e) == [2, 4]
    r = P.step(np.array([[6, 2]]), np.array([[0.9, 0.1]]), 1.0, 10.0)
    assert r.hits == [2] and r.q == 0 and r.host == [6] and list(r.s2e) == [2, 4]
    r = P.step(np.array([[7, 6]]), np.array([[0.55, 0.45]]), 1.0, 2.5)
    assert r.q == 1 and r.streamed == [7] and r.host == [6] and r.evicted == [(1, 4)]
    assert list(r.s2e) == [2, 7]


def test_lru_no_takeable_slot_goes_to_host():
    P = policy.LruPool(E=4, S=1)
    r = P.step(np.array([[0, 1]]), np.array([[0.6, 0.4]]), 1.0, 1.0)
    assert r.streamed == [0] and r.host == [1] and r.q == 2


def test_lru_invariants_random():
    rng = np.random.default_rng(3)
    E, S, k = 32, 6, 4
    P = policy.LruPool(E, S)
    for step in range(300):
        T = int(rng.integers(1, 4))
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
        w = rng.random((T, k))
        w /= w.sum(1, keepdims=True)
        bh = float(rng.uniform(0.5, 4.0))
        r = P.step(idx, w, 1.0, bh)
        res = np.nonzero(r.e2s >= 0)[0]
        assert len(res) <= S
        for e in res:
            assert r.s2e[r.e2s[e]] == e
        for s in range(S):
            if r.s2e[s] >= 0:
                assert r.e2s[r.s2e[s]] == s
        sel = set(int(e) for e in idx.ravel())
        parts = [set(r.hits), set(r.streamed), set(r.host)]
        assert set().union(*parts) == sel
        assert sum(len(p) for p in parts) == len(sel)
        for e in r.streamed + r.hits:
            assert r.e2s[e] >= 0


def test_prefetch_scripted_sequence():
    """Worked by hand from the prefetch reading: predicted residents are protected, new ones
    are admitted in weight order up to the depth, and a prefetched slot survives the step it
    was fetched for and counts as a prefetch hit when used."""
    P = policy.LruPool(E=8, S=3)
    r = P.step(np.array([[0, 1]]), np.array([[0.6, 0.4]]), 1.0, 1.0)
    assert list(r.s2e) == [0, 1, -1]
    # predicted weights: 0 -> 1.2, 2 -> 0.5, 3 -> 0.3; 0 is resident and gets protected
    f = P.prefetch(np.array([[2, 0], [3, 0]]), np.array([[0.5, 0.5], [0.3, 0.7]]), depth=2)
    assert f.step == 1 and f.predicted == [0, 2, 3]
    assert f.admitted == [2, 3] and f.evicted == [(1, 1)] and list(f.s2e) == [0, 3, 2]
    # step 1: 2 is a prefetch hit; 4 misses, but every slot was used or fetched for step 1
    r = P.step(np.array([[2, 4]]), np.array([[0.8, 0.2]]), 1.0, 1.0)
    assert r.hits == [2] and r.prefetch_hits == 1 and r.host == [4] and r.streamed == []
    # step 2: 3 (fetched for step 1, unused there) still counts; 5 evicts slot 0 (last use 1,
    # tied with slot 2, lower index)
    r = P.step(np.array([[3, 5]]), np.array([[0.5, 0.5]]), 1.0, 1.0)
    assert r.hits == [3] and r.prefetch_hits == 1 and r.evicted == [(0, 0)]
    assert list(r.s2e) == [5, 3, 2]
    # a used slot is no longer a prefetched one
    r = P.step(np.array([[3, 2]]), np.array([[0.5, 0.5]]), 1.0, 1.0)
    assert r.prefetch_hits == 0
    # depth 0 admits nothing; all-resident predictions admit nothing
    assert P.prefetch(np.array([[7]]), np.array([[1.0]]), depth=0).admitted == []
    assert P.prefetch(np.array([[3, 2]]), np.array([[0.5, 0.5]]), depth=4).admitted == []


def test_prefetch_invariants_random():
    rng = np.random.default_rng(11)
    E, S, k = 24, 5, 3
    P = policy.LruPool(E, S)
    pending = set()          # experts a prefetch brought in that no step has used since
    for it in range(400):
        T = int(rng.integers(1, 3))
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
        w = rng.random((T, k))
        w /= w.sum(1, keepdims=True)
        if rng.random() < 0.5:
            depth = int(rng.integers(0, 4))
            before = set(int(e) for e in np.nonzero(P.e2s >= 0)[0])
            f = P.prefetch(idx, w, depth)
            pred = set(int(e) for e in idx.ravel())
            assert len(f.admitted) <= depth and set(f.admitted) <= pred - before
            for e in pred & before:          # predicted residents are never evicted
                assert f.e2s[e] >= 0
            for e in f.admitted:
                assert f.e2s[e] >= 0 and f.s2e[f.e2s[e]] == e
            pending -= {old for _, old in f.evicted}
            pending |= set(f.admitted)
            continue
        r = P.step(idx, w, 1.0, float(rng.uniform(0.5, 3.0)))
        assert r.prefetch_hits == len(pending & set(r.hits))
        pending -= set(r.hits)
        pending -= {old for _, old in r.evicted}
        for s in range(S):
            if r.s2e[s] >= 0:
                assert r.e2s[r.s2e[s]] == s


def test_host_tier_scripted_sequence():
    """Worked by hand: the host-memory tier under the VRAM pool (3 host slots, 2 VRAM slots)."""
    V, H = policy.LruPool(E=8, S=2), policy.LruPool(E=8, S=3)
    r = V.step(np.array([[3, 5]]), np.array([[0.6, 0.4]]), 1.0, 1.0)
    t = policy.tier_step(H, r.misses)
    assert r.misses == [3, 5] and t.loaded == [3, 5] and list(t.s2e) == [3, 5, -1]
    r = V.step(np.array([[5, 1]]), np.array([[0.7, 0.3]]), 1.0, 1.0)
    t = policy.tier_step(H, r.misses)          # 1 misses VRAM, read into the empty slot 2
    assert r.misses == [1] and t.loaded == [1] and list(t.s2e) == [3, 5, 1]
    r = V.step(np.array([[3, 6]]), np.array([[0.4, 0.6]]), 1.0, 1.0)
    # VRAM held [1, 5]: both miss, 6 first (heavier); host tier: 3 resident (touched at 2),
    # 6 evicts the oldest untouched slot: slot 1 (expert 5, last use 0)
    t = policy.tier_step(H, r.misses)
    assert r.misses == [6, 3] and t.loaded == [6] and t.evicted == [(1, 5)]
    assert list(t.s2e) == [3, 6, 1]
    r = V.step(np.array([[6, 3]]), np.array([[0.5, 0.5]]), 1.0, 1.0)
    t = policy.tier_step(H, r.misses)          # all VRAM hits: nothing needed
    assert r.misses == [] and t.loaded == [] and list(t.s2e) == [3, 6, 1]
    with pytest.raises(ValueError):
        policy.tier_step(policy.LruPool(E=8, S=1), [2, 4])


def test_host_tier_invariants_random():
    rng = np.random.default_rng(5)
    E, S, R, k = 30, 4, 9, 3
    V, H = policy.LruPool(E, S), policy.LruPool(E, R)
    for it in range(300):
        T = int(rng.integers(1, 4))
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
        w = rng.random((T, k))
        r = V.step(idx, w, 1.0, float(rng.uniform(0.5, 3.0)))
        before = set(int(e) for e in np.nonzero(H.e2s >= 0)[0])
        t = policy.tier_step(H, r.misses)
        assert set(t.loaded) == set(r.misses) - before
        for e in r.misses:                    # every miss is in host memory afterwards
            assert t.e2s[e] >= 0 and t.s2e[t.e2s[e]] == e
        assert len(set(int(e) for e in t.s2e if e >= 0)) == int((t.s2e >= 0).sum())


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (7, 2, 5), (64, 8, 16), (200, 6, 256)])
def test_permutation_matches_stable_sort(T, k, E):
    rng = np.random.default_rng(T * 31 + k)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    counts, offsets, pos, rows = perm.permutation(idx, E)
    assert counts.sum() == T * k and offsets[-1] == T * k
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    order = np.argsort(idx.ravel(), kind="stable")       # library stable sort
    assert np.array_equal(rows[:, 0] * k + rows[:, 1], order)
    flat = pos.ravel()
    assert np.array_equal(np.sort(flat), np.arange(T * k))
    for p in range(T * k):
        t, j = rows[p]
        assert pos[t, j] == p
        e = idx[t, j]
        assert offsets[e] <= p < offsets[e + 1]


def test_load_rule_hand_worked():
    """blob = 1, Bp = 1, Bh = 3 (a copy takes 1, a host expert 1/2), m = 6 misses, g0 = 4
    experts already on the GPU.
    t_gpu = 1/4: q = 0: max(1, 0) + 0 = 1 vs 3 -> 3; q = 1: max(1, 1) + 1/4 vs 5/2 -> 5/2;
      q = 2: max(1, 2) + 1/2 vs 2 -> 5/2; q = 3: 3 + 3/4 vs 3/2 -> 15/4: the tie of q = 1 and
      q = 2 goes to q = 1 (the makespan variant, with no GPU term, picks 2: max(2, 2)).
    t_gpu = 1 (a busy GPU): q = 0: max(4, 0) vs 3 -> 4; q = 1: max(4, 1) + 1 -> 5: q = 0."""
    assert policy.qstar_load(6, 4, 1.0, 3.0, 1.0, 0.25) == 1
    assert policy.qstar_makespan(6, 1.0, 3.0) == 2
    assert policy.qstar_load(6, 4, 1.0, 3.0, 1.0, 1.0) == 0
    assert policy.qstar_load(0, 4, 1.0, 3.0, 1.0, 1.0) == 0
    assert policy.qstar_load(5, 0, 2.0, 1.5, 1.0, 0.1) == 5          # Bh <= Bp: every miss streams


def test_load_rule_without_gpu_term_is_the_makespan_variant():
    rng = np.random.default_rng(11)
    for _ in range(300):
        m, g0 = int(rng.integers(0, 20)), int(rng.integers(0, 12))
        Bp, Bh = float(rng.uniform(1, 60)), float(rng.uniform(1, 250))
        assert policy.qstar_load(m, g0, Bp, Bh, 13.4, 0.0) == policy.qstar_makespan(m, Bp, Bh)


def test_load_rule_never_streams_more_than_the_makespan_variant():
    """A GPU term only lengthens the GPU side, so the balance point cannot move toward more
    copies; and a heavier GPU term never streams more."""
    rng = np.random.default_rng(12)
    for _ in range(300):
        m, g0 = int(rng.integers(0, 20)), int(rng.integers(0, 12))
        Bp, Bh = float(rng.uniform(1, 60)), float(rng.uniform(1, 250))
        t1 = float(rng.uniform(0, 0.5))
        t2 = t1 + float(rng.uniform(0, 0.5))
        q1 = policy.qstar_load(m, g0, Bp, Bh, 13.4, t1)
        assert q1 <= policy.qstar_makespan(m, Bp, Bh)
        assert policy.qstar_load(m, g0, Bp, Bh, 13.4, t2) <= q1
