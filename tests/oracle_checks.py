"""Checks that pin the CPU oracle to facts fixed independently of it.

Each check takes the oracle function(s) under test as arguments, so the same
check runs against the real oracle (tests/test_oracle_pins.py) and against
deliberately broken copies of it (tests/test_oracle_mutations.py), which shows
that a plausible mistake in the oracle fails at least one pin.

The facts used: the min/max bound dominates every token's q.k and is exact
for a one-token block; q+ . kmax + q- . kmin is the same bound written another
way; brute-force ordering with Python's sorted and heapq; set algebra of the
resident maps; torch's scaled_dot_product_attention in fp64 on the CPU for
dense attention; one-token and zero-query closed forms.
"""
from __future__ import annotations

import heapq
import math

import numpy as np
import torch

BLOCK = 16


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- O1 meta
def check_meta_brute(block_meta, seed=0, n=53, d=5):
    K = _rand(seed, 64, d)
    K[n:] = 1e9  # tokens at or past n must not be pooled
    kmin, kmax = block_meta(K, n)
    N = (n + BLOCK - 1) // BLOCK
    assert kmin.shape == (N, d) and kmax.shape == (N, d)
    for b in range(N):
        for c in range(d):
            vals = [K[j, c] for j in range(b * BLOCK, min(b * BLOCK + BLOCK, n))]
            lo, hi = vals[0], vals[0]
            for v in vals:
                lo = v if v < lo else lo
                hi = v if v > hi else hi
            assert kmin[b, c] == lo and kmax[b, c] == hi


def check_meta_append(block_meta, block_meta_append, seed=1, n0=13, n1=70, d=4):
    K = _rand(seed, n1, d)
    kmin, kmax = block_meta(K, n0)
    for n in range(n0, n1):
        kmin, kmax = block_meta_append(kmin, kmax, n, K[n])
        rmin, rmax = block_meta(K, n + 1)
        assert np.array_equal(kmin, rmin) and np.array_equal(kmax, rmax)


# ---------------------------------------------------------------- O2 score
def check_bound_dominates(block_meta, block_bound, seed=2, n=45, d=8, trials=20):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        K = rng.standard_normal((n, d)) * rng.uniform(0.1, 3)
        q = rng.standard_normal(d)
        kmin, kmax = block_meta(K, n)
        bnd = block_bound(q, kmin, kmax)
        for j in range(n):
            assert bnd[j // BLOCK] >= float(q @ K[j]) - 1e-12


def check_bound_single_token(block_meta, block_bound, seed=3, d=7):
    # n = 33: block 2 holds one token, so the bound equals q.k exactly.
    K = _rand(seed, 33, d)
    q = _rand(seed + 1, d)
    kmin, kmax = block_meta(K, 33)
    bnd = block_bound(q, kmin, kmax)
    assert math.isclose(bnd[2], float(q @ K[32]), rel_tol=1e-12, abs_tol=1e-12)


def check_bound_split_form(block_meta, block_bound, seed=4, n=40, d=6):
    K = _rand(seed, n, d)
    q = _rand(seed + 1, d)
    q[0] = 0.0
    kmin, kmax = block_meta(K, n)
    bnd = block_bound(q, kmin, kmax)
    for b in range(kmin.shape[0]):
        acc = 0.0
        for c in range(d):
            acc += (q[c] * kmax[b, c]) if q[c] > 0 else (q[c] * kmin[b, c])
        assert math.isclose(bnd[b], acc, rel_tol=1e-12, abs_tol=1e-12)


def check_bound_zero_and_homogeneous(block_meta, block_bound, seed=5, n=48, d=5):
    K = _rand(seed, n, d)
    kmin, kmax = block_meta(K, n)
    assert np.all(block_bound(np.zeros(d), kmin, kmax) == 0.0)
    q = _rand(seed + 1, d)
    for a in (0.5, 2.0, 7.25):
        np.testing.assert_allclose(block_bound(a * q, kmin, kmax), a * block_bound(q, kmin, kmax),
                                   rtol=1e-12, atol=1e-12)


def check_score_max_over_rows(block_meta, lookahead_score, seed=6, n=70, d=4, D=3, G=2):
    K = _rand(seed, n, d)
    qd = _rand(seed + 1, D, G, d)
    kmin, kmax = block_meta(K, n)
    sc = lookahead_score(qd, kmin, kmax)
    for b in range(kmin.shape[0]):
        best = -math.inf
        for t in range(D):
            for g in range(G):
                tot = 0.0
                for c in range(d):
                    tot += max(qd[t, g, c] * kmin[b, c], qd[t, g, c] * kmax[b, c])
                best = max(best, tot)
        assert math.isclose(sc[b], best, rel_tol=1e-12, abs_tol=1e-12)


# ---------------------------------------------------------------- O3 select
def brute_select(score, N, k):
    """Independent statement: forced sink/newest, then the best others."""
    forced = [0] if N == 1 else [0, N - 1]
    others = list(range(1, N - 1))
    want = max(0, min(k - len(forced), len(others)))
    keyed = [((0.0 if score[b] == 0 else -float(score[b])), b) for b in others]
    best = heapq.nsmallest(want, keyed)
    return forced + [b for _, b in best] + [-1] * (k - len(forced) - want)


def check_select_brute(topk_select, seed=7, trials=200):
    rng = np.random.default_rng(seed)
    for i in range(trials):
        N = int(rng.integers(1, 60))
        k = int(rng.integers(2, 20))
        kind = i % 3
        if kind == 0:
            s = rng.standard_normal(N)
        elif kind == 1:
            s = rng.choice([-1.5, -0.0, 0.0, 0.25, 3.0], size=N)
        else:
            s = np.zeros(N)
        got = topk_select(s, N, k)
        assert got == brute_select(s, N, k), (N, k, s)


def check_select_special(topk_select):
    # worked example: forced 0 and 5, then 2 and 3 (tie at 3.0 broken by index)
    assert topk_select(np.array([5.0, 1.0, 3.0, 3.0, 0.5, 2.0]), 6, 4) == [0, 5, 2, 3]
    # all-equal scores (q = 0): forced, then the lowest indices
    assert topk_select(np.zeros(10), 10, 5) == [0, 9, 1, 2, 3]
    # N <= k: every block, rank order, padded
    assert topk_select(np.array([0.0, 2.0, 1.0, 9.0]), 4, 6) == [0, 3, 1, 2, -1, -1]
    assert topk_select(np.array([7.0]), 1, 3) == [0, -1, -1]
    assert topk_select(np.array([7.0, 1.0]), 2, 3) == [0, 1, -1]
    # -0.0 ranks equal to +0.0: lower index first
    assert topk_select(np.array([1.0, 0.0, -0.0, -0.0, 0.0, 1.0]), 6, 4) == [0, 5, 1, 2]
    assert topk_select(np.array([1.0, -0.0, 0.0, 0.0, 1.0]), 5, 4) == [0, 4, 1, 2]
    # the sink and newest are kept even when they score lowest
    assert topk_select(np.array([-9.0, 5.0, 4.0, -9.0]), 4, 3) == [0, 3, 1]


# ---------------------------------------------------------------- O4 diff/cap/evict
def random_maps(rng, N, k, n_res):
    s2b = np.full(k, -1, dtype=np.int64)
    blocks = rng.choice(N, size=min(n_res, N, k), replace=False)
    slots = rng.choice(k, size=len(blocks), replace=False)
    s2b[slots] = blocks
    b2s = np.full(N, -1, dtype=np.int64)
    b2s[blocks] = slots
    return b2s, s2b


def check_diff_invariants(topk_select, diff, seed=8, trials=300):
    rng = np.random.default_rng(seed)
    for i in range(trials):
        N = int(rng.integers(1, 50))
        k = int(rng.integers(2, 16))
        cap = int(rng.choice([0, 1, 3, 1000, int(rng.integers(0, k + 1))]))
        n_res = int(rng.integers(0, k + 1))
        if i % 4 == 0:
            score = rng.choice([0.0, -0.0, 1.0, 2.0], size=N)
        else:
            score = rng.standard_normal(N)
        b2s, s2b = random_maps(rng, N, k, n_res)
        sel = topk_select(score, N, k)
        res = diff(sel, score, b2s, s2b, cap)
        S = [b for b in sel if b >= 0]
        R_old = {int(b) for b in s2b if b >= 0}
        M = [b for b in S if b not in R_old]
        F = [b for b, _ in res.fetch]
        V = list(res.evict)
        free = sorted(s for s in range(k) if s2b[s] < 0)
        assert len(F) == min(cap, len(M)) and F == M[: len(F)]       # highest-ranked missing first
        assert not (set(F) & R_old)                                    # only missing blocks fetched
        assert set(F) <= set(S) and len(F) <= cap
        assert not (set(V) & set(S)) and set(V) <= R_old
        assert len(V) == max(0, len(F) - len(free))
        R_new = {int(b) for b in res.slot_to_block if b >= 0}
        assert R_new == (R_old - set(V)) | set(F)
        assert len(R_new) <= k
        for s in range(k):                                             # maps are inverse
            b = res.slot_to_block[s]
            if b >= 0:
                assert res.block_to_slot[b] == s
        for b in range(N):
            s = res.block_to_slot[b]
            if s >= 0:
                assert res.slot_to_block[s] == b
        # targets: free slots ascending first, then the victims' former slots
        tg = [s for _, s in res.fetch]
        nf = min(len(F), len(free))
        assert tg[:nf] == free[:nf]
        assert tg[nf:] == [int(b2s[v]) for v in V]
        # victims are the lowest-ranked residents outside S
        outside = R_old - set(S)
        kv = lambda b: ((0.0 if score[b] == 0 else -float(score[b])), b)  # noqa: E731
        for v in V:
            for w in outside - set(V):
                assert kv(v) > kv(w)
        assert V == sorted(V, key=kv, reverse=True)
        if cap >= len(M):
            assert set(S) <= R_new


def check_diff_worked_example(diff):
    # k = 4 slots; slot 0 holds block 7, slot 2 holds block 3, slot 3 holds block 5; slot 1 free.
    s2b = np.array([7, -1, 3, 5])
    b2s = np.full(10, -1)
    b2s[7], b2s[3], b2s[5] = 0, 2, 3
    score = np.array([9.0, 1.0, 8.0, 6.0, 4.0, 0.5, 2.0, 0.5, 3.0, 5.0])
    sel = [0, 9, 2, 3]          # missing in rank order: 0, 9, 2 (3 is resident)
    res = diff(sel, score, b2s, s2b, 2)
    # cap 2: fetch 0 and 9; one free slot (1), so one victim: residents outside S are
    # 7 (0.5) and 5 (0.5); tie broken toward evicting the higher index, 7.
    assert res.fetch == [(0, 1), (9, 0)]
    assert res.evict == [7]
    assert list(res.slot_to_block) == [9, 0, 3, 5]
    res = diff(sel, score, b2s, s2b, 3)
    assert res.fetch == [(0, 1), (9, 0), (2, 3)] and res.evict == [7, 5]
    res = diff(sel, score, b2s, s2b, 0)
    assert res.fetch == [] and res.evict == [] and list(res.slot_to_block) == [7, -1, 3, 5]


def check_diff_lru(topk_select, diff, diff_lru, seed=11, trials=300):
    """LRU eviction: with every stamp equal it is the lowest-score policy; with
    random stamps every victim is at least as old as every resident block
    outside S that stays (and at equal stamps ranks after it in the score
    order); the fetch and the maps obey the same rules; the next attention's
    slots carry the step's stamp and no other slot changes."""
    rng = np.random.default_rng(seed)
    for i in range(trials):
        N = int(rng.integers(1, 50))
        k = int(rng.integers(2, 16))
        cap = int(rng.choice([0, 1, 3, 1000, int(rng.integers(0, k + 1))]))
        n_res = int(rng.integers(0, k + 1))
        score = rng.choice([0.0, -0.0, 1.0, 2.0], size=N) if i % 3 == 0 else rng.standard_normal(N)
        b2s, s2b = random_maps(rng, N, k, n_res)
        sel = topk_select(score, N, k)
        step = int(rng.integers(0, 50))
        same = np.full(k, int(rng.integers(-1, 5)))
        a = diff(sel, score, b2s, s2b, cap)
        b = diff_lru(sel, score, b2s, s2b, same, cap, step)
        assert a.fetch == b.fetch and a.evict == b.evict
        assert np.array_equal(a.block_to_slot, b.block_to_slot) and np.array_equal(a.slot_to_block, b.slot_to_block)
        lu = rng.integers(-1, 4, size=k)
        r = diff_lru(sel, score, b2s, s2b, lu, cap, step)
        S = {x for x in sel if x >= 0}
        V = list(r.evict)
        stay = [int(x) for x in s2b if x >= 0 and int(x) not in S and int(x) not in V]
        key = lambda x: (int(lu[b2s[x]]), float(score[x]) + 0.0, -x)
        assert [key(v) for v in V] == sorted(key(v) for v in V)          # eviction order
        for v in V:
            for w in stay:
                assert key(v) < key(w)
        ref = diff(sel, score, b2s, s2b, cap)                            # same fetch list and count
        assert [f for f, _ in r.fetch] == [f for f, _ in ref.fetch] and len(V) == len(ref.evict)
        nxt = {int(r.block_to_slot[x]) for x in S if r.block_to_slot[x] >= 0}
        for s in range(k):
            assert r.last_use[s] == (step if s in nxt else lu[s])
        for s in range(k):                                               # maps are inverse
            x = r.slot_to_block[s]
            if x >= 0:
                assert r.block_to_slot[x] == s


def check_diff_lru_worked_example(diff_lru):
    # the lowest-score worked example above, with stamps: slot 0 (block 7) last read
    # at step 5, slot 2 (block 3) at step 2, slot 3 (block 5) at step 1; slot 1 free
    s2b = np.array([7, -1, 3, 5])
    b2s = np.full(10, -1)
    b2s[7], b2s[3], b2s[5] = 0, 2, 3
    score = np.array([9.0, 1.0, 8.0, 6.0, 4.0, 0.5, 2.0, 0.5, 3.0, 5.0])
    sel = [0, 9, 2, 3]
    lu = np.array([5, -1, 2, 1])
    res = diff_lru(sel, score, b2s, s2b, lu, 2, 6)
    # cap 2: fetch 0 into free slot 1, then 9 into the slot of the least recently
    # read resident block outside S: 5 (stamp 1), where the score policy takes 7
    assert res.fetch == [(0, 1), (9, 3)] and res.evict == [5]
    assert list(res.slot_to_block) == [7, 0, 3, 9]
    assert list(res.last_use) == [5, 6, 6, 6]   # 0, 9 and 3 are read next; 7 keeps its stamp
    res = diff_lru(sel, score, b2s, s2b, lu, 3, 6)
    assert res.fetch == [(0, 1), (9, 3), (2, 0)] and res.evict == [5, 7]
    assert list(res.last_use) == [6, 6, 6, 6]
    res = diff_lru(sel, score, b2s, s2b, lu, 0, 6)
    assert res.fetch == [] and res.evict == [] and list(res.last_use) == [5, -1, 6, 1]


# ---------------------------------------------------------------- O6 attention
def _sdpa(q, K, V):
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64)).reshape(1, 1, -1, q.shape[-1])
    kt = torch.from_numpy(np.asarray(K, dtype=np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(V, dtype=np.float64))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return o.reshape(q.shape).numpy()


def check_attention_dense(sparse_attention, seed=9, n=45, d=16):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n + 11, d)) * 2
    V = rng.standard_normal((n + 11, d))
    q = rng.standard_normal((3, 2, d))
    N = (n + BLOCK - 1) // BLOCK
    out = sparse_attention(q, K, V, list(range(N)), n)
    ref = _sdpa(q, K[:n], V[:n])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # subset of blocks == dense attention over those tokens; block order is irrelevant
    blocks = [2, 0]
    J = [j for b in sorted(blocks) for j in range(b * BLOCK, min(b * BLOCK + BLOCK, n))]
    np.testing.assert_allclose(sparse_attention(q, K, V, blocks, n), _sdpa(q, K[J], V[J]),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sparse_attention(q, K, V, [0, 2], n),
                               sparse_attention(q, K, V, [2, 0], n), rtol=0, atol=1e-15)


def check_attention_closed_forms(sparse_attention, seed=10, d=8):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((40, d))
    V = rng.standard_normal((40, d))
    q = rng.standard_normal((2, d))
    # one valid token (n = 33, block 2): output is that token's value row
    np.testing.assert_allclose(sparse_attention(q, K, V, [2], 33), np.tile(V[32], (2, 1)), atol=1e-15)
    # q = 0: uniform weights, the mean of V over the attended tokens
    np.testing.assert_allclose(sparse_attention(np.zeros((1, d)), K, V, [0, 1], 40),
                               V[:32].mean(axis=0)[None], atol=1e-14)
    assert np.all(sparse_attention(q, K, V, [], 40) == 0)
