"""Plant plausible mistakes in copies of the oracle and show a pin catches each (CPU only)."""
import math

import numpy as np
import pytest

from oracle import oasis_oracle as O
from tests import oracle_checks as C

B = 16


def meta_off_by_one(K, n):
    N = (n + B - 1) // B
    kmin = np.array([K[b * B: min(b * B + B, n + 1)].min(0) for b in range(N)])
    kmax = np.array([K[b * B: min(b * B + B, n + 1)].max(0) for b in range(N)])
    return kmin, kmax


def meta_whole_block(K, n):
    N = (n + B - 1) // B
    return (np.array([K[b * B: b * B + B].min(0) for b in range(N)]),
            np.array([K[b * B: b * B + B].max(0) for b in range(N)]))


def append_no_reset(kmin, kmax, n, k_new):
    b = n // B
    if n % B == 0:
        kmin = np.vstack([kmin, np.minimum(kmin[-1], k_new)[None]])
        kmax = np.vstack([kmax, np.maximum(kmax[-1], k_new)[None]])
        return kmin, kmax
    return O.block_meta_append(kmin, kmax, n, k_new)


def bound_min(q, kmin, kmax):
    return np.minimum(kmin * q, kmax * q).sum(1)


def bound_scaled(q, kmin, kmax):
    return O.block_bound(q, kmin, kmax) / math.sqrt(len(q))


def bound_swapped(q, kmin, kmax):
    return (np.maximum(q, 0) * kmin + np.minimum(q, 0) * kmax).sum(1)


def score_mean(qd, kmin, kmax):
    rows = np.asarray(qd).reshape(-1, kmin.shape[1])
    return np.mean([O.block_bound(q, kmin, kmax) for q in rows], axis=0)


def score_first_row(qd, kmin, kmax):
    rows = np.asarray(qd).reshape(-1, kmin.shape[1])
    return O.block_bound(rows[0], kmin, kmax)


def select_high_index_ties(score, N, k):
    forced = [0] if N == 1 else [0, N - 1]
    cand = sorted(range(1, N - 1), key=lambda b: (-score[b], -b))
    sel = forced + cand[: k - len(forced)]
    return sel + [-1] * (k - len(sel))


def select_no_newest(score, N, k):
    cand = sorted(range(1, N), key=lambda b: (-score[b], b))
    sel = [0] + cand[: k - 1]
    return sel + [-1] * (k - len(sel))


def select_ascending(score, N, k):
    forced = [0] if N == 1 else [0, N - 1]
    cand = sorted(range(1, N - 1), key=lambda b: (score[b], b))
    sel = forced + cand[: k - len(forced)]
    return sel + [-1] * (k - len(sel))


def _diff_variant(victim_from_head=False, lowest_missing_first=False, free_desc=False):
    def diff(sel, score, b2s_in, s2b_in, cap):
        k = len(s2b_in)
        b2s = np.array(b2s_in).copy()
        s2b = np.array(s2b_in).copy()
        S = [b for b in sel if b >= 0]
        missing = [b for b in S if b2s[b] < 0]
        if lowest_missing_first:
            missing = missing[::-1]
        F = missing[: min(cap, len(missing))]
        free = [s for s in range(k) if s2b[s] < 0]
        if free_desc:
            free = free[::-1]
        need = max(0, len(F) - len(free))
        outside = [int(s2b[s]) for s in range(k) if s2b[s] >= 0 and s2b[s] not in S]
        ranked = sorted(outside, key=lambda b: O.order_key(score[b], b))
        V = (ranked if victim_from_head else ranked[::-1])[:need]
        targets = free[: min(len(F), len(free))] + [int(b2s[v]) for v in V]
        for v in V:
            b2s[v] = -1
        for b, s in zip(F, targets):
            s2b[s] = b
            b2s[b] = s
        return O.DiffResult(list(zip(F, targets)), V, b2s, s2b)
    return diff


def attn_unscaled(q, K, V, blocks, n):
    d = q.shape[-1]
    return O.sparse_attention(np.asarray(q) / math.sqrt(d), K, V, blocks, n)


def attn_mask_off_by_one(q, K, V, blocks, n):
    return O.sparse_attention(q, K, V, blocks, n + 1)


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _lru_variant(newest_first=False, index_ties=False, no_stamp=False, stamp_all=False):
    def f(sel, score, b2s, s2b, last_use, cap, step):
        r = O.resident_diff_cap_evict_lru(sel, score, b2s, s2b, last_use, cap, step)
        if not (newest_first or index_ties):
            lu = r.last_use
        if newest_first or index_ties:
            k = len(s2b)
            S = {int(b) for b in sel if b >= 0}
            outside = [int(s2b[s]) for s in range(k) if s2b[s] >= 0 and int(s2b[s]) not in S]
            if newest_first:
                key = lambda b: (-int(last_use[b2s[b]]), float(score[b]) + 0.0, -b)  # noqa: E731
            else:
                key = lambda b: (int(last_use[b2s[b]]), b)  # noqa: E731
            V = sorted(outside, key=key)[: len(r.evict)]
            b2 = np.array(b2s).copy()
            s2 = np.array(s2b).copy()
            F = [f for f, _ in r.fetch]
            free = [s for s in range(k) if s2[s] < 0]
            tg = free[: min(len(F), len(free))] + [int(b2[v]) for v in V]
            for v in V:
                b2[v] = -1
            for b, s in zip(F, tg):
                s2[s] = b
                b2[b] = s
            lu = np.array(last_use).copy()
            for b in S:
                if b2[b] >= 0:
                    lu[b2[b]] = step
            return O.DiffResult(fetch=list(zip(F, tg)), evict=V, block_to_slot=b2, slot_to_block=s2, last_use=lu)
        if no_stamp:
            lu = np.array(last_use).copy()
        if stamp_all:
            lu = np.full(len(s2b), step)
        return O.DiffResult(fetch=r.fetch, evict=r.evict, block_to_slot=r.block_to_slot,
                            slot_to_block=r.slot_to_block, last_use=lu)
    return f


def _fails_lru(variant):
    try:
        C.check_diff_lru(O.topk_select, O.resident_diff_cap_evict, variant)
        C.check_diff_lru_worked_example(variant)
    except AssertionError:
        return True
    return False


MUTANTS = [
    ("LRU evicts the newest", lambda: _fails_lru(_lru_variant(newest_first=True))),
    ("LRU ties by block index", lambda: _fails_lru(_lru_variant(index_ties=True))),
    ("LRU stamps nothing", lambda: _fails_lru(_lru_variant(no_stamp=True))),
    ("LRU stamps every slot", lambda: _fails_lru(_lru_variant(stamp_all=True))),
    ("meta includes token n", lambda: _fails(C.check_meta_brute, meta_off_by_one)),
    ("meta ignores context length", lambda: _fails(C.check_meta_brute, meta_whole_block)),
    ("append does not reset a new block", lambda: _fails(C.check_meta_append, O.block_meta, append_no_reset)),
    ("bound takes min", lambda: _fails(C.check_bound_dominates, O.block_meta, bound_min)),
    ("bound scaled by 1/sqrt(d)", lambda: _fails(C.check_bound_single_token, O.block_meta, bound_scaled)),
    ("bound pairs q+ with kmin", lambda: _fails(C.check_bound_split_form, O.block_meta, bound_swapped)),
    ("score averages rows", lambda: _fails(C.check_score_max_over_rows, O.block_meta, score_mean)),
    ("score uses one row", lambda: _fails(C.check_score_max_over_rows, O.block_meta, score_first_row)),
    ("ties to higher index", lambda: _fails(C.check_select_brute, select_high_index_ties)),
    ("newest not forced", lambda: _fails(C.check_select_special, select_no_newest)),
    ("ascending ranking", lambda: _fails(C.check_select_brute, select_ascending)),
    ("victims from the head", lambda: _fails(C.check_diff_invariants, O.topk_select,
                                             _diff_variant(victim_from_head=True))),
    ("lowest-ranked missing first", lambda: _fails(C.check_diff_invariants, O.topk_select,
                                                   _diff_variant(lowest_missing_first=True))),
    ("free slots descending", lambda: _fails(C.check_diff_invariants, O.topk_select,
                                             _diff_variant(free_desc=True))),
    ("attention without 1/sqrt(d)", lambda: _fails(C.check_attention_dense, attn_unscaled)),
    ("attention mask off by one", lambda: _fails(C.check_attention_closed_forms, attn_mask_off_by_one)),
]


@pytest.mark.parametrize("name,caught", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, caught):
    assert caught(), f"pin did not catch mutant: {name}"
