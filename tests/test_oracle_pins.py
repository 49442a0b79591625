"""Pins of the CPU oracle (CPU only)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import oasis_oracle as O
from tests import oracle_checks as C
from workload import CONFIGS, synth


def test_meta_brute():
    C.check_meta_brute(O.block_meta)
    C.check_meta_brute(O.block_meta, seed=11, n=16, d=3)
    C.check_meta_brute(O.block_meta, seed=12, n=1, d=3)


def test_meta_append_equals_rebuild():
    C.check_meta_append(O.block_meta, O.block_meta_append)


def test_bound_dominates_every_token():
    C.check_bound_dominates(O.block_meta, O.block_bound)


def test_bound_exact_on_one_token_block():
    C.check_bound_single_token(O.block_meta, O.block_bound)


def test_bound_split_positive_negative_form():
    C.check_bound_split_form(O.block_meta, O.block_bound)


def test_bound_zero_query_and_homogeneity():
    C.check_bound_zero_and_homogeneous(O.block_meta, O.block_bound)


def test_score_is_max_over_drafts_and_group():
    C.check_score_max_over_rows(O.block_meta, O.lookahead_score)


def test_select_brute_force():
    C.check_select_brute(O.topk_select)


def test_select_special_cases():
    C.check_select_special(O.topk_select)


@settings(max_examples=150, deadline=None)
@given(st.lists(st.sampled_from([-2.0, -0.0, 0.0, 0.5, 1.0, 4.0]), min_size=1, max_size=40),
       st.integers(2, 12))
def test_select_hypothesis(scores, k):
    s = np.array(scores)
    N = len(s)
    got = O.topk_select(s, N, k)
    assert got == C.brute_select(s, N, k)
    S = [b for b in got if b >= 0]
    assert len(S) == min(k, N) and len(set(S)) == len(S)
    assert 0 in S and (N - 1) in S


def test_diff_invariants():
    C.check_diff_invariants(O.topk_select, O.resident_diff_cap_evict)


def test_diff_lru_pins():
    C.check_diff_lru(O.topk_select, O.resident_diff_cap_evict, O.resident_diff_cap_evict_lru)


def test_diff_lru_worked_example():
    C.check_diff_lru_worked_example(O.resident_diff_cap_evict_lru)


def test_diff_worked_example():
    C.check_diff_worked_example(O.resident_diff_cap_evict)


def test_attention_dense_equivalence():
    C.check_attention_dense(O.sparse_attention)


def test_attention_closed_forms():
    C.check_attention_closed_forms(O.sparse_attention)


# ------------------------------------------------------------- chain pins
def _chain(cfg, r=0, l=0, h=0, with_attention=True, eviction="score"):
    ud = synth.unit_data(cfg, r, l, h)
    K = ud.keys()
    return ud, K, O.run_unit(
        K_at=lambda t: K, V=ud.V, queries=ud.queries, drafts_prologue=ud.drafts[0],
        n0=cfg.ctx_of(r), k=cfg.k, cap=cfg.fetch_cap, steps=cfg.steps,
        initial_slots=lambda S0: synth.initial_residency(cfg, r, l, h, S0),
        append=cfg.append, max_blocks=cfg.max_blocks, with_attention=with_attention, eviction=eviction)


def _check_chain_invariants(cfg, recs):
    prev_res = None
    for rec in recs:
        R = {int(b) for b in rec.slot_to_block if b >= 0}
        F = [b for b, _ in rec.fetch]
        assert len(F) <= cfg.fetch_cap
        if prev_res is not None:
            assert not (set(F) & prev_res)
        S = [b for b in rec.sel if b >= 0]
        if rec.n_missing <= cfg.fetch_cap:
            assert set(S) <= R
            if len(R) == cfg.k:
                assert R == set(S) or len(S) < cfg.k
        prev_res = R


def test_chain_tiny_invariants():
    cfg = CONFIGS["tiny"]
    ud, K, recs = _chain(cfg)
    assert len(recs) == cfg.steps + 1
    _check_chain_invariants(cfg, recs)
    # the planted blocks dominate the ranking (structure of the synthetic input)
    planted = set(int(b) for b in ud.planted0)
    assert planted <= set(recs[-1].sel)


def test_chain_full_budget_is_dense_attention():
    # budget >= context and cap >= missing: the chain converges to all blocks resident and
    # the attention equals dense attention over the whole context.
    cfg = CONFIGS["tiny"].with_(ctx=200, budget_tokens=256, fetch_cap=16, steps=3)
    ud, K, recs = _chain(cfg)
    n = cfg.ctx
    for rec in recs[1:]:
        assert rec.attended and sorted(rec.attended) == list(range((n + 15) // 16))
        q = ud.queries(rec.t)
        ref = C._sdpa(q.astype(np.float64), K[:n].astype(np.float64), ud.V[:n].astype(np.float64))
        np.testing.assert_allclose(rec.out, ref, rtol=1e-10, atol=1e-12)


def test_chain_append_meta_and_newest_forced():
    cfg = CONFIGS["tiny"].with_(ctx=1000, steps=40, append=True, fetch_cap=2)
    ud, K, recs = _chain(cfg, with_attention=False)
    for rec in recs[1:]:
        N = (rec.n_score + 15) // 16
        assert rec.sel[0] == 0 and rec.sel[1] == N - 1
    _check_chain_invariants(cfg, recs)


@pytest.mark.parametrize("cap", [0, 1])
def test_chain_small_cap(cap):
    cfg = CONFIGS["tiny"].with_(fetch_cap=cap, steps=4)
    ud, K, recs = _chain(cfg, with_attention=False)
    _check_chain_invariants(cfg, recs)
    if cap == 0:
        for rec in recs:
            assert rec.fetch == [] and rec.evict == []


@pytest.mark.parametrize("cap", [1, 3, 16])
def test_chain_lru_stamps_are_last_reads(cap):
    """LRU chain: after every step a slot's stamp is the index of the last
    attention that read it (-1 if none has), recomputed here from the attended
    sets alone; every victim is at least as old as every resident block outside
    the selection that stays; the chain invariants hold."""
    cfg = CONFIGS["tiny"].with_(fetch_cap=cap, steps=8, append=True, ctx=1000)
    ud, K, recs = _chain(cfg, with_attention=False, eviction="lru")
    _check_chain_invariants(cfg, recs)
    last = {}
    for a, rec in enumerate(recs):
        # attention a (of step a) reads the selected resident blocks this record leaves
        for b in O.attended_blocks(rec.sel, rec.block_to_slot):
            last[int(rec.block_to_slot[b])] = a
        assert [last.get(s, -1) for s in range(cfg.k)] == [int(x) for x in rec.last_use], a
        if a > 0:
            prev = recs[a - 1].last_use
            S = {b for b in rec.sel if b >= 0}
            before = rec.slot_to_block_before
            stay = [int(x) for x in before if x >= 0 and int(x) not in S and int(x) not in rec.evict]
            slot_of = {int(x): s for s, x in enumerate(before) if x >= 0}
            for v in rec.evict:
                assert all(prev[slot_of[v]] <= prev[slot_of[w]] for w in stay), (a, v)


def test_chain_lru_equals_score_policy_without_eviction_pressure():
    """With a cap that never needs a victim beyond the free slots (cap 0) the
    two eviction policies leave identical chains."""
    cfg = CONFIGS["tiny"].with_(fetch_cap=0, steps=4)
    _, _, a = _chain(cfg, with_attention=False)
    _, _, b = _chain(cfg, with_attention=False, eviction="lru")
    for x, y in zip(a, b):
        assert x.sel == y.sel and x.fetch == y.fetch and x.evict == y.evict
        assert np.array_equal(x.block_to_slot, y.block_to_slot)
