"""Chained comparison of the GPU decode chain with the oracle, unit by unit.

Discrete state (selection, fetch list, eviction list, both maps) must match the
oracle bit for bit.  The only admitted difference is a near tie: the GPU scores
in fp32, the oracle in fp64, so blocks whose oracle scores lie within 1e-5
relative of each other at a decision boundary may be ordered either way.  When
the GPU's choice differs from the oracle's only through such a near tie, the
GPU's result is checked for validity against the oracle's scores and the unit's
chain is not compared further (its state legitimately differs from then on).
Attention outputs are compared at every step before that, to max abs 2e-2 and
relative L2 5e-3; scores to the fp32 summation bound.
"""
from __future__ import annotations

import numpy as np

from oracle import oasis_oracle as O
from tests import gpu_util as U
from workload import synth

REL_TIE = 1e-5


def oracle_unit(cfg, l, u):
    H = cfg.kv_heads
    r, h = divmod(u, H)
    ud = synth.unit_data(cfg, r, l, h)
    K0 = ud.keys()
    if cfg.drift_blocks:
        sched = synth.drift_schedule(cfg, r, l, h, ud.planted0)
        Ks = {-1: K0}
        for t in range(cfg.steps):
            Ks[t] = ud.keys(sched[t][2])
        K_at = Ks.__getitem__
    else:
        K_at = lambda t: K0  # noqa: E731
    recs = O.run_unit(K_at=K_at, V=ud.V, queries=ud.queries, drafts_prologue=ud.drafts[0],
                      n0=cfg.ctx, k=cfg.k, cap=cfg.fetch_cap, steps=cfg.steps,
                      initial_slots=lambda S0: synth.initial_residency(cfg, r, l, h, S0),
                      append=cfg.append, max_blocks=cfg.max_blocks)
    return ud, K_at, recs


def _key(score, b):
    return O.order_key(score, b)


def _near(a, b, ref):
    return abs(a - b) <= REL_TIE * max(abs(ref), 1e-30)


def selection_valid(sel_gpu, o_score, k, N):
    """The GPU selection is a valid ranking of the oracle's scores up to near ties."""
    forced = [0] if N == 1 else [0, N - 1]
    S = [int(b) for b in sel_gpu if b >= 0]
    if S[: len(forced)] != forced or len(S) != min(k, N) or len(set(S)) != len(S):
        return False
    cand = S[len(forced):]
    # adjacent order: no inversion beyond a near tie
    for a, b in zip(cand, cand[1:]):
        if _key(o_score[a], a) > _key(o_score[b], b) and not _near(o_score[a], o_score[b], o_score[a]):
            return False
    if not cand:
        return True
    worst = min(o_score[b] for b in cand)
    chosen = set(S)
    for b in range(1, N - 1):
        if b not in chosen and o_score[b] > worst and not _near(o_score[b], worst, worst):
            return False
    return True


def evict_valid(ev_gpu, s2b_before, sel, o_score, need):
    """GPU victims are the lowest-ranked residents outside S up to near ties."""
    S = {int(b) for b in sel if b >= 0}
    outside = [int(b) for b in s2b_before if b >= 0 and int(b) not in S]
    if len(ev_gpu) != need or not set(ev_gpu) <= set(outside):
        return False
    if need == 0:
        return True
    hi = max(o_score[v] for v in ev_gpu)
    for b in outside:
        if b not in ev_gpu and o_score[b] < hi and not _near(o_score[b], hi, hi):
            return False
    return True


def compare_unit(cfg, l, u, gpu_recs, oracle, check_scores=True):
    """Returns dict(compared_steps, diverged_at, reason); raises AssertionError on a real mismatch."""
    ud, K_at, recs = oracle
    d = cfg.head_dim
    stats = {"compared_steps": 0, "diverged_at": None, "reason": None, "attn_max_abs": 0.0,
             "attn_rel_l2": 0.0, "score_max_err_over_tol": 0.0}
    for o in recs:
        t = o.t
        g = gpu_recs[t]
        if t >= 0 and "out" in g:
            ma, rl = U.attn_errors(g["out"].astype(np.float64), o.out)
            stats["attn_max_abs"] = max(stats["attn_max_abs"], ma)
            stats["attn_rel_l2"] = max(stats["attn_rel_l2"], rl)
            assert ma <= U.ATTN_MAX_ABS and rl <= U.ATTN_REL_L2, (l, u, t, ma, rl)
        N = len(o.score)
        assert g["n_scoring"] == o.n_score, (t, g["n_scoring"], o.n_score)
        if check_scores:
            K = K_at(t)
            kmin, kmax = O.block_meta(K.astype(np.float64), o.n_score)
            q = ud.drafts[t + 1].reshape(-1, d).astype(np.float64)
            tol = U.score_tolerance(q, kmin, kmax)
            err = np.abs(g["scores"][:N].astype(np.float64) - o.score)
            stats["score_max_err_over_tol"] = max(stats["score_max_err_over_tol"], float(np.max(err / tol)))
            assert np.all(err <= tol), (l, u, t, float(err.max()))
        stats["compared_steps"] += 1
        sel_g = [int(x) for x in g["sel"]]
        if sel_g != o.sel:
            assert selection_valid(sel_g, o.score, cfg.k, N), (l, u, t, "invalid selection")
            if set(sel_g) != set(o.sel):
                stats["diverged_at"], stats["reason"] = t, "near-tie selection"
                return stats
            # same set, near-tied blocks ranked the other way: harmless unless it
            # changes which missing blocks make the capped fetch list
            stats["order_swaps"] = stats.get("order_swaps", 0) + 1
            missing_g = [b for b in sel_g if b >= 0 and o.slot_to_block_before is not None
                         and b not in set(int(x) for x in o.slot_to_block_before)]
            if [b for b, _ in g["fetch"]] != missing_g[: len(g["fetch"])] or len(g["fetch"]) != len(o.fetch):
                raise AssertionError((l, u, t, "fetch list is not the capped missing prefix"))
            if g["fetch"] != [tuple(p) for p in o.fetch]:
                stats["diverged_at"], stats["reason"] = t, "near-tie order changed the capped fetch"
                return stats
        if g["fetch"] != [tuple(p) for p in o.fetch] or g["evict"] != o.evict:
            same_blocks = [b for b, _ in g["fetch"]] == [b for b, _ in o.fetch]
            if same_blocks and evict_valid(g["evict"], o.slot_to_block_before, o.sel, o.score, len(o.evict)):
                stats["diverged_at"], stats["reason"] = t, "near-tie eviction"
                return stats
            raise AssertionError((l, u, t, "fetch/evict mismatch", g["fetch"], o.fetch, g["evict"], o.evict))
        assert np.array_equal(g["s2b"], o.slot_to_block), (l, u, t, "slot_to_block")
        assert np.array_equal(g["b2s"], o.block_to_slot), (l, u, t, "block_to_slot")
    return stats
