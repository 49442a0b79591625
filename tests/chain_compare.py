"""Chained comparison of the GPU decode chain with the oracle, unit by unit.

Discrete state (selection, fetch list, eviction list, both maps, LRU stamps)
must match the oracle bit for bit at every step.  The only admitted
difference is a near tie: the GPU scores in fp32, the oracle in fp64, so
blocks whose oracle scores lie within 1e-5 relative of each other at a
decision boundary may be ordered either way.  When the GPU's selection or its
victims differ from the oracle's, the GPU's choice is checked to be a valid
ranking of the oracle's scores up to such near ties; the oracle then adopts it
for that step (the event is counted) and the comparison continues from the
common state, so every unit is compared over every step.  Attention outputs
are compared at every step to max abs 2e-2 and relative L2 5e-3, scores to the
fp32 summation bound.
"""
from __future__ import annotations

import os
from collections import Counter

import numpy as np

from oracle import oasis_oracle as O
from tests import gpu_util as U
from workload import synth

REL_TIE = 1e-5
EVENTS = ("selection_near_tie", "rank_order_near_tie", "eviction_near_tie")


def _near(a, b, ref):
    return abs(a - b) <= REL_TIE * max(abs(ref), 1e-30)


def selection_valid(sel_gpu, o_score, k, N):
    """The GPU selection is a valid ranking of the oracle's scores up to near ties."""
    forced = [0] if N == 1 else [0, N - 1]
    S = [int(b) for b in sel_gpu if b >= 0]
    if S[: len(forced)] != forced or len(S) != min(k, N) or len(set(S)) != len(S):
        return False
    if any(int(b) != -1 for b in sel_gpu[len(S):]) or any(b >= N for b in S):
        return False
    cand = S[len(forced):]
    # adjacent order: no inversion beyond a near tie
    for a, b in zip(cand, cand[1:]):
        if O.order_key(o_score[a], a) > O.order_key(o_score[b], b) and not _near(o_score[a], o_score[b], o_score[a]):
            return False
    if not cand:
        return True
    worst = min(o_score[b] for b in cand)
    chosen = set(S)
    for b in range(1, N - 1):
        if b not in chosen and o_score[b] > worst and not _near(o_score[b], worst, worst):
            return False
    return True


def evict_valid(ev_gpu, s2b_before, sel, o_score, need, key=None):
    """GPU victims are resident blocks outside S, as many as needed, ranked last
    by the eviction order up to near ties of the oracle's scores.  key: the LRU
    order key (stamp first), or None for the lowest-score order."""
    S = {int(b) for b in sel if b >= 0}
    outside = [int(b) for b in s2b_before if b >= 0 and int(b) not in S]
    if len(ev_gpu) != need or len(set(ev_gpu)) != need or not set(ev_gpu) <= set(outside):
        return False
    if need == 0:
        return True
    if key is not None:
        # LRU: stamps are exact integers; only the score part of the key may tie
        stamp = {b: key(b)[0] for b in outside}
        oldest_kept = min((stamp[b] for b in outside if b not in ev_gpu), default=None)
        if oldest_kept is not None and any(stamp[v] > oldest_kept for v in ev_gpu):
            return False
        top = max(stamp[v] for v in ev_gpu)
        boundary = [b for b in outside if stamp[b] == top]
        chosen = [v for v in ev_gpu if stamp[v] == top]
        if not boundary or len(chosen) == len(boundary):
            return True
        hi = max(o_score[v] for v in chosen)
        return all(not (o_score[b] < hi and not _near(o_score[b], hi, hi))
                   for b in boundary if b not in chosen)
    hi = max(o_score[v] for v in ev_gpu)
    for b in outside:
        if b not in ev_gpu and o_score[b] < hi and not _near(o_score[b], hi, hi):
            return False
    return True


class ComparingChain(O.UnitChain):
    """The oracle chain of one unit, adopting the GPU's choice at a near tie."""

    def __init__(self, cfg, l, u, gpu_recs, ud, check_scores=True, **kw):
        super().__init__(**kw)
        self.cfg, self.l, self.u, self.gpu, self.ud = cfg, l, u, gpu_recs, ud
        self.check_scores = check_scores
        self.events = Counter()
        self.score_over_tol = 0.0

    def _g(self, rec):
        return self.gpu[rec.t]

    def choose_selection(self, rec, sel):
        g = self._g(rec)
        where = (self.l, self.u, rec.t)
        N = len(rec.score)
        assert g["n_scoring"] == rec.n_score, (where, "context length", g["n_scoring"], rec.n_score)
        if self.check_scores:
            d = self.cfg.head_dim
            q = self.ud.drafts[rec.t + 1].reshape(-1, d).astype(np.float64)
            tol = U.score_tolerance(q, self.kmin, self.kmax)
            err = np.abs(g["scores"][:N].astype(np.float64) - rec.score)
            self.score_over_tol = max(self.score_over_tol, float(np.max(err / tol)))
            assert np.all(err <= tol), (where, "score", float(err.max()))
        sel_g = [int(x) for x in g["sel"]]
        if sel_g == sel:
            return sel
        assert selection_valid(sel_g, rec.score, self.k, N), (where, "invalid selection", sel_g, sel)
        self.events["selection_near_tie" if set(sel_g) != set(sel) else "rank_order_near_tie"] += 1
        return sel_g

    def choose_victims(self, rec, F, V):
        g = self._g(rec)
        where = (self.l, self.u, rec.t)
        assert [b for b, _ in g["fetch"]] == list(F), (where, "fetch blocks", g["fetch"], F)
        if g["evict"] == list(V):
            return V
        key = None
        if self.eviction == "lru":
            lu, b2s = self.last_use, self.b2s
            key = lambda b: (int(lu[b2s[b]]), float(rec.score[b]) + 0.0, -b)  # noqa: E731
        assert evict_valid(g["evict"], rec.slot_to_block_before, rec.sel, rec.score, len(V), key), \
            (where, "invalid victims", g["evict"], V)
        self.events["eviction_near_tie"] += 1
        return list(g["evict"])

    def check_record(self, rec):
        """Everything the step left must now equal the GPU's, bit for bit."""
        g = self._g(rec)
        where = (self.l, self.u, rec.t)
        assert g["fetch"] == [tuple(p) for p in rec.fetch], (where, "fetch", g["fetch"], rec.fetch)
        assert g["evict"] == list(rec.evict), (where, "evict", g["evict"], rec.evict)
        assert np.array_equal(g["s2b"], rec.slot_to_block), (where, "slot_to_block")
        assert np.array_equal(g["b2s"], rec.block_to_slot), (where, "block_to_slot")
        if self.eviction == "lru":
            assert np.array_equal(g["last_use"], rec.last_use), (where, "LRU stamps")


def unit_inputs(cfg, l, u):
    """The unit's seeded data and its key truth per step (recomputed for drift)."""
    H = cfg.kv_heads
    r, h = divmod(u, H)
    ud = synth.unit_data(cfg, r, l, h)
    K0 = ud.keys()
    if cfg.drift_blocks:
        sched = synth.drift_schedule(cfg, r, l, h, ud.planted0)
        K_at = lambda t: K0 if t < 0 else ud.keys(sched[t][2])  # noqa: E731
    else:
        K_at = lambda t: K0  # noqa: E731
    return ud, K_at


def compare_unit(cfg, l, u, gpu_recs, check_scores=True, eviction="score"):
    """Compares one unit's whole chain; returns its statistics, raises
    AssertionError on a real mismatch."""
    H = cfg.kv_heads
    r, h = divmod(u, H)
    ud, K_at = unit_inputs(cfg, l, u)
    chain = ComparingChain(cfg, l, u, gpu_recs, ud, check_scores=check_scores,
                           K_at=K_at, V=ud.V, queries=ud.queries, n0=cfg.ctx_of(r), k=cfg.k,
                           cap=cfg.fetch_cap, steps=cfg.steps, append=cfg.append, max_blocks=cfg.max_blocks,
                           eviction=eviction)
    stats = {"compared_steps": 0, "attn_max_abs": 0.0, "attn_rel_l2": 0.0}
    rec = chain.prologue(ud.drafts[0], lambda S0: synth.initial_residency(cfg, r, l, h, S0))
    chain.check_record(rec)
    stats["compared_steps"] += 1
    for t in range(cfg.steps):
        rec = chain.step(t)
        g = gpu_recs[t]
        ma, rl = U.attn_errors(g["out"].astype(np.float64), rec.out)
        stats["attn_max_abs"] = max(stats["attn_max_abs"], ma)
        stats["attn_rel_l2"] = max(stats["attn_rel_l2"], rl)
        assert ma <= U.ATTN_MAX_ABS and rl <= U.ATTN_REL_L2, ((l, u, t), "attention", ma, rl)
        chain.check_record(rec)
        stats["compared_steps"] += 1
    stats["score_max_err_over_tol"] = chain.score_over_tol
    for e in EVENTS:
        stats[e] = chain.events[e]
    return stats


def _job(args):
    cfg, l, u, recs, check_scores, eviction = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return compare_unit(cfg, l, u, recs, check_scores=check_scores, eviction=eviction)


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def compare_units(cfg, units, records, check_scores=True, eviction="score", log=print):
    """compare_unit over many units; with more than a few units, in worker
    processes started fresh (spawn: the caller may hold a GPU context)."""
    jobs = [(cfg, l, u, records.pop((l, u)), check_scores, eviction) for (l, u) in units]
    out = {}
    if len(jobs) <= 4:
        for j in jobs:
            out[(j[1], j[2])] = _job(j)
    else:
        import multiprocessing as mp
        from concurrent.futures import ProcessPoolExecutor
        with ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn")) as ex:
            futs = {(j[1], j[2]): ex.submit(_job, j) for j in jobs}
            del jobs
            for i, (key, f) in enumerate(futs.items()):
                out[key] = f.result()
                if log is not None and (i % 64 == 63 or i == len(futs) - 1):
                    log(f"{cfg.name}: {i + 1}/{len(futs)} units compared")
    return out


def summarize(name, results):
    """One line: units, unit-steps compared, near-tie events, worst errors."""
    tot = Counter()
    for st in results.values():
        for e in EVENTS:
            tot[e] += st[e]
        tot["unit_steps"] += st["compared_steps"]
    worst_abs = max((st["attn_max_abs"] for st in results.values()), default=0.0)
    worst_rel = max((st["attn_rel_l2"] for st in results.values()), default=0.0)
    worst_sc = max((st["score_max_err_over_tol"] for st in results.values()), default=0.0)
    return (f"{name}: {len(results)} units, {tot['unit_steps']} unit-steps compared, near ties: "
            f"selection {tot['selection_near_tie']}, rank order {tot['rank_order_near_tie']}, "
            f"eviction {tot['eviction_near_tie']}; attention max abs {worst_abs:.2e}, rel L2 {worst_rel:.2e}; "
            f"score error / bound {worst_sc:.3f}")
