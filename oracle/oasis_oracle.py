"""CPU oracle for the lookahead sparse-KV decode step (test infrastructure only).

This is a plain, slow, fp64 numpy statement of what one decode step of one
(request, layer, KV head) unit computes.  It shares no code with the HIP
library and imports nothing from it.  Only the tests, the smoke entry point
and the benchmark's CPU-baseline leg may use it; the product path never does.

Sources (the OasisKV pages, cited by title and section/figure/table):
  [EXPL]  METAL MEDIA explainer "OasisKV: Scaling In-Decode KV Cache Beyond HBM
          with Lookahead Sparse Prefetching" (metalmedia.ai, arXiv 2608.08097)
  [INDEX] mlsanity.com index entry for arXiv 2608.08097 (abstract, "Builds on")
  [POD]   researchpod.app episode on the same paper (abstract and dialogue)

Where the pages leave a step open, this oracle takes the readings listed in the
repository's design notes; each function below names the reading it applies.

Parity pins (see tests/test_oracle_*.py): every function here is pinned by
invariants, closed forms, brute force or a library routine, except the
multi-step fetch sequence when the cap binds, whose order (highest-ranked
missing block first, free slots ascending, then victims from the tail of the
ranking) is fixed by the readings, not by the pages: parity unpinned by the
pages for that ordering.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 16


# --------------------------------------------------------------------------
# O1  block metadata ("compressed keys")
# --------------------------------------------------------------------------
def block_meta(K: np.ndarray, n: int):
    """Per-block, per-channel min and max of the keys of tokens < n.

    [EXPL] Figure 7 (left): the GPU keeps compressed keys made by min/max
    pooling each KV block.  Block b covers tokens 16b .. 16b+15, clipped to the
    context length n, so a partially filled newest block pools only its valid
    tokens.  Returns (kmin, kmax), each [N][d] with N = ceil(n / 16).
    """
    K = np.asarray(K, dtype=np.float64)
    N = (n + BLOCK - 1) // BLOCK
    d = K.shape[1]
    kmin = np.empty((N, d))
    kmax = np.empty((N, d))
    for b in range(N):
        rows = K[b * BLOCK: min((b + 1) * BLOCK, n)]
        kmin[b] = rows.min(axis=0)
        kmax[b] = rows.max(axis=0)
    return kmin, kmax


def block_meta_append(kmin: np.ndarray, kmax: np.ndarray, n: int, k_new: np.ndarray):
    """Metadata after appending the token at position n (O7).

    A token that starts a new block initialises that block's min and max to
    itself; otherwise the block's min/max absorb it.  Returns new (kmin, kmax)
    with ceil((n + 1) / 16) rows.
    """
    b = n // BLOCK
    k_new = np.asarray(k_new, dtype=np.float64)
    if n % BLOCK == 0:
        assert kmin.shape[0] == b
        kmin = np.vstack([kmin, k_new[None]])
        kmax = np.vstack([kmax, k_new[None]])
    else:
        kmin = kmin.copy()
        kmax = kmax.copy()
        kmin[b] = np.minimum(kmin[b], k_new)
        kmax[b] = np.maximum(kmax[b], k_new)
    return kmin, kmax


# --------------------------------------------------------------------------
# O2  lookahead score
# --------------------------------------------------------------------------
def block_bound(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Upper bound of q.k over every key k of each block: sum_c max(q_c kmin_c, q_c kmax_c).

    The pages leave the scoring function open ([EXPL] Figure 7 says only that the
    draft query scans the compressed keys); the reading is the Quest bound
    (Quest appears in [INDEX] "Builds on").  No 1/sqrt(d) scale: a positive
    scale does not change a ranking.
    """
    q = np.asarray(q, dtype=np.float64)
    return np.maximum(kmin * q[None, :], kmax * q[None, :]).sum(axis=1)


def lookahead_score(q_draft: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Score of each block: the max of block_bound over every draft query row.

    q_draft is [D][G][d] (or any [..., d]): all draft tokens of the step times
    the G query heads sharing the KV head.  Only draft queries score ([EXPL]
    Figure 7 right: the draft query predicts the next step's top-K blocks).
    """
    rows = np.asarray(q_draft, dtype=np.float64).reshape(-1, kmin.shape[1])
    per_row = np.stack([block_bound(q, kmin, kmax) for q in rows])
    return per_row.max(axis=0)


# --------------------------------------------------------------------------
# O3  top-k selection
# --------------------------------------------------------------------------
def order_key(score: float, b: int):
    """Total order used to rank blocks: higher score first, then lower index.

    -0.0 is treated as +0.0 (adding +0.0 canonicalises it).
    """
    return (-(float(score) + 0.0), int(b))


def topk_select(score: np.ndarray, N: int, k: int) -> list:
    """Selected blocks S in rank order, padded with -1 to length k.

    Forced blocks come first: the sink block 0 and then the newest block N-1
    (one block when N = 1); attention sinks are in [INDEX] "Builds on".  The
    remaining k - |forced| places go to the other blocks in order_key order,
    i.e. the top-k blocks that fill the token budget ([EXPL] Figure 7 right,
    Figure 4).  With N <= k every block is selected.
    """
    assert k >= 2
    forced = [0] if N == 1 else [0, N - 1]
    cand = sorted(range(1, N - 1), key=lambda b: order_key(score[b], b))
    sel = forced + cand[: k - len(forced)]
    return sel + [-1] * (k - len(sel))


# --------------------------------------------------------------------------
# O4  set difference, capped fetch, capped eviction
# --------------------------------------------------------------------------
@dataclass
class DiffResult:
    fetch: list            # [(block, slot)] in fetch order
    evict: list            # victim blocks in eviction order
    block_to_slot: np.ndarray
    slot_to_block: np.ndarray
    last_use: np.ndarray = None  # LRU policy only: per-slot stamp after the step


def plan_fetch_evict(sel, score, block_to_slot, slot_to_block, cap: int):
    """O4 steps 1-5: the fetch list F and the victims V, both in order.

    [EXPL] explanatory diagram step 3 and "What they did" item 3: predicted
    blocks are compared with the resident ones, only the missing blocks are
    fetched, and a capped-eviction policy bounds the blocks fetched per step
    (Table 2 sweeps that cap).

    Readings: the fetch takes the highest-ranked missing blocks first; victims
    are resident blocks outside S taken from the tail of the ranking order
    (lowest score first, and among equal scores the higher block index first),
    as many as the free slots do not cover.
    """
    k = len(slot_to_block)
    b2s = np.asarray(block_to_slot)
    s2b = np.asarray(slot_to_block)
    S = [int(b) for b in sel if b >= 0]
    Sset = set(S)
    missing = [b for b in S if b2s[b] < 0]
    F = missing[: min(cap, len(missing))]
    n_free = sum(1 for s in range(k) if s2b[s] < 0)
    need = max(0, len(F) - n_free)
    outside = [int(s2b[s]) for s in range(k) if s2b[s] >= 0 and int(s2b[s]) not in Sset]
    ranked = sorted(outside, key=lambda b: order_key(score[b], b))
    V = list(reversed(ranked))[:need]
    assert len(V) == need, "fewer victims than needed: |S| must not exceed k"
    return F, V


def apply_fetch_evict(block_to_slot, slot_to_block, F, V) -> DiffResult:
    """O4 steps 6-8: target slots and the updated head-wise resident maps.

    [EXPL] Figure 9: a per-KV-head table maps each GPU block (slot) to a CPU
    block; block_to_slot is its inverse.  Reading: the fetched blocks take the
    free slots in ascending order first, then the victims' slots in victim
    order.
    """
    k = len(slot_to_block)
    b2s = np.array(block_to_slot, dtype=np.int64).copy()
    s2b = np.array(slot_to_block, dtype=np.int64).copy()
    free = [s for s in range(k) if s2b[s] < 0]
    assert len(V) == max(0, len(F) - len(free)), "victims must cover exactly what the free slots do not"
    assert all(b2s[v] >= 0 for v in V) and all(b2s[b] < 0 for b in F)
    targets = free[: min(len(F), len(free))] + [int(b2s[v]) for v in V]
    for v in V:
        b2s[v] = -1
    for b, s in zip(F, targets):
        s2b[s] = b
        b2s[b] = s
    return DiffResult(fetch=list(zip(F, targets)), evict=list(V), block_to_slot=b2s, slot_to_block=s2b)


def resident_diff_cap_evict(sel, score, block_to_slot, slot_to_block, cap: int) -> DiffResult:
    """Fetch list, eviction list and updated head-wise resident maps (O4):
    plan_fetch_evict, then apply_fetch_evict."""
    F, V = plan_fetch_evict(sel, score, block_to_slot, slot_to_block, cap)
    return apply_fetch_evict(block_to_slot, slot_to_block, F, V)


def plan_fetch_evict_lru(sel, score, block_to_slot, slot_to_block, last_use, cap: int):
    """O4 steps 1-5 with least-recently-used eviction ([EXPL] Table 2: the
    fetch-ratio ablation runs with LRU eviction).

    Readings (the pages name the policy only): victims are the resident blocks
    outside S with the oldest stamp first (a slot never read holds -1); among
    equal stamps, the lowest-score order of plan_fetch_evict (lowest score
    first, then the higher block index).  The fetch list is as there.
    """
    k = len(slot_to_block)
    b2s = np.asarray(block_to_slot)
    s2b = np.asarray(slot_to_block)
    lu = np.asarray(last_use)
    S = [int(b) for b in sel if b >= 0]
    Sset = set(S)
    missing = [b for b in S if b2s[b] < 0]
    F = missing[: min(cap, len(missing))]
    n_free = sum(1 for s in range(k) if s2b[s] < 0)
    need = max(0, len(F) - n_free)
    outside = [int(s2b[s]) for s in range(k) if s2b[s] >= 0 and int(s2b[s]) not in Sset]
    # oldest stamp first; then lowest score (-0.0 as +0.0), then higher index
    ranked = sorted(outside, key=lambda b: (int(lu[b2s[b]]), float(score[b]) + 0.0, -b))
    V = ranked[:need]
    assert len(V) == need, "fewer victims than needed: |S| must not exceed k"
    return F, V


def stamp_last_use(sel, block_to_slot, last_use, step: int) -> np.ndarray:
    """LRU stamps after a step's diff.  Reading: a slot is used when an
    attention reads it, so the slots of the next attention's blocks (the
    selection that is resident after this step's fetch) get `step`."""
    lu = np.array(last_use, dtype=np.int64).copy()
    for b in sel:
        if b >= 0 and block_to_slot[b] >= 0:
            lu[block_to_slot[b]] = step
    return lu


def resident_diff_cap_evict_lru(sel, score, block_to_slot, slot_to_block, last_use, cap: int,
                                step: int) -> DiffResult:
    """The O4 step with LRU eviction: plan_fetch_evict_lru, apply_fetch_evict,
    then stamp_last_use with `step`."""
    F, V = plan_fetch_evict_lru(sel, score, block_to_slot, slot_to_block, last_use, cap)
    res = apply_fetch_evict(block_to_slot, slot_to_block, F, V)
    res.last_use = stamp_last_use(sel, res.block_to_slot, last_use, step)
    return res


# --------------------------------------------------------------------------
# O6  sparse attention over the resident selected blocks
# --------------------------------------------------------------------------
def attended_blocks(sel, block_to_slot) -> list:
    """A = blocks of S that are resident (S intersect R), in rank order."""
    return [int(b) for b in sel if b >= 0 and block_to_slot[b] >= 0]


def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, blocks, n: int) -> np.ndarray:
    """softmax(q.K_J / sqrt(d)) V_J for every query row, J = tokens of `blocks` below n.

    [EXPL] Figure 7 (right): the normal (verify) and draft queries attend
    together over the sparse working set.  q is [..., d]; the result has the
    same shape.  No mask between the query rows (their own keys are not in the
    cache during the step).  An empty J gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    shape = q.shape
    qr = q.reshape(-1, shape[-1])
    J = sorted(j for b in blocks for j in range(b * BLOCK, min((b + 1) * BLOCK, n)))
    if not J:
        return np.zeros(shape)
    Kj = np.asarray(K, dtype=np.float64)[J]
    Vj = np.asarray(V, dtype=np.float64)[J]
    logits = qr @ Kj.T / math.sqrt(shape[-1])
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return (p @ Vj).reshape(shape)


# --------------------------------------------------------------------------
# Step loop of one unit
# --------------------------------------------------------------------------
@dataclass
class StepRecord:
    t: int                 # -1 = prologue
    n_attn: int = 0        # context length seen by this step's attention
    attended: list = field(default_factory=list)
    out: np.ndarray | None = None      # [G][T][d] attention output
    n_score: int = 0       # context length when scoring
    score: np.ndarray | None = None    # [N] fp64
    sel: list = field(default_factory=list)
    fetch: list = field(default_factory=list)
    evict: list = field(default_factory=list)
    block_to_slot: np.ndarray | None = None  # after this step's update
    slot_to_block: np.ndarray | None = None
    slot_to_block_before: np.ndarray | None = None  # before this step's update
    block_to_slot_before: np.ndarray | None = None
    last_use: np.ndarray | None = None  # LRU stamps after this step (LRU eviction only)
    n_missing: int = 0


class UnitChain:
    """Multi-step chain of one unit ([EXPL] Figure 8).

    The draft queries of step t drive scoring, selection and transfer, and the
    transferred blocks serve that layer's attention at step t+1.  Per step t:
    attention with step t's queries over S_t intersect R_t; append token n (if
    `append`); score with step t's drafts; select S_{t+1}; diff/cap/evict into
    R_{t+1}.  The prologue scores the drafts of step -1, selects S_0, applies
    the initial residency initial_slots(S_0) and runs one diff/cap/evict.

    K_at(t) gives the key truth valid after step t's drift (t = -1 for the
    prologue; the same array object when nothing changed); V is fixed;
    queries(t) is [G][T][d] (row 0 verify, rows 1..D the drafts).  In this
    oracle the HBM pool is a view of the host truth, so a fetched or patched
    page always holds the current keys and values.

    eviction: "score" (lowest-score victims) or "lru" (least recently used;
    the diff that prepares the attention of step t stamps its slots with t, the
    prologue's with 0).

    Two choices have more than one correct result when scores tie within the
    comparison's tolerance: the selection of a step and the victims of its
    diff.  They pass through choose_selection and choose_victims, which return
    the oracle's own choice; a comparison may override them to continue from
    another implementation's choice after checking that it is valid.
    """

    def __init__(self, *, K_at, V, queries, n0: int, k: int, cap: int, steps: int, append: bool = False,
                 max_blocks: int | None = None, with_attention: bool = True, eviction: str = "score"):
        assert eviction in ("score", "lru")
        self.K_at, self.V, self.queries = K_at, V, queries
        self.n = n0
        self.k, self.cap = k, cap
        self.append, self.with_attention, self.eviction = append, with_attention, eviction
        self.Nmax = max_blocks if max_blocks is not None else (n0 + BLOCK - 1) // BLOCK + (steps if append else 0)
        self.K = K_at(-1)
        self.kmin, self.kmax = block_meta(self.K, self.n)
        self.sel = None
        self.b2s = self.s2b = self.last_use = None

    # ---- decision points (near ties) ----
    def choose_selection(self, rec: StepRecord, sel: list) -> list:
        return sel

    def choose_victims(self, rec: StepRecord, F: list, V: list) -> list:
        return V

    # ---- stages ----
    def _predict(self, rec: StepRecord, drafts):
        rec.n_score = self.n
        rec.score = lookahead_score(drafts, self.kmin, self.kmax)
        rec.sel = self.choose_selection(rec, topk_select(rec.score, self.kmin.shape[0], self.k))

    def _diff(self, rec: StepRecord, stamp: int):
        rec.n_missing = sum(1 for b in rec.sel if b >= 0 and self.b2s[b] < 0)
        rec.slot_to_block_before = self.s2b.copy()
        rec.block_to_slot_before = self.b2s.copy()
        if self.eviction == "lru":
            F, V = plan_fetch_evict_lru(rec.sel, rec.score, self.b2s, self.s2b, self.last_use, self.cap)
        else:
            F, V = plan_fetch_evict(rec.sel, rec.score, self.b2s, self.s2b, self.cap)
        V = self.choose_victims(rec, F, V)
        res = apply_fetch_evict(self.b2s, self.s2b, F, V)
        if self.eviction == "lru":
            self.last_use = stamp_last_use(rec.sel, res.block_to_slot, self.last_use, stamp)
            rec.last_use = self.last_use.copy()
        self.b2s, self.s2b = res.block_to_slot, res.slot_to_block
        rec.fetch, rec.evict = res.fetch, res.evict
        rec.block_to_slot, rec.slot_to_block = self.b2s.copy(), self.s2b.copy()
        self.sel = rec.sel

    def prologue(self, drafts_prologue, initial_slots) -> StepRecord:
        """drafts_prologue is [D][G][d] or [G][D][d] (only its rows matter)."""
        rec = StepRecord(t=-1)
        self._predict(rec, drafts_prologue)
        self.s2b = np.asarray(initial_slots(rec.sel), dtype=np.int64).copy()
        self.b2s = np.full(self.Nmax, -1, dtype=np.int64)
        for s, b in enumerate(self.s2b):
            if b >= 0:
                self.b2s[b] = s
        self.last_use = np.full(self.k, -1, dtype=np.int64)
        self._diff(rec, stamp=0)
        return rec

    def step(self, t: int) -> StepRecord:
        rec = StepRecord(t=t, n_attn=self.n)
        q = self.queries(t)
        rec.attended = attended_blocks(self.sel, self.b2s)
        if self.with_attention:
            rec.out = sparse_attention(q, self.K, self.V, rec.attended, self.n)
        if self.append:
            self.kmin, self.kmax = block_meta_append(self.kmin, self.kmax, self.n, self.K[self.n])
            self.n += 1
        K_new = self.K_at(t)
        if K_new is not self.K:
            self.K = K_new
            self.kmin, self.kmax = block_meta(self.K, self.n)
        self._predict(rec, q[:, 1:, :])
        self._diff(rec, stamp=t + 1)
        return rec


def run_unit(*, K_at, V, queries, drafts_prologue, n0: int, k: int, cap: int, steps: int,
             initial_slots, append: bool = False, max_blocks: int | None = None,
             with_attention: bool = True, eviction: str = "score") -> list:
    """The prologue and `steps` steps of one unit's chain (UnitChain), as records."""
    chain = UnitChain(K_at=K_at, V=V, queries=queries, n0=n0, k=k, cap=cap, steps=steps, append=append,
                      max_blocks=max_blocks, with_attention=with_attention, eviction=eviction)
    recs = [chain.prologue(drafts_prologue, initial_slots)]
    for t in range(steps):
        recs.append(chain.step(t))
    return recs
