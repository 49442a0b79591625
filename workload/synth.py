"""Seeded synthetic inputs for the lookahead sparse-KV decode step.

Both the product path and the CPU oracle draw their inputs from here; this
module holds none of the method's arithmetic (no pooling, scoring, selection,
eviction or attention).  It only draws random tensors, plants structure into
them and rounds them to the element type.

Recipe (per unit = one (request r, layer l, KV head h); each unit has its own
PCG64 streams so any unit can be regenerated alone, which lets the oracle
check sampled units of a full-size run):

* stream (r, l, h, 0), fixed draw order:
  K_raw [max_blocks*16][d] ~ N(0, 1), V_raw [max_blocks*16][d] ~ N(0, 1),
  q_base [G][d] ~ N(0, 1), the planted block set (uniform without replacement
  over the request's prompt blocks), draft noise [steps + 1][D][G][d] ~ N(0, 0.1^2).
* u = normalize(sum_g q_base[g]), the unit mean query direction of the group.
* K = round(round(K_raw) + s * u) per token, s = planted_shift if the token's
  block is planted, plus recency_shift if the token lies in the last
  `recency_blocks` prompt blocks or was appended after the prompt.
* V = round(V_raw); verify query = round(q_base) at every step;
  drafts of step t (t = -1 .. steps-1) = round(q_base + noise[t + 1]).
* stream (r, l, h, 1): initial residency; stream (r, l, h, 2): drift schedule.

round() is the identity for fp32 workloads and round-to-nearest-even to
bfloat16 for bf16 workloads (the rounding torch's float32 -> bfloat16
conversion performs).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .configs import BLOCK, Config


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bfloat16 value (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array of bf16-representable values -> uint16 bf16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("value is not representable in bfloat16")
    return (bits >> 16).astype(np.uint16)


def round_elem(cfg: Config, x: np.ndarray) -> np.ndarray:
    if cfg.dtype == "bf16":
        return round_bf16(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def _rng(cfg: Config, r: int, l: int, h: int, purpose: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(cfg.seed, spawn_key=(r, l, h, purpose)))


@dataclass
class UnitData:
    """Synthetic tensors of one (request, layer, KV head) unit, element-typed float32."""
    cfg: Config
    r: int
    l: int
    h: int
    K_base: np.ndarray    # [max_blocks * 16][d] round(K_raw), before any shift
    V: np.ndarray         # [max_blocks * 16][d]
    q_base: np.ndarray    # [G][d] verify query (element-typed)
    drafts: np.ndarray    # [steps + 1][D][G][d]; drafts[t + 1] are the drafts of step t
    u: np.ndarray         # [d] float32 unit mean query direction
    planted0: np.ndarray  # sorted planted blocks at the start

    def shift_per_token(self, planted: np.ndarray) -> np.ndarray:
        """Per-token shift multiplier s for the given planted block set."""
        cfg = self.cfg
        s = np.zeros(cfg.max_blocks * BLOCK, dtype=np.float32)
        if len(planted):
            blk = np.arange(cfg.max_blocks * BLOCK) // BLOCK
            s += cfg.planted_shift * np.isin(blk, planted).astype(np.float32)
        if cfg.recency_blocks:
            start = max(0, (cfg.n_blocks0_of(self.r) - cfg.recency_blocks) * BLOCK)
            s[start:] += cfg.recency_shift  # last prompt blocks and every appended token
        return s

    def keys(self, planted: np.ndarray | None = None) -> np.ndarray:
        """K [max_blocks * 16][d] for a planted set (default: the initial one)."""
        if planted is None:
            planted = self.planted0
        s = self.shift_per_token(np.asarray(planted))
        return round_elem(self.cfg, self.K_base + s[:, None] * self.u[None, :])

    def keys_of_blocks(self, blocks: np.ndarray, planted: np.ndarray) -> np.ndarray:
        """K rows of the given blocks [len(blocks)][16][d] for a planted set."""
        s = self.shift_per_token(np.asarray(planted)).reshape(-1, BLOCK)[blocks]
        kb = self.K_base.reshape(-1, BLOCK, self.cfg.head_dim)[blocks]
        return round_elem(self.cfg, kb + s[:, :, None] * self.u[None, None, :])

    def queries(self, t: int) -> np.ndarray:
        """Queries of step t as [G][T][d]: index 0 verify, 1..D the drafts of step t."""
        cfg = self.cfg
        q = np.empty((cfg.group, cfg.T, cfg.head_dim), dtype=np.float32)
        q[:, 0, :] = self.q_base
        q[:, 1:, :] = self.drafts[t + 1].transpose(1, 0, 2)
        return q


def unit_data(cfg: Config, r: int, l: int, h: int) -> UnitData:
    rng = _rng(cfg, r, l, h, 0)
    n, d, G, D = cfg.max_blocks * BLOCK, cfg.head_dim, cfg.group, cfg.n_draft
    K_raw = rng.standard_normal((n, d), dtype=np.float32)
    V_raw = rng.standard_normal((n, d), dtype=np.float32)
    q_raw = rng.standard_normal((G, d), dtype=np.float32)
    nb0 = cfg.n_blocks0_of(r)
    planted = np.sort(rng.choice(nb0, size=min(cfg.planted, nb0), replace=False))
    noise = rng.standard_normal((cfg.steps + 1, D, G, d), dtype=np.float32)
    noise *= np.float32(cfg.draft_sigma)
    su = q_raw.sum(axis=0)
    u = (su / np.float32(np.linalg.norm(su))).astype(np.float32)
    return UnitData(
        cfg=cfg, r=r, l=l, h=h,
        K_base=round_elem(cfg, K_raw),
        V=round_elem(cfg, V_raw),
        q_base=round_elem(cfg, q_raw),
        drafts=round_elem(cfg, q_raw[None, None] + noise),
        u=u,
        planted0=planted.astype(np.int64),
    )


def initial_residency(cfg: Config, r: int, l: int, h: int, S0) -> np.ndarray:
    """slot_to_block [k] (-1 = empty) of the initial resident set.

    "random": k distinct random prompt blocks in random slot order.
    "half":   a random half of the first selection S0 plus random blocks outside
              S0 in the remaining slots, all in random slot order.
    S0 is the selection the caller computed for the prologue (entries < 0 ignored).
    """
    rng = _rng(cfg, r, l, h, 1)
    k, N = cfg.k, cfg.n_blocks0_of(r)
    if cfg.init_resident == "random":
        blocks = rng.choice(N, size=min(k, N), replace=False)
    elif cfg.init_resident == "half":
        s0 = np.array(sorted(int(b) for b in S0 if b >= 0), dtype=np.int64)
        half = rng.choice(s0, size=len(s0) // 2, replace=False) if len(s0) else s0
        others = np.setdiff1d(np.arange(N), s0)
        n_other = min(k - len(half), len(others))
        extra = rng.choice(others, size=n_other, replace=False) if n_other > 0 else others[:0]
        blocks = rng.permutation(np.concatenate([half, extra]))
    else:
        raise ValueError(cfg.init_resident)
    s2b = np.full(k, -1, dtype=np.int32)
    s2b[: len(blocks)] = blocks
    return s2b


def drift_schedule(cfg: Config, r: int, l: int, h: int, planted0: np.ndarray):
    """Per step t: (unplant, plant, planted_after) block arrays.

    Each step swaps `drift_blocks` planted blocks for as many unplanted ones,
    so the important set drifts by that many blocks per step.
    """
    rng = _rng(cfg, r, l, h, 2)
    cur = np.array(sorted(planted0), dtype=np.int64)
    out = []
    for _ in range(cfg.steps):
        m = min(cfg.drift_blocks, len(cur))
        unplant = np.sort(rng.choice(cur, size=m, replace=False)) if m else cur[:0]
        pool = np.setdiff1d(np.arange(cfg.n_blocks0_of(r)), cur)
        m2 = min(cfg.drift_blocks, len(pool))
        plant = np.sort(rng.choice(pool, size=m2, replace=False)) if m2 else pool[:0]
        cur = np.sort(np.concatenate([np.setdiff1d(cur, unplant), plant]))
        out.append((unplant, plant, cur.copy()))
    return out


def random_scores(rng: np.random.Generator, n: int, kind: str = "normal") -> np.ndarray:
    """Synthetic fp32 block scores for stage-wise selection tests.

    kind "normal": N(0, 1); "ties": few distinct values (many exact ties, with
    -0.0 and +0.0 mixed in); "const": all equal.
    """
    if kind == "normal":
        s = rng.standard_normal(n).astype(np.float32)
    elif kind == "ties":
        vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 3.0], dtype=np.float32)
        s = vals[rng.integers(0, len(vals), size=n)]
    elif kind == "const":
        s = np.full(n, 0.5, dtype=np.float32)
    else:
        raise ValueError(kind)
    return s
