"""Workload shapes for the lookahead sparse-KV decode step.

Each configuration is one decode workload: batch, layers, GQA head layout,
head dimension, element type, context, token budget, number of draft queries,
per-step fetch cap and the synthetic structure planted into the keys.  The
shapes imitate the models and contexts the OasisKV pages evaluate (OasisKV
explainer, Table 1: Llama-3.1-8B-Instruct and Qwen3-8B on long input at a
2,048-token budget; Table 2: Qwen3-8B long-output reasoning; Figure 2:
Qwen3-32B at 32K context).  No dataset content is used: only shapes and the
structure of the sparsity are imitated.

This module holds shapes only; it contains none of the method's arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

BLOCK = 16  # tokens per KV block (page)


@dataclass(frozen=True)
class Config:
    name: str
    batch: int            # B, requests
    layers: int           # layers run back to back
    kv_heads: int         # H
    group: int            # G, query heads per KV head
    head_dim: int         # d
    dtype: str            # "f32" or "bf16": element type of K, V, Q and block metadata
    ctx: int              # prompt length n0 in tokens
    budget_tokens: int    # HBM token budget per (request, layer, KV head)
    n_draft: int          # D draft queries per step (plus one verify query)
    fetch_cap: int        # max blocks fetched per (request, layer, KV head) per step
    steps: int            # decode steps
    append: bool = False  # append one token per step (long-output reasoning)
    planted: int = 0      # number of planted blocks per (request, layer, KV head)
    planted_shift: float = 2.0
    recency_blocks: int = 0      # last prompt blocks shifted toward u
    recency_shift: float = 1.0
    drift_blocks: int = 0        # planted blocks swapped per step
    init_resident: str = "half"  # "random": k random blocks; "half": half of S0 + random others
    draft_sigma: float = 0.1
    seed: int = 20260807
    ctx_list: tuple = ()  # per-request prompt lengths (empty: every request has `ctx`)

    # ---- derived sizes ----
    @property
    def block(self) -> int:
        return BLOCK

    @property
    def n_blocks0(self) -> int:
        return (self.ctx + BLOCK - 1) // BLOCK

    def ctx_of(self, r: int) -> int:
        """Prompt length of request r."""
        return int(self.ctx_list[r]) if self.ctx_list else self.ctx

    def n_blocks0_of(self, r: int) -> int:
        return (self.ctx_of(r) + BLOCK - 1) // BLOCK

    @property
    def ctx_max(self) -> int:
        top = max(self.ctx_list) if self.ctx_list else self.ctx
        return top + (self.steps if self.append else 0)

    @property
    def max_blocks(self) -> int:
        return (self.ctx_max + BLOCK - 1) // BLOCK

    @property
    def k(self) -> int:
        return self.budget_tokens // BLOCK

    @property
    def T(self) -> int:
        return 1 + self.n_draft

    @property
    def q_heads(self) -> int:
        return self.kv_heads * self.group

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def units_per_layer(self) -> int:
        return self.batch * self.kv_heads

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


def _planted(frac: float, n_blocks: int) -> int:
    return int(round(frac * n_blocks))


CONFIGS = {
    # 1 request, 4 query heads over 1 KV head, d=64, fp32, 1024 tokens (64 blocks),
    # budget 256 tokens (16 blocks), 3 drafts, cap 4, 16 random initially resident blocks.
    "tiny": Config(
        name="tiny", batch=1, layers=1, kv_heads=1, group=4, head_dim=64, dtype="f32",
        ctx=1024, budget_tokens=256, n_draft=3, fetch_cap=4, steps=8,
        planted=3, init_resident="random", seed=20260807 + 0),
    # Llama-3.1-8B-shaped single layer at 32K context.
    "llama8b_32k": Config(
        name="llama8b_32k", batch=8, layers=1, kv_heads=8, group=4, head_dim=128, dtype="bf16",
        ctx=32768, budget_tokens=2048, n_draft=4, fetch_cap=32, steps=32,
        planted=_planted(0.05, 2048), init_resident="half", seed=20260807 + 1),
    # Qwen3-32B-shaped, 8 layers, 64 query / 8 KV heads, drifting important set.
    "qwen32b_32k": Config(
        name="qwen32b_32k", batch=16, layers=8, kv_heads=8, group=8, head_dim=128, dtype="bf16",
        ctx=32768, budget_tokens=2048, n_draft=4, fetch_cap=16, steps=32,
        planted=_planted(0.05, 2048), drift_blocks=_planted(0.02, 2048),
        init_resident="half", seed=20260807 + 2),
    # Qwen3-8B-shaped long-output reasoning: 8192-token prompt, 256 appended tokens.
    "qwen8b_reason": Config(
        name="qwen8b_reason", batch=64, layers=1, kv_heads=8, group=4, head_dim=128, dtype="bf16",
        ctx=8192, budget_tokens=2048, n_draft=5, fetch_cap=24, steps=256, append=True,
        planted=_planted(0.03, 512), recency_blocks=64, recency_shift=1.0,
        init_resident="half", seed=20260807 + 3),
    # Llama-3.1-8B-shaped 128K context, 8 layers (4 x 8 x 512 MiB = 16 GiB host tier).
    "llama8b_128k": Config(
        name="llama8b_128k", batch=4, layers=8, kv_heads=8, group=4, head_dim=128, dtype="bf16",
        ctx=131072, budget_tokens=2048, n_draft=4, fetch_cap=32, steps=32,
        planted=_planted(0.01, 8192), init_resident="half", seed=20260807 + 4),
}

CONFIG_ORDER = ["tiny", "llama8b_32k", "qwen32b_32k", "qwen8b_reason", "llama8b_128k"]
