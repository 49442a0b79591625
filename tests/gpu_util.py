"""Helpers shared by the GPU parity tests (inputs, conversions, tolerances)."""
from __future__ import annotations

import numpy as np
import torch

from lookahead_sparse_kv_draft_amd.runtime import Shape
from workload.synth import round_bf16, to_bf16_bits

# Attention tolerance: max abs error and relative L2 error against the fp64 oracle
# on the same element-typed inputs.
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3


def elem_round(dtype: str, x: np.ndarray) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def to_elem_np(dtype: str, x: np.ndarray) -> np.ndarray:
    """Element-typed float32 values -> the library's element array (bf16 bits or f32)."""
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def to_dev(dtype: str, x: np.ndarray, tiled_meta: bool = False) -> torch.Tensor:
    """Element-typed float32 numpy values -> device tensor of the element type
    (exact).  tiled_meta: x is logical block metadata [units][N][2][d], stored in
    the library's tile layout."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    if tiled_meta:
        from lookahead_sparse_kv_draft_amd.runtime import tile_meta
        bits = t.view(torch.int16) if dtype == "bf16" else t
        t = torch.from_numpy(tile_meta(bits.numpy())).view(t.dtype)
    return t.cuda()


def from_dev_elem(dtype: str, t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def i32(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).cuda()


def score_tolerance(q_rows: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Per-block bound on the fp32 summation error of the Quest bound (256 terms):
    4e-5 * max over rows of sum_c |q_c| * max(|kmin_c|, |kmax_c|)."""
    mag = np.maximum(np.abs(kmin), np.abs(kmax))  # [N][d]
    s = np.abs(q_rows) @ mag.T                    # [rows][N]
    return 4e-5 * s.max(axis=0) + 1e-6


def attn_errors(got: np.ndarray, ref: np.ndarray):
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def make_shape(**kw) -> Shape:
    base = dict(batch=2, kv_heads=2, group=4, head_dim=128, max_blocks=64, budget_blocks=16,
                n_draft=4, fetch_cap=4, dtype="bf16")
    base.update(kw)
    return Shape(**base)
