"""Chained GPU parity: the whole multi-step decode chain (prologue, attention,
append, scoring, selection, diff/cap/evict, transfer) against the oracle.

Small workloads are compared on every unit; the full-size workloads, in the
launch configuration the benchmark times, on sampled units (each unit's chain
is independent of the others).
"""
import numpy as np
import pytest

from lookahead_sparse_kv_draft_amd.synthetic import SyntheticRun
from tests import chain_compare as CC
from workload import CONFIGS

pytestmark = pytest.mark.gpu


def _run_and_compare(cfg, units, steps=None, layers=None, max_diverged_frac=0.25):
    cfg = cfg if steps is None else cfg.with_(steps=steps)
    run = SyntheticRun(cfg, layers=layers, record_units=units)
    try:
        run.run()
        results = []
        for (l, u) in units:
            st = CC.compare_unit(cfg, l, u, run.records[(l, u)], CC.oracle_unit(cfg, l, u))
            results.append(st)
            print(f"{cfg.name} layer {l} unit {u}: {st}", flush=True)
    finally:
        run.close()
    total = sum(r["compared_steps"] for r in results)
    possible = len(units) * (cfg.steps + 1)
    assert total >= (1 - max_diverged_frac) * possible, (total, possible)
    return results


def test_chain_tiny_full():
    cfg = CONFIGS["tiny"]
    res = _run_and_compare(cfg, [(0, 0)], max_diverged_frac=0.0)
    assert res[0]["diverged_at"] is None


def test_chain_small_bf16_ragged():
    # ragged context (partial newest block), several tiles and splits, cap binding
    cfg = CONFIGS["llama8b_32k"].with_(batch=2, ctx=16 * 300 + 7, steps=6, fetch_cap=8,
                                       planted=15, budget_tokens=16 * 32)
    _run_and_compare(cfg, [(0, u) for u in range(cfg.batch * cfg.kv_heads)])


def test_chain_small_append():
    cfg = CONFIGS["qwen8b_reason"].with_(batch=2, ctx=16 * 40 + 13, steps=40, recency_blocks=8,
                                         planted=4, budget_tokens=16 * 16, fetch_cap=3)
    _run_and_compare(cfg, [(0, u) for u in range(cfg.batch * cfg.kv_heads)])


def test_chain_small_drift():
    cfg = CONFIGS["qwen32b_32k"].with_(batch=1, layers=2, ctx=16 * 200, steps=5, planted=10,
                                       drift_blocks=4, budget_tokens=16 * 24, fetch_cap=4)
    _run_and_compare(cfg, [(l, u) for l in range(2) for u in range(cfg.kv_heads)])


def test_chain_llama8b_32k_full_size_sampled():
    cfg = CONFIGS["llama8b_32k"]
    units = [(0, u) for u in (0, 9, 22, 35, 47, 63)]
    _run_and_compare(cfg, units, steps=12)
