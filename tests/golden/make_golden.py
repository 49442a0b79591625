"""Writes tests/golden/tiny_chain_oracle.json from the CPU oracle alone.

The OasisKV pages print no worked numeric example for the per-step kernels, so
the only stored expected values here are snapshots of the oracle itself on the
tiny workload (1 request, 1 KV head, 4 query heads, d = 64, fp32, 64 blocks,
budget 16 blocks, 3 drafts, cap 4, 8 steps).  They guard the oracle against
unintended changes; a deliberate change regenerates them with this script and
names the passage (or reading) that justifies it in the commit message.

Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import oasis_oracle as O  # noqa: E402
from workload import CONFIGS, synth  # noqa: E402


def tiny_chain():
    cfg = CONFIGS["tiny"]
    ud = synth.unit_data(cfg, 0, 0, 0)
    K = ud.keys()
    recs = O.run_unit(K_at=lambda t: K, V=ud.V, queries=ud.queries, drafts_prologue=ud.drafts[0],
                      n0=cfg.ctx, k=cfg.k, cap=cfg.fetch_cap, steps=cfg.steps,
                      initial_slots=lambda S0: synth.initial_residency(cfg, 0, 0, 0, S0),
                      max_blocks=cfg.max_blocks)
    out = []
    for r in recs:
        out.append({
            "t": r.t,
            "sel": [int(b) for b in r.sel],
            "fetch": [[int(b), int(s)] for b, s in r.fetch],
            "evict": [int(v) for v in r.evict],
            "slot_to_block": [int(b) for b in r.slot_to_block],
            "attended": [int(b) for b in r.attended],
            "out_row0_head0_first4": [] if r.out is None else [float(x) for x in r.out[0, 0, :4]],
            "score_first4": [float(x) for x in r.score[:4]],
        })
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_chain_oracle.json"), "w") as f:
        json.dump({"config": "tiny", "steps": tiny_chain()}, f, indent=1)
    print("wrote tiny_chain_oracle.json")
