"""The oracle still reproduces its committed snapshot on the tiny workload (CPU only)."""
import json
import os

import numpy as np

from tests.golden.make_golden import tiny_chain

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_chain_snapshot():
    with open(os.path.join(HERE, "tiny_chain_oracle.json")) as f:
        ref = json.load(f)["steps"]
    got = tiny_chain()
    assert len(got) == len(ref)
    for g, r in zip(got, ref):
        for key in ("t", "sel", "fetch", "evict", "slot_to_block", "attended"):
            assert g[key] == r[key], (g["t"], key)
        np.testing.assert_allclose(g["out_row0_head0_first4"], r["out_row0_head0_first4"], rtol=1e-12)
        np.testing.assert_allclose(g["score_first4"], r["score_first4"], rtol=1e-12)
