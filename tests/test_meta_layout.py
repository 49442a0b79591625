"""The metadata tile layout: the runtime's un-tiling view against the layout
rule stated in include/oasiskv.h (chunk c of block 16t + j at chunk position
16c + j of tile t), written out element by element here."""
import numpy as np
import pytest
import torch

from lookahead_sparse_kv_draft_amd.runtime import tile_meta, untile_meta


@pytest.mark.parametrize("dtype,d,units,nmax", [("bf16", 128, 3, 37), ("bf16", 64, 2, 16), ("f32", 64, 2, 21),
                                                 ("f32", 128, 1, 5)])
def test_untile_meta_inverts_the_layout(dtype, d, units, nmax):
    rng = np.random.default_rng(7)
    ce = 8 if dtype == "bf16" else 4
    np_t = np.int16 if dtype == "bf16" else np.float32
    logical = rng.integers(-30000, 30000, size=(units, nmax, 2 * d)).astype(np_t)
    tiles = (nmax + 15) // 16
    flat = np.zeros(units * tiles * 16 * 2 * d, dtype=np_t)
    nc = 2 * d // ce
    for u in range(units):
        for b in range(nmax):
            t, j = divmod(b, 16)
            for e in range(2 * d):
                c, o = divmod(e, ce)
                flat[((u * tiles + t) * nc + c) * 16 * ce + j * ce + o] = logical[u, b, e]
    got = untile_meta(torch.from_numpy(flat.view(np.uint8)), units, nmax, d, dtype).numpy()
    assert got.shape == (units, nmax, 2, d)
    assert np.array_equal(got.reshape(units, nmax, 2 * d), logical)


@pytest.mark.parametrize("dtype,d,units,nmax", [("bf16", 128, 2, 75), ("f32", 64, 3, 16)])
def test_tile_meta_round_trip(dtype, d, units, nmax):
    rng = np.random.default_rng(8)
    np_t = np.int16 if dtype == "bf16" else np.float32
    logical = rng.integers(-30000, 30000, size=(units, nmax, 2, d)).astype(np_t)
    flat = tile_meta(logical)
    assert flat.size == units * ((nmax + 15) // 16) * 16 * 2 * d
    back = untile_meta(torch.from_numpy(flat.view(np.uint8)), units, nmax, d, dtype).numpy()
    assert np.array_equal(back, logical)
