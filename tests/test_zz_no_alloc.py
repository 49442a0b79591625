"""The attention entry point that allocates nothing (its split partials in the
library's per-GPU scratch array) against the entry point with a caller
workspace: bit-identical outputs, and within the attention tolerance of the
oracle, on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

from lookahead_sparse_kv_draft_amd import _lib as L
from lookahead_sparse_kv_draft_amd.runtime import DecodeRuntime
from oracle import oasis_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
BLK = 16


def _case(B, H, G, D, k, ctxs, seed):
    """A runtime with packed pages, a selection with unselected and missing
    blocks, resident pages fetched into the pool; returns (rt, q, oracle outputs)."""
    d = 128
    T = 1 + D
    Nmax = max((c + BLK - 1) // BLK for c in ctxs)
    sh = U.make_shape(batch=B, kv_heads=H, group=G, head_dim=d, max_blocks=Nmax, budget_blocks=k, n_draft=D,
                      fetch_cap=k, dtype="bf16")
    rt = DecodeRuntime(sh)
    rng = np.random.default_rng(seed)
    units = B * H
    K = U.elem_round("bf16", rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32) * 1.5)
    V = U.elem_round("bf16", rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32))
    q = U.elem_round("bf16", rng.standard_normal((B, H * G, T, d)).astype(np.float32))
    for u in range(units):
        rt.pack_unit(0, u, U.to_elem_np("bf16", K[u]), U.to_elem_np("bf16", V[u]))
    rt.set_ctx(ctxs)
    sel = np.full((units, k), -1, dtype=np.int32)
    s2b = np.full((units, k), -1, dtype=np.int32)
    b2s = np.full((units, Nmax), -1, dtype=np.int32)
    fetch = np.full((units, k, 2), -1, dtype=np.int32)
    nfe = np.zeros(units, dtype=np.int32)
    for u in range(units):
        N = (ctxs[u // H] + BLK - 1) // BLK
        m = min(k, N)
        chosen = rng.choice(N, size=m, replace=False)
        sel[u, :m] = chosen
        resident = [b for i, b in enumerate(chosen) if i % 7 != 3][:k]
        slots = rng.permutation(k)[: len(resident)]
        for b, s in zip(resident, slots):
            s2b[u, s] = b
            b2s[u, b] = s
            fetch[u, nfe[u]] = (b, s)
            nfe[u] += 1
    st = rt.state[0][0]
    st.sel.copy_(torch.from_numpy(sel))
    st.b2s.copy_(torch.from_numpy(b2s))
    st.s2b.copy_(torch.from_numpy(s2b))
    L.oasis_fetch_issue(rt.h, st.host_tier, st.pool, fetch, nfe, torch.cuda.current_stream())
    torch.cuda.synchronize()
    refs = {}
    for u in range(units):
        r, hh = divmod(u, H)
        A = O.attended_blocks(sel[u], b2s[u])
        refs[u] = O.sparse_attention(q[r, hh * G:(hh + 1) * G].astype(np.float64), K[u].astype(np.float64),
                                     V[u].astype(np.float64), A, ctxs[r])
    return rt, U.to_dev("bf16", q), refs


def _check(rt, q_d, refs):
    st = rt.state[0][0]
    B, HG = rt.out.shape[0], rt.out.shape[1]
    H, G = rt.shape.kv_heads, rt.shape.group
    # the existing entry point, with a caller workspace
    rt.out.fill_(float("nan"))
    L.oasis_sparse_paged_decode_attn(rt.h, q_d, st.pool, st.sel, st.b2s, rt.ctx_len, rt.out, rt.ws_ptr)
    torch.cuda.synchronize()
    want = rt.out.cpu().numpy().copy()
    # the entry point that allocates nothing
    got_out = torch.full_like(rt.out, float("nan"))
    L.oasis_sparse_paged_decode_attn_noalloc(rt.h, q_d, st.pool, st.sel, st.b2s, rt.ctx_len, got_out)
    torch.cuda.synchronize()
    got = got_out.cpu().numpy()
    assert np.array_equal(got, want)
    for u, ref in refs.items():
        r, hh = divmod(u, H)
        ma, rl = U.attn_errors(got[r, hh * G:(hh + 1) * G].astype(np.float64), ref)
        assert ma <= U.ATTN_MAX_ABS and rl <= U.ATTN_REL_L2, (u, ma, rl)


def test_noalloc_attention_matches_workspace_entry_point():
    # first call: 64 units, 4 attention splits of 128 selected blocks (split partials in the scratch)
    rt, q, refs = _case(B=8, H=8, G=4, D=4, k=128, ctxs=[32768, 2050, 16 * 900 + 5, 4096, 32768, 3000, 2048, 16 * 129],
                        seed=21)
    try:
        _check(rt, q, refs)
    finally:
        rt.close()
    # second call: a smaller input (4 units, 16 selected blocks, ragged contexts)
    rt, q, refs = _case(B=2, H=2, G=4, D=4, k=16, ctxs=[263, 1024], seed=22)
    try:
        _check(rt, q, refs)
    finally:
        rt.close()
