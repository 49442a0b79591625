"""Stage-wise GPU parity: each HIP kernel against the fp64 oracle on the same inputs.

Inputs come from the seeded generators; discrete stages (selection, diff) must
match bit for bit, metadata exactly, scores within the fp32 summation bound and
attention within max-abs 2e-2 / relative-L2 5e-3.
"""
import numpy as np
import pytest
import torch

from lookahead_sparse_kv_draft_amd import _lib as L
from lookahead_sparse_kv_draft_amd.runtime import DecodeRuntime, tile_meta
from oracle import oasis_oracle as O
from tests import gpu_util as U
from workload.synth import random_scores

pytestmark = pytest.mark.gpu
BLK = 16


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ score
@pytest.mark.parametrize("dtype,d,G,D,Nmax,ctxs", [
    ("bf16", 128, 4, 4, 75, [1190, 700]),      # 16 rows, ragged tiles
    ("bf16", 128, 8, 4, 40, [640, 17]),        # 32 rows (two row tiles)
    ("bf16", 128, 4, 5, 33, [528, 513]),       # 20 rows (padded row tile)
    ("bf16", 64, 4, 3, 70, [1024, 1]),         # d = 64, a one-block request
    ("bf16", 128, 16, 3, 300, [4800, 3333]),   # 48 rows, several tiles per wave
    ("f32", 64, 4, 3, 64, [1024, 999]),
    ("f32", 128, 2, 2, 20, [300, 20]),
    # every tile count mod 2, 3 and 4 below the capacity of 19 tiles, so that the
    # last run of some wavefront holds a single in-context tile with capacity past it
    ("bf16", 128, 4, 4, 300, [16 * 16 * 4 + 5, 16 * 16 * 3 + 1, 16 * 16 * 9 + 16, 16 * 16 * 6 + 9, 16 * 16 * 18]),
])
@pytest.mark.parametrize("tpw", [None, 2, 3, 4])
def test_score_parity(dtype, d, G, D, Nmax, ctxs, tpw):
    # tpw: 16-block tiles per scoring wavefront (None: the default for the shape,
    # one tile here)
    B, H = len(ctxs), 2
    sh = U.make_shape(batch=B, kv_heads=H, group=G, head_dim=d, max_blocks=Nmax, n_draft=D, dtype=dtype)
    h = sh.handle(options=None if tpw is None else dict(score_tpw=tpw))
    rng = _rng(1)
    units = B * H
    a = rng.standard_normal((units, Nmax, d)).astype(np.float32)
    b = rng.standard_normal((units, Nmax, d)).astype(np.float32)
    kmin = U.elem_round(dtype, np.minimum(a, b) * 1.5)
    kmax = U.elem_round(dtype, np.maximum(a, b) * 1.5)
    q = U.elem_round(dtype, rng.standard_normal((B, H * G, 1 + D, d)).astype(np.float32))
    meta = np.stack([kmin, kmax], axis=2)  # [units][Nmax][2][d]
    meta_d = U.to_dev(dtype, meta, tiled_meta=True)
    q_d = U.to_dev(dtype, q)
    ctx_d = U.i32(ctxs)
    # the drafts' lookahead score, then the same bound from the verify query rows
    for fn, rows in ((L.oasis_lookahead_score, slice(1, None)), (L.oasis_verify_score, slice(0, 1))):
        scores = torch.full((units, Nmax), float("nan"), device="cuda")
        fn(h, q_d, meta_d, ctx_d, scores)
        torch.cuda.synchronize()
        got = scores.cpu().numpy().astype(np.float64)
        for u in range(units):
            r, hh = divmod(u, H)
            N = (ctxs[r] + BLK - 1) // BLK
            qd = q[r, hh * G:(hh + 1) * G, rows, :].astype(np.float64)
            ref = O.lookahead_score(qd, kmin[u, :N].astype(np.float64), kmax[u, :N].astype(np.float64))
            tol = U.score_tolerance(qd.reshape(-1, d), kmin[u, :N].astype(np.float64),
                                    kmax[u, :N].astype(np.float64))
            err = np.abs(got[u, :N] - ref)
            assert np.all(err <= tol), (fn.__name__, u, float(err.max()), float(tol.min()))
            assert np.all(np.isnan(got[u, N:])), "blocks past the context must not be written"
    L.oasis_destroy(h)


def test_score_standalone_matches_step_launch():
    """At 64 units x 2048 blocks (8192 tiles of 16 blocks) the scoring on its own
    runs 4 tiles per wavefront and the decode step's first launch, beside the
    attention, 2; every block's bound is the same MFMA sequence either way, so
    the two must agree bit for bit, and with the oracle on every unit.  Several
    contexts end on a tile count of 1 mod 4 (and odd) below the capacity: the
    last wavefront of those units holds one in-context tile."""
    B, H, G, D, d, Nmax, k = 8, 8, 4, 4, 128, 2048, 16
    ctxs = [32768, 32768 - 5, 16 * 2000 + 3, 16 * 16 * 65, 16 * 65, 16 * 1024, 16 * (16 * 96 + 1) + 9, 16 * 2047]
    sh = U.make_shape(batch=B, kv_heads=H, group=G, head_dim=d, max_blocks=Nmax, budget_blocks=k, n_draft=D)
    h = sh.handle()
    rng = _rng(11)
    units = B * H
    a = rng.standard_normal((units, Nmax, d), dtype=np.float32)
    b = rng.standard_normal((units, Nmax, d), dtype=np.float32)
    kmin = U.elem_round("bf16", np.minimum(a, b))
    kmax = U.elem_round("bf16", np.maximum(a, b))
    del a, b
    q = U.elem_round("bf16", rng.standard_normal((B, H * G, 1 + D, d)).astype(np.float32))
    meta_d = U.to_dev("bf16", np.stack([kmin, kmax], axis=2), tiled_meta=True)
    q_d = U.to_dev("bf16", q)
    ctx_d = U.i32(ctxs)
    solo = torch.full((units, Nmax), float("nan"), device="cuda")
    L.oasis_lookahead_score(h, q_d, meta_d, ctx_d, solo)
    # the step's first launch with nothing to attend (empty attended lists)
    pool = torch.zeros(L.oasis_pool_bytes(h), dtype=torch.uint8, device="cuda")
    sel = torch.full((units, k), -1, dtype=torch.int32, device="cuda")
    b2s = torch.full((units, Nmax), -1, dtype=torch.int32, device="cuda")
    attend = torch.full((units, k), -1, dtype=torch.int32, device="cuda")
    n_attend = torch.zeros(units, dtype=torch.int32, device="cuda")
    out = torch.zeros((B, H * G, 1 + D, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(L.oasis_workspace_bytes(h) + 256, dtype=torch.uint8, device="cuda")
    ws_ptr = ws.data_ptr() + (-ws.data_ptr()) % 256
    fused = torch.full((units, Nmax), float("nan"), device="cuda")
    L.oasis_attend_and_score(h, q_d, pool, meta_d, ctx_d, ctx_d, sel, b2s, attend, n_attend, fused, out, ws_ptr)
    torch.cuda.synchronize()
    got_solo, got_fused = solo.cpu().numpy(), fused.cpu().numpy()
    assert np.array_equal(got_solo, got_fused, equal_nan=True)
    for u in range(units):
        r, hh = divmod(u, H)
        N = (ctxs[r] + BLK - 1) // BLK
        qd = q[r, hh * G:(hh + 1) * G, 1:].reshape(-1, d).astype(np.float64)
        ref = O.lookahead_score(qd, kmin[u, :N].astype(np.float64), kmax[u, :N].astype(np.float64))
        tol = U.score_tolerance(qd, kmin[u, :N].astype(np.float64), kmax[u, :N].astype(np.float64))
        assert np.all(np.abs(got_solo[u, :N] - ref) <= tol), u
        assert np.all(np.isnan(got_solo[u, N:])), "blocks past the context must not be written"
    L.oasis_destroy(h)


# ------------------------------------------------------------------ top-k
@pytest.mark.parametrize("k,ctxs,kind", [
    (128, [32768, 16 * 130, 16 * 128, 16 * 127 + 3], "normal"),
    (128, [32768, 16 * 3000 + 1, 17, 16], "ties"),
    (16, [1024, 16 * 16, 16 * 17, 5], "ties"),
    (16, [1024, 999, 33, 16 * 18], "const"),
    (2, [1024, 16, 32, 48], "normal"),
    (128, [131072, 131072 - 5, 16 * 129, 16 * 8191], "normal"),   # N = 8192: largest fast-path case
    (128, [16 * 4096, 16 * 4000 + 9, 16 * 200, 16 * 130], "ties"),
    (512, [16 * 3000, 16 * 600, 16 * 513, 77], "normal"),          # k = 512: largest fast-path budget
    (256, [16 * 3000, 16 * 600, 16 * 257, 16 * 200], "ties"),
    # all keys equal: 512 candidates fit the winner list beside the threshold
    # bin (taken whole, trimmed by rank), 513 and more take the ordered tie pass
    (128, [16 * 514, 16 * 515, 16 * 513, 16 * 516], "const"),
    # the workgroup kernel (N > 8192 or k > 514): normal scores, few distinct
    # values and all equal; with ties the threshold's equal keys overflow its
    # list (2 * 128 or 2 * 1024 entries) and take the ordered lowest-index pass
    (128, [16 * 9000, 16 * 8200 + 3, 16 * 8193 + 1, 16 * 300], "normal"),
    (128, [16 * 9000, 16 * 8200 + 3, 16 * 8193 + 1, 16 * 300], "ties"),
    (128, [16 * 9000, 16 * 8200 + 3, 16 * 8193 + 1, 16 * 300], "const"),
    (1024, [16 * 4000, 16 * 3000 + 9, 16 * 2051, 16 * 1030], "normal"),
    (1024, [16 * 9000, 16 * 4000 + 9, 16 * 2051, 16 * 1030], "ties"),
    (1024, [16 * 9000, 16 * 4000 + 9, 16 * 2051, 16 * 100], "const"),
])
def test_topk_parity(k, ctxs, kind):
    B, H = len(ctxs), 3
    Nmax = max((c + BLK - 1) // BLK for c in ctxs)
    sh = U.make_shape(batch=B, kv_heads=H, max_blocks=Nmax, budget_blocks=k)
    h = sh.handle()
    rng = _rng(2)
    sc = np.stack([random_scores(rng, Nmax, kind) for _ in range(B * H)])
    sc_d = torch.from_numpy(sc).cuda()
    sel = torch.full((B * H, k), -7, dtype=torch.int32, device="cuda")
    L.oasis_topk_select(h, sc_d, U.i32(ctxs), sel)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    for u in range(B * H):
        N = (ctxs[u // H] + BLK - 1) // BLK
        ref = O.topk_select(sc[u].astype(np.float64), N, k)
        assert list(got[u]) == ref, (u, N)
    L.oasis_destroy(h)


# ------------------------------------------------------------------ diff / cap / evict
def _random_state(rng, N, k, n_res, kind):
    """A valid selection (forced blocks first) and consistent resident maps."""
    forced = [0] if N == 1 else [0, N - 1]
    others = rng.permutation(np.arange(1, N - 1))[: max(0, min(k, N) - len(forced))]
    sel = forced + [int(b) for b in others]
    sel += [-1] * (k - len(sel))
    s2b = np.full(k, -1, dtype=np.int64)
    res = rng.choice(N, size=min(n_res, N, k), replace=False)
    slots = rng.choice(k, size=len(res), replace=False)
    s2b[slots] = res
    b2s = np.full(N, -1, dtype=np.int64)
    b2s[res] = slots
    sc = random_scores(rng, N, kind)
    return sel, sc, b2s, s2b


@pytest.mark.parametrize("k,cap,N,kind", [
    (128, 32, 2048, "normal"), (128, 16, 2048, "ties"), (128, 0, 2048, "normal"),
    (128, 128, 500, "ties"), (16, 4, 64, "normal"), (16, 1, 20, "const"), (8, 8, 8, "ties"),
    (2, 2, 1, "normal"), (128, 24, 528, "normal"), (128, 32, 8192, "ties"),
    (512, 64, 3000, "ties"), (1024, 200, 4000, "normal"), (300, 300, 700, "const"),
])
def test_diff_parity(k, cap, N, kind):
    B, H = 3, 4
    units = B * H
    sh = U.make_shape(batch=B, kv_heads=H, max_blocks=N, budget_blocks=k, fetch_cap=cap)
    h = sh.handle()
    rng = _rng(3)
    sels, scs, b2ss, s2bs = [], [], [], []
    for u in range(units):
        n_res = [0, k // 2, k, int(rng.integers(0, k + 1))][u % 4]
        sel, sc, b2s, s2b = _random_state(rng, N, k, n_res, kind)
        sels.append(sel), scs.append(sc), b2ss.append(b2s), s2bs.append(s2b)
    sel_d = U.i32(sels)
    sc_d = torch.from_numpy(np.stack(scs)).cuda()
    b2s_d = U.i32(b2ss)
    s2b_d = U.i32(s2bs)
    cw = max(cap, 1)
    fetch = torch.full((units, cw, 2), -9, dtype=torch.int32, device="cuda")
    nf = torch.full((units,), -9, dtype=torch.int32, device="cuda")
    ev = torch.full((units, cw), -9, dtype=torch.int32, device="cuda")
    att = torch.full((units, k), -9, dtype=torch.int32, device="cuda")
    natt = torch.full((units,), -9, dtype=torch.int32, device="cuda")
    L.oasis_resident_diff_cap_evict(h, sel_d, sc_d, b2s_d, s2b_d, fetch, nf, ev, att, natt)
    torch.cuda.synchronize()
    g_b2s, g_s2b = b2s_d.cpu().numpy(), s2b_d.cpu().numpy()
    g_f, g_nf, g_ev = fetch.cpu().numpy(), nf.cpu().numpy(), ev.cpu().numpy()
    g_att, g_natt = att.cpu().numpy(), natt.cpu().numpy()
    for u in range(units):
        ref = O.resident_diff_cap_evict(sels[u], scs[u].astype(np.float64), b2ss[u], s2bs[u], cap)
        # attended list of the next attention: S ∩ R after this fetch, rank order
        exp_att = [(b << 10) | int(ref.block_to_slot[b]) for b in O.attended_blocks(sels[u], ref.block_to_slot)]
        assert g_natt[u] == len(exp_att), u
        assert list(g_att[u][: len(exp_att)]) == exp_att, u
        assert g_nf[u] == len(ref.fetch)
        exp_f = np.full((cw, 2), -9 if cap == 0 else -1)
        for i, (b, s) in enumerate(ref.fetch):
            exp_f[i] = (b, s)
        if cap > 0:
            assert np.array_equal(g_f[u], exp_f), u
            exp_e = np.full(cap, -1)
            exp_e[: len(ref.evict)] = ref.evict
            assert np.array_equal(g_ev[u], exp_e), u
        assert np.array_equal(g_b2s[u], ref.block_to_slot), u
        assert np.array_equal(g_s2b[u], ref.slot_to_block), u
    L.oasis_destroy(h)


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("dtype,d,G,D,k,ctxs", [
    ("bf16", 128, 4, 4, 128, [32768, 2050]),    # 20 rows, split-K over 128 blocks
    ("bf16", 128, 8, 4, 128, [4000, 2048]),     # 40 rows (three row tiles)
    ("bf16", 128, 4, 5, 16, [263, 100]),        # 24 rows, partial newest block
    ("bf16", 64, 4, 3, 16, [1024, 17]),         # d = 64
    ("bf16", 128, 16, 3, 8, [150, 15]),         # 64 rows; one-block request with 15 tokens
    ("f32", 64, 4, 3, 16, [1024, 250]),
    ("f32", 128, 2, 1, 8, [200, 33]),
])
@pytest.mark.parametrize("waves,pf,splits", [(None, None, None), (1, 2, 1), (2, 4, 3), (4, 2, 0), (4, 8, 2),
                                             (1, 8, 5)])
def test_attention_parity(dtype, d, G, D, k, ctxs, waves, pf, splits):
    # launch variants: default shape; 1-, 2- and 4-wavefront workgroups merged in
    # LDS; rings of 2, 4 or 8 pages over runs that are shorter than, equal to or
    # (padded) multiples of the ring; one split or several
    opts = None if waves is None else dict(attn_waves=waves, attn_pf=pf, attn_splits=splits)
    B, H = len(ctxs), 2
    T = 1 + D
    Nmax = max((c + BLK - 1) // BLK for c in ctxs)
    sh = U.make_shape(batch=B, kv_heads=H, group=G, head_dim=d, max_blocks=Nmax, budget_blocks=k,
                      n_draft=D, fetch_cap=k, dtype=dtype)
    rt = DecodeRuntime(sh, options=opts)
    rng = _rng(4)
    units = B * H
    K = U.elem_round(dtype, rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32) * 1.5)
    V = U.elem_round(dtype, rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32))
    q = U.elem_round(dtype, rng.standard_normal((B, H * G, T, d)).astype(np.float32))
    for u in range(units):
        rt.pack_unit(0, u, U.to_elem_np(dtype, K[u]), U.to_elem_np(dtype, V[u]))
    rt.set_ctx(ctxs)
    # selection with some -1 entries and some selected blocks not resident
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
        if m > 2:
            sel[u, m - 1] = -1
        resident = [b for i, b in enumerate(chosen) if i % 5 != 3] + \
            [b for b in rng.choice(N, size=min(N, 4), replace=False) if b not in chosen]
        resident = resident[:k]
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
    q_d = U.to_dev(dtype, q)
    # repeated calls give the same output (deterministic merge)
    outs = []
    for _ in range(3):
        rt.out.fill_(float("nan"))
        rt.attention(0, q_d)
        torch.cuda.synchronize()
        outs.append(rt.out.cpu().numpy().astype(np.float64))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    got = outs[0]
    # the attended-list entry point, on the list the maps define, is bit-identical
    att = np.full((units, k), -1, dtype=np.int32)
    natt = np.zeros(units, dtype=np.int32)
    for u in range(units):
        lst = [(int(b) << 10) | int(b2s[u, b]) for b in O.attended_blocks(sel[u], b2s[u])]
        natt[u] = len(lst)
        att[u, : len(lst)] = lst
    rt.out.fill_(float("nan"))
    L.oasis_sparse_paged_decode_attn_list(rt.h, q_d, st.pool, U.i32(att), U.i32(natt), rt.ctx_len, rt.out,
                                          rt.ws_ptr)
    torch.cuda.synchronize()
    got_list = rt.out.cpu().numpy().astype(np.float64)
    if dtype == "bf16":
        assert np.array_equal(got_list, got)
    else:  # the fp32 kernel splits the list, not the selection: same sums, another order
        assert np.allclose(got_list, got, rtol=1e-5, atol=1e-6)
    if waves is None:
        # the decode step's first half (attention beside the scoring, in one grid
        # where the shape allows) then the split combine: the same attention
        # output as the separate calls (to fp32 reordering) and the same scores,
        # bit for bit
        rt.build_meta(0)
        st.scores.fill_(float("nan"))  # blocks past the context are left unwritten
        L.oasis_lookahead_score(rt.h, q_d, st.meta, rt.ctx_len, st.scores)
        torch.cuda.synchronize()
        ref_scores = st.scores.cpu().numpy().copy()
        variants = [(st.sel, st.b2s, None, None)]
        if dtype == "bf16":
            variants += [(None, None, U.i32(att), U.i32(natt)), (st.sel, st.b2s, U.i32(att), U.i32(natt))]
        for sel_a, b2s_a, att_a, natt_a in variants:
            rt.out.fill_(float("nan"))
            st.scores.fill_(float("nan"))
            L.oasis_attend_and_score(rt.h, q_d, st.pool, st.meta, rt.ctx_len, rt.ctx_len, sel_a, b2s_a, att_a,
                                     natt_a, st.scores, rt.out, rt.ws_ptr)
            L.oasis_attn_combine(rt.h, rt.ws_ptr, rt.out)
            torch.cuda.synchronize()
            # the step's launch may split the list differently from the attention on
            # its own (its own split count): the same sums in another fp32 order
            assert np.allclose(rt.out.cpu().numpy().astype(np.float64), got, rtol=1e-5, atol=1e-6)
            assert np.array_equal(st.scores.cpu().numpy(), ref_scores, equal_nan=True)
    for u in range(units):
        r, hh = divmod(u, H)
        A = O.attended_blocks(sel[u], b2s[u])
        ref = O.sparse_attention(q[r, hh * G:(hh + 1) * G].astype(np.float64), K[u].astype(np.float64),
                                 V[u].astype(np.float64), A, ctxs[r])
        g = got[r, hh * G:(hh + 1) * G]
        ma, rl = U.attn_errors(g, ref)
        assert ma <= U.ATTN_MAX_ABS and rl <= U.ATTN_REL_L2, (u, ma, rl)
    rt.close()


def test_attention_empty_selection_gives_zero():
    sh = U.make_shape(batch=1, kv_heads=1, max_blocks=8, budget_blocks=4)
    rt = DecodeRuntime(sh)
    rt.set_ctx([100])
    q = torch.ones((1, 4, 5, 128), dtype=torch.bfloat16, device="cuda")
    rt.out.fill_(float("nan"))
    rt.attention(0, q)  # sel all -1
    torch.cuda.synchronize()
    assert torch.all(rt.out == 0)
    rt.close()


@pytest.mark.parametrize("waves,pf", [(None, None), (1, 8)])
def test_attention_growing_logits(waves, pf):
    """Logits that grow along the selection order by far more than the lazy
    rescaling threshold, so the running reference max moves many times."""
    opts = None if waves is None else dict(attn_waves=waves, attn_pf=pf)
    B, H, G, D, d, k = 2, 2, 4, 4, 128, 64
    ctxs = [2048, 1500]
    T = 1 + D
    Nmax = 128
    sh = U.make_shape(batch=B, kv_heads=H, group=G, head_dim=d, max_blocks=Nmax, budget_blocks=k,
                      n_draft=D, fetch_cap=k, dtype="bf16")
    rt = DecodeRuntime(sh, options=opts)
    rng = _rng(9)
    units = B * H
    q = U.elem_round("bf16", rng.standard_normal((B, H * G, T, d)).astype(np.float32))
    K = np.empty((units, Nmax * BLK, d), dtype=np.float32)
    V = U.elem_round("bf16", rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32))
    sel = np.full((units, k), -1, dtype=np.int32)
    s2b = np.full((units, k), -1, dtype=np.int32)
    b2s = np.full((units, Nmax), -1, dtype=np.int32)
    fetch = np.full((units, k, 2), -1, dtype=np.int32)
    nfe = np.zeros(units, dtype=np.int32)
    for u in range(units):
        r, hh = divmod(u, H)
        N = (ctxs[r] + BLK - 1) // BLK
        chosen = rng.choice(N, size=k, replace=False)
        sel[u] = chosen
        # keys aligned with the mean query of the unit, scaled up along the rank
        qm = q[r, hh * G:(hh + 1) * G].reshape(-1, d).mean(axis=0)
        qm /= np.linalg.norm(qm)
        base = rng.standard_normal((Nmax * BLK, d)).astype(np.float32)
        for i, b in enumerate(chosen):
            base[b * BLK:(b + 1) * BLK] += qm * (3.0 * i)
        K[u] = U.elem_round("bf16", base)
        for i, b in enumerate(chosen):
            s2b[u, i] = b
            b2s[u, b] = i
            fetch[u, i] = (b, i)
        nfe[u] = k
        rt.pack_unit(0, u, U.to_elem_np("bf16", K[u]), U.to_elem_np("bf16", V[u]))
    rt.set_ctx(ctxs)
    st = rt.state[0][0]
    st.sel.copy_(torch.from_numpy(sel))
    st.b2s.copy_(torch.from_numpy(b2s))
    st.s2b.copy_(torch.from_numpy(s2b))
    L.oasis_fetch_issue(rt.h, st.host_tier, st.pool, fetch, nfe, torch.cuda.current_stream())
    torch.cuda.synchronize()
    rt.out.fill_(float("nan"))
    rt.attention(0, U.to_dev("bf16", q))
    torch.cuda.synchronize()
    got = rt.out.cpu().numpy().astype(np.float64)
    for u in range(units):
        r, hh = divmod(u, H)
        A = O.attended_blocks(sel[u], b2s[u])
        ref = O.sparse_attention(q[r, hh * G:(hh + 1) * G].astype(np.float64), K[u].astype(np.float64),
                                 V[u].astype(np.float64), A, ctxs[r])
        ma, rl = U.attn_errors(got[r, hh * G:(hh + 1) * G], ref)
        assert ma <= U.ATTN_MAX_ABS and rl <= U.ATTN_REL_L2, (u, ma, rl)
    rt.close()


# ------------------------------------------------------------------ metadata
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_meta_build_and_append(dtype, d):
    B, H, Nmax, k = 2, 2, 12, 4
    ctxs = [150, 33]
    steps = 40
    sh = U.make_shape(batch=B, kv_heads=H, head_dim=d, max_blocks=Nmax, budget_blocks=k, fetch_cap=k,
                      dtype=dtype)
    rt = DecodeRuntime(sh)
    rng = _rng(5)
    units = B * H
    K = U.elem_round(dtype, rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32))
    V = U.elem_round(dtype, rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32))
    for u in range(units):
        rt.pack_unit(0, u, U.to_elem_np(dtype, K[u]), U.to_elem_np(dtype, V[u]))
    rt.set_ctx(ctxs)
    rt.build_meta(0)
    st = rt.state[0][0]
    # make the block holding each request's next token resident in slot 1
    s2b = np.full((units, k), -1, dtype=np.int32)
    b2s = np.full((units, Nmax), -1, dtype=np.int32)
    for u in range(units):
        b = ctxs[u // H] // BLK
        s2b[u, 1], b2s[u, b] = b, 1
    st.s2b.copy_(torch.from_numpy(s2b))
    st.b2s.copy_(torch.from_numpy(b2s))
    st.pool.zero_()

    def check(n_per_req):
        m = rt.meta_view(0)
        mv = m.view(torch.bfloat16).float() if dtype == "bf16" else m
        mv = mv.cpu().numpy().astype(np.float64)
        for u in range(units):
            n = n_per_req[u // H]
            kmin, kmax = O.block_meta(K[u].astype(np.float64), n)
            N = kmin.shape[0]
            assert np.array_equal(mv[u, :N, 0], kmin) and np.array_equal(mv[u, :N, 1], kmax), (u, n)

    check(ctxs)
    n = list(ctxs)
    for t in range(steps):
        pos = np.array(n)
        kn = np.stack([K[u, pos[u // H]] for u in range(units)]).reshape(B, H, d)
        vn = np.stack([V[u, pos[u // H]] for u in range(units)]).reshape(B, H, d)
        rt.append(0, U.to_dev(dtype, kn), U.to_dev(dtype, vn), U.to_elem_np(dtype, kn), U.to_elem_np(dtype, vn))
        rt.end_step()
        n = [x + 1 for x in n]
        torch.cuda.synchronize()
        check(n)
        assert list(rt.ctx_len.cpu().numpy()) == n
    # resident page rows written by the append == host tier rows
    pages = rt.pool_pages(0).cpu().numpy()
    eb = sh.elem_bytes
    for u in range(units):
        b = ctxs[u // H] // BLK
        first = ctxs[u // H]
        last = min(n[u // H], (b + 1) * BLK)
        pg = pages[u, 1].view(np.uint16 if dtype == "bf16" else np.float32)
        kp = pg[: BLK * d].reshape(BLK, d)
        vt = pg[BLK * d:].reshape(d, BLK)
        for j in range(first - b * BLK, last - b * BLK):
            assert np.array_equal(kp[j], U.to_elem_np(dtype, K[u, b * BLK + j])), (u, j)
            assert np.array_equal(vt[:, j], U.to_elem_np(dtype, V[u, b * BLK + j])), (u, j)
        ht = rt.host_tier_view(0).numpy().view(np.uint16 if dtype == "bf16" else np.float32)
        ht = ht.reshape(units, Nmax, 2 * BLK * d)
        hp = ht[u, b]
        for j in range(first - b * BLK, last - b * BLK):
            assert np.array_equal(hp[: BLK * d].reshape(BLK, d)[j], U.to_elem_np(dtype, K[u, b * BLK + j]))
    rt.close()


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_append_outside_capacity_keeps_the_context(dtype, d):
    """A request whose position is at the capacity (16 * max_blocks) appends
    nothing: no metadata, no page row, and its grown context stays the
    position; the other requests of the same launch (one of them at the last
    position inside the capacity) append as usual."""
    from lookahead_sparse_kv_draft_amd import _lib as L
    B, H, Nmax, k = 3, 2, 4, 4
    cap = Nmax * BLK
    ctxs = [cap, 40, cap - 1]
    sh = U.make_shape(batch=B, kv_heads=H, head_dim=d, max_blocks=Nmax, budget_blocks=k, fetch_cap=k,
                      dtype=dtype)
    rt = DecodeRuntime(sh)
    rng = _rng(6)
    units = B * H
    K = U.elem_round(dtype, rng.standard_normal((units, cap, d)).astype(np.float32))
    V = U.elem_round(dtype, rng.standard_normal((units, cap, d)).astype(np.float32))
    for u in range(units):
        rt.pack_unit(0, u, U.to_elem_np(dtype, K[u]), U.to_elem_np(dtype, V[u]))
    rt.set_ctx(ctxs)
    rt.build_meta(0)
    st = rt.state[0][0]
    # the block of every request's position (the last one where it is at the capacity) resident in slot 0
    s2b = np.full((units, k), -1, dtype=np.int32)
    b2s = np.full((units, Nmax), -1, dtype=np.int32)
    for u in range(units):
        b = min(ctxs[u // H], cap - 1) // BLK
        s2b[u, 0], b2s[u, b] = b, 0
    st.s2b.copy_(torch.from_numpy(s2b))
    st.b2s.copy_(torch.from_numpy(b2s))
    st.pool.zero_()
    torch.cuda.synchronize()
    meta0 = rt.meta_view(0).clone()
    # new tokens: fresh rows (request 0's would go past the capacity)
    kn = U.elem_round(dtype, rng.standard_normal((B, H, d)).astype(np.float32) * 3)
    vn = U.elem_round(dtype, rng.standard_normal((B, H, d)).astype(np.float32))
    ctx_in = torch.tensor(ctxs, dtype=torch.int32, device="cuda")
    ctx_out = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    L.oasis_block_meta_update(rt.h, U.to_dev(dtype, kn), U.to_dev(dtype, vn), ctx_in, ctx_out, st.meta, st.pool,
                              st.b2s)
    torch.cuda.synchronize()
    assert ctx_out.cpu().tolist() == [cap, 41, cap]
    m = rt.meta_view(0)
    assert torch.equal(m[0:H], meta0[0:H])  # request 0: untouched
    mv = (m.view(torch.bfloat16).float() if dtype == "bf16" else m).cpu().numpy().astype(np.float64)
    pages = rt.pool_pages(0).cpu().numpy()
    for u in range(H, units):
        n = ctxs[u // H]
        kmin, kmax = O.block_meta(K[u].astype(np.float64), n)
        kmin, kmax = O.block_meta_append(kmin, kmax, n, kn.reshape(units, d)[u].astype(np.float64))
        N = kmin.shape[0]
        assert np.array_equal(mv[u, :N, 0], kmin) and np.array_equal(mv[u, :N, 1], kmax), u
        pg = pages[u, 0].view(np.uint16 if dtype == "bf16" else np.float32)
        j = n % BLK
        assert np.array_equal(pg[: BLK * d].reshape(BLK, d)[j], U.to_elem_np(dtype, kn.reshape(units, d)[u])), u
        assert np.array_equal(pg[BLK * d:].reshape(d, BLK)[:, j], U.to_elem_np(dtype, vn.reshape(units, d)[u])), u
    assert not pages[0:H].any()  # request 0's resident page: nothing written
    with pytest.raises(ValueError, match="capacity"):
        rt.append(0, U.to_dev(dtype, kn), U.to_dev(dtype, vn))
    rt.close()


@pytest.mark.parametrize("dtype,d,nmax", [("bf16", 128, 37), ("f32", 64, 16), ("bf16", 64, 5)])
def test_meta_export_and_import(dtype, d, nmax):
    """The tiles built from pages, read back through the export, equal the
    oracle's per-block min/max; the import of those logical rows rebuilds the
    very same tile bytes, and the host packing agrees with both."""
    B, H = 2, 3
    ctxs = [nmax * BLK, nmax * BLK - 7]
    sh = U.make_shape(batch=B, kv_heads=H, head_dim=d, max_blocks=nmax, budget_blocks=4, fetch_cap=4,
                      dtype=dtype)
    rt = DecodeRuntime(sh)
    rng = _rng(11)
    units = B * H
    K = U.elem_round(dtype, rng.standard_normal((units, nmax * BLK, d)).astype(np.float32))
    for u in range(units):
        rt.pack_unit(0, u, U.to_elem_np(dtype, K[u]), U.to_elem_np(dtype, K[u]))
    rt.set_ctx(ctxs)
    rt.build_meta(0)
    torch.cuda.synchronize()
    exported = rt.meta_view(0)
    torch.cuda.synchronize()
    ev = exported.view(torch.bfloat16).float() if dtype == "bf16" else exported
    ev = ev.cpu().numpy().astype(np.float64)
    for u in range(units):
        kmin, kmax = O.block_meta(K[u].astype(np.float64), ctxs[u // H])
        N = kmin.shape[0]
        assert np.array_equal(ev[u, :N, 0], kmin) and np.array_equal(ev[u, :N, 1], kmax), u
    built = rt.state[0][0].meta.clone()
    fresh = torch.zeros_like(built)
    L.oasis_block_meta_import(rt.h, exported, fresh)
    torch.cuda.synchronize()
    n_valid = units * ((nmax + 15) // 16) * 16 * 2 * d * sh.elem_bytes
    assert torch.equal(fresh[:n_valid], built[:n_valid])
    host = tile_meta(exported.cpu().numpy())
    assert np.array_equal(fresh[:n_valid].cpu().numpy(), host.view(np.uint8))
    rt.state[0][0].meta.zero_()
    rt.load_meta(0, exported)
    torch.cuda.synchronize()
    assert torch.equal(rt.state[0][0].meta[:n_valid], built[:n_valid])
    rt.close()


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_meta_build_from_key_rows(dtype, d):
    """The metadata from key rows and a token range: every block the range
    touches equals the oracle's min/max over the block's tokens below the
    context, the others keep what they held, and a whole-range build equals the
    build from staged pages."""
    B, H, Nmax = 3, 2, 40
    ctxs = [Nmax * BLK, 16 * 21 + 5, 16 * 3]
    sh = U.make_shape(batch=B, kv_heads=H, head_dim=d, max_blocks=Nmax, budget_blocks=4, fetch_cap=4, dtype=dtype)
    rt = DecodeRuntime(sh)
    rng = _rng(17)
    units = B * H
    K = U.elem_round(dtype, rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32))
    for u in range(units):
        rt.pack_unit(0, u, U.to_elem_np(dtype, K[u]), U.to_elem_np(dtype, K[u]))
    rt.set_ctx(ctxs)
    rt.build_meta(0)
    torch.cuda.synchronize()
    staged = rt.state[0][0].meta.clone()
    k_rows = U.to_dev(dtype, K.reshape(B, H, Nmax * BLK, d))
    n_tiles = units * ((Nmax + 15) // 16) * 16 * 2 * d * sh.elem_bytes
    meta = torch.zeros_like(staged)
    L.oasis_block_meta_build_rows(rt.h, k_rows, 0, Nmax * BLK, rt.ctx_len, meta)
    torch.cuda.synchronize()
    assert torch.equal(meta[:n_tiles], staged[:n_tiles])
    # a range that starts and ends inside blocks: blocks 5 .. 12 only
    meta2 = torch.zeros_like(staged)
    L.oasis_block_meta_build_rows(rt.h, k_rows, 16 * 5 + 3, 16 * 12 + 1, rt.ctx_len, meta2)
    torch.cuda.synchronize()
    lg = torch.empty((units, Nmax, 2, d), dtype=torch.int16 if dtype == "bf16" else torch.float32, device="cuda")
    L.oasis_block_meta_export(rt.h, meta2, lg)
    torch.cuda.synchronize()
    mv = (lg.view(torch.bfloat16).float() if dtype == "bf16" else lg).cpu().numpy().astype(np.float64)
    for u in range(units):
        n = ctxs[u // H]
        kmin, kmax = O.block_meta(K[u].astype(np.float64), n)
        N = kmin.shape[0]
        for b in range(Nmax):
            if 5 <= b <= 12 and b < N:
                assert np.array_equal(mv[u, b, 0], kmin[b]) and np.array_equal(mv[u, b, 1], kmax[b]), (u, b)
            else:
                assert not mv[u, b].any(), (u, b)
    rt.close()


def test_fetch_issue_copies_pages():
    sh = U.make_shape(batch=2, kv_heads=2, max_blocks=40, budget_blocks=8, fetch_cap=5)
    rt = DecodeRuntime(sh)
    rng = _rng(6)
    ht = rt.host_tier_view(0)
    ht.copy_(torch.from_numpy(rng.integers(0, 255, size=ht.numel(), dtype=np.uint8)))
    st = rt.state[0][0]
    st.pool.zero_()
    fetch = np.full((4, 5, 2), -1, dtype=np.int32)
    nf = np.array([5, 0, 3, 1], dtype=np.int32)
    for u in range(4):
        blocks = rng.choice(40, size=nf[u], replace=False)
        slots = rng.choice(8, size=nf[u], replace=False)
        fetch[u, : nf[u]] = np.stack([blocks, slots], axis=1)
    L.oasis_fetch_issue(rt.h, st.host_tier, st.pool, fetch, nf, rt.side)
    rt.side.synchronize()
    pb = L.oasis_page_bytes(rt.h)
    host = ht.numpy().reshape(4, 40, pb)
    pool = st.pool.cpu().numpy().reshape(4, 8, pb)
    for u in range(4):
        used = set()
        for i in range(nf[u]):
            b, s = fetch[u, i]
            assert np.array_equal(pool[u, s], host[u, b])
            used.add(s)
        for s in set(range(8)) - used:
            assert not pool[u, s].any()
    rt.close()


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_fetch_gather_matches_fetch_issue(dtype, d):
    """The device-driven gather copies exactly the pages the host-issued copies
    do, skips entries beyond n_fetch and entries out of range, and touches no
    other slot."""
    B, H, Nmax, k, cap = 2, 2, 40, 8, 5
    sh = U.make_shape(batch=B, kv_heads=H, head_dim=d, max_blocks=Nmax, budget_blocks=k, fetch_cap=cap,
                      dtype=dtype)
    rt = DecodeRuntime(sh)
    rng = _rng(16)
    ht = rt.host_tier_view(0)
    ht.copy_(torch.from_numpy(rng.integers(0, 255, size=ht.numel(), dtype=np.uint8)))
    st = rt.state[0][0]
    units = B * H
    fetch = np.full((units, cap, 2), -1, dtype=np.int32)
    nf = np.array([5, 0, 3, 2], dtype=np.int32)
    for u in range(units):
        blocks = rng.choice(Nmax, size=cap, replace=False)
        slots = rng.choice(k, size=cap, replace=False)
        fetch[u] = np.stack([blocks, slots], axis=1)   # entries >= n_fetch hold valid-looking pairs
    fetch_bad = fetch.copy()
    fetch_bad[0, 1] = (Nmax + 3, 2)   # block out of range: skipped by the gather
    fetch_bad[2, 0] = (4, k)          # slot out of range: skipped
    pb = L.oasis_page_bytes(rt.h)
    host = ht.numpy().reshape(units, Nmax, pb)
    # host-issued copies of the valid lists
    st.pool.zero_()
    L.oasis_fetch_issue(rt.h, st.host_tier, st.pool, fetch, nf, rt.side)
    rt.side.synchronize()
    ref = st.pool.cpu().numpy().reshape(units, k, pb).copy()
    # the gather from device-resident lists
    st.pool.zero_()
    L.oasis_fetch_gather(rt.h, st.host_tier, st.pool, U.i32(fetch), U.i32(nf))
    torch.cuda.synchronize()
    got = st.pool.cpu().numpy().reshape(units, k, pb)
    assert np.array_equal(got, ref)
    # out-of-range entries are skipped, the rest of the list still lands
    st.pool.zero_()
    L.oasis_fetch_gather(rt.h, st.host_tier, st.pool, U.i32(fetch_bad), U.i32(nf))
    torch.cuda.synchronize()
    got = st.pool.cpu().numpy().reshape(units, k, pb)
    for u in range(units):
        filled = set()
        for i in range(nf[u]):
            b, s = fetch_bad[u, i]
            if 0 <= b < Nmax and 0 <= s < k:
                assert np.array_equal(got[u, s], host[u, b]), (u, i)
                filled.add(s)
        for s in set(range(k)) - filled:
            assert not got[u, s].any(), (u, s)
    # pageable host memory is refused before any launch (empty lists, so even a
    # launch would touch nothing)
    plain = np.zeros(ht.numel(), dtype=np.uint8)
    with pytest.raises(L.OasisError) as e:
        L.oasis_fetch_gather(rt.h, plain, st.pool, U.i32(fetch), U.i32(np.zeros(units, dtype=np.int32)))
    assert e.value.code == L.OASIS_EINVAL
    rt.close()


@pytest.mark.parametrize("k,cap,ctxs,kind", [
    (128, 32, [32768, 16 * 700 + 3, 16 * 130, 100], "normal"),
    (128, 16, [32768, 32768, 16 * 129, 16 * 2], "ties"),
    (16, 4, [1024, 999, 16 * 17, 16], "const"),
    (128, 0, [16 * 528, 16 * 600, 16 * 300, 16 * 129], "normal"),
    (512, 100, [16 * 3000, 16 * 600, 16 * 513, 77], "ties"),       # largest fused budget
    (128, 32, [131072 + 16 * 10, 16 * 900, 16 * 130, 16 * 50], "normal"),  # N > 8192: two launches
    # k = 2: only the sink and the newest block are selected (nothing to rank), yet
    # resident blocks must still be ranked as victims by their order keys
    (2, 2, [16 * 100, 16 * 37 + 5, 33, 16], "normal"),
    (2, 1, [16 * 300, 16 * 64, 16 * 3, 100], "ties"),
    # the workgroup selection's larger sizes: 1024 threads with 4 and 8 keys each
    (128, 32, [16 * 3000, 16 * 2100, 16 * 700, 16 * 2049], "normal"),
    (128, 16, [131072, 16 * 5000, 16 * 4097, 16 * 300], "ties"),
    # a cap above the budget (at most k blocks move; the lists are cap long)
    (64, 100, [16 * 700, 16 * 64, 16 * 200, 40], "normal"),
])
def test_select_and_diff_matches_separate_calls_and_oracle(k, cap, ctxs, kind):
    B, H = len(ctxs), 3
    Nmax = max((c + BLK - 1) // BLK for c in ctxs)
    units = B * H
    sh = U.make_shape(batch=B, kv_heads=H, max_blocks=Nmax, budget_blocks=k, fetch_cap=cap)
    h = sh.handle()
    rng = _rng(7)
    sc = np.stack([random_scores(rng, Nmax, kind) for _ in range(units)])
    b2s0 = np.full((units, Nmax), -1, dtype=np.int32)
    s2b0 = np.full((units, k), -1, dtype=np.int32)
    for u in range(units):
        N = (ctxs[u // H] + BLK - 1) // BLK
        n_res = [0, k // 2, k, int(rng.integers(0, k + 1))][u % 4]
        res = rng.choice(N, size=min(n_res, N), replace=False)
        slots = rng.choice(k, size=len(res), replace=False)
        s2b0[u, slots] = res
        b2s0[u, res] = slots
    cw = max(cap, 1)
    outs = []
    for fused in (False, True):
        sel = torch.full((units, k), -7, dtype=torch.int32, device="cuda")
        b2s, s2b = U.i32(b2s0), U.i32(s2b0)
        fetch = torch.full((units, cw, 2), -9, dtype=torch.int32, device="cuda")
        nf = torch.full((units,), -9, dtype=torch.int32, device="cuda")
        ev = torch.full((units, cw), -9, dtype=torch.int32, device="cuda")
        att = torch.full((units, k), -9, dtype=torch.int32, device="cuda")
        natt = torch.full((units,), -9, dtype=torch.int32, device="cuda")
        sc_d, ctx_d = torch.from_numpy(sc).cuda(), U.i32(ctxs)
        if fused:
            L.oasis_select_and_diff(h, sc_d, ctx_d, sel, b2s, s2b, fetch, nf, ev, att, natt)
        else:
            L.oasis_topk_select(h, sc_d, ctx_d, sel)
            L.oasis_resident_diff_cap_evict(h, sel, sc_d, b2s, s2b, fetch, nf, ev, att, natt)
        torch.cuda.synchronize()
        na = natt.cpu().numpy()
        am = att.cpu().numpy()
        am = [list(am[u][: na[u]]) for u in range(units)]
        outs.append([x.cpu().numpy() for x in (sel, b2s, s2b, fetch, nf, ev, natt)] + [am])
    for a, b in zip(*outs):
        assert (a == b) if isinstance(a, list) else np.array_equal(a, b)
    sel, b2s, s2b, fetch, nf, ev, natt, am = outs[1]
    for u in range(units):
        N = (ctxs[u // H] + BLK - 1) // BLK
        ref_sel = O.topk_select(sc[u].astype(np.float64), N, k)
        assert list(sel[u]) == ref_sel, u
        ref = O.resident_diff_cap_evict(ref_sel, sc[u].astype(np.float64), b2s0[u], s2b0[u], cap)
        assert nf[u] == len(ref.fetch)
        assert [tuple(p) for p in fetch[u][: nf[u]]] == ref.fetch, u
        assert list(ev[u][: len(ref.evict)]) == ref.evict
        assert np.array_equal(b2s[u], ref.block_to_slot) and np.array_equal(s2b[u], ref.slot_to_block)
        assert am[u] == [(b << 10) | int(ref.block_to_slot[b]) for b in O.attended_blocks(ref_sel, ref.block_to_slot)]
    L.oasis_destroy(h)


@pytest.mark.parametrize("Nmax,k,cap,kind,ctxs", [
    (300, 64, 16, "ties", [16 * 300, 16 * 170 + 5]),          # 4 keys per thread
    (2048, 128, 32, "ties", [16 * 2048, 16 * 1500 + 9]),      # 16 keys per thread
    (2048, 128, 32, "const", [16 * 2048, 16 * 131]),
    (8192, 128, 32, "ties", [16 * 8192, 16 * 6000 + 3]),      # 64 keys per thread
    (8192, 128, 16, "const", [16 * 8192, 16 * 4100]),
    (8192, 128, 32, "normal", [16 * 8000, 16 * 129]),
    # one to three blocks: only the forced blocks, or a single candidate
    (300, 64, 16, "normal", [1, 16 * 2 + 1]),
    (2048, 128, 8, "ties", [16, 17]),
])
def test_carried_selection_matches_select_and_diff(Nmax, k, cap, kind, ctxs):
    """The selection and diff carried by a decode step's first launch (128-thread
    workgroups, 4 to 64 keys per thread) on tie-heavy and constant scores, which
    take the radix select's later passes and its ordered tie pass: selection,
    both maps, fetch and evict lists and the attended list bit-identical to
    oasis_select_and_diff on the same state, and the selection the oracle's."""
    B, H = len(ctxs), 2
    units = B * H
    sh = U.make_shape(batch=B, kv_heads=H, max_blocks=Nmax, budget_blocks=k, fetch_cap=cap)
    h = sh.handle()
    rng = _rng(31)
    # this step's own inputs: zeros, nothing attended (its outputs are not compared)
    d, T = sh.head_dim, sh.T
    q = torch.zeros((B, sh.q_heads, T, d), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((units * k * 2 * 16 * d,), dtype=torch.bfloat16, device="cuda")
    meta = torch.zeros((L.oasis_meta_bytes(h),), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((L.oasis_workspace_bytes(h),), dtype=torch.uint8, device="cuda")
    ctx_own = U.i32([16 * Nmax] * B)
    att_own = torch.zeros((units, k), dtype=torch.int32, device="cuda")
    natt_own = torch.zeros((units,), dtype=torch.int32, device="cuda")
    sc_own = torch.zeros((units, Nmax), dtype=torch.float32, device="cuda")
    out = torch.zeros((B, sh.q_heads, T, d), dtype=torch.float32, device="cuda")
    # the carried state
    sc = np.stack([random_scores(rng, Nmax, kind) for _ in range(units)])
    b2s0 = np.full((units, Nmax), -1, dtype=np.int32)
    s2b0 = np.full((units, k), -1, dtype=np.int32)
    for u in range(units):
        N = (ctxs[u // H] + BLK - 1) // BLK
        n_res = [k, k // 2, int(rng.integers(0, k + 1)), 0][u % 4]
        res = rng.choice(N, size=min(n_res, N), replace=False)
        slots = rng.choice(k, size=len(res), replace=False)
        s2b0[u, slots] = res
        b2s0[u, res] = slots
    sc_d, ctx_d = torch.from_numpy(sc).cuda(), U.i32(ctxs)
    outs = []
    for carried in (True, False):
        sel = torch.full((units, k), -7, dtype=torch.int32, device="cuda")
        b2s, s2b = U.i32(b2s0), U.i32(s2b0)
        fetch = torch.full((units, cap, 2), -9, dtype=torch.int32, device="cuda")
        nf = torch.full((units,), -9, dtype=torch.int32, device="cuda")
        ev = torch.full((units, cap), -9, dtype=torch.int32, device="cuda")
        att = torch.full((units, k), -9, dtype=torch.int32, device="cuda")
        natt = torch.full((units,), -9, dtype=torch.int32, device="cuda")
        if carried:
            L.oasis_decode_step_carry(h, q, pool, meta, ctx_own, ctx_own, att_own, natt_own, sc_own, out, ws,
                                      job=(sc_d, ctx_d, sel, b2s, s2b, fetch, nf, ev, att, natt))
        else:
            L.oasis_select_and_diff(h, sc_d, ctx_d, sel, b2s, s2b, fetch, nf, ev, att, natt)
        torch.cuda.synchronize()
        na = natt.cpu().numpy()
        am = att.cpu().numpy()
        am = [list(am[u][: na[u]]) for u in range(units)]
        outs.append([x.cpu().numpy() for x in (sel, b2s, s2b, fetch, nf, ev, natt)] + [am])
    for i, (a, b) in enumerate(zip(*outs)):
        assert (a == b) if isinstance(a, list) else np.array_equal(a, b), i
    sel = outs[0][0]
    for u in range(units):
        N = (ctxs[u // H] + BLK - 1) // BLK
        assert list(sel[u]) == O.topk_select(sc[u].astype(np.float64), N, k), u
    L.oasis_destroy(h)


# ------------------------------------------------------------------ LRU eviction
@pytest.mark.parametrize("k,cap,N,kind,steps", [
    (128, 32, 2048, "normal", 6), (128, 8, 700, "ties", 6), (16, 4, 64, "normal", 8),
    (64, 64, 300, "normal", 5), (128, 0, 500, "normal", 3), (8, 3, 40, "const", 6), (2, 2, 9, "normal", 4),
    (128, 32, 5000, "normal", 4), (32, 50, 200, "normal", 4),
])
def test_select_and_diff_lru_parity(k, cap, N, kind, steps):
    """Several steps in a row of selection + diff with least-recently-used
    eviction against the oracle, bit for bit: selection, fetch and eviction
    lists, both maps, the per-slot stamps and the attended list."""
    B, H = 2, 3
    units = B * H
    ctxs = [N * BLK, max(1, N * BLK - 37)]
    sh = U.make_shape(batch=B, kv_heads=H, max_blocks=N, budget_blocks=k, fetch_cap=cap)
    h = sh.handle()
    rng = _rng(21)
    b2ss, s2bs, lus = [], [], []
    for u in range(units):
        Nu = (ctxs[u // H] + BLK - 1) // BLK
        _, _, b2s, s2b = _random_state(rng, Nu, k, [0, k // 2, k][u % 3], kind)
        full = np.full(N, -1, dtype=np.int64)
        full[:Nu] = b2s
        b2ss.append(full), s2bs.append(s2b), lus.append(rng.integers(-1, 3, size=k))
    b2s_d, s2b_d, lu_d = U.i32(b2ss), U.i32(s2bs), U.i32(lus)
    ctx_d = U.i32(ctxs)
    cw = max(cap, 1)
    sel_d = torch.full((units, k), -9, dtype=torch.int32, device="cuda")
    for t in range(steps):
        scs = np.stack([random_scores(rng, N, kind) for _ in range(units)])
        sc_d = torch.from_numpy(scs).cuda()
        fetch = torch.full((units, cw, 2), -9, dtype=torch.int32, device="cuda")
        nf = torch.full((units,), -9, dtype=torch.int32, device="cuda")
        ev = torch.full((units, cw), -9, dtype=torch.int32, device="cuda")
        att = torch.full((units, k), -9, dtype=torch.int32, device="cuda")
        natt = torch.full((units,), -9, dtype=torch.int32, device="cuda")
        L.oasis_select_and_diff_lru(h, sc_d, ctx_d, sel_d, b2s_d, s2b_d, lu_d, 100 + t, fetch, nf, ev, att, natt)
        torch.cuda.synchronize()
        g = [x.cpu().numpy() for x in (sel_d, b2s_d, s2b_d, lu_d, fetch, nf, ev, att, natt)]
        for u in range(units):
            Nu = (ctxs[u // H] + BLK - 1) // BLK
            sel = O.topk_select(scs[u].astype(np.float64), Nu, k)
            ref = O.resident_diff_cap_evict_lru(sel, scs[u].astype(np.float64), b2ss[u], s2bs[u], lus[u], cap, 100 + t)
            assert list(g[0][u]) == sel, (t, u)
            assert np.array_equal(g[1][u], ref.block_to_slot), (t, u)
            assert np.array_equal(g[2][u], ref.slot_to_block), (t, u)
            assert np.array_equal(g[3][u], ref.last_use), (t, u)
            assert g[5][u] == len(ref.fetch), (t, u)
            if cap > 0:
                exp_f = np.full((cw, 2), -1)
                for i, (b, s) in enumerate(ref.fetch):
                    exp_f[i] = (b, s)
                assert np.array_equal(g[4][u], exp_f), (t, u)
                exp_e = np.full(cap, -1)
                exp_e[: len(ref.evict)] = ref.evict
                assert np.array_equal(g[6][u], exp_e), (t, u)
            exp_att = [(b << 10) | int(ref.block_to_slot[b]) for b in O.attended_blocks(sel, ref.block_to_slot)]
            assert g[8][u] == len(exp_att) and list(g[7][u][: len(exp_att)]) == exp_att, (t, u)
            b2ss[u], s2bs[u], lus[u] = ref.block_to_slot, ref.slot_to_block, ref.last_use
    # more than 128 blocks of budget: not supported by the LRU variant
    h2 = U.make_shape(batch=1, kv_heads=1, max_blocks=300, budget_blocks=256, fetch_cap=4).handle()
    z = torch.zeros(1024, dtype=torch.int32, device="cuda")
    with pytest.raises(L.OasisError) as e:
        L.oasis_select_and_diff_lru(h2, z, z, z, z, z, z, 0, z, z, z)
    assert e.value.code == L.OASIS_EUNSUPPORTED
    L.oasis_destroy(h2)
    L.oasis_destroy(h)


def test_select_diff_combine_lru_matches_two_calls():
    """The step's second launch with LRU eviction leaves the same output and
    state as the split combine followed by the LRU selection + diff."""
    from workload import CONFIGS
    from lookahead_sparse_kv_draft_amd.synthetic import SyntheticRun
    cfg = CONFIGS["llama8b_32k"].with_(batch=2, ctx=16 * 300 + 7, steps=3, fetch_cap=8, planted=15,
                                       budget_tokens=16 * 32)
    run = SyntheticRun(cfg, overlap=False, replicas=2)
    try:
        run.prologue()
        rt = run.rt
        rt.state[0][1].copy_from(rt.state[0][0])
        lus = [torch.full((rt.shape.units, rt.shape.budget_blocks), -1, dtype=torch.int32, device="cuda")
               for _ in range(2)]
        outs = [torch.zeros_like(rt.out) for _ in range(2)]
        for t in range(cfg.steps):
            q = run.q[0, t + 1]
            for rep in range(2):
                st = rt.state[0][rep]
                L.oasis_attend_and_score(rt.h, q, st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.sel, st.b2s, st.attend,
                                         st.n_attend, st.scores, outs[rep], rt.ws_ptr)
                if rep == 0:
                    L.oasis_select_diff_combine_lru(rt.h, st.scores, rt.ctx_len, st.sel, st.b2s, st.s2b, lus[rep], t,
                                                    st.fetch, st.n_fetch, st.evict, st.attend, st.n_attend,
                                                    outs[rep], rt.ws_ptr)
                else:
                    L.oasis_attn_combine(rt.h, rt.ws_ptr, outs[rep])
                    L.oasis_select_and_diff_lru(rt.h, st.scores, rt.ctx_len, st.sel, st.b2s, st.s2b, lus[rep], t,
                                                st.fetch, st.n_fetch, st.evict, st.attend, st.n_attend)
            torch.cuda.synchronize()
            a, b = rt.state[0][0], rt.state[0][1]
            assert torch.equal(outs[0], outs[1]), t
            assert torch.equal(lus[0], lus[1]), t
            for name in ("sel", "b2s", "s2b", "fetch", "n_fetch", "evict", "attend", "n_attend"):
                assert torch.equal(getattr(a, name), getattr(b, name)), (t, name)
    finally:
        run.close()


# ------------------------------------------------------------------ prefill admission
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_admit_parity(dtype, d):
    """Admission of a device-resident prefill: every page below the context in
    the pinned host tier (K token-major, V channel-major, bytes as given), the
    metadata rows equal to the oracle's min/max, resident blocks' pages in their
    pool slots, and nothing past the context touched."""
    B, H, Nmax, k = 2, 2, 13, 8
    ctxs = [Nmax * BLK, 7 * BLK + 5]
    sh = U.make_shape(batch=B, kv_heads=H, head_dim=d, max_blocks=Nmax, budget_blocks=k, dtype=dtype)
    rt = DecodeRuntime(sh)
    rt.set_ctx(ctxs)
    units = B * H
    rng = _rng(31)
    K = U.elem_round(dtype, rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32))
    V = U.elem_round(dtype, rng.standard_normal((units, Nmax * BLK, d)).astype(np.float32))
    b2s = np.full((units, Nmax), -1, dtype=np.int32)
    for u in range(units):
        N = (ctxs[u // H] + BLK - 1) // BLK
        for s, b in enumerate(rng.choice(N, size=min(k, N, 5), replace=False)):
            b2s[u, b] = s
    st = rt.state[0][0]
    L.oasis_admit(rt.h, U.to_dev(dtype, K), U.to_dev(dtype, V), rt.ctx_len, st.host_tier, st.meta, st.pool,
                  U.i32(b2s))
    torch.cuda.synchronize()
    Ke, Ve = U.to_elem_np(dtype, K), U.to_elem_np(dtype, V)
    tier = st.host_tier.numpy().view(Ke.dtype).reshape(units, Nmax, -1)
    pool = st.pool.cpu().numpy().view(Ke.dtype).reshape(units, k, -1)
    m = rt.meta_view(0)
    mv = (m.view(torch.bfloat16).float() if dtype == "bf16" else m).cpu().numpy().astype(np.float64)
    for u in range(units):
        n = ctxs[u // H]
        N = (n + BLK - 1) // BLK
        kmin, kmax = O.block_meta(K[u].astype(np.float64), n)
        assert np.array_equal(mv[u, :N, 0], kmin) and np.array_equal(mv[u, :N, 1], kmax), u
        for b in range(Nmax):
            if b >= N:
                assert not tier[u, b].any(), (u, b)   # untouched (the tier starts zeroed)
                continue
            page = np.concatenate([Ke[u, b * BLK:(b + 1) * BLK].reshape(-1),
                                   Ve[u, b * BLK:(b + 1) * BLK].T.reshape(-1)])
            assert np.array_equal(tier[u, b], page), (u, b)
            if b2s[u, b] >= 0:
                assert np.array_equal(pool[u, b2s[u, b]], page), (u, b)
    rt.close()
