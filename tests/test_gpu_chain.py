"""Chained GPU parity: the whole multi-step decode chain (prologue, attention,
append, scoring, selection, diff/cap/evict, transfer) against the oracle.

Every recorded unit is compared over every step; where the GPU's fp32 scores
order near-tied blocks differently from the oracle's fp64 ones, the oracle
adopts the GPU's valid choice, counts the event and continues.  Small workloads
are recorded on every unit; the full-size workloads run in the launch
configuration the benchmark times, on every unit of the benchmark's workload
and of the reasoning workload, and on one whole layer plus samples of the
other layers of the two eight-layer workloads (each unit's chain is
independent of the others).
"""
import numpy as np
import pytest
import torch

from lookahead_sparse_kv_draft_amd.synthetic import SyntheticRun
from oracle import oasis_oracle as O
from tests import chain_compare as CC
from workload import CONFIGS, synth

pytestmark = pytest.mark.gpu


def _run_and_compare(cfg, units, steps=None, layers=None, overlap=False, gather=True, options=None,
                     eviction="score", transfer_group=1, transfer_mode="side", carry_select=False):
    """Runs the chain on the GPU recording `units`, then compares every recorded
    unit with the oracle over every step (near ties adopted and counted)."""
    cfg = cfg if steps is None else cfg.with_(steps=steps)
    print(f"{cfg.name}: filling host tier and metadata ({len(units)} units recorded)", flush=True)
    run = SyntheticRun(cfg, layers=layers, record_units=units, overlap=overlap, gather=gather, options=options,
                       eviction=eviction, transfer_group=transfer_group, transfer_mode=transfer_mode,
                       carry_select=carry_select)
    try:
        run.run(log=lambda msg: print(msg, flush=True))
        records = run.records
    finally:
        run.close()
    del run
    results = CC.compare_units(cfg, units, records, eviction=eviction, log=lambda m: print(m, flush=True))
    print(CC.summarize(f"{cfg.name} [{eviction}{', overlap' if overlap else ''}"
                       f"{', host copies' if not gather else ''}"
                       f"{', carried selection' if carry_select else ''}]", results),
          flush=True)
    for key, st in results.items():
        assert st["compared_steps"] == cfg.steps + 1, (key, st)
    return results


def _all_units(cfg, layer=0):
    return [(layer, u) for u in range(cfg.batch * cfg.kv_heads)]


def _layer_plus_samples(cfg, full_layer, per_layer, seed):
    rng = np.random.default_rng(seed)
    units = _all_units(cfg, full_layer)
    for l in range(cfg.layers):
        if l != full_layer:
            units += [(l, int(u)) for u in rng.choice(cfg.batch * cfg.kv_heads, size=per_layer, replace=False)]
    return units


@pytest.mark.parametrize("overlap,gather", [(False, True), (True, True), (False, False)])
def test_chain_tiny_full(overlap, gather):
    _run_and_compare(CONFIGS["tiny"], [(0, 0)], overlap=overlap, gather=gather)


def test_chain_small_bf16_ragged():
    # ragged context (partial newest block), several tiles and splits, cap binding
    cfg = CONFIGS["llama8b_32k"].with_(batch=2, ctx=16 * 300 + 7, steps=6, fetch_cap=8,
                                       planted=15, budget_tokens=16 * 32)
    _run_and_compare(cfg, _all_units(cfg))


@pytest.mark.parametrize("tpw", [2, 3])
def test_chain_ragged_contexts(tpw):
    """A different prompt length per request, with runs of several 16-block
    scoring tiles per wavefront: tile counts of 1 modulo the run below the
    capacity leave some wavefront a single in-context tile."""
    cfg = CONFIGS["llama8b_32k"].with_(batch=5, steps=6, fetch_cap=8, planted=6, budget_tokens=16 * 32,
                                       ctx_list=(16 * 16 * 4 + 5, 16 * 16 * 3 + 1, 16 * 16 * 9 + 16,
                                                 16 * 16 * 6 + 9, 16 * 16 * 12 - 5))
    _run_and_compare(cfg, _all_units(cfg), options=dict(score_tpw=tpw))


@pytest.mark.parametrize("overlap,gather", [(False, True), (True, True), (False, False)])
def test_chain_small_append(overlap, gather):
    cfg = CONFIGS["qwen8b_reason"].with_(batch=2, ctx=16 * 40 + 13, steps=40, recency_blocks=8,
                                         planted=4, budget_tokens=16 * 16, fetch_cap=3)
    _run_and_compare(cfg, _all_units(cfg), overlap=overlap, gather=gather)


def test_chain_small_drift():
    cfg = CONFIGS["qwen32b_32k"].with_(batch=1, layers=2, ctx=16 * 200, steps=5, planted=10,
                                       drift_blocks=4, budget_tokens=16 * 24, fetch_cap=4)
    _run_and_compare(cfg, [(l, u) for l in range(2) for u in range(cfg.kv_heads)])


@pytest.mark.parametrize("overlap,gather,group", [(False, True, 2), (False, True, 3), (True, True, 4),
                                                  (False, False, 4)])
def test_chain_layer_batched_transfers(overlap, gather, group):
    """Several layers' transfers handed to the side stream as one batch behind one
    event (groups of 2, 3 and 4 over 5 layers, the last group short): every
    layer's next attention still sees its fetched pages."""
    cfg = CONFIGS["llama8b_32k"].with_(batch=1, layers=5, ctx=16 * 150 + 3, steps=5, planted=8,
                                       budget_tokens=16 * 16, fetch_cap=4)
    _run_and_compare(cfg, [(l, u) for l in range(5) for u in (0, 3, 6)], overlap=overlap, gather=gather,
                     transfer_group=group)


@pytest.mark.parametrize("layers", [1, 2, 5])
def test_chain_inline_transfers(layers):
    """Each layer's fetched pages carried in the first launch of the next decode
    step on the compute stream (no second stream): over five layers, two, and one
    (where a layer's own pending transfer moves as a gather before its step)."""
    cfg = CONFIGS["llama8b_32k"].with_(batch=1, layers=layers, ctx=16 * 150 + 3, steps=5, planted=8,
                                       budget_tokens=16 * 16, fetch_cap=4)
    _run_and_compare(cfg, [(l, u) for l in range(layers) for u in (0, 3, 6)], transfer_mode="inline")


@pytest.mark.parametrize("layers", [1, 3])
def test_chain_inline_transfers_append(layers):
    """Inline transfers with a token appended per step (a new newest block is
    fetched first and then written by the next append)."""
    cfg = CONFIGS["qwen8b_reason"].with_(batch=2, ctx=16 * 40 + 13, steps=24, recency_blocks=8, planted=4,
                                         budget_tokens=16 * 16, fetch_cap=3)
    _run_and_compare(cfg, [(l, u) for l in range(layers) for u in range(cfg.batch * cfg.kv_heads)],
                     layers=layers, transfer_mode="inline")


@pytest.mark.parametrize("overlap", [False, True])
def test_chain_small_lru(overlap):
    """Least-recently-used eviction over a drifting chain with a binding cap,
    stamps compared at every step.  The drift makes the LRU victims differ
    from the lowest-score ones at most steps (checked on the oracle)."""
    cfg = CONFIGS["qwen32b_32k"].with_(batch=1, layers=2, ctx=16 * 200, steps=8, planted=10, drift_blocks=4,
                                       budget_tokens=16 * 24, fetch_cap=4)
    units = [(l, u) for l in range(2) for u in range(cfg.kv_heads)]
    _run_and_compare(cfg, units, overlap=overlap, eviction="lru")
    differ = 0
    for (l, u) in units[:3]:
        r, h = divmod(u, cfg.kv_heads)
        ud, K_at = CC.unit_inputs(cfg, l, u)
        recs = {ev: O.run_unit(K_at=K_at, V=ud.V, queries=ud.queries, drafts_prologue=ud.drafts[0], n0=cfg.ctx, k=cfg.k,
                               cap=cfg.fetch_cap, steps=cfg.steps,
                               initial_slots=lambda S0: synth.initial_residency(cfg, r, l, h, S0),
                               max_blocks=cfg.max_blocks, with_attention=False, eviction=ev)
                for ev in ("score", "lru")}
        differ += sum(a.evict != b.evict for a, b in zip(recs["score"], recs["lru"]))
    assert differ >= 3, differ


def test_chain_small_lru_append():
    """Least-recently-used eviction over a chain with appends (the newest block
    turns over), stamps compared at every step."""
    cfg = CONFIGS["qwen8b_reason"].with_(batch=2, ctx=16 * 40 + 13, steps=30, recency_blocks=8,
                                         planted=4, budget_tokens=16 * 16, fetch_cap=3)
    _run_and_compare(cfg, _all_units(cfg), eviction="lru")


def _state_snapshot(run):
    rt = run.rt
    snap = [rt.out.cpu().numpy().copy()]
    for l in range(run.L):
        st = rt.state[l][0]
        snap += [x.cpu().numpy().copy() for x in (st.scores, st.sel, st.b2s, st.s2b, st.fetch, st.n_fetch,
                                                   st.evict, st.meta, st.pool)]
        na = st.n_attend.cpu().numpy().copy()
        att = st.attend.cpu().numpy()
        snap += [na, np.stack([np.where(np.arange(att.shape[1]) < n, a, -1) for a, n in zip(att, na)])]
    return snap


@pytest.mark.parametrize("name,kw", [
    ("llama8b_32k", dict(batch=2, ctx=16 * 300 + 7, steps=5, fetch_cap=8, planted=15, budget_tokens=16 * 32)),
    ("llama8b_32k", dict(batch=2, ctx=16 * 40, steps=4, fetch_cap=4, planted=3, budget_tokens=16 * 8)),
    ("qwen8b_reason", dict(batch=2, ctx=16 * 40 + 13, steps=6, recency_blocks=8, planted=4,
                           budget_tokens=16 * 16, fetch_cap=3)),
    ("qwen32b_32k", dict(batch=1, layers=2, ctx=16 * 200, steps=4, planted=10, budget_tokens=16 * 24,
                         fetch_cap=4, drift_blocks=0)),                 # 40 attention rows
    ("llama8b_32k", dict(batch=2, ctx=16 * 40, steps=3, fetch_cap=2, planted=1, budget_tokens=32)),  # 1 split
    ("tiny", dict(steps=4)),                                              # f32
])
def test_decode_step_matches_separate_calls(name, kw):
    """The single decode-step call (attention and scoring in one launch, then
    selection, diff and the split combine) leaves bit-identical outputs and
    state to the separate entry points, step after step."""
    _decode_step_vs_separate(CONFIGS[name].with_(**kw))


@pytest.mark.parametrize("launches,order,waves", [(2, 1, 2), (2, 2, 2), (3, 0, 2), (2, 0, 4), (2, 2, 4)])
def test_decode_step_launch_variants(launches, order, waves):
    """Both workgroup orders of the fused attention + scoring launch other than
    the default, workgroups of 4 wavefronts, and the three-launch step give the
    same bit-identical result as the separate calls."""
    opts = dict(step_launches=launches, step_order=order, attn_waves=waves)
    _decode_step_vs_separate(CONFIGS["llama8b_32k"].with_(batch=2, ctx=16 * 300 + 7, steps=4, fetch_cap=8,
                                                          planted=15, budget_tokens=16 * 32), options=opts)


@pytest.mark.parametrize("launches", [2, 3])
def test_decode_step_halves(launches):
    """The decode step's two halves as separate calls (attention + scoring, then
    selection + diff + split combine) leave bit-identical outputs and state to
    the single decode-step call."""
    opts = dict(step_launches=launches)
    cfg = CONFIGS["llama8b_32k"].with_(batch=2, ctx=16 * 300 + 7, steps=4, fetch_cap=8, planted=15,
                                       budget_tokens=16 * 32)
    _decode_step_vs_separate(cfg, runs=[SyntheticRun(cfg, overlap=False, two_calls=tc, options=opts)
                                        for tc in (True, False)])


def _decode_step_vs_separate(cfg, runs=None, options=None, exact=False):
    runs = runs or [SyntheticRun(cfg, overlap=False, fused_step=f, options=options) for f in (True, False)]
    try:
        for r in runs:
            r.prologue()
        for t in range(cfg.steps):
            snaps = []
            for r in runs:
                r.step(t)
                snaps.append(_state_snapshot(r))
            for i, (a, b) in enumerate(zip(*snaps)):
                if i == 0 and not exact:
                    # the attention output: the standalone attention may split the
                    # attended list differently (its own split count), which only
                    # reorders fp32 sums; every discrete output must be identical
                    assert np.allclose(a, b, rtol=1e-5, atol=1e-6), (t, float(np.abs(a - b).max()))
                else:
                    assert np.array_equal(a, b, equal_nan=True), (t, i)
            print(f"{cfg.name} step {t}: identical", flush=True)
    finally:
        for r in runs:
            r.close()


CARRY_SHAPES = [
    # (config, overrides): three layers, a ragged context of 301 blocks (keys per
    # selecting thread 4), cap binding
    ("llama8b_32k", dict(batch=2, layers=3, ctx=16 * 300 + 7, steps=5, fetch_cap=8, planted=15,
                         budget_tokens=16 * 32)),
    # two layers of one request with 2048 blocks, the full budget (128 blocks) and cap (16 keys per thread)
    ("llama8b_32k", dict(batch=1, layers=2, steps=4)),
    # 8192 blocks over two KV heads (64 keys per thread)
    ("llama8b_128k", dict(batch=1, kv_heads=2, layers=2, steps=3)),
    # a prompt length per request
    ("llama8b_32k", dict(batch=5, layers=2, steps=4, fetch_cap=8, planted=6, budget_tokens=16 * 32,
                         ctx_list=(16 * 16 * 4 + 5, 16 * 16 * 3 + 1, 16 * 16 * 9 + 16, 16 * 16 * 6 + 9,
                                   16 * 16 * 12 - 5))),
    # appends (the newest block turns over) with two layers
    ("qwen8b_reason", dict(batch=2, layers=2, ctx=16 * 40 + 13, steps=20, recency_blocks=8, planted=4,
                           budget_tokens=16 * 16, fetch_cap=3)),
    # 40 attention rows and 32 scoring rows, three layers
    ("qwen32b_32k", dict(batch=1, layers=3, ctx=16 * 200, steps=4, planted=10, budget_tokens=16 * 24,
                         fetch_cap=4, drift_blocks=0)),
    # k = 2 (no candidates to rank, one attention split), cap = k, no cap, one layer
    ("llama8b_32k", dict(batch=2, layers=2, ctx=16 * 40, steps=3, fetch_cap=2, planted=1, budget_tokens=32)),
    ("llama8b_32k", dict(batch=2, layers=2, ctx=16 * 90 + 1, steps=4, fetch_cap=16, planted=6,
                         budget_tokens=16 * 16)),
    ("llama8b_32k", dict(batch=2, layers=2, ctx=16 * 90 + 1, steps=3, fetch_cap=0, planted=6,
                         budget_tokens=16 * 16)),
    ("llama8b_32k", dict(batch=2, layers=1, ctx=16 * 300 + 7, steps=4, fetch_cap=8, planted=15,
                         budget_tokens=16 * 32)),
]


@pytest.mark.parametrize("name,kw", CARRY_SHAPES)
def test_carry_step_matches_decode_step(name, kw):
    """Each layer's selection and diff carried by the next layer's first launch
    (the last layer's run on its own at the end of each step) leave
    bit-identical outputs and state, attended list included, to the decode step
    that selects in its own second launch, step after step."""
    cfg = CONFIGS[name].with_(**kw)
    print(f"{name} {kw}", flush=True)
    _decode_step_vs_separate(cfg, runs=[SyntheticRun(cfg, overlap=False, carry_select=c) for c in (True, False)])


@pytest.mark.parametrize("name,kw", [CARRY_SHAPES[0], CARRY_SHAPES[4], CARRY_SHAPES[5]])
def test_carry_step_matches_separate_calls(name, kw):
    """The carried step against the separate entry points (attention, score,
    selection and diff each on their own): every selection, list and map bit
    for bit, the attention output up to the split order of its fp32 sums."""
    cfg = CONFIGS[name].with_(**kw)
    _decode_step_vs_separate(cfg, runs=[SyntheticRun(cfg, overlap=False, carry_select=True),
                                        SyntheticRun(cfg, overlap=False, fused_step=False)])


@pytest.mark.parametrize("shape,splits,carry,waves,d", [
    (0, 4, False, 2, 128),   # three layers, 16 units, the two-launch step
    (0, 4, False, 4, 128),   # 4-wavefront attention workgroups (each merges 2 of the 8 channel tiles)
    (0, 3, False, 2, 64),    # head dim 64 (4 channel tiles; the two-launch step)
    (0, 8, True, 2, 128),    # the carried selection, the largest split count merged in launch
    (0, 3, True, 2, 128),    # a split count that is no power of two
    (5, 2, False, 2, 128),   # 40 attention rows (three row tiles)
    (5, 3, True, 2, 128),
    (4, 3, True, 2, 128),    # appends over 20 steps
    (2, 8, True, 2, 128),    # 8192 blocks per head
])
def test_split_merge_in_launch_matches_the_combine(shape, splits, carry, waves, d):
    """The attention's splits merged inside the fused first launch (the last
    workgroup of each unit to finish merges, attn_merge = 2) against the same
    split count merged by the combine (attn_merge = 1): every output, the
    attention's included, and all state bit for bit, step after step (the
    arrival counters return to zero after every launch, or a later step would
    merge early, late or never)."""
    from lookahead_sparse_kv_draft_amd import _lib as L
    name, kw = CARRY_SHAPES[shape]
    cfg = CONFIGS[name].with_(**dict(kw, head_dim=d))
    print(f"{name} {kw} d {d} splits {splits} carry {carry} waves {waves}", flush=True)
    runs = [SyntheticRun(cfg, overlap=False, carry_select=carry,
                         options=dict(attn_splits=splits, attn_merge=m, attn_waves=waves)) for m in (2, 1)]
    got = [L.oasis_get_launch_options(r.rt.h) for r in runs]
    assert got[0]["attn_splits"] == splits and got[0]["attn_merge"] == 2, got[0]
    assert got[0]["attn_waves"] == waves, got[0]
    assert got[1]["attn_merge"] == 1, got[1]
    _decode_step_vs_separate(cfg, runs=runs, exact=True)


def test_split_merge_in_launch_under_graph_replay():
    """The fused first launch with its splits merged inside it, captured as a
    HIP graph and replayed three times, with eager calls on the same workspace
    between the replays: every replay and every eager call gives the eager
    output and scores bit for bit (each launch leaves the arrival counters
    zero for the next, captured or not)."""
    from lookahead_sparse_kv_draft_amd import _lib as L
    name, kw = CARRY_SHAPES[0]
    cfg = CONFIGS[name].with_(**dict(kw, layers=1))
    run = SyntheticRun(cfg, overlap=False, options=dict(attn_splits=4, attn_merge=2))
    try:
        run.prologue()
        rt = run.rt
        st = rt.state[0][0]
        assert L.oasis_get_launch_options(rt.h)["attn_merge"] == 2

        def call(out, scores, stream):
            L.oasis_attend_and_score(rt.h, run.q[0, 1], st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.sel, st.b2s,
                                     st.attend, st.n_attend, scores, out, rt.ws_ptr, stream)

        out_e, sc_e = torch.zeros_like(rt.out), torch.zeros_like(st.scores)
        call(out_e, sc_e, torch.cuda.current_stream())
        torch.cuda.synchronize()
        out_g, sc_g = torch.zeros_like(rt.out), torch.zeros_like(st.scores)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(out_g, sc_g, torch.cuda.current_stream())
        torch.cuda.synchronize()
        for r in range(3):
            out_g.zero_()
            sc_g.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_g, out_e) and torch.equal(sc_g, sc_e), r
            out_x, sc_x = torch.zeros_like(rt.out), torch.zeros_like(st.scores)
            call(out_x, sc_x, torch.cuda.current_stream())
            torch.cuda.synchronize()
            assert torch.equal(out_x, out_e) and torch.equal(sc_x, sc_e), r
        # and the same output as the combine after the launch
        h1 = run.shape.handle(options=dict(attn_splits=4, attn_merge=1))
        try:
            out_c = torch.zeros_like(rt.out)
            L.oasis_attend_and_score(h1, run.q[0, 1], st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.sel, st.b2s,
                                     st.attend, st.n_attend, torch.zeros_like(st.scores), out_c, rt.ws_ptr)
            L.oasis_attn_combine(h1, rt.ws_ptr, out_c)
            torch.cuda.synchronize()
            assert torch.equal(out_c, out_e)
        finally:
            L.oasis_destroy(h1)
    finally:
        run.close()


@pytest.mark.parametrize("dtype,options,full", [
    ("bf16", {"attn_splits": 1}, False),   # attention and scoring launches carry the metadata and page rows
    ("bf16", {"attn_splits": 1}, True),    # the same, request 0 reaching the capacity
    ("bf16", {"step_launches": 3}, False),  # three launches (with a split combine: the append launch first)
    ("bf16", None, False),                 # attention beside the scoring: the append launch goes first
    ("f32", None, True),                   # fp32: the append launch goes first
])
def test_decode_step_append_matches_separate_calls(dtype, options, full):
    """oasis_decode_step_append against oasis_block_meta_update followed by
    oasis_decode_step on an identical copy of the state, over steps that cross
    a block boundary: every output, the grown context, the metadata, the pool
    and every list and map bit for bit.  With `full`, request 0 starts two
    tokens below the capacity and stays at it once there: its later appends
    leave the context as it was."""
    from lookahead_sparse_kv_draft_amd import _lib as L
    cfg = CONFIGS["qwen8b_reason"].with_(batch=2, ctx=16 * 40 + 13, steps=5, dtype=dtype, budget_tokens=16 * 16,
                                         fetch_cap=4, planted=6)
    print(f"{dtype} {options} {full}", flush=True)
    run = SyntheticRun(cfg, replicas=2, overlap=False, options=options)
    try:
        run.prologue()
        rt = run.rt
        a, b = rt.state[0][0], rt.state[0][1]
        b.copy_from(a)
        torch.cuda.synchronize()
        cap = run.shape.max_blocks * 16
        base = torch.tensor([cfg.ctx_of(r) for r in range(cfg.batch)], dtype=torch.int32, device="cuda")
        if full:
            base[0] = cap - 2
        out_a, out_b = torch.zeros_like(rt.out), torch.zeros_like(rt.out)
        for t in range(cfg.steps):
            ctx_in = torch.clamp(base + t, max=cap)
            grown_a, grown_b = torch.zeros_like(ctx_in), torch.zeros_like(ctx_in)
            q, kn, vn = run.q[0, t + 1], run.k_new_dev[0, t], run.v_new_dev[0, t]
            L.oasis_block_meta_update(rt.h, kn, vn, ctx_in, grown_a, a.meta, a.pool, a.b2s)
            L.oasis_decode_step(rt.h, q, a.pool, a.meta, ctx_in, grown_a, a.sel, a.b2s, a.s2b, a.scores, out_a,
                                rt.ws_ptr, a.fetch, a.n_fetch, a.evict, a.attend, a.n_attend)
            L.oasis_decode_step_append(rt.h, q, b.pool, b.meta, ctx_in, grown_b, b.sel, b.b2s, b.s2b, b.scores,
                                       out_b, rt.ws_ptr, b.fetch, b.n_fetch, b.evict, b.attend, b.n_attend, kn, vn)
            torch.cuda.synchronize()
            assert torch.equal(out_a, out_b), t
            assert torch.equal(grown_a, grown_b), t
            assert torch.equal(grown_a, torch.where(ctx_in < cap, ctx_in + 1, ctx_in)), t
            for name in ("meta", "pool", "b2s", "s2b", "scores", "sel", "fetch", "n_fetch", "evict", "attend",
                         "n_attend"):
                assert torch.equal(getattr(a, name), getattr(b, name)), (t, name)
    finally:
        run.close()


def _outputs_without_step_syncs(cfg, **kw):
    """All steps enqueued back to back (carried selections and inline transfers
    cross step boundaries); every layer's output copied on the stream; the
    final state after one flush."""
    run = SyntheticRun(cfg, overlap=False, **kw)
    try:
        run.prologue()
        torch.cuda.synchronize()
        rt = run.rt
        outs = torch.empty((cfg.steps, run.L) + tuple(rt.out.shape), dtype=rt.out.dtype, device="cuda")
        for t in range(cfg.steps):
            for l in range(run.L):
                q = run.q[l, t + 1]
                if cfg.append:
                    rt.append(l, run.k_new_dev[l, t], run.v_new_dev[l, t], run.k_new_host[l, t],
                              run.v_new_host[l, t])
                rt.decode_step(l, q, stamp=t + 1)
                outs[t, l].copy_(rt.out)
                run._transfer_after(l)
            rt.end_step()
        rt.wait_transfers()
        torch.cuda.synchronize()
        return outs.cpu().numpy(), _state_snapshot(run)[1:]
    finally:
        run.close()


@pytest.mark.parametrize("layers,mode", [(3, "side"), (3, "inline"), (5, "inline"), (2, "inline"), (1, "side")])
def test_carry_across_steps(layers, mode):
    """Carried selections and transfers pending across step boundaries (the last
    layer's selection rides in the next step's first layer): every output and
    the final state bit-identical to the decode step that selects itself."""
    cfg = CONFIGS["llama8b_32k"].with_(batch=1, layers=layers, ctx=16 * 150 + 3, steps=6, planted=8,
                                       budget_tokens=16 * 16, fetch_cap=4)
    ref_out, ref_state = _outputs_without_step_syncs(cfg, transfer_mode=mode)
    out, state = _outputs_without_step_syncs(cfg, transfer_mode=mode, carry_select=True)
    for t in range(cfg.steps):
        for l in range(layers):
            assert np.array_equal(out[t, l], ref_out[t, l]), (t, l)
    for i, (a, b) in enumerate(zip(state, ref_state)):
        assert np.array_equal(a, b), i


@pytest.mark.parametrize("layers,mode", [(3, "side"), (3, "inline")])
def test_chain_carry_small(layers, mode):
    """Carried selections against the oracle over a chain, every unit of every layer."""
    cfg = CONFIGS["llama8b_32k"].with_(batch=2, layers=layers, ctx=16 * 300 + 7, steps=6, fetch_cap=8,
                                       planted=15, budget_tokens=16 * 32)
    _run_and_compare(cfg, [(l, u) for l in range(layers) for u in range(cfg.batch * cfg.kv_heads)],
                     transfer_mode=mode, carry_select=True)


@pytest.mark.timeout(1100)
def test_chain_llama8b_128k_full_layer_carry():
    """The 128K workload with every layer's selection carried by the next
    layer's first launch: every unit of layer 2, two sampled units of the rest."""
    cfg = CONFIGS["llama8b_128k"]
    _run_and_compare(cfg, _layer_plus_samples(cfg, 2, 2, seed=129), carry_select=True)


@pytest.mark.timeout(1100)
def test_chain_qwen32b_32k_full_layer_carry():
    """The Qwen3-32B-shaped workload (without the drift, which rebuilds metadata
    mid-step) with carried selections: every unit of layer 6, two sampled units
    of the rest."""
    cfg = CONFIGS["qwen32b_32k"].with_(drift_blocks=0)
    _run_and_compare(cfg, _layer_plus_samples(cfg, 6, 2, seed=33), carry_select=True)


@pytest.mark.timeout(1100)
def test_chain_llama8b_32k_full_size():
    """The benchmark's workload: every unit over all 32 steps."""
    cfg = CONFIGS["llama8b_32k"]
    _run_and_compare(cfg, _all_units(cfg))


@pytest.mark.timeout(1100)
def test_chain_llama8b_32k_full_size_lru():
    """The benchmark's workload with least-recently-used eviction ([EXPL] Table 2's
    policy): every unit over all 32 steps."""
    cfg = CONFIGS["llama8b_32k"]
    _run_and_compare(cfg, _all_units(cfg), eviction="lru")


@pytest.mark.timeout(1100)
def test_chain_llama8b_32k_full_size_host_copies():
    """The benchmark's workload with the host-issued per-page copies on the side
    stream (hipMemcpyAsync) instead of the device gather: sampled units, all
    32 steps."""
    cfg = CONFIGS["llama8b_32k"]
    _run_and_compare(cfg, [(0, u) for u in (0, 5, 13, 22, 35, 41, 50, 63)], gather=False)


@pytest.mark.timeout(1100)
def test_chain_qwen32b_32k_full_layer():
    # 8 layers, 64 query / 8 KV heads (40 attention rows, 32 scoring rows), drifting
    # set: every unit of layer 3 and two sampled units of each other layer
    cfg = CONFIGS["qwen32b_32k"]
    _run_and_compare(cfg, _layer_plus_samples(cfg, 3, 2, seed=32))


@pytest.mark.timeout(1100)
def test_chain_qwen8b_reason_full_size():
    # 64 requests, 256 appended tokens (the newest block turns over 16 times): every unit
    cfg = CONFIGS["qwen8b_reason"]
    _run_and_compare(cfg, _all_units(cfg))


@pytest.mark.timeout(1100)
def test_chain_llama8b_128k_full_layer():
    # 8192 blocks per head, 8 layers, 16 GiB host tier: every unit of layer 5 and
    # two sampled units of each other layer
    cfg = CONFIGS["llama8b_128k"]
    _run_and_compare(cfg, _layer_plus_samples(cfg, 5, 2, seed=128))


def test_corrective_fetch_makes_exact_set_resident():
    """After a few capped prefetch steps, the corrective path selects the verify
    query's own top-k (bit for bit the oracle's selection on the same scores),
    fetches every block of it the prefetch missed, and leaves the attended list
    equal to that set with the host tier's pages in its slots."""
    cfg = CONFIGS["llama8b_32k"].with_(batch=2, ctx=16 * 300 + 7, steps=4, fetch_cap=2, planted=15,
                                       budget_tokens=16 * 32)
    run = SyntheticRun(cfg, overlap=False)
    try:
        run.prologue()
        for t in range(2):
            run.step(t)
        rt = run.rt
        st = rt.state[0][0]
        q = run.q[0, 3]
        rt.corrective(0, q)
        torch.cuda.synchronize()
        H = cfg.kv_heads
        vs, vsel = st.vscores.cpu().numpy(), st.vsel.cpu().numpy()
        b2s, att, natt = st.b2s.cpu().numpy(), st.attend.cpu().numpy(), st.n_attend.cpu().numpy()
        ncf = st.cn_fetch.cpu().numpy()
        pool = rt.pool_pages(0).cpu().numpy()
        tier = rt.host_tier_view(0).numpy().reshape(rt.shape.units, rt.shape.max_blocks, -1)
        assert ncf.sum() > 0, "the capped prefetch left nothing for the corrective fetch to do"
        for u in range(rt.shape.units):
            N = (int(rt.ctx_host[u // H]) + 15) // 16
            ref = O.topk_select(vs[u].astype(np.float64), N, rt.shape.budget_blocks)
            assert list(vsel[u]) == ref, u
            S = [b for b in ref if b >= 0]
            assert all(b2s[u, b] >= 0 for b in S), u
            assert natt[u] == len(S) and [e >> 10 for e in att[u, :natt[u]]] == S, u
            for e in att[u, :natt[u]]:
                b, s = e >> 10, e & 1023
                assert s == b2s[u, b] and np.array_equal(pool[u, s], tier[u, b]), (u, b)
    finally:
        run.close()
