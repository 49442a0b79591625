"""Delayed transfers: each side-stream transfer is held back on the GPU (gated
behind a bounded spin kernel on a third stream), while the host enqueues the
following layers and steps without any synchronisation.  The transfer must
still land before that layer's next attention and must not overwrite a victim
slot while an attention reads it (the explainer's Figure 8 ordering: the
transfer precedes that layer's attention at step t+1).  Every output and the
final state must be bit-identical to a run that synchronises after every
transfer.  Every kernel exits normally: the delay is a fixed-length spin."""
import numpy as np
import pytest
import torch

from lookahead_sparse_kv_draft_amd.synthetic import SyntheticRun
from workload import CONFIGS

pytestmark = pytest.mark.gpu

DELAY_CYCLES = 400_000  # a few hundred microseconds of spinning per transfer batch


def _chain(cfg, overlap, group, delayed):
    run = SyntheticRun(cfg, overlap=overlap, transfer_group=group)
    rt = run.rt
    try:
        run.prologue()
        torch.cuda.synchronize()
        L, steps = run.L, cfg.steps
        outs = torch.empty((steps, L) + tuple(rt.out.shape), dtype=rt.out.dtype, device="cuda")
        gate = torch.cuda.Stream()
        plain = rt.transfer_group
        fetched = [0]

        def transfer_group(layers, replica=0, stream=None):
            if delayed:
                src = rt._pred() if stream is None else stream
                gate.wait_stream(src)  # the spin starts once the diffs are done
                with torch.cuda.stream(gate):
                    torch.cuda._sleep(DELAY_CYCLES)
                ev = torch.cuda.Event()
                ev.record(gate)
                rt.side.wait_event(ev)
            plain(layers, replica, stream)
            if not delayed:
                torch.cuda.synchronize()
                fetched[0] += sum(int(rt.state[l][replica].n_fetch.sum()) for l in layers)

        rt.transfer_group = transfer_group
        cs = torch.cuda.current_stream()
        for t in range(steps):
            for l in range(L):
                q = run.q[l, t + 1]
                if overlap:
                    rt.attention(l, q)
                    outs[t, l].copy_(rt.out)
                    rt.predict_select(l, q, stamp=t + 1)
                else:
                    rt.decode_step(l, q, stamp=t + 1)
                    outs[t, l].copy_(rt.out)
                run._transfer_after(l)
        rt.wait_transfers()
        cs.synchronize()
        torch.cuda.synchronize()
        state = []
        for l in range(L):
            st = rt.state[l][0]
            state += [x.cpu().numpy().copy() for x in (st.sel, st.b2s, st.s2b, st.fetch, st.n_fetch, st.evict,
                                                       st.attend, st.n_attend, st.pool)]
        return outs.cpu().numpy(), state, fetched[0]
    finally:
        run.close()


@pytest.mark.parametrize("overlap,group", [(False, 1), (False, 2), (True, 1)])
def test_delayed_transfers_match_synchronous(overlap, group):
    cfg = CONFIGS["llama8b_32k"].with_(batch=1, layers=3, ctx=16 * 150 + 3, steps=6, planted=8,
                                       budget_tokens=16 * 16, fetch_cap=4)
    ref_out, ref_state, n_fetched = _chain(cfg, overlap, group, delayed=False)
    out, state, _ = _chain(cfg, overlap, group, delayed=True)
    for t in range(cfg.steps):
        for l in range(cfg.layers):
            assert np.array_equal(out[t, l], ref_out[t, l]), (t, l)
    for i, (a, b) in enumerate(zip(state, ref_state)):
        assert np.array_equal(a, b), i
    # pages were fetched over the run (the delayed transfers carried work)
    assert n_fetched > 0
