"""Per-layer decode-step runtime over liboasiskv.

Holds the device and pinned-host buffers of each layer (torch is used only to
allocate memory, to provide streams and events, and for plain copies) and
enqueues the per-step chain of the OasisKV explainer's Figure 8: the draft
queries of step t drive prediction, selection and transfer, which land in HBM
before that layer's attention at step t+1.

Per layer and step (compute stream unless noted):
    wait for the layer's previous transfer
    sparse_paged_decode_attn     verify + draft queries over S_t and R_t
    [block_meta_update]          long-output decode: append the step's token
    lookahead_score              drafts of step t against the block metadata
    topk_select                  S_{t+1}
    resident_diff_cap_evict      fetch / evict lists, maps -> R_{t+1}
    fetch list -> host, fetch_issue on the side stream (transfer mode only)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L

BLOCK = 16


@dataclass(frozen=True)
class Shape:
    batch: int
    kv_heads: int
    group: int
    head_dim: int
    max_blocks: int
    budget_blocks: int
    n_draft: int
    fetch_cap: int
    dtype: str  # "bf16" | "f32"

    @property
    def units(self) -> int:
        return self.batch * self.kv_heads

    @property
    def T(self) -> int:
        return 1 + self.n_draft

    @property
    def q_heads(self) -> int:
        return self.kv_heads * self.group

    @property
    def code(self) -> int:
        return L.OASIS_BF16 if self.dtype == "bf16" else L.OASIS_F32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def np_elem(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    def handle(self, fetch_cap: int | None = None, options: dict | None = None) -> int:
        """A library handle of this shape (options: launch options, see
        oasis_launch_options; None = the library's defaults)."""
        return L.oasis_create_with_options(self.batch, self.kv_heads, self.group, self.head_dim, self.max_blocks,
                                           self.budget_blocks, self.n_draft,
                                           self.fetch_cap if fetch_cap is None else fetch_cap, self.code,
                                           options=options)


def untile_meta(meta: torch.Tensor, units: int, max_blocks: int, d: int, dtype: str) -> torch.Tensor:
    """[units][max_blocks][2][d] elements (int16 bit patterns for bf16, float32
    otherwise) of a metadata buffer in the library's chunk-major 16-block tiles."""
    el = meta.view(torch.int16 if dtype == "bf16" else torch.float32)
    ce = 16 // el.element_size()
    tiles = (max_blocks + 15) // 16
    t = el.view(units, tiles, 2 * d // ce, 16, ce).permute(0, 1, 3, 2, 4)
    return t.reshape(units, tiles * 16, 2, d)[:, :max_blocks].contiguous()


def tile_meta(meta: np.ndarray) -> np.ndarray:
    """Host-side packing of logical metadata [units][max_blocks][2][d] (bf16 bit
    patterns as uint16/int16, or float32) into the library's chunk-major tiles of
    16 blocks; flat, zero-padded to whole tiles (the inverse of untile_meta)."""
    units, nmax, two, d = meta.shape
    assert two == 2
    ce = 16 // meta.dtype.itemsize
    tiles = (nmax + 15) // 16
    pad = np.zeros((units, tiles * 16, 2 * d), dtype=meta.dtype)
    pad[:, :nmax] = meta.reshape(units, nmax, 2 * d)
    t = pad.reshape(units, tiles, 16, 2 * d // ce, ce).transpose(0, 1, 3, 2, 4)
    return np.ascontiguousarray(t).reshape(-1)


class PendingTransfer:
    """One batch of page transfers on the side stream (the gathers or copies of
    one or more layers): its completion event and the streams that have already
    waited for it, so that each stream waits once per batch however many of the
    batch's layers it then touches."""

    def __init__(self, event):
        self.event = event
        self.waited = set()

    def wait(self, stream):
        key = stream.cuda_stream
        if key not in self.waited:
            stream.wait_event(self.event)
            self.waited.add(key)


class LayerState:
    """Device state of one layer (one replica) plus its pinned host tier."""

    def __init__(self, rt: "DecodeRuntime", host_tier: torch.Tensor | None):
        s, dev = rt.shape, rt.device
        h = rt.h
        u, k, N, cap = s.units, s.budget_blocks, s.max_blocks, s.fetch_cap
        self.meta = torch.zeros(L.oasis_meta_bytes(h), dtype=torch.uint8, device=dev)
        self.pool = torch.zeros(L.oasis_pool_bytes(h), dtype=torch.uint8, device=dev)
        self.b2s = torch.full((u, N), -1, dtype=torch.int32, device=dev)
        self.s2b = torch.full((u, k), -1, dtype=torch.int32, device=dev)
        self.scores = torch.zeros((u, N), dtype=torch.float32, device=dev)
        self.sel = torch.full((u, k), -1, dtype=torch.int32, device=dev)
        self.fetch = torch.full((u, max(cap, 1), 2), -1, dtype=torch.int32, device=dev)
        self.n_fetch = torch.zeros(u, dtype=torch.int32, device=dev)
        self.evict = torch.full((u, max(cap, 1)), -1, dtype=torch.int32, device=dev)
        # attended list for the next attention (written by every diff)
        self.attend = torch.full((u, k), -1, dtype=torch.int32, device=dev)
        self.n_attend = torch.zeros(u, dtype=torch.int32, device=dev)
        # least-recently-used eviction: per-slot stamp of the last attention that read it
        self.last_use = (torch.full((u, k), -1, dtype=torch.int32, device=dev) if rt.eviction == "lru"
                         else None)
        self.vscores = None  # corrective path buffers (allocated on first use)
        self.host_tier = host_tier
        self.fetch_host = torch.empty((u, max(cap, 1), 2), dtype=torch.int32, pin_memory=True)
        self.n_fetch_host = torch.empty(u, dtype=torch.int32, pin_memory=True)
        # the last transfer into this layer's pool (a PendingTransfer): the next
        # attention and the next token append wait for it; events: attention done
        # reading the maps (compute stream), selection/diff done (predict stream)
        self.pending = None
        self.attn_done = torch.cuda.Event()
        self.select_done = torch.cuda.Event()
        self.select_pending = False

    def ensure_corrective(self, rt: "DecodeRuntime"):
        """Buffers of the corrective path: the verify query's scores and selection,
        and an uncapped fetch / evict list."""
        if self.vscores is not None:
            return
        s, dev = rt.shape, rt.device
        u, k, N = s.units, s.budget_blocks, s.max_blocks
        self.vscores = torch.zeros((u, N), dtype=torch.float32, device=dev)
        self.vsel = torch.full((u, k), -1, dtype=torch.int32, device=dev)
        self.cfetch = torch.full((u, k, 2), -1, dtype=torch.int32, device=dev)
        self.cn_fetch = torch.zeros(u, dtype=torch.int32, device=dev)
        self.cevict = torch.full((u, k), -1, dtype=torch.int32, device=dev)

    def copy_from(self, other: "LayerState"):
        for name in ("meta", "pool", "b2s", "s2b", "scores", "sel", "fetch", "n_fetch", "evict", "attend",
                     "n_attend"):
            getattr(self, name).copy_(getattr(other, name))
        if self.last_use is not None:
            self.last_use.copy_(other.last_use)


class DecodeRuntime:
    """Buffers and step chain for `layers` layers of one shape on one GPU."""

    def __init__(self, shape: Shape, layers: int = 1, device: str = "cuda", replicas: int = 1,
                 host_tier: bool = True, fused_select: bool = True, overlap: bool = False,
                 gather: bool = True, options: dict | None = None, eviction: str = "score",
                 transfer_mode: str = "side", carry_select: bool = False):
        """overlap: run scoring / selection on a second stream so that they overlap
        the attention of the same step (and of other layers); the selection waits
        only for the attention that reads the maps it rewrites.  options: launch
        options of the library handle (None = defaults).  eviction: "score"
        (lowest-score victims) or "lru" (least recently read slot first; the diff
        that prepares attention t stamps that attention's slots with t).
        transfer_mode: "side" (each layer's transfer on the side stream,
        transfer_group) or "inline" (a layer's fetched pages ride in the first
        launch of the next decode step enqueued on the compute stream,
        oasis_decode_step_gather: no second stream, no event; defer_transfer).
        carry_select: decode_step leaves the layer's selection and diff pending
        and runs them as leading workgroups of the next decode step's first
        launch (another layer's, or the next step's first layer's;
        oasis_decode_step_carry: the second launch is the split combine alone),
        then hands that layer's transfer on; score eviction."""
        if eviction not in ("score", "lru"):
            raise ValueError(eviction)
        if transfer_mode not in ("side", "inline"):
            raise ValueError(transfer_mode)
        if transfer_mode == "inline" and (overlap or not gather):
            raise ValueError("inline transfers run on the compute stream with the device gather")
        if carry_select and (eviction != "score" or overlap):
            raise ValueError("a carried selection evicts by score, on the compute stream")
        self.carry_select = carry_select
        self.pending_select = None  # (layer, replica, ctx tensor) whose selection and diff have not run
        self.transfer_mode = transfer_mode
        self.inline_pending = None  # (layer, replica) whose fetched pages await their transfer
        self.shape = shape
        self.options = options
        self.eviction = eviction
        self.fused_select = fused_select
        self.overlap = overlap
        self.gather = gather
        self.device = torch.device(device)
        self.h = shape.handle(options=options)
        self._h_full = None
        s = shape
        self.n_layers = layers
        self.replicas = replicas
        tiers = []
        for _ in range(layers):
            # zero-filled: pages of blocks that appends create later are fetched
            # with their not-yet-written rows, which then hold defined values
            tiers.append(torch.zeros(L.oasis_host_tier_bytes(self.h), dtype=torch.uint8, pin_memory=True)
                         if host_tier else None)
        # state[layer][replica]; replicas share the layer's host tier
        self.state = [[LayerState(self, tiers[l]) for _ in range(replicas)] for l in range(layers)]
        self.ctx = [torch.zeros(s.batch, dtype=torch.int32, device=self.device) for _ in range(2)]
        self.ctx_cur = 0
        self.ctx_host = np.zeros(s.batch, dtype=np.int32)
        self.out = torch.zeros((s.batch, s.q_heads, s.T, s.head_dim), dtype=torch.float32, device=self.device)
        ws = L.oasis_workspace_bytes(self.h)
        # zeroed: the tail holds the in-launch split merge's arrival counters
        self.ws = torch.zeros(ws + 256, dtype=torch.uint8, device=self.device)
        off = (-self.ws.data_ptr()) % 256
        self.ws_ptr = self.ws.data_ptr() + off
        self.side = torch.cuda.Stream(device=self.device)
        self.pstream = torch.cuda.Stream(device=self.device) if overlap else None

    def close(self):
        if self.h:
            L.oasis_destroy(self.h)
            self.h = 0
        if self._h_full:
            L.oasis_destroy(self._h_full)
            self._h_full = None

    # ------------------------------------------------------------ setup (untimed)
    @property
    def ctx_len(self) -> torch.Tensor:
        return self.ctx[self.ctx_cur]

    def set_ctx(self, ctx_host):
        self.ctx_host = np.asarray(ctx_host, dtype=np.int32).copy()
        self.ctx[self.ctx_cur].copy_(torch.from_numpy(self.ctx_host))

    def host_tier_view(self, layer: int) -> torch.Tensor:
        return self.state[layer][0].host_tier

    def pack_unit(self, layer: int, unit: int, k_rows: np.ndarray, v_rows: np.ndarray | None,
                  blocks: np.ndarray | None = None):
        """Write blocks of one unit into the layer's host tier.

        k_rows/v_rows: element-typed arrays [n_blocks * 16][d] (uint16 bf16 bits or float32);
        blocks: destination block ids (default 0 .. n_blocks-1).
        """
        s = self.shape
        k_rows = np.ascontiguousarray(k_rows, dtype=s.np_elem)
        nb = k_rows.shape[0] // BLOCK
        assert k_rows.shape == (nb * BLOCK, s.head_dim)
        if v_rows is not None:
            v_rows = np.ascontiguousarray(v_rows, dtype=s.np_elem)
            assert v_rows.shape == k_rows.shape
        bl = None if blocks is None else np.ascontiguousarray(blocks, dtype=np.int32)
        L.oasis_pack_pages(self.h, k_rows, v_rows, bl, nb, unit, self.host_tier_view(layer))

    def build_meta(self, layer: int, stream=None):
        """Stage the layer's whole host tier to the device and build its block metadata."""
        tier = self.host_tier_view(layer)
        staged = tier.to(self.device, non_blocking=False)
        for st in self.state[layer]:
            L.oasis_block_meta_build(self.h, staged, None, self.shape.units * self.shape.max_blocks,
                                     self.ctx_len, st.meta, None, None, stream)
        torch.cuda.current_stream().synchronize()
        del staged

    def rebuild_blocks(self, layer: int, page_ids: np.ndarray):
        """After host-tier pages changed: restage them, rebuild their metadata and patch
        the resident copies (page_ids = unit * max_blocks + block)."""
        s = self.shape
        ids = np.ascontiguousarray(page_ids, dtype=np.int64)
        if len(ids) == 0:
            return
        pb = L.oasis_page_bytes(self.h)
        tier = self.host_tier_view(layer).view(-1, pb)
        torch.cuda.synchronize()  # after this layer's attention and every earlier selection
        staged = tier[torch.from_numpy(ids)].to(self.device)
        ids_dev = torch.from_numpy(ids.astype(np.int32)).to(self.device)
        for st in self.state[layer]:
            L.oasis_block_meta_build(self.h, staged, ids_dev, len(ids), self.ctx_len, st.meta, st.pool,
                                     st.b2s)
        torch.cuda.synchronize()

    def prologue(self, layer: int, q: torch.Tensor, initial_slots):
        """Score the step -1 drafts, select S_0, install the initial residency
        (initial_slots(unit, sel_row) -> slot_to_block row), then one diff + transfer."""
        s = self.shape
        for st in self.state[layer]:
            L.oasis_lookahead_score(self.h, q, st.meta, self.ctx_len, st.scores)
            L.oasis_topk_select(self.h, st.scores, self.ctx_len, st.sel)
        st0 = self.state[layer][0]
        sel = st0.sel.cpu().numpy()
        s2b = np.stack([np.asarray(initial_slots(u, sel[u]), dtype=np.int32) for u in range(s.units)])
        b2s = np.full((s.units, s.max_blocks), -1, dtype=np.int32)
        for u in range(s.units):
            for slot, b in enumerate(s2b[u]):
                if b >= 0:
                    b2s[u, b] = slot
        # initial pages through the transfer path (a handle whose cap covers every slot)
        h_all = s.handle(fetch_cap=s.budget_blocks)
        try:
            lst = np.full((s.units, s.budget_blocks, 2), -1, dtype=np.int32)
            cnt = np.zeros(s.units, dtype=np.int32)
            for u in range(s.units):
                rows = [(int(b), slot) for slot, b in enumerate(s2b[u]) if b >= 0]
                cnt[u] = len(rows)
                if rows:
                    lst[u, : len(rows)] = rows
            for st in self.state[layer]:
                st.s2b.copy_(torch.from_numpy(s2b))
                st.b2s.copy_(torch.from_numpy(b2s))
                torch.cuda.current_stream().synchronize()
                L.oasis_fetch_issue(h_all, st.host_tier, st.pool, lst, cnt, torch.cuda.current_stream())
                torch.cuda.current_stream().synchronize()
        finally:
            L.oasis_destroy(h_all)
        for st in self.state[layer]:
            if self.eviction == "lru":
                # the selection again (same scores, same result) with the diff
                # that stamps the slots attention 0 reads
                L.oasis_select_and_diff_lru(self.h, st.scores, self.ctx_len, st.sel, st.b2s, st.s2b, st.last_use, 0,
                                            st.fetch, st.n_fetch, st.evict, st.attend, st.n_attend)
            else:
                L.oasis_resident_diff_cap_evict(self.h, st.sel, st.scores, st.b2s, st.s2b, st.fetch, st.n_fetch,
                                                st.evict, st.attend, st.n_attend)
        self.transfer(layer, stream=torch.cuda.current_stream())

    # ------------------------------------------------------------ per-step chain
    def _pred(self):
        return self.pstream if self.overlap else torch.cuda.current_stream()

    def attention(self, layer: int, q: torch.Tensor, replica: int = 0, out: torch.Tensor | None = None):
        """Sparse attention of step t on the current stream, after the last transfer
        and the last selection of this layer."""
        st = self.state[layer][replica]
        cs = torch.cuda.current_stream()
        self._flush_select_of(layer, replica, cs)
        if st.pending is not None:
            st.pending.wait(cs)
        if self.inline_pending == (layer, replica):
            self.flush_inline(cs)
        if st.select_pending:
            cs.wait_event(st.select_done)
            st.select_pending = False
        L.oasis_sparse_paged_decode_attn(self.h, q, st.pool, st.sel, st.b2s, self.ctx_len,
                                         self.out if out is None else out, self.ws_ptr, cs)
        if self.overlap:
            st.attn_done.record(cs)

    def decode_step(self, layer: int, q: torch.Tensor, replica: int = 0, out: torch.Tensor | None = None,
                    two_calls: bool = False, stamp: int = 0):
        """Attention of step t, scoring of its drafts, selection of S_{t+1} and the
        diff, in one library call (two launches for the default shape) on the
        current stream, or (two_calls) as its two halves: attention + scoring,
        then selection + diff + the attention's split combine.  An append of this
        step is enqueued before it (the attention does not read what the append
        writes; the scoring sees the grown context).  stamp: with LRU eviction,
        the index of the next attention (step t + 1), whose slots the diff stamps."""
        st = self.state[layer][replica]
        cs = torch.cuda.current_stream()
        self._flush_select_of(layer, replica, cs)  # its own attention needs it
        if st.pending is not None:
            st.pending.wait(cs)
        if st.select_pending:
            cs.wait_event(st.select_done)
            st.select_pending = False
        o = self.out if out is None else out
        carry = None
        if self.inline_pending is not None:
            if self.inline_pending != (layer, replica) and self.eviction == "score" and not two_calls:
                pst = self.state[self.inline_pending[0]][self.inline_pending[1]]
                carry = (pst.host_tier, pst.pool, pst.fetch, pst.n_fetch)
                self.inline_pending = None
            else:
                self.flush_inline(cs)
        if self.carry_select and not two_calls:
            job = None
            pend = self.pending_select
            if pend is not None:
                pst = self.state[pend[0]][pend[1]]
                job = (pst.scores, pend[2], pst.sel, pst.b2s, pst.s2b, pst.fetch, pst.n_fetch, pst.evict,
                       pst.attend, pst.n_attend)
            L.oasis_decode_step_carry(self.h, q, st.pool, st.meta, self.ctx_len, self.ctx_scoring, st.attend,
                                      st.n_attend, st.scores, o, self.ws_ptr, job=job, transfer=carry, stream=cs)
            self.pending_select = (layer, replica, self.ctx_scoring)
            if pend is not None:
                self._selected(pend[0], pend[1], cs)
            return
        if carry is not None:
            L.oasis_decode_step_gather(self.h, q, st.pool, st.meta, self.ctx_len, self.ctx_scoring, st.sel, st.b2s,
                                       st.s2b, st.scores, o, self.ws_ptr, st.fetch, st.n_fetch, st.evict, st.attend,
                                       st.n_attend, transfer=carry, stream=cs)
            return
        if self.eviction == "lru":
            L.oasis_attend_and_score(self.h, q, st.pool, st.meta, self.ctx_len, self.ctx_scoring, st.sel, st.b2s,
                                     st.attend, st.n_attend, st.scores, o, self.ws_ptr, cs)
            L.oasis_select_diff_combine_lru(self.h, st.scores, self.ctx_scoring, st.sel, st.b2s, st.s2b, st.last_use,
                                            stamp, st.fetch, st.n_fetch, st.evict, st.attend, st.n_attend, o,
                                            self.ws_ptr, cs)
            return
        if two_calls:
            L.oasis_attend_and_score(self.h, q, st.pool, st.meta, self.ctx_len, self.ctx_scoring, st.sel, st.b2s,
                                     st.attend, st.n_attend, st.scores, o, self.ws_ptr, cs)
            L.oasis_select_diff_combine(self.h, st.scores, self.ctx_scoring, st.sel, st.b2s, st.s2b, st.fetch,
                                        st.n_fetch, st.evict, st.attend, st.n_attend, o, self.ws_ptr, cs)
            return
        L.oasis_decode_step(self.h, q, st.pool, st.meta, self.ctx_len, self.ctx_scoring, st.sel, st.b2s, st.s2b,
                            st.scores, o, self.ws_ptr, st.fetch, st.n_fetch, st.evict, st.attend, st.n_attend,
                            stream=cs)

    def append(self, layer: int, k_new_dev, v_new_dev, k_new_host=None, v_new_host=None,
               replica: int = 0):
        """Append one token per unit at the current context lengths (positions).

        Every layer of a step appends at the same positions; the scoring that
        follows sees the grown context (ctx_scoring) while later layers' attention
        of the same step still sees the old one; end_step() makes it current.
        The append may run beside this step's attention: it writes the metadata,
        the other context buffer and page row n % 16, none of which the attention
        reads (it sees tokens < n).  Raises ValueError if a request's context
        is already at the capacity (max_blocks * 16 tokens).
        """
        cap_tokens = self.shape.max_blocks * 16
        if (self.ctx_host >= cap_tokens).any():
            raise ValueError(f"append: a context length is at the capacity of {cap_tokens} tokens")
        st = self.state[layer][replica]
        ps = self._pred()
        self._flush_select_of(layer, replica, ps)
        if st.pending is not None:
            st.pending.wait(ps)
        if self.inline_pending == (layer, replica):
            self.flush_inline(ps)
        L.oasis_block_meta_update(self.h, k_new_dev, v_new_dev, self.ctx[self.ctx_cur],
                                  self.ctx[1 - self.ctx_cur], st.meta, st.pool, st.b2s, ps)
        if k_new_host is not None and replica == 0:
            L.oasis_host_tier_append(self.h, np.ascontiguousarray(k_new_host),
                                     np.ascontiguousarray(v_new_host), self.ctx_host, st.host_tier)
        self._appended = True

    @property
    def ctx_scoring(self) -> torch.Tensor:
        return self.ctx[1 - self.ctx_cur] if getattr(self, "_appended", False) else self.ctx[self.ctx_cur]

    def end_step(self):
        if getattr(self, "_appended", False):
            self.ctx_cur = 1 - self.ctx_cur
            self.ctx_host = self.ctx_host + 1
            self._appended = False

    def predict_select(self, layer: int, q: torch.Tensor, replica: int = 0, stamp: int = 0):
        """Score the drafts of step t, select S_{t+1}, diff against the resident set.

        With overlap the scoring runs beside the attention of step t; the
        selection/diff waits for that attention (it rewrites the selection and
        maps the attention reads)."""
        st = self.state[layer][replica]
        ctx = self.ctx_scoring
        ps = self._pred()
        self._flush_select_of(layer, replica, ps)
        if self.inline_pending == (layer, replica):  # its fetch list is about to be rewritten
            self.flush_inline(ps)
        L.oasis_lookahead_score(self.h, q, st.meta, ctx, st.scores, ps)
        if self.overlap:
            ps.wait_event(st.attn_done)
        if self.eviction == "lru":
            L.oasis_select_and_diff_lru(self.h, st.scores, ctx, st.sel, st.b2s, st.s2b, st.last_use, stamp, st.fetch,
                                        st.n_fetch, st.evict, st.attend, st.n_attend, stream=ps)
        elif self.fused_select:
            L.oasis_select_and_diff(self.h, st.scores, ctx, st.sel, st.b2s, st.s2b, st.fetch, st.n_fetch,
                                    st.evict, st.attend, st.n_attend, stream=ps)
        else:
            L.oasis_topk_select(self.h, st.scores, ctx, st.sel, ps)
            L.oasis_resident_diff_cap_evict(self.h, st.sel, st.scores, st.b2s, st.s2b, st.fetch, st.n_fetch,
                                            st.evict, st.attend, st.n_attend, stream=ps)
        if self.overlap:
            st.select_done.record(ps)
            st.select_pending = True

    def exact_select(self, layer: int, q: torch.Tensor, replica: int = 0):
        """The set the verify query itself selects (same bound and top-k rule, from
        the verify rows instead of the drafts) into st.vsel, with its scores in
        st.vscores, on the current stream."""
        st = self.state[layer][replica]
        st.ensure_corrective(self)
        cs = torch.cuda.current_stream()
        L.oasis_verify_score(self.h, q, st.meta, self.ctx_len, st.vscores, cs)
        L.oasis_topk_select(self.h, st.vscores, self.ctx_len, st.vsel, cs)

    def corrective(self, layer: int, q: torch.Tensor, replica: int = 0):
        """Blocking corrective fetch before this step's attention: the verify
        query's own selection (exact_select), the blocks of it the prefetch missed
        fetched without a cap on the current stream (victims: the lowest-scoring
        resident blocks outside that set), and the attended list set to that set.
        The next decode_step of the layer then attends over the exact set."""
        st = self.state[layer][replica]
        cs = torch.cuda.current_stream()
        self._flush_select_of(layer, replica, cs)
        if st.pending is not None:  # a pending prefetch may target the same slots
            st.pending.wait(cs)
        if self.inline_pending == (layer, replica):
            self.flush_inline(cs)
        if st.select_pending:
            cs.wait_event(st.select_done)
            st.select_pending = False
        self.exact_select(layer, q, replica)
        hf = self.full_cap_handle()
        L.oasis_resident_diff_cap_evict(hf, st.vsel, st.vscores, st.b2s, st.s2b, st.cfetch, st.cn_fetch, st.cevict,
                                        st.attend, st.n_attend, cs)
        L.oasis_fetch_gather(hf, st.host_tier, st.pool, st.cfetch, st.cn_fetch, cs)

    def full_cap_handle(self) -> int:
        """A handle of the same shape whose fetch cap is the whole budget (the
        corrective fetch is not capped)."""
        if self._h_full is None:
            self._h_full = self.shape.handle(fetch_cap=self.shape.budget_blocks, options=self.options)
        return self._h_full

    def transfer(self, layer: int, replica: int = 0, stream=None):
        """Move this step's fetched pages of one layer into its pool on the side
        stream, after the diff (transfer_group of that layer alone)."""
        self.transfer_group([layer], replica, stream)

    def transfer_group(self, layers, replica: int = 0, stream=None):
        """Move this step's fetched pages of several layers into their pools on the
        side stream, after their diffs, as one batch: the side stream waits once
        (for the work enqueued so far on the stream that ran the diffs), then
        transfers every layer of the batch; later attention and appends of those
        layers wait for the batch's one event.  Default: the device-driven gather
        (reads the fetch list in HBM and the pages from the pinned host tier, no
        host synchronisation); with gather=False: copy the fetch lists to the
        host, wait for them once, and issue one copy per page."""
        ps = self._pred() if stream is None else stream
        states = [self.state[l][replica] for l in layers]
        if self.gather:
            ready = torch.cuda.Event()
            ready.record(ps)
            self.side.wait_event(ready)
            for st in states:
                L.oasis_fetch_gather(self.h, st.host_tier, st.pool, st.fetch, st.n_fetch, self.side)
        else:
            with torch.cuda.stream(ps):
                for st in states:
                    st.fetch_host.copy_(st.fetch, non_blocking=True)
                    st.n_fetch_host.copy_(st.n_fetch, non_blocking=True)
            ready = torch.cuda.Event()
            ready.record(ps)
            ready.synchronize()
            self.side.wait_event(ready)
            for st in states:
                L.oasis_fetch_issue(self.h, st.host_tier, st.pool, st.fetch_host, st.n_fetch_host, self.side)
        done = torch.cuda.Event()
        done.record(self.side)
        batch = PendingTransfer(done)
        for st in states:
            st.pending = batch

    def _selected(self, layer: int, replica: int, stream):
        """The layer's carried selection and diff are enqueued on `stream`: hand
        its transfer on (inline: to the next decode step's first launch; else
        the side stream, behind `stream`)."""
        if self.transfer_mode == "inline":
            self.defer_transfer(layer, replica)
        else:
            self.transfer_group([layer], replica, stream)

    def flush_select(self, stream):
        """The pending carried selection and diff as a launch of their own on
        `stream` (oasis_select_and_diff: the same results), then its transfer."""
        if self.pending_select is None:
            return
        layer, replica, ctx = self.pending_select
        self.pending_select = None
        st = self.state[layer][replica]
        L.oasis_select_and_diff(self.h, st.scores, ctx, st.sel, st.b2s, st.s2b, st.fetch, st.n_fetch, st.evict,
                                st.attend, st.n_attend, stream=stream)
        self._selected(layer, replica, stream)

    def _flush_select_of(self, layer: int, replica: int, stream):
        if self.pending_select is not None and self.pending_select[:2] == (layer, replica):
            self.flush_select(stream)

    def defer_transfer(self, layer: int, replica: int = 0):
        """Inline mode: the layer's fetched pages move in the first launch of the
        next decode step enqueued on the compute stream (or in flush_inline)."""
        if self.inline_pending is not None:
            self.flush_inline(torch.cuda.current_stream())
        self.inline_pending = (layer, replica)

    def flush_inline(self, stream):
        """The pending inline transfer as a gather launch of its own on `stream`."""
        if self.inline_pending is None:
            return
        st = self.state[self.inline_pending[0]][self.inline_pending[1]]
        L.oasis_fetch_gather(self.h, st.host_tier, st.pool, st.fetch, st.n_fetch, stream)
        self.inline_pending = None

    def wait_transfers(self):
        """Make the current stream wait for every pending transfer and selection."""
        cs = torch.cuda.current_stream()
        self.flush_select(cs)
        self.flush_inline(cs)
        for layer in self.state:
            for st in layer:
                if st.pending is not None:
                    st.pending.wait(cs)
                if st.select_pending:
                    cs.wait_event(st.select_done)
                    st.select_pending = False

    # ------------------------------------------------------------ inspection
    def pool_pages(self, layer: int, replica: int = 0) -> torch.Tensor:
        s = self.shape
        st = self.state[layer][replica]
        return st.pool.view(s.units, s.budget_blocks, -1)

    def meta_view(self, layer: int, replica: int = 0) -> torch.Tensor:
        """The layer's block metadata as [units][max_blocks][2][d] (a copy on the
        device, int16 bit patterns for bf16): the library's export of its
        chunk-major tiles into the logical layout."""
        s = self.shape
        st = self.state[layer][replica]
        out = torch.empty((s.units, s.max_blocks, 2, s.head_dim),
                          dtype=torch.int16 if s.dtype == "bf16" else torch.float32, device=self.device)
        L.oasis_block_meta_export(self.h, st.meta, out)
        return out

    def load_meta(self, layer: int, meta: torch.Tensor, replica: int = 0):
        """Write logical metadata [units][max_blocks][2][d] (device, element
        type or its bit patterns) into the layer's tiles."""
        s = self.shape
        assert meta.is_cuda and meta.is_contiguous()
        assert tuple(meta.shape) == (s.units, s.max_blocks, 2, s.head_dim)
        assert meta.element_size() == s.elem_bytes
        L.oasis_block_meta_import(self.h, meta, self.state[layer][replica].meta)
