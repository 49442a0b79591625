"""Runs the decode chain on the seeded synthetic workloads (workload/).

Fills the pinned host tier of every layer from the generator, builds the block
metadata on the GPU, runs the prologue (first selection, initial residency,
first transfer) and then decode steps, optionally recording the per-step
state of selected units for parity checks.  Used by the benchmark, the smoke
check and the GPU tests.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from workload import synth
from workload.configs import BLOCK, Config

from .runtime import DecodeRuntime, Shape


def shape_of(cfg: Config) -> Shape:
    return Shape(batch=cfg.batch, kv_heads=cfg.kv_heads, group=cfg.group, head_dim=cfg.head_dim,
                 max_blocks=cfg.max_blocks, budget_blocks=cfg.k, n_draft=cfg.n_draft,
                 fetch_cap=cfg.fetch_cap, dtype=cfg.dtype)


def _elem(cfg: Config, x: np.ndarray) -> np.ndarray:
    return synth.to_bf16_bits(x) if cfg.dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class SyntheticRun:
    """The decode chain of one workload configuration on cuda:0."""

    def __init__(self, cfg: Config, layers: int | None = None, replicas: int = 1,
                 record_units=None, device: str = "cuda", overlap: bool = True, fused_step: bool = True,
                 gather: bool = True, two_calls: bool = False, options: dict | None = None,
                 eviction: str = "score", transfer_group: int = 1, transfer_mode: str = "side",
                 carry_select: bool = False):
        """fused_step: without overlap and drift, run each layer's step through the
        single decode-step call (attention, scoring, selection, diff), or through
        its two halves (two_calls).  gather: move the fetched pages with the
        device-driven gather (else host-issued copies).  options: the library's
        launch options (None = defaults).  eviction: "score" or "lru".
        transfer_group: layers whose transfers go to the side stream as one
        batch (one cross-stream hand-off and one completion event per batch).
        transfer_mode: "side" or "inline" (each layer's pages ride in the next
        decode step's first launch on the compute stream).
        carry_select: each layer's selection and diff run in the next decode
        step's first launch (oasis_decode_step_carry), which also hands that
        layer's transfer on; used where the fused step runs."""
        self.cfg = cfg
        self.fused_step = fused_step and not overlap
        self.two_calls = two_calls
        self.group = max(1, int(transfer_group))
        self.L = cfg.layers if layers is None else layers
        self.shape = shape_of(cfg)
        self.rt = DecodeRuntime(self.shape, layers=self.L, device=device, replicas=replicas, overlap=overlap,
                                gather=gather, options=options, eviction=eviction,
                                transfer_mode=(transfer_mode if self.fused_step and not cfg.drift_blocks
                                               else "side"),
                                carry_select=(carry_select and self.fused_step and not cfg.drift_blocks
                                              and not two_calls))
        self.record_units = record_units  # list of (layer, unit) to record, or None
        self.records = {}
        B, H, G, T, d = cfg.batch, cfg.kv_heads, cfg.group, cfg.T, cfg.head_dim
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        # queries: [layer][step + 1][B][Hq][T][d]; index 0 = the prologue's drafts (step -1)
        self.q = torch.empty((self.L, cfg.steps + 1, B, H * G, T, d), dtype=tdt, device=device)
        self.kv_new = None
        self.drift = None
        if cfg.append:
            self.k_new_host = np.empty((self.L, cfg.steps, B, H, d), dtype=self.shape.np_elem)
            self.v_new_host = np.empty_like(self.k_new_host)
        self._fill()

    # ----------------------------------------------------------------- setup
    def _fill(self):
        cfg, rt = self.cfg, self.rt
        B, H, G, T, d = cfg.batch, cfg.kv_heads, cfg.group, cfg.T, cfg.head_dim
        qh = np.empty((cfg.steps + 1, B, H * G, T, d), dtype=np.float32)
        if cfg.drift_blocks:
            self.drift = {}  # (l, u) -> (unit data, schedule)
        for l in range(self.L):
            def work(u, l=l):
                r, h = divmod(u, H)
                ud = synth.unit_data(cfg, r, l, h)
                K = ud.keys()
                N0 = cfg.n_blocks0_of(r)
                rt.pack_unit(l, u, _elem(cfg, K[: N0 * BLOCK]), _elem(cfg, ud.V[: N0 * BLOCK]))
                for t in range(-1, cfg.steps):
                    qq = ud.queries(t)  # [G][T][d]
                    if t == -1:
                        qq = qq.copy()
                        qq[:, 0, :] = 0.0  # the prologue scores drafts only
                    qh[t + 1, r, h * G:(h + 1) * G] = qq
                if cfg.append:
                    pos = cfg.ctx_of(r) + np.arange(cfg.steps)
                    self.k_new_host[l, :, r, h] = _elem(cfg, K[pos])
                    self.v_new_host[l, :, r, h] = _elem(cfg, ud.V[pos])
                if self.drift is not None:
                    self.drift[(l, u)] = (ud, synth.drift_schedule(cfg, r, l, h, ud.planted0))
            with ThreadPoolExecutor(max_workers=_threads()) as ex:
                list(ex.map(work, range(cfg.units_per_layer)))
            self.q[l].copy_(torch.from_numpy(qh).to(self.q.dtype))
        if cfg.append:
            self.k_new_dev = torch.from_numpy(self.k_new_host.view(np.int16) if cfg.dtype == "bf16"
                                              else self.k_new_host).to(self.rt.device)
            self.v_new_dev = torch.from_numpy(self.v_new_host.view(np.int16) if cfg.dtype == "bf16"
                                              else self.v_new_host).to(self.rt.device)
        rt.set_ctx(np.array([cfg.ctx_of(r) for r in range(cfg.batch)], dtype=np.int32))
        for l in range(self.L):
            rt.build_meta(l)

    def prologue(self):
        cfg = self.cfg
        H = cfg.kv_heads
        for l in range(self.L):
            def init(u, sel_row, l=l):
                r, h = divmod(u, H)
                return synth.initial_residency(cfg, r, l, h, sel_row)
            self.rt.prologue(l, self.q[l, 0], init)
        self.rt.wait_transfers()
        self._record(-1)

    # ----------------------------------------------------------------- steps
    def _apply_drift(self, l: int, t: int):
        cfg, rt = self.cfg, self.rt
        ids = []
        for u in range(cfg.units_per_layer):
            ud, sched = self.drift[(l, u)]
            unplant, plant, planted_after = sched[t]
            blocks = np.concatenate([unplant, plant]).astype(np.int64)
            if len(blocks) == 0:
                continue
            kb = ud.keys_of_blocks(blocks, planted_after)  # [m][16][d]
            rt.pack_unit(l, u, _elem(cfg, kb.reshape(-1, cfg.head_dim)), None, blocks.astype(np.int32))
            ids.append(u * cfg.max_blocks + blocks)
        if ids:
            rt.rebuild_blocks(l, np.concatenate(ids))

    def step(self, t: int, transfer: bool = True, sync: bool = True):
        """One decode step over the layers; sync: end it with every selection and
        transfer enqueued and waited for (else carried selections and inline
        transfers stay pending into the next step)."""
        cfg, rt = self.cfg, self.rt
        if self.fused_step and self.drift is None:
            for l in range(self.L):
                q = self.q[l, t + 1]
                if cfg.append:
                    rt.append(l, self.k_new_dev[l, t], self.v_new_dev[l, t],
                              self.k_new_host[l, t], self.v_new_host[l, t])
                rt.decode_step(l, q, two_calls=self.two_calls, stamp=t + 1)
                if self.record_units is not None:
                    self._record_out(l, t)
                if transfer:
                    self._transfer_after(l)
            rt.end_step()
            if transfer and sync:
                rt.wait_transfers()
            if sync:
                self._record(t)
            return
        for l in range(self.L):
            q = self.q[l, t + 1]
            rt.attention(l, q)
            if self.record_units is not None:
                self._record_out(l, t)
            if cfg.append:
                rt.append(l, self.k_new_dev[l, t], self.v_new_dev[l, t],
                          self.k_new_host[l, t], self.v_new_host[l, t])
            if self.drift is not None:
                self._apply_drift(l, t)
            rt.predict_select(l, q, stamp=t + 1)
            if transfer:
                self._transfer_after(l)
        rt.end_step()
        if transfer:
            rt.wait_transfers()
        self._record(t)

    def _transfer_after(self, l: int):
        """After layer l's diff: hand the batch that ends at layer l to the side
        stream (or, inline, leave the pages to the next decode step's launch).
        A carried selection hands its transfer on itself."""
        if self.rt.carry_select:
            return
        if self.rt.transfer_mode == "inline":
            self.rt.defer_transfer(l)
            return
        if (l + 1) % self.group == 0 or l == self.L - 1:
            first = l - (l % self.group)
            self.rt.transfer_group(range(first, l + 1))

    def run(self, steps: int | None = None, transfer: bool = True, log=None):
        """Prologue plus `steps` decode steps; `log(msg)` receives progress lines."""
        self.prologue()
        total = self.cfg.steps if steps is None else steps
        for t in range(total):
            self.step(t, transfer=transfer)
            if log is not None and (t % 8 == 7 or t == total - 1):
                log(f"{self.cfg.name}: step {t + 1}/{total} done")

    # ----------------------------------------------------------------- records
    def _record_out(self, l: int, t: int):
        cfg = self.cfg
        out = self.rt.out.cpu().numpy()
        for (rl, u) in self.record_units:
            if rl != l:
                continue
            r, h = divmod(u, cfg.kv_heads)
            self.records.setdefault((l, u), {}).setdefault(t, {})["out"] = \
                out[r, h * cfg.group:(h + 1) * cfg.group].copy()

    def _record(self, t: int):
        if self.record_units is None:
            return
        torch.cuda.synchronize()
        cache = {}
        for (l, u) in self.record_units:
            if l not in cache:
                st = self.rt.state[l][0]
                cache[l] = {k: getattr(st, k).cpu().numpy() for k in
                            ("sel", "scores", "fetch", "n_fetch", "evict", "s2b", "b2s")}
                if st.last_use is not None:
                    cache[l]["last_use"] = st.last_use.cpu().numpy()
            c = cache[l]
            rec = self.records.setdefault((l, u), {}).setdefault(t, {})
            nf = int(c["n_fetch"][u])
            rec.update(sel=c["sel"][u].copy(), scores=c["scores"][u].copy(),
                       fetch=[tuple(int(x) for x in p) for p in c["fetch"][u][:nf]],
                       evict=[int(v) for v in c["evict"][u][:nf] if v >= 0],
                       s2b=c["s2b"][u].copy(), b2s=c["b2s"][u].copy(),
                       n_scoring=int(self.rt.ctx_len.cpu().numpy()[u // self.cfg.kv_heads]))
            if "last_use" in c:
                rec["last_use"] = c["last_use"][u].copy()

    def close(self):
        self.rt.close()
