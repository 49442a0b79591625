"""Benchmark of the lookahead sparse-KV decode step on one MI355X.

A step is one pass of the whole hot path for every layer of one batch:
sparse paged decode attention (verify + drafts over the resident selected
blocks), lookahead scoring of every block, top-k selection and the
resident-set diff with capped fetch / eviction.  The timed loop keeps all
inputs resident in HBM and leaves the host-tier transfer out (the maps still
update every step, so every step moves the same bytes); the workload's state is
replicated so that the working set exceeds the 256 MB Infinity Cache and every
step streams from HBM.

Prints one JSON line: throughput in (request x layer) decode steps per second,
the roofline of the dominant kernel (algorithmic bytes / measured duration
against 8 TB/s), per-kernel timings, and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LEAD_US = 300.0  # spin ahead of each event-timed region (covers the host's first launches)
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2**20
CALIB_ELEMS = 2**28  # float32: 1 GiB
CSRC = os.path.join(ROOT, "lookahead_sparse_kv_draft_amd", "csrc")
# source files of each op's kernels (a traffic measurement is valid while they are unchanged)
# (api.cpp holds the launch shapes)
OP_SOURCES = {"attend_and_score": ["step.hip", "step_kernel.h", "attn_body.h", "score_body.h", "select_wg.h",
                                   "topk_body.h", "diff_body.h", "oasis_internal.h", "api.cpp"],
              "select_diff_combine": ["select.hip", "select_wg.h", "topk_body.h", "diff_body.h", "block_ops.h",
                                      "attn_combine.h", "oasis_internal.h"],
              "sparse_paged_decode_attn": ["attn.hip", "attn_body.h", "attn_combine.h", "oasis_internal.h"],
              "lookahead_score": ["score.hip", "score_body.h", "oasis_internal.h"],
              "select_and_diff": ["select.hip", "select_wg.h", "topk_body.h", "diff_body.h", "block_ops.h",
                                  "oasis_internal.h"]}
# (budgets of at most 128 blocks run the workgroup selection kernels, larger ones the
# 1024-thread kernels; only one of each pair runs for a shape)
OP_KERNELS = {"attend_and_score": ["attn_score_kernel"],
              "select_diff_combine": ["select_wg_combine_kernel", "select_diff_combine_kernel"],
              "sparse_paged_decode_attn": ["attn_mfma_kernel", "attn_combine_kernel"],
              "lookahead_score": ["score_mfma_kernel"], "select_and_diff": ["select_wg_kernel", "select_diff_kernel"]}
# the two launches of the decode step, then the stages on their own
OPS = ["attend_and_score", "select_diff_combine", "sparse_paged_decode_attn", "lookahead_score", "select_and_diff"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # the warm-up runs long enough (~10 ms at the default workload) for the GPU to
    # reach its steady state; 20 steps measured ~4 % slow in the first timed steps
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--config", default="llama8b_32k")
    p.add_argument("--replicas", type=int, default=0,
                   help="0 = enough for each op's own footprint to exceed the Infinity Cache twice")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--calib-copy", action="store_true", help="also run a plain 1 GiB device copy (counter calibration)")
    p.add_argument("--no-h2", action="store_true", help="skip the end-to-end (transfer-inclusive) measurement")
    p.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT"),
                   help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                        "`bench.py --calib-copy` into a traffic file and exit")
    p.add_argument("--counter-summary", nargs="+", metavar="CSV",
                   help="average per kernel every counter of rocprofv3 --pmc counter_collection.csv "
                        "files, the last argument being the output text file, and exit")
    p.add_argument("--pipeline", action="store_true",
                   help="cross-layer transfer pipeline: exposed transfer per step against the fetch cap "
                        "(one JSON line per sweep instead of the headline)")
    p.add_argument("--layers", type=int, default=8, help="layers of the --pipeline run")
    p.add_argument("--groups", default="carry,inline,1,4",
                   help="--pipeline: layers per side-stream transfer batch (one hand-off and one event each), "
                        "'inline' (each layer's pages ride in the next decode step's first launch), or 'carry' "
                        "(as inline, with each layer's selection also carried by the next layer's first launch)")
    p.add_argument("--recall", action="store_true",
                   help="prediction recall of the drafts' selection against the verify query's own selection, "
                        "and the cost of a blocking corrective fetch (one JSON line)")
    p.add_argument("--cap-fracs", default="0,0.01,0.02,0.05,0.10,0.20,1.0",
                   help="--pipeline fetch caps as fractions of the block budget k (1.0 = fetch all)")
    p.add_argument("--eviction", choices=["score", "lru", "both"], default="both",
                   help="--pipeline eviction policies: lowest score, least recently used, or both")
    p.add_argument("--launch-options", default=None, metavar="JSON",
                   help="the library's launch options as a JSON object (oasis_launch_options fields), "
                        "e.g. '{\"attn_merge\": 2}'; default: the library's own choice")
    p.add_argument("--mode", choices=["auto", "graph", "overlap", "eager", "carry", "two_streams",
                                      "two_streams_graph"], default="auto",
                   help="graph: steps captured as a HIP graph on one stream; overlap: the scoring on a "
                        "second stream beside the attention, captured likewise; eager: plain launches; "
                        "carry: plain launches, each layer's selection and diff carried by the next layer's "
                        "first launch (several layers only); two_streams: plain launches, each layer's "
                        "selection and diff on a second stream beside the next layer's attention and scoring; "
                        "two_streams_graph: the same captured as a HIP graph; auto: carry for several layers, "
                        "else eager")
    return p.parse_args()


def algorithmic_bytes(cfg, attended_blocks: int):
    """Bytes each kernel must move per launch (whole batch, one layer)."""
    e = cfg.elem_bytes
    units = cfg.batch * cfg.kv_heads
    N = cfg.n_blocks0
    d = cfg.head_dim
    score = units * N * 2 * d * e + units * N * 4 + cfg.batch * cfg.q_heads * cfg.n_draft * d * e
    attn = (attended_blocks * 2 * 16 * d * e + cfg.batch * cfg.q_heads * cfg.T * d * (e + 4)
            + units * cfg.k * 8)
    sel_diff = units * N * 4 + units * cfg.k * 4 * 5 + units * cfg.fetch_cap * 12
    out = cfg.batch * cfg.q_heads * cfg.T * d * 4  # the attention output, written by the split combine
    return {"lookahead_score": score, "sparse_paged_decode_attn": attn, "select_and_diff": sel_diff,
            "attend_and_score": attn - out + score, "select_diff_combine": sel_diff + out}


def attn_flops(cfg, attended_blocks: int):
    return attended_blocks * 16 * cfg.group * cfg.T * cfg.head_dim * 4


def _oracle_unit_job(args):
    """Prologue + `steps` oracle steps of one unit; returns its CPU seconds."""
    cfg_name, cfg_kw, r, h, steps = args
    from threadpoolctl import threadpool_limits

    from oracle import oasis_oracle as O
    from workload import CONFIGS, synth
    cfg = CONFIGS[cfg_name].with_(**cfg_kw) if cfg_kw else CONFIGS[cfg_name]
    with threadpool_limits(limits=1):
        ud = synth.unit_data(cfg, r, 0, h)
        K = ud.keys()
        t0 = time.perf_counter()
        O.run_unit(K_at=lambda t: K, V=ud.V, queries=ud.queries, drafts_prologue=ud.drafts[0],
                   n0=cfg.ctx, k=cfg.k, cap=cfg.fetch_cap, steps=steps,
                   initial_slots=lambda S0: synth.initial_residency(cfg, r, 0, h, S0),
                   append=cfg.append, max_blocks=cfg.max_blocks)
        return time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, target_s: float):
    """The oracle (fp64 numpy, one BLAS thread per worker) timed on a bounded
    sample of the same workload: layer-0 units, prologue + 16 steps each, over a
    process pool of the host's cores (at most 16), after a one-worker run."""
    import concurrent.futures as cf
    import multiprocessing as mp

    H = cfg.kv_heads
    steps = min(cfg.steps, 16)
    units = [(u // H, u % H) for u in range(cfg.batch * H)]
    # one worker: units until the time target
    t1, n1 = 0.0, 0
    for (r, h) in units:
        if t1 >= target_s / 3:
            break
        t1 += _oracle_unit_job((cfg.name, None, r, h, steps))
        n1 += 1
    one = (n1 * steps / H) / t1
    # pool: as many units as fit the target at the measured per-unit cost
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    per_unit = t1 / n1
    n_units = int(min(len(units) * 8, max(workers, target_s * workers / per_unit)))
    jobs = [(cfg.name, None, units[i % len(units)][0], units[i % len(units)][1], steps) for i in range(n_units)]
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        list(ex.map(_oracle_unit_job, jobs))
    wall = time.perf_counter() - t0
    value = (n_units * steps / H) / wall
    return {"value": value, "unit": "decode steps/s (request x layer)", "cores": workers, "kind": "oracle",
            "sample": f"{n_units} (request, KV head) units of layer 0 (cycled over the {len(units)} units), "
                      f"prologue + {steps} steps each, fp64 numpy, {workers} worker processes x 1 BLAS "
                      f"thread, {wall:.1f} s wall (incl. worker start-up); CPU {_cpu_model()}",
            "one_worker": {"value": one, "units": n1, "seconds": t1}}


def op_source_hash(op: str) -> str:
    """Hash of the code of an op's sources: comments and whitespace removed, so
    that only a change of the code itself invalidates measured traffic."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in OP_SOURCES[op]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _counter_means(path: str):
    """Mean counter value (KiB per dispatch) per kernel from a rocprofv3
    counter_collection.csv: keyed by base name for the library's kernels and by
    full name for elementwise kernels (the calibration add)."""
    import csv
    import re
    acc = {}
    for r in csv.DictReader(open(path)):
        full = r["Kernel_Name"]
        m = re.search(r"(\w+)(<[^(]*>)?\(", full)
        name = m.group(1) if m else full
        key = full if "elementwise" in name else name
        acc.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic_summary(fetch_csv: str, write_csv: str, out: str, cmdline: str):
    """HBM bytes per launch of each op: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what it reads for the calibration add (1 GiB in,
    1 GiB out)."""
    fe, wr = _counter_means(fetch_csv), _counter_means(write_csv)
    gib_kib = CALIB_ELEMS * 4 / 1024
    calib = [k for k in wr if "elementwise" in k and abs(wr[k] - gib_kib) < 0.05 * gib_kib and k in fe]
    if not calib:
        raise SystemExit("no calibration kernel in the counter files (run bench.py with --calib-copy)")
    c = calib[0]
    f_fac = gib_kib / fe[c]
    w_fac = gib_kib / wr[c]
    short = c.split("(")[0][:90]
    lines = [f"# HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, llama8b_32k",
             "# counters: cd /tmp && rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'oasis|elementwise' "
             "--output-format csv -d <dir> -o f -- python <repo>/bench.py --steps 8 --warmup 2 --no-cpu-baseline "
             "--no-h2 --calib-copy  (then the same with WRITE_SIZE and -o w)",
             f"# summary: {cmdline}",
             f"calibration {short.replace(' ', '')} fetch_kib {fe[c]:.1f} write_kib {wr[c]:.1f} "
             f"expected_kib {gib_kib:.1f} fetch_factor {f_fac:.4f} write_factor {w_fac:.4f}"]
    for op, kernels in OP_KERNELS.items():
        tot = 0.0
        for k in kernels:
            f_kib, w_kib = fe.get(k, 0.0), wr.get(k, 0.0)
            b = (f_kib * f_fac + w_kib * w_fac) * 1024
            tot += b
            lines.append(f"kernel {k} op {op} fetch_kib {f_kib:.1f} write_kib {w_kib:.1f} hbm_bytes {b:.0f}")
        lines.append(f"op {op} source {op_source_hash(op)} hbm_bytes {tot:.0f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counter_summary(paths, out: str, cmdline: str):
    """Mean of every counter per kernel (template arguments kept) over the
    dispatches of rocprofv3 --pmc counter_collection.csv files."""
    import csv
    import re
    acc, calls = {}, {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            m = re.search(r"(\w+_kernel)(<[^(]*>)?", r["Kernel_Name"])
            k = (m.group(1) + (m.group(2) or "")) if m else r["Kernel_Name"][:60]
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for v in acc.values() for c in v})
    lines = [f"# rocprofv3 --pmc counters per kernel (mean over dispatches), llama8b_32k",
             "# counters: cd /tmp && rocprofv3 --pmc MfmaUtil VALUBusy --kernel-include-regex 'oasis' "
             "--output-format csv -d <dir1> -o m -- python <repo>/bench.py --steps 8 --warmup 2 --no-cpu-baseline "
             "--no-h2  (then the same with --pmc MfmaFlopsBF16 OccupancyPercent and -d <dir2>)",
             "# MfmaUtil, VALUBusy, OccupancyPercent: percent of the kernel's active time (derived counters); "
             "MfmaFlopsBF16: bf16 MFMA flops per dispatch",
             f"# summary: {cmdline}",
             "kernel " + " ".join(f"{n}(calls)" for n in names)]
    for k in sorted(acc):
        cells = []
        for n in names:
            v = acc[k].get(n)
            cells.append("-" if v is None else f"{sum(v) / len(v):.4g}({len(v)})")
        lines.append(f"{k.replace(' ', '')} " + " ".join(cells))
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_traffic(workload: str):
    """op -> measured HBM bytes per launch, only for ops whose sources are unchanged."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return {}
    res = {}
    for ln in open(path):
        t = ln.split()
        if len(t) >= 6 and t[0] == "op" and t[2] == "source" and t[4] == "hbm_bytes":
            if t[3] == op_source_hash(t[1]):
                res[t[1]] = float(t[5])
    return res


def measure_h2(args, cfg, run, rt, replicas, sequential_step, h1_step_us):
    """End to end: every step's fetched pages move from the pinned host tier into
    the pool on the side stream and the next step's attention of the layer waits
    for them, as in a single-layer decode chain.  Two transfer paths: the
    device-driven gather (the fetch list stays in HBM, one kernel reads the
    pages from pinned host memory) and host-issued copies (the fetch list is
    copied to pinned host memory, the host waits for it and issues one
    hipMemcpyAsync per page).  Reports per path the step time, the exposed
    transfer (end-to-end minus HBM-resident step time) and fetched bytes per
    step, plus the gather's PCIe rate and a plain pinned host-to-device copy rate
    for reference."""
    import torch

    from lookahead_sparse_kv_draft_amd import _lib as L

    cs = torch.cuda.current_stream()
    side = rt.side
    ev_sel = [torch.cuda.Event() for _ in range(run.L)]
    ev_fetch = [torch.cuda.Event() for _ in range(run.L)]
    nf_tot = torch.zeros((), dtype=torch.int64, device="cuda")
    page = L.oasis_page_bytes(rt.h)

    def step(i, first, mode, count=False):
        rep = i % replicas
        t = i % cfg.steps
        for l in range(run.L):
            st = rt.state[l][rep]
            if not first:
                cs.wait_event(ev_fetch[l])
            L.oasis_decode_step(rt.h, run.q[l, t + 1], st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.sel, st.b2s,
                                st.s2b, st.scores, rt.out, rt.ws_ptr, st.fetch, st.n_fetch, st.evict, st.attend,
                                st.n_attend, stream=cs)
            if count:
                nf_tot.add_(st.n_fetch.sum())
            if mode == "gather":
                ev_sel[l].record(cs)
                side.wait_event(ev_sel[l])
                L.oasis_fetch_gather(rt.h, st.host_tier, st.pool, st.fetch, st.n_fetch, side)
            else:
                st.fetch_host.copy_(st.fetch, non_blocking=True)
                st.n_fetch_host.copy_(st.n_fetch, non_blocking=True)
                ev_sel[l].record(cs)
                ev_sel[l].synchronize()
                side.wait_event(ev_sel[l])
                L.oasis_fetch_issue(rt.h, st.host_tier, st.pool, st.fetch_host, st.n_fetch_host, side)
            ev_fetch[l].record(side)

    def chain(mode, K):
        for i in range(min(args.warmup, 20)):
            step(i, i == 0, mode)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(i, False, mode)
        cs.wait_event(ev_fetch[run.L - 1])
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / K * 1e6
        nf_tot.zero_()
        for i in range(K):  # untimed: fetched pages per step
            step(i, False, mode, count=True)
        torch.cuda.synchronize()
        return {"ms_per_step": us * 1e-3,
                "steps_per_s": cfg.batch * run.L * 1e6 / us,
                "exposed_transfer_us_per_step": us - h1_step_us * run.L,
                "fetched_bytes_per_step": float(nf_tot.item()) * page / K,
                "steps_timed": K}

    res = {"gather": chain("gather", min(args.steps, 200))}
    # the gather alone, back to back on the side stream, over the last lists
    eb, ee = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    Kg = min(args.steps, 200)
    eb.record(side)
    for i in range(Kg):
        st = rt.state[0][i % replicas]
        L.oasis_fetch_gather(rt.h, st.host_tier, st.pool, st.fetch, st.n_fetch, side)
    ee.record(side)
    torch.cuda.synchronize()
    gather_us = eb.elapsed_time(ee) * 1e3 / Kg
    nf_last = sum(int(rt.state[0][r].n_fetch.sum()) for r in range(replicas)) / replicas
    res["gather"]["gather_us"] = gather_us
    res["gather"]["gather_pcie_GBs"] = (nf_last * page) / (gather_us * 1e-6) / 1e9 if gather_us > 0 else None
    # host-issued copies: one hipMemcpyAsync per page (a few microseconds each), fewer steps
    res["host_copies"] = chain("host_copies", min(args.steps, 40))
    # pinned host -> device copy reference (64 MiB)
    hbuf = torch.empty(64 * 2**20, dtype=torch.uint8, pin_memory=True)
    dbuf = torch.empty(64 * 2**20, dtype=torch.uint8, device="cuda")
    dbuf.copy_(hbuf, non_blocking=True)
    torch.cuda.synchronize()
    # three rounds of 5 copies: the host link's rate varies from run to run, the
    # best round is the achievable reference
    memcpy_rounds = []
    for _ in range(3):
        eb.record(cs)
        for _ in range(5):
            dbuf.copy_(hbuf, non_blocking=True)
        ee.record(cs)
        torch.cuda.synchronize()
        memcpy_rounds.append(5 * hbuf.numel() / (eb.elapsed_time(ee) * 1e-3) / 1e9)
    res["h2d_pinned_memcpy_GBs"] = max(memcpy_rounds)
    res["h2d_pinned_memcpy_rounds_GBs"] = memcpy_rounds
    res["note"] = ("PCIe-inclusive single-layer chain, host wall clock: each step's fetch lands before the next "
                   "attention; not the headline value")
    return res


def pipeline_sweep(args):
    """Cross-layer pipeline: per step, every layer runs its decode step on the
    compute stream and its fetched pages move with the device-driven gather on
    the side stream; layer l's next attention waits only for layer l's gather, so
    each layer's transfer runs while the later layers (and the next step's
    earlier layers) compute.  For each eviction policy (lowest score; least
    recently used) and fetch cap, from the same starting state: the
    HBM-resident step time (H1, no transfer), the end-to-end step time (H2),
    exposed transfer = H2 - H1, bytes fetched per step and the gather's PCIe
    rate."""
    import torch

    from lookahead_sparse_kv_draft_amd import _lib as L
    from lookahead_sparse_kv_draft_amd.synthetic import SyntheticRun
    from workload import CONFIGS

    base = CONFIGS[args.config]
    kb = base.k
    fracs = [float(x) for x in args.cap_fracs.split(",")]
    caps = sorted({min(kb, int(round(f * kb))) if f < 1.0 else kb for f in fracs})
    policies = ["score", "lru"] if args.eviction == "both" else [args.eviction]
    cfg = base.with_(layers=args.layers, fetch_cap=max(caps))
    torch.cuda.set_device(0)
    print(f"# pipeline: {cfg.name} x {cfg.layers} layers, caps {caps}, eviction {policies}", file=sys.stderr,
          flush=True)
    run = SyntheticRun(cfg, overlap=False, replicas=2)  # replica 1 keeps the starting state
    run.prologue()
    rt = run.rt
    nl = run.L
    for l in range(nl):
        rt.state[l][1].copy_from(rt.state[l][0])
    torch.cuda.synchronize()
    cs = torch.cuda.current_stream()
    side = rt.side
    page = L.oasis_page_bytes(rt.h)
    units, k = rt.shape.units, rt.shape.budget_blocks
    lus = [torch.full((units, k), -1, dtype=torch.int32, device="cuda") for _ in range(nl)]
    ev_sel = [torch.cuda.Event() for _ in range(nl)]
    ev_fetch = [torch.cuda.Event() for _ in range(nl)]
    nf_tot = torch.zeros((), dtype=torch.int64, device="cuda")
    points = []
    # layers per side-stream batch; 0 ("inline"): each layer's pages ride in the next
    # decode step's first launch on the compute stream (oasis_decode_step_gather);
    # -1 ("carry"): the same, each layer's selection carried by the next layer's
    # first launch too (oasis_decode_step_carry), its pages by the one after
    groups = [{"inline": 0, "carry": -1}.get(x.strip()) if x.strip() in ("inline", "carry") else int(x)
              for x in args.groups.split(",")]
    runs = [(p, c, g) for p in policies for c in caps
            for g in (groups if p == policies[0] else [x for x in groups if x > 0][-1:])]
    for policy, cap, group in runs:
        h = rt.shape.handle(fetch_cap=cap)
        for l in range(nl):
            rt.state[l][0].copy_from(rt.state[l][1])
            lus[l].fill_(-1)
        clock = [0]

        pending = [None]  # inline: the layer whose fetched pages await the next launch
        pending_sel = [None]  # carry: the layer whose selection awaits the next launch

        def job_of(l):
            sj = rt.state[l][0]
            return (sj.scores, rt.ctx_len, sj.sel, sj.b2s, sj.s2b, sj.fetch, sj.n_fetch, sj.evict, sj.attend,
                    sj.n_attend)

        def step(i, transfer, first=False, count=False):
            t = i % cfg.steps
            clock[0] += 1
            for l in range(nl):
                st = rt.state[l][0]
                q = run.q[l, t + 1]
                if group == -1:
                    if pending_sel[0] == l:  # one layer: its own next attention needs the selection
                        L.oasis_select_and_diff(h, *job_of(l), stream=cs)
                        pending_sel[0] = None
                        pending[0] = l if transfer else None
                    carry = None
                    if transfer and pending[0] is not None:
                        ps_ = rt.state[pending[0]][0]
                        if pending[0] == l:
                            L.oasis_fetch_gather(h, ps_.host_tier, ps_.pool, ps_.fetch, ps_.n_fetch, cs)
                        else:
                            carry = (ps_.host_tier, ps_.pool, ps_.fetch, ps_.n_fetch)
                        pending[0] = None
                    js = pending_sel[0]
                    L.oasis_decode_step_carry(h, q, st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.attend,
                                              st.n_attend, st.scores, rt.out, rt.ws_ptr,
                                              job=None if js is None else job_of(js), transfer=carry, stream=cs)
                    if count and js is not None:
                        nf_tot.add_(rt.state[js][0].n_fetch.sum())
                    pending[0] = js if transfer else None
                    pending_sel[0] = l
                    continue
                if group == 0:
                    pl = pending[0]
                    carry = None
                    if transfer and pl is not None:
                        ps_ = rt.state[pl][0]
                        if pl == l:
                            L.oasis_fetch_gather(h, ps_.host_tier, ps_.pool, ps_.fetch, ps_.n_fetch, cs)
                        else:
                            carry = (ps_.host_tier, ps_.pool, ps_.fetch, ps_.n_fetch)
                    L.oasis_decode_step_gather(h, q, st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.sel, st.b2s,
                                               st.s2b, st.scores, rt.out, rt.ws_ptr, st.fetch, st.n_fetch, st.evict,
                                               st.attend, st.n_attend, transfer=carry, stream=cs)
                    pending[0] = l if transfer else None
                    if count:
                        nf_tot.add_(st.n_fetch.sum())
                    continue
                gi = l // group  # layers [gi * group, ...) hand their transfers over as one batch
                if transfer and not first and l % group == 0:
                    cs.wait_event(ev_fetch[gi])
                if policy == "score":
                    L.oasis_decode_step(h, q, st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.sel, st.b2s, st.s2b,
                                        st.scores, rt.out, rt.ws_ptr, st.fetch, st.n_fetch, st.evict, st.attend,
                                        st.n_attend, stream=cs)
                else:
                    L.oasis_attend_and_score(h, q, st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.sel, st.b2s,
                                             st.attend, st.n_attend, st.scores, rt.out, rt.ws_ptr, cs)
                    L.oasis_select_diff_combine_lru(h, st.scores, rt.ctx_len, st.sel, st.b2s, st.s2b, lus[l],
                                                    clock[0], st.fetch, st.n_fetch, st.evict, st.attend,
                                                    st.n_attend, rt.out, rt.ws_ptr, cs)
                if count:
                    nf_tot.add_(st.n_fetch.sum())
                if transfer and ((l + 1) % group == 0 or l == nl - 1):
                    ev_sel[gi].record(cs)
                    side.wait_event(ev_sel[gi])
                    for ll in range(gi * group, l + 1):
                        sl = rt.state[ll][0]
                        L.oasis_fetch_gather(h, sl.host_tier, sl.pool, sl.fetch, sl.n_fetch, side)
                    ev_fetch[gi].record(side)

        def flush(transfer=True):
            if pending_sel[0] is not None:
                js = pending_sel[0]
                L.oasis_select_and_diff(h, *job_of(js), stream=cs)
                pending_sel[0] = None
                if transfer and pending[0] is not None:
                    ps_ = rt.state[pending[0]][0]
                    L.oasis_fetch_gather(h, ps_.host_tier, ps_.pool, ps_.fetch, ps_.n_fetch, cs)
                pending[0] = js if transfer else None
            if pending[0] is not None:
                ps_ = rt.state[pending[0]][0]
                L.oasis_fetch_gather(h, ps_.host_tier, ps_.pool, ps_.fetch, ps_.n_fetch, cs)
                pending[0] = None

        K = args.steps
        res = {}
        for transfer in (False, True):
            for i in range(args.warmup):
                step(i, transfer, first=(i == 0))
            flush(transfer)
            cs.wait_stream(side)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(K):
                step(i, transfer)
            flush(transfer)
            cs.wait_stream(side)
            torch.cuda.synchronize()
            res[transfer] = (time.perf_counter() - t0) / K * 1e6
        nf_tot.zero_()
        for i in range(K):  # untimed: pages fetched per step
            step(i, True, count=True)
        flush()
        cs.wait_stream(side)
        torch.cuda.synchronize()
        fetched = float(nf_tot.item()) * page / K
        # the gather alone, back to back on the side stream, over the last lists of every layer
        eb, ee = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eb.record(side)
        for _ in range(4):
            for l in range(nl):
                st = rt.state[l][0]
                L.oasis_fetch_gather(h, st.host_tier, st.pool, st.fetch, st.n_fetch, side)
        ee.record(side)
        torch.cuda.synchronize()
        g_us = eb.elapsed_time(ee) * 1e3 / 4
        last = sum(int(rt.state[l][0].n_fetch.sum()) for l in range(nl)) * page
        points.append({"eviction": policy, "cap": cap, "cap_frac_of_k": cap / kb, "layers_per_transfer": group,
                       "h1_us_per_step": res[False], "h2_us_per_step": res[True],
                       "exposed_transfer_us_per_step": res[True] - res[False],
                       "fetched_MB_per_step": fetched / 1e6, "gather_us_per_step": g_us,
                       "gather_GBs": last / (g_us * 1e-6) / 1e9 if g_us > 0 else None,
                       "h2_steps_per_s": cfg.batch * nl * 1e6 / res[True]})
        print(f"# {policy} cap {cap} group {group}: H1 {res[False]:.1f} us, H2 {res[True]:.1f} us, "
              f"{fetched / 1e6:.2f} MB/step", file=sys.stderr, flush=True)
        L.oasis_destroy(h)
    run.close()
    print(json.dumps({
        "metric": "cross-layer pipeline: exposed transfer per decode step vs fetch cap and eviction policy",
        "unit": "us per step (all layers, whole batch)",
        "config": {"workload": f"{cfg.name} shape, {nl} layers, batch {cfg.batch}, ctx {cfg.ctx}, k {kb} blocks",
                   "layers": nl, "steps": args.steps, "warmup": args.warmup},
        "data": "synthetic", "points": points,
        "note": "H1 = decode steps with inputs resident (no transfer); H2 = with every step's fetched pages "
                "moved: layers_per_transfer > 0: by the device-driven gather on a side stream, that many layers "
                "handing their gathers over as one batch behind one event, each batch's layers waiting at the "
                "next step for that batch only; 0: inline, each layer's gather carried by the next decode "
                "step's first launch on the compute stream (no second stream, no event); -1: carry, each "
                "layer's selection and diff carried by the next layer's first launch and its gather by the one "
                "after (H1 is then the carried step's own time); every (policy, cap, batch) run starts from "
                "the same state"}))


def recall_measure(args):
    """Prediction recall and corrective fetch on one layer.  At step t the drafts
    of step t-1 predicted S_pred(t) (the selection in place before step t's decode
    call); the verify query of step t selects S_exact(t) with the same bound and
    top-k rule.  Reports recall |S_pred & S_exact| / |S_exact| and the recall of
    S_exact's 20 highest-ranked blocks, the blocks of S_exact not resident after
    the prefetch (what a corrective fetch moves), and the step time of the chain
    without and with the blocking corrective fetch (each step's prefetch lands
    before the next step, as in a single-layer chain)."""
    import torch

    from lookahead_sparse_kv_draft_amd import _lib as L
    from lookahead_sparse_kv_draft_amd.synthetic import SyntheticRun
    from workload import CONFIGS

    cfg = CONFIGS[args.config]
    torch.cuda.set_device(0)
    run = SyntheticRun(cfg, overlap=False, replicas=2)
    run.prologue()
    rt = run.rt
    rt.state[0][1].copy_from(rt.state[0][0])  # the starting state of every pass
    cs = torch.cuda.current_stream()
    page = L.oasis_page_bytes(rt.h)
    steps = min(args.steps, cfg.steps)

    def chain(corrective, stats=None):
        st = rt.state[0][0]
        st.copy_from(rt.state[0][1])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(steps):
            q = run.q[0, t + 1]
            if stats is not None:
                rt.exact_select(0, q)
                pred = st.sel.cpu().numpy()
                exact = st.vsel.cpu().numpy()
                b2s = st.b2s.cpu().numpy()
                for u in range(pred.shape[0]):
                    P = {int(b) for b in pred[u] if b >= 0}
                    E = [int(b) for b in exact[u] if b >= 0]
                    stats["recall"].append(len(P & set(E)) / len(E))
                    stats["recall20"].append(len(P & set(E[:20])) / min(20, len(E)))
                    stats["missed"].append(sum(1 for b in E if b2s[u, b] < 0))
            if corrective:
                rt.corrective(0, q)
            L.oasis_decode_step(rt.h, q, st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.sel, st.b2s, st.s2b,
                                st.scores, rt.out, rt.ws_ptr, st.fetch, st.n_fetch, st.evict, st.attend,
                                st.n_attend, stream=cs)
            L.oasis_fetch_gather(rt.h, st.host_tier, st.pool, st.fetch, st.n_fetch, cs)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    chain(False)  # warm-up
    chain(True)
    t_pred = chain(False)
    t_corr = chain(True)
    stats = {"recall": [], "recall20": [], "missed": []}
    chain(True, stats)
    run.close()
    units = cfg.batch * cfg.kv_heads
    missed = np.array(stats["missed"], dtype=np.float64).reshape(steps, units)
    print(json.dumps({
        "metric": "prediction recall of the draft-predicted selection vs the verify query's selection; "
                  "corrective fetch cost",
        "config": {"workload": f"{cfg.name}: batch {cfg.batch}, 1 layer, ctx {cfg.ctx}, k {cfg.k} blocks, "
                               f"{cfg.n_draft} drafts, cap {cfg.fetch_cap}", "steps": steps},
        "data": "synthetic",
        "recall_at_k": {"mean": float(np.mean(stats["recall"])), "min": float(np.min(stats["recall"]))},
        "recall_top20": {"mean": float(np.mean(stats["recall20"])), "min": float(np.min(stats["recall20"]))},
        "corrective_pages_per_step": float(missed.sum(1).mean()),
        "corrective_MB_per_step": float(missed.sum(1).mean() * page / 1e6),
        "units_with_a_miss_frac": float((missed > 0).mean()),
        "step_us_prefetch_only": t_pred,
        "step_us_with_corrective_fetch": t_corr,
        "note": "single-layer chain, every transfer on the compute stream (nothing hides it); recall per "
                "(request, KV head) unit and step"}))


def main():
    args = parse()
    if args.recall:
        recall_measure(args)
        return
    if args.pipeline:
        pipeline_sweep(args)
        return
    if args.counter_summary:
        if len(args.counter_summary) < 2:
            raise SystemExit("--counter-summary needs at least one CSV and the output file")
        counter_summary(args.counter_summary[:-1], args.counter_summary[-1], " ".join(sys.argv))
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, cmdline=" ".join(sys.argv))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path shards by request or "
              f"KV head with no exchange, so N GPUs would run N independent copies of this benchmark.",
              file=sys.stderr)
        sys.exit(2)

    from workload import CONFIGS

    cfg = CONFIGS[args.config]
    if args.mode == "auto":
        args.mode = "carry" if cfg.layers > 1 else "eager"
    if args.mode == "carry" and cfg.layers < 2:
        raise SystemExit("--mode carry needs several layers: with one layer the next step's attention needs the "
                         "selection that would be carried")
    cpu = None
    if not args.no_cpu_baseline:
        # first, before anything initialises the GPU: the worker processes start clean
        print("# cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, args.cpu_seconds)

    import torch

    from lookahead_sparse_kv_draft_amd import _lib as L
    from lookahead_sparse_kv_draft_amd.synthetic import SyntheticRun

    torch.cuda.set_device(0)
    # per-layer HBM state (metadata + pool) and the replica count that defeats the MALL
    shape_meta = cfg.batch * cfg.kv_heads * cfg.max_blocks * 2 * cfg.head_dim * cfg.elem_bytes
    shape_pool = cfg.batch * cfg.kv_heads * cfg.k * 2 * 16 * cfg.head_dim * cfg.elem_bytes
    state_bytes = (shape_meta + shape_pool) * cfg.layers
    # every op on its own (the scoring reads only the metadata, the attention
    # only the pool) cycles through at least twice the Infinity Cache
    smallest = min(shape_meta, shape_pool) * cfg.layers
    replicas = args.replicas or min(64, max(1, math.ceil(2 * MALL_BYTES / smallest)))
    print(f"# config {cfg.name}: state {state_bytes / 2**20:.0f} MiB per replica, {replicas} replicas",
          file=sys.stderr, flush=True)

    launch_options = json.loads(args.launch_options) if args.launch_options else None
    run = SyntheticRun(cfg, replicas=replicas, overlap=args.mode == "overlap", options=launch_options)
    rt = run.rt
    run.prologue()
    for l in range(run.L):
        for rep in range(1, replicas):
            rt.state[l][rep].copy_from(rt.state[l][0])
    torch.cuda.synchronize()
    print("# prologue done", file=sys.stderr, flush=True)

    names = OPS
    # side stream (default priority) of the overlap and two-stream modes
    ps = rt.pstream if rt.pstream is not None else (torch.cuda.Stream() if args.mode.startswith("two_streams")
                                                    else None)
    ev_attn = [torch.cuda.Event() for _ in range(run.L)]
    ev_sel = [torch.cuda.Event() for _ in range(run.L)]

    def chain_step(i, cs, first):
        """One decode step over all layers with the real dependencies: the score
        runs beside the attention (it needs only the step's drafts), the fused
        selection/diff waits for the attention (it rewrites the selection and maps
        the attention reads), and the next step's attention of the layer waits
        for that selection."""
        rep = i % replicas
        t = i % cfg.steps
        for l in range(run.L):
            q = run.q[l, t + 1]
            st = rt.state[l][rep]
            if not first:
                cs.wait_event(ev_sel[l])
            L.oasis_sparse_paged_decode_attn(rt.h, q, st.pool, st.sel, st.b2s, rt.ctx_len, rt.out, rt.ws_ptr, cs)
            ev_attn[l].record(cs)
            append(l, t, st, ps)  # writes token n only, which the attention does not read
            L.oasis_lookahead_score(rt.h, q, st.meta, ctx_score, st.scores, ps)
            ps.wait_event(ev_attn[l])
            L.oasis_select_and_diff(rt.h, st.scores, ctx_score, st.sel, st.b2s, st.s2b, st.fetch, st.n_fetch,
                                    st.evict, st.attend, st.n_attend, stream=ps)
            ev_sel[l].record(ps)

    # Appending workloads: every step of every layer first appends one token per
    # request (oasis_block_meta_update at the current context length, written to
    # the other context buffer, which the step's scoring then sees).  The timed
    # loop does not advance the context, so each step appends at the same
    # position: the same work as a growing context.
    ctx_in, ctx_grown = rt.ctx[rt.ctx_cur], rt.ctx[1 - rt.ctx_cur]
    ctx_score = ctx_grown if cfg.append else ctx_in

    def append(l, t, st, cs):
        if cfg.append:
            L.oasis_block_meta_update(rt.h, run.k_new_dev[l, t], run.v_new_dev[l, t], ctx_in, ctx_grown, st.meta,
                                      st.pool, st.b2s, cs)

    def sequential_step(i, cs):
        """One decode step over all layers: the single decode-step call per layer
        (attention beside the scoring in one launch; selection, diff and the
        attention's split combine in the second; other shapes in three); with
        an append, the call that carries the layer's token append."""
        rep = i % replicas
        t = i % cfg.steps
        for l in range(run.L):
            q = run.q[l, t + 1]
            st = rt.state[l][rep]
            if cfg.append:
                L.oasis_decode_step_append(rt.h, q, st.pool, st.meta, ctx_in, ctx_grown, st.sel, st.b2s, st.s2b,
                                           st.scores, rt.out, rt.ws_ptr, st.fetch, st.n_fetch, st.evict,
                                           st.attend, st.n_attend, run.k_new_dev[l, t], run.v_new_dev[l, t], cs)
                continue
            L.oasis_decode_step(rt.h, q, st.pool, st.meta, rt.ctx_len, ctx_score, st.sel, st.b2s, st.s2b,
                                st.scores, rt.out, rt.ws_ptr, st.fetch, st.n_fetch, st.evict, st.attend,
                                st.n_attend, stream=cs)

    pending = [None]

    def carry_step(i, cs):
        """One decode step over all layers with each layer's selection and diff
        carried by the next call's first launch (the last layer's by the next
        step's first layer): per layer, one call of two launches, the second
        being the split combine alone."""
        rep = i % replicas
        t = i % cfg.steps
        for l in range(run.L):
            q = run.q[l, t + 1]
            st = rt.state[l][rep]
            append(l, t, st, cs)
            L.oasis_decode_step_carry(rt.h, q, st.pool, st.meta, rt.ctx_len, ctx_score, st.attend, st.n_attend,
                                      st.scores, rt.out, rt.ws_ptr, job=pending[0], stream=cs)
            pending[0] = (st.scores, ctx_score, st.sel, st.b2s, st.s2b, st.fetch, st.n_fetch, st.evict, st.attend,
                          st.n_attend)

    def carry_flush(cs):
        """The selection still pending after the last step, as a launch of its own."""
        if pending[0] is not None:
            j = pending[0]
            L.oasis_select_and_diff(rt.h, j[0], j[1], j[2], j[3], j[4], j[5], j[6], j[7], j[8], j[9], stream=cs)
            pending[0] = None

    ev_scored = torch.cuda.Event()
    ev_state = [[torch.cuda.Event() for _ in range(replicas)] for _ in range(run.L)]

    def two_stream_step(i, cs, first=False):
        """One decode step over all layers, the cross-layer pipeline: on the
        compute stream each layer's attention beside the scoring, then the
        attention's split combine (the layer's output, which the next layer
        needs); on the side stream, once the layer's first launch is done, its
        selection and diff, which only the same layer's next step reads. A
        state's next first launch waits for its previous selection."""
        rep = i % replicas
        t = i % cfg.steps
        for l in range(run.L):
            q = run.q[l, t + 1]
            st = rt.state[l][rep]
            if not first:
                cs.wait_event(ev_state[l][rep])
            append(l, t, st, cs)
            L.oasis_attend_and_score(rt.h, q, st.pool, st.meta, rt.ctx_len, ctx_score, st.sel, st.b2s, st.attend,
                                     st.n_attend, st.scores, rt.out, rt.ws_ptr, cs)
            ev_scored.record(cs)
            ps.wait_event(ev_scored)
            L.oasis_select_and_diff(rt.h, st.scores, ctx_score, st.sel, st.b2s, st.s2b, st.fetch, st.n_fetch,
                                    st.evict, st.attend, st.n_attend, stream=ps)
            ev_state[l][rep].record(ps)
            L.oasis_attn_combine(rt.h, rt.ws_ptr, rt.out, cs)

    cs0 = torch.cuda.current_stream()
    for i in range(args.warmup):
        if args.mode.startswith("two_streams"):
            two_stream_step(i, cs0)
        elif args.mode == "carry":
            carry_step(i, cs0)
        else:
            sequential_step(i, cs0)
    carry_flush(cs0)
    torch.cuda.synchronize()

    def attended():
        tot = 0
        for l in range(run.L):
            st = rt.state[l][0]
            sel = st.sel.long()
            valid = sel >= 0
            slots = torch.gather(st.b2s, 1, sel.clamp(min=0).to(torch.int64))
            tot += int(((slots >= 0) & valid).sum())
        return tot // run.L

    attended_before = attended()

    # Headline: G steps captured once as a HIP graph and replayed (or plain launches).
    G = 2 * replicas
    cs = torch.cuda.current_stream()
    graph = None
    if args.mode not in ("eager", "two_streams", "carry"):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            gs = torch.cuda.current_stream()
            if args.mode == "two_streams_graph":
                # a state's first use in the graph follows the previous replay's join
                ps.wait_stream(gs)
                for j in range(G):
                    two_stream_step(j, gs, first=(j < replicas))
                gs.wait_stream(ps)
            elif args.mode == "overlap":
                ps.wait_stream(gs)
                for j in range(G):
                    chain_step(j, gs, first=(j == 0))
                gs.wait_stream(ps)
            else:
                for j in range(G):
                    sequential_step(j, gs)
        for _ in range(max(1, args.warmup // G)):
            graph.replay()
        torch.cuda.synchronize()

    def eager_steps(n):
        for j in range(n):
            if args.mode == "overlap":
                ps.wait_stream(cs)
                chain_step(j, cs, first=(j == 0))
                cs.wait_stream(ps)
            elif args.mode.startswith("two_streams"):
                two_stream_step(j, cs)
            elif args.mode == "carry":
                carry_step(j, cs)
            else:
                sequential_step(j, cs)
        if args.mode == "carry":
            carry_flush(cs)  # every step's selection inside the timed region

    # Every event-timed region starts with a short spin kernel ahead of its begin
    # event: the GPU stays busy while the host enqueues the first calls, so the
    # events time K back-to-back calls and not the host's launch latency after a
    # synchronisation (which added 10-30 us to the first step).  The spin's
    # length is calibrated here, untimed, on a second spin (the first launch of
    # the spin kernel also loads its code, which made the calibrated lead a
    # quarter of its intended length).
    torch.cuda._sleep(1_000)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(cs0)
    torch.cuda._sleep(1_000_000)
    c1.record(cs0)
    torch.cuda.synchronize()
    lead_cycles = int(1_000_000 * LEAD_US / max(1.0, c0.elapsed_time(c1) * 1e3))

    def lead():
        torch.cuda._sleep(lead_cycles)

    # timed region 1 (headline): K steps = K // G graph replays + an eager remainder,
    # HIP events on the compute stream around the K steps (GPU time; the host's
    # wall clock around the same region is reported beside it)
    torch.cuda.synchronize()
    h_beg, h_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h_lead = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    h_lead.record(cs)
    lead()
    h_beg.record(cs)
    if graph is not None:
        for _ in range(args.steps // G):
            graph.replay()
        eager_steps(args.steps % G)
    else:
        eager_steps(args.steps)
    h_end.record(cs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    elapsed = h_beg.elapsed_time(h_end) * 1e-3
    lead_s = h_lead.elapsed_time(h_beg) * 1e-3  # the spin, as the GPU ran it

    # timed region 2: each op alone, K back-to-back calls over the replicas on
    # the compute stream, HIP events around the K calls (per-op durations for
    # the roofline; the op order inside a step does not matter for these)
    ops = {
        "attend_and_score": lambda st, q: L.oasis_attend_and_score(
            rt.h, q, st.pool, st.meta, rt.ctx_len, rt.ctx_len, st.sel, st.b2s, st.attend, st.n_attend, st.scores,
            rt.out, rt.ws_ptr, cs0),
        "select_diff_combine": lambda st, q: L.oasis_select_diff_combine(
            rt.h, st.scores, rt.ctx_len, st.sel, st.b2s, st.s2b, st.fetch, st.n_fetch, st.evict, st.attend,
            st.n_attend, rt.out, rt.ws_ptr, cs0),
        "sparse_paged_decode_attn": lambda st, q: L.oasis_sparse_paged_decode_attn_list(
            rt.h, q, st.pool, st.attend, st.n_attend, rt.ctx_len, rt.out, rt.ws_ptr, cs0),
        "lookahead_score": lambda st, q: L.oasis_lookahead_score(rt.h, q, st.meta, rt.ctx_len, st.scores, cs0),
        "select_and_diff": lambda st, q: L.oasis_select_and_diff(
            rt.h, st.scores, rt.ctx_len, st.sel, st.b2s, st.s2b, st.fetch, st.n_fetch, st.evict, st.attend,
            st.n_attend, stream=cs0),
    }
    avg = {}
    t1 = time.perf_counter()
    for n in names:
        e_beg, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for l in range(run.L):  # untimed first call: loads the op's code objects
            ops[n](rt.state[l][0], run.q[l, 1])
        torch.cuda.synchronize()
        lead()
        e_beg.record(cs0)
        for i in range(args.steps):
            for l in range(run.L):
                ops[n](rt.state[l][i % replicas], run.q[l, i % cfg.steps + 1])
        e_end.record(cs0)
        torch.cuda.synchronize()
        avg[n] = e_beg.elapsed_time(e_end) * 1e-3 / (args.steps * run.L)
    elapsed_ops = time.perf_counter() - t1
    # the whole per-layer step as one call, back to back over the replicas
    e_beg, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    lead()
    e_beg.record(cs0)
    for i in range(args.steps):
        sequential_step(i, cs0)
    e_end.record(cs0)
    torch.cuda.synchronize()
    step_call_us = e_beg.elapsed_time(e_end) * 1e3 / (args.steps * run.L)
    # the same with each layer's selection carried by the next call (several layers)
    carry_call_us = None
    if run.L > 1:
        torch.cuda.synchronize()
        lead()
        e_beg.record(cs0)
        for i in range(args.steps):
            carry_step(i, cs0)
        carry_flush(cs0)
        e_end.record(cs0)
        torch.cuda.synchronize()
        carry_call_us = e_beg.elapsed_time(e_end) * 1e3 / (args.steps * run.L)
    attended_after = attended()

    h2 = None if args.no_h2 else measure_h2(args, cfg, run, rt, replicas, sequential_step, step_call_us)

    # achievable-bandwidth reference on this machine: torch's device copy of 1 GiB
    # (1 GiB read + 1 GiB written), HIP events around 5 copies after a warm-up
    src = torch.empty(CALIB_ELEMS, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    eb, ee = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eb.record(cs0)
    for _ in range(5):
        dst.copy_(src)
    ee.record(cs0)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * CALIB_ELEMS * 4 / (eb.elapsed_time(ee) * 1e-3) / 1e9
    # launch 1 cold, after two kinds of 1 GiB sweep (each evicts the L2 and the
    # Infinity Cache): the device copy (1 GiB read and 1 GiB written, whose
    # written lines the launch's reads then push out to HBM) and a read-only sum;
    # HIP events around the launch alone
    def cold_after(flush, op="attend_and_score"):
        t = []
        for i in range(10):
            flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cs0)
            ops[op](rt.state[0][i % replicas], run.q[0, i % cfg.steps + 1])
            e1.record(cs0)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e3)
        return float(np.mean(t))

    cold_us = cold_after(lambda: dst.copy_(src))
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    read_flush = lambda: torch.sum(src, dim=(0,), out=sink)  # noqa: E731
    cold_clean_us = cold_after(read_flush)
    # every op cold after the read-only sweep (the selection ops read the
    # scores and maps the step left, the attention the attended list)
    cold_ops = {n: cold_after(read_flush, n) for n in names}
    del src, dst

    if args.calib_copy:
        # counter calibration: an elementwise add that reads 1 GiB and writes 1 GiB
        a = torch.ones(CALIB_ELEMS, dtype=torch.float32, device="cuda")
        for _ in range(3):
            b = a + 1.0
            del b
        torch.cuda.synchronize()
        del a

    steps_total = cfg.batch * run.L * args.steps
    value = steps_total / elapsed
    ab = algorithmic_bytes(cfg, attended_before)
    # the append per layer step: per unit the new K and V rows read, the block's
    # metadata row read and written, the K and V rows written into a resident page
    append_bytes = (cfg.batch * cfg.kv_heads * cfg.head_dim * cfg.elem_bytes * (2 + 4 + 2)) if cfg.append else 0
    kern = {}
    for n in names:
        gbs = ab[n] / avg[n] / 1e9
        kern[n] = {"avg_us": avg[n] * 1e6, "bytes": ab[n], "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                   "cold_us": cold_ops[n]}
    dominant = "attend_and_score"  # the step's first launch: attention beside the scoring, ~3/4 of the step
    traffic = load_traffic(cfg.name)
    for n in names:
        kern[n]["traffic_bytes"] = traffic.get(n)
    roof = {"bound": "hbm", "achieved": kern[dominant]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kern[dominant]["GB/s"] / HBM_PEAK_GBS, "traffic": traffic.get(dominant), "kernel": dominant,
            "kernels": OP_KERNELS[dominant],
            "bytes_per_launch": ab[dominant], "avg_launch_us": avg[dominant] * 1e6}
    res = {
        "metric": "predict+select+sparse-attn decode steps/s at 32K ctx; % of peak HBM GB/s",
        "value": value,
        "unit": "decode steps/s (request x layer)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: batch {cfg.batch}, {run.L} layer(s), {cfg.q_heads}q/{cfg.kv_heads}kv "
                               f"heads, d {cfg.head_dim}, ctx {cfg.ctx}, budget {cfg.budget_tokens} tokens, "
                               f"{cfg.n_draft} drafts + 1 verify, cap {cfg.fetch_cap}",
                   "batch": cfg.batch, "layers": run.L, "ctx": cfg.ctx, "replicas": replicas,
                   "attended_blocks": [attended_before, attended_after]},
        "roofline": roof,
        "kernels": kern,
        "launch_options": L.oasis_get_launch_options(rt.h),
        "step_mode": {"graph": f"HIP graph of {G} steps on one stream",
                      "overlap": f"HIP graph of {G} steps; scoring on a second stream beside the attention",
                      "eager": ("one oasis_decode_step_append call per layer on one stream (the token's "
                                "metadata row carried by the step's attention launch and its page row by the "
                                "scoring launch where the two run on their own)" if cfg.append else
                                "one decode-step call per layer (2 launches) on one stream"),
                      "carry": "one call per layer (2 launches) on one stream whose first launch carries the "
                               "previous layer's selection and diff (the last layer's in the next step's first "
                               "layer; the last step's run on its own) and whose second is the split combine",
                      "two_streams": "per layer: attention + scoring, then the split combine, on one stream; "
                                  "the selection and diff on a second stream beside the next layer",
                      "two_streams_graph": f"HIP graph of {G} steps of the two_streams mode"}[args.mode],
        "hbm_bytes_per_step": (ab["attend_and_score"] + ab["select_diff_combine"] + append_bytes) * run.L,
        "step_includes_append": bool(cfg.append),
        "decode_step_call_us": step_call_us,
        "decode_step_carry_call_us": carry_call_us,
        "headline_timing": {"clock": "HIP events on the compute stream around the K timed steps, after a "
                                     f"{LEAD_US:g} us spin kernel that keeps the GPU busy while the host enqueues "
                                     "the first steps",
                            # host wall clock around the region, less the lead spin
                            "lead_us": lead_s * 1e6,
                            "wall_ms_per_step": (wall - lead_s) / args.steps * 1e3,
                            "wall_steps_per_s": steps_total / (wall - lead_s)},
        "hbm_reference": {"kernel": "torch device copy, 1 GiB read + 1 GiB written", "GB/s": copy_gbs,
                          "frac": copy_gbs / HBM_PEAK_GBS},
        "attend_and_score_cold_us": {"after_1GiB_copy": cold_us, "after_1GiB_read": cold_clean_us},
        "h2": h2,
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    run.close()
    print(json.dumps(res))


if __name__ == "__main__":
    main()
