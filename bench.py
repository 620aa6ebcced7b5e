"""Benchmark: training steps of the sparse-embedding hot path on one MI355X.

A step = idmap_find_or_insert -> embedding_bag_fwd -> embedding_bag_bwd_update
over one batch, with inputs synthetic, seeded and resident in HBM before the
timed region starts.  The default run measures all five workloads and prints
ONE JSON line whose `value` is the click-log workload's lookups/s:

  1. multi-hot: 8 tables x batch 1024, bags U[1,8], dim 16 fp32, SGD, tables
     start empty (new ids inserted on first sight), G = 2 * pooled output;
  2. click-log (the headline): 26 one-hot tables x batch 65536, dim 128 fp32,
     cardinalities log-uniform in [10, 4e7], Zipf(1.1), Adagrad;
  3. behaviour sequence: 4 tables x batch 8192, bags U[1,100], mean pooling,
     dim 64 fp32, Adam, 1% never-seen ids in every step;
  4. billion-scale ID space: 2e8 live int64 keys at map load 0.7, batch
     131072 x 50 uniform lookups, dim 64 fp32, Adam (154 GB of rows);
  5. merged tables: 100 tables merged into one map keyed by (t << 56) | id,
     bf16 weights + fp32 Adagrad state, dim 32, batch 32768, bags Poisson(20).

Per workload: lookups/s and updated rows/s, the step's compulsory HBM bytes
per second against the 8 TB/s peak, the segmented-update kernel's roofline
(algorithmic bytes / its average launch time, timed live with HIP events on
its stream; HBM traffic from committed rocprofv3 counter summaries when they
were taken on the same kernel sources) and the CPU oracle timed on the host
on a bounded sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config N] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import gc
import glob
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
# 2^24 rows per chunk: the tables live in a few large allocations (16 GB per
# chunk for the click-log table's 1 KB rows).  Against 2^20-row chunks the
# click-log step measured 0.540 against 0.566 ms in alternating processes on
# one GPU; the other workloads did not change beyond the run-to-run spread.
CHUNK_LOG2 = 24
# map load of each workload's prepopulated key set (the billion-scale
# workload is defined at 0.7)
MAP_LOAD = {1: 0.5, 2: 0.5, 3: 0.5, 4: 0.7, 5: 0.5}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=0,
                   help="run only this workload (1-5); default: all five, value = workload 2")
    p.add_argument("--batches", type=int, default=4,
                   help="distinct batches cycled through (workloads whose ids are all live)")
    p.add_argument("--other-steps", type=int, default=10,
                   help="timed steps of workloads 1, 3, 4 and 5 in the default run")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--map-load", type=float, default=0.0, help="override the workload's map load")
    p.add_argument("--ceilings", action="store_true",
                   help="only measure plain reference kernels (torch's read, write, copy and row gathers) "
                        "that bound what the library's kernels can reach on this GPU")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of COPY_BYTES (an elementwise kernel that reads and "
                        "writes each byte once), to scale the FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


COPY_BYTES = 872_415_232


def copy_calibration():
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(10):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "dispatches": 10}))


def ceilings():
    """Bandwidth of plain kernels on this GPU (torch's own, one launch
    each, median of 10 after warm-up): a read-only reduction, a fill, a
    copy, and gathers of 512-byte rows (the click-log update's gradient
    rows) in random and in sorted order of a [65536 * 26, 128] fp32 array,
    1.7M rows gathered."""
    import torch

    dev = torch.device("cuda:0")
    n = 1 << 28                                            # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    rows = torch.randn(65536 * 26, 128, device=dev)
    g = torch.Generator(device=dev).manual_seed(3)
    idx = torch.randint(0, rows.shape[0], (1703936,), device=dev, generator=g)
    idx_sorted = torch.sort(idx).values
    out = torch.empty(idx.numel(), 128, device=dev)

    def timed(fn, nbytes):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        return {"ms": round(ms, 4), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}

    res = {
        "read (sum of 1 GiB)": timed(lambda: a.sum(), 4 * n),
        "write (fill of 1 GiB)": timed(lambda: b.fill_(2.0), 4 * n),
        "copy (neg, 1 GiB read + 1 GiB written)": timed(lambda: torch.neg(a, out=b), 8 * n),
        "gather 512 B rows, random order (872 MB read + written)":
            timed(lambda: torch.index_select(rows, 0, idx, out=out), 2 * out.numel() * 4),
        "gather 512 B rows, sorted order": timed(lambda: torch.index_select(rows, 0, idx_sorted, out=out),
                                                 2 * out.numel() * 4),
    }
    print(json.dumps({"ceilings": res, "peak_gbs": PEAK_HBM_GBS}))


def kernel_sources_sha() -> str:
    """Hash of the HIP sources and headers the library is built from: stored
    counter summaries apply only to the kernels they were taken on."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "recommender_sparse_embedding_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "rse.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def compulsory_bytes(cfg, L, U, n_new, row_bytes):
    """Bytes the step must move at least once: ids, bag offsets, one map slot
    per distinct key, read+write of every touched row (weights + state), the
    pooled output write and the upstream-gradient read, new-row init."""
    TB = cfg.n_tables * cfg.batch
    return (L * 8 + (TB + 1) * 8 + U * 16 + U * row_bytes * 2 + TB * cfg.dim * 4 * 2
            + n_new * row_bytes)


def logical_bytes(cfg, L, U, n_new, row_bytes):
    """Bytes the step moves with no reuse across lookups: the compulsory
    bytes plus, for every lookup beyond the first of its row, the forward's
    row-weight gather and one map slot."""
    import synth

    w_bytes = cfg.dim * (2 if cfg.wdtype == synth.BF16 else 4)
    return compulsory_bytes(cfg, L, U, n_new, row_bytes) + (L - U) * (w_bytes + 16)


def read_traffic(workload: int, sha: str):
    """HBM bytes per launch of the segmented update from the committed
    counter summary of this workload (profiles/seg_update_<name>.txt), or
    None if absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"seg_update_{PROFILE_NAME[workload]}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.split("#")[0].strip()
    if vals.get("kernel_sources_sha") != sha or "hbm_bytes_per_launch" not in vals:
        return None
    return int(float(vals["hbm_bytes_per_launch"]))


PROFILE_NAME = {1: "multihot", 2: "clicklog", 3: "sequence", 4: "billion", 5: "merged"}

_SIDE_STREAMS = {}


def side_streams(dev):
    """The two extra streams of the step schedules (default priority),
    created once per process: the runtime places each new stream on one of
    a few hardware queues, and streams made afresh for every workload can
    land on the queue of the main stream, whose work then runs one after
    the other (measured: the billion-scale lookahead step as slow as the
    serial one)."""
    import torch

    if dev not in _SIDE_STREAMS:
        _SIDE_STREAMS[dev] = (torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev))
    return _SIDE_STREAMS[dev]


def run_workload(n: int, args, full_schedules: bool, steps: int, warmup: int) -> dict:
    """Builds the workload's map and blocks, inserts every key, stages the
    batches on the device and times the step.  Returns the workload's
    result object; frees its device memory before returning."""
    import torch

    import recommender_sparse_embedding_amd as rse
    import synth

    dev = torch.device("cuda:0")
    cfg = synth.config(n)
    wl = synth.Workload(cfg)
    T, B, D = cfg.n_tables, cfg.batch, cfg.dim
    map_load = args.map_load or MAP_LOAD[n]
    t0 = time.time()
    # every step of a workload with never-seen ids (or whose tables start
    # empty) gets its own batch, so that every timed step inserts what the
    # workload says it inserts; the others cycle a few batches
    distinct = cfg.fresh_frac > 0 or not cfg.prepopulate
    n_ref = max(2, steps // 2)
    n_warm_sched = 4 if full_schedules else 2
    n_ref_sched = 3 if full_schedules else 1
    # batches the run finds: warmup runs of every schedule (each primed up
    # to two batches ahead), the two lookahead calibration runs, the timed
    # run (two ahead), the traced run and the other lookahead (two ahead),
    # the other reference runs (one ahead)
    n_cal = max(3, warmup)
    n_finds = ((n_warm_sched + 1) * (warmup + 2) + 2 * (n_cal + 2) + steps + 2
               + n_ref_sched * (n_ref + 1) + 2 * (n_ref + 2) + 4)
    n_batches = n_finds if distinct else max(3, args.batches)

    # ---------------------------------------------------------- setup ----
    total_keys = int(wl.card.sum())
    max_bag = {"fixed": cfg.bag[1], "uniform": cfg.bag[-1], "poisson": 3 * cfg.bag[1]}[cfg.bag[0]]
    if not cfg.prepopulate:
        headroom = total_keys
    else:
        headroom = int(cfg.fresh_frac * cfg.n_bags * max_bag * n_finds * 1.1)
    if cfg.merged:
        slots = [int((total_keys + headroom) / map_load) + 1024]
    else:
        per_table = headroom // T if cfg.prepopulate else 0
        slots = [int((int(c) + per_table) / map_load) + 1024 for c in wl.card]
    idm = rse.IdMap(slots, max_load=0.9, merged=cfg.merged, hash_seed=12345, device=dev)
    blk = rse.EmbeddingBlocks(D, cfg.wdtype, cfg.optim, CHUNK_LOG2, max_chunks=4096, seed=cfg.seed, device=dev)
    blk.grow(-(-((total_keys if cfg.prepopulate else 0) + headroom + (1 << CHUNK_LOG2)) // (1 << CHUNK_LOG2)))
    opt = rse.Optim(cfg.optim, cfg.lr, cfg.eps, cfg.beta1, cfg.beta2)
    n_new = torch.zeros(1, dtype=torch.int64, device=dev)
    pre_ws = idm.workspace(1 << 24)
    for ids, bounds in wl.prepopulation(chunk=1 << 24):
        t_ids = torch.from_numpy(ids).to(dev)
        ro = torch.empty_like(t_ids)
        rse.idmap_find_or_insert(idm, blk, t_ids, torch.from_numpy(bounds).to(dev), 1, T, ro, n_new, ws=pre_ws)
    torch.cuda.synchronize()
    del pre_ws
    used0, st = blk.status()
    assert st == 0 and used0 == (total_keys if cfg.prepopulate else 0), (used0, st)
    log(f"[{n}] prepopulated {used0} keys in {time.time() - t0:.1f}s")

    batches = []
    for k in range(n_batches):
        ids, bo = wl.batch_inputs(k)
        g = torch.from_numpy(wl.grad(k)).to(dev) if (cfg.grad == "normal" and k < max(3, args.batches)) else None
        batches.append(dict(ids=torch.from_numpy(ids).to(dev), bo=torch.from_numpy(bo).to(dev), grad=g,
                            L=len(ids), ro=torch.empty(len(ids), dtype=torch.int64, device=dev),
                            nu=torch.zeros(1, dtype=torch.int64, device=dev),
                            nn=torch.zeros(1, dtype=torch.int64, device=dev)))
    if cfg.grad == "normal" and distinct:      # gradients cycle; the lookups do not
        for k, b in enumerate(batches):
            b["grad"] = batches[k % max(3, args.batches)]["grad"]
    L_max = max(b["L"] for b in batches)
    find_ws = idm.workspace(L_max)
    ws2 = [rse.bwd_workspace(L_max, T, B, D, dev), rse.bwd_workspace(L_max, T, B, D, dev)]
    out = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    log(f"[{n}] staged {len(batches)} batches ({L_max} lookups max), setup {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()
    # second stream (default priority) for work that does not wait for the
    # previous phase: the backward's sort, and the next batch's find
    side, finder = side_streams(dev)
    step_no = [0]

    def batch_at(k):
        return batches[k % len(batches)]

    def grad_of(b):
        return b["grad"] if b["grad"] is not None else 2.0 * out

    def find(b, s=None):
        rse.idmap_find_or_insert(idm, blk, b["ids"], b["bo"], B, T, b["ro"], b["nn"], ws=find_ws, stream=s)

    def step_serial(i):
        b = batch_at(i)
        find(b)
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        step_no[0] += 1
        rse.embedding_bag_bwd_update(blk, b["ro"], b["bo"], T, B, cfg.pooling, grad_of(b), opt, step_no[0],
                                     b["nu"], ws=ws2[0])

    def step_overlap(i, ev=None):
        """find; then the forward (stream 1) and the backward's sort (stream
        2) together; then the apply."""
        b = batch_at(i)
        if ev:
            ev[0].record(stream)
        find(b)
        if ev:
            ev[1].record(stream)
        found_ = torch.cuda.Event()
        found_.record(stream)
        side.wait_event(found_)
        plan = rse.embedding_bag_bwd_prepare(blk, b["ro"], b["bo"], T, B, ws2[0], stream=side)
        srt = torch.cuda.Event()
        srt.record(side)
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        if ev:
            ev[2].record(stream)
        g = grad_of(b)
        step_no[0] += 1
        stream.wait_event(srt)
        rse.embedding_bag_bwd_apply(blk, plan, b["bo"], T, B, cfg.pooling, g, opt, step_no[0], b["nu"], ws2[0])
        if ev:
            ev[3].record(stream)

    # Pipelined: the find and sort of batch i+1 (stream 2) run while batch
    # i's forward and apply run (stream 1).  The find of batch i+1 touches
    # only the map, rows it creates and its own outputs, none of which batch
    # i's apply reads or writes; the forward of batch i+1 waits for both.
    # Sort workspaces alternate; a sort waits for the apply that last used
    # its workspace.
    applied = [torch.cuda.Event(), torch.cuda.Event()]
    fronted = [torch.cuda.Event(), torch.cuda.Event()]
    plans = [None, None]

    def front(i):
        b = batch_at(i)
        side.wait_event(applied[i % 2])
        find(b, side)
        plans[i % 2] = rse.embedding_bag_bwd_prepare(blk, b["ro"], b["bo"], T, B, ws2[i % 2], stream=side)
        fronted[i % 2].record(side)

    def back(i):
        b = batch_at(i)
        stream.wait_event(fronted[i % 2])
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        g = grad_of(b)
        step_no[0] += 1
        rse.embedding_bag_bwd_apply(blk, plans[i % 2], b["bo"], T, B, cfg.pooling, g, opt, step_no[0], b["nu"],
                                    ws2[i % 2])
        applied[i % 2].record(stream)

    # Lookahead (the value): stream 2 runs one more batch ahead.  While
    # stream 1 runs batch i's forward and apply, stream 2 sorts batch i+1
    # (found during the previous step) and then finds batch i+2.  The find
    # of i+2 writes only the map, rows it creates and batch i+2's offsets (a
    # buffer last read by the forward of batch i-2 when at least three
    # batches cycle); finds still run in batch order, so every result is
    # that of the plain order.
    ready = [torch.cuda.Event() for _ in range(3)]        # find of batch k done: ready[k % 3]
    prepared = [torch.cuda.Event(), torch.cuda.Event()]   # prepare of batch k done: prepared[k % 2]

    def la_find(k):
        find(batch_at(k), side)
        ready[k % 3].record(side)

    def la_prepare(k):
        side.wait_event(applied[k % 2])               # the apply that last used this workspace
        b = batch_at(k)
        plans[k % 2] = rse.embedding_bag_bwd_prepare(blk, b["ro"], b["bo"], T, B, ws2[k % 2], stream=side)
        prepared[k % 2].record(side)

    # Lookahead over three streams: the finds move to a third stream, so the
    # find chain of batch i+2 and the sort chain of batch i+1 (both made of
    # short dependent kernels) run side by side instead of one after the
    # other.  Finds still run in batch order (one stream); a prepare waits
    # for its batch's find; the find of batch i+2 waits for the apply of
    # batch i-1, as in the two-stream schedule (there through the sort that
    # precedes it): the offsets buffer it overwrites was last read by the
    # forward and the sort of batch i+2-nb (nb >= 3 batches cycle), both
    # done before that apply.  This also bounds how far the finds run ahead.

    def la3_find(k):
        finder.wait_event(applied[(k - 1) % 2])       # the apply of batch k-3 (recorded at step k-3)
        find(batch_at(k), finder)
        ready[k % 3].record(finder)

    def la3_prepare(k):
        side.wait_event(applied[k % 2])
        side.wait_event(ready[k % 3])
        b = batch_at(k)
        plans[k % 2] = rse.embedding_bag_bwd_prepare(blk, b["ro"], b["bo"], T, B, ws2[k % 2], stream=side)
        prepared[k % 2].record(side)

    def la3_step(i):
        la3_find(i + 2)
        la3_prepare(i + 1)
        b = batch_at(i)
        stream.wait_event(ready[i % 3])
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        g = grad_of(b)
        step_no[0] += 1
        stream.wait_event(prepared[i % 2])
        rse.embedding_bag_bwd_apply(blk, plans[i % 2], b["bo"], T, B, cfg.pooling, g, opt, step_no[0], b["nu"],
                                    ws2[i % 2])
        applied[i % 2].record(stream)

    def la_step(i):
        la_prepare(i + 1)
        la_find(i + 2)
        b = batch_at(i)
        stream.wait_event(ready[i % 3])
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        g = grad_of(b)
        step_no[0] += 1
        stream.wait_event(prepared[i % 2])
        rse.embedding_bag_bwd_apply(blk, plans[i % 2], b["bo"], T, B, cfg.pooling, g, opt, step_no[0], b["nu"],
                                    ws2[i % 2])
        applied[i % 2].record(stream)

    host_ms = {}
    cursor = [0]       # next batch index: every batch is found exactly once per pass over them

    def timed(schedule, n_steps, evs=None):
        """n_steps steps starting at the next unused batch, timed between
        events on stream 1 (every stream's work inside is waited for);
        returns (ms, first batch index)."""
        first = cursor[0]
        torch.cuda.synchronize()
        if schedule == "pipelined":
            front(first)
        if schedule == "lookahead":
            la_find(first)
            la_prepare(first)
            la_find(first + 1)
        if schedule == "lookahead3":
            la3_find(first)
            la3_prepare(first)
            la3_find(first + 1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        h0 = time.perf_counter()
        for k in range(n_steps):
            i = first + k
            if schedule == "serial":
                step_serial(i)
            elif schedule == "overlap":
                step_overlap(i, evs[k] if evs else None)
            elif schedule == "lookahead":
                la_step(i)
            elif schedule == "lookahead3":
                la3_step(i)
            else:
                front(i + 1)          # the next batch: one find + sort per step
                back(i)
        if schedule == "pipelined":
            stream.wait_event(fronted[(first + n_steps) % 2])
        if schedule in ("lookahead", "lookahead3"):
            stream.wait_event(prepared[(first + n_steps) % 2])
            stream.wait_event(ready[(first + n_steps + 1) % 3])
        e1.record(stream)
        host_ms[schedule] = (time.perf_counter() - h0) * 1e3 / max(n_steps, 1)
        torch.cuda.synchronize()
        # batches found ahead by the two-stream schedules are skipped: the
        # next run starts at a batch nobody has found yet
        cursor[0] = first + n_steps + (2 if schedule in ("lookahead", "lookahead3") else
                                       1 if schedule == "pipelined" else 0)
        return e0.elapsed_time(e1), first

    others = ("serial", "overlap", "pipelined") if full_schedules else ("serial",)
    for name in others + ("lookahead", "lookahead3"):
        timed(name, warmup)
    idm_st, _ = idm.status()
    _, st = blk.status()
    assert idm_st == 0 and st == 0, (idm_st, st)

    # The step's schedule: two streams, or three (finds beside the sorts)
    # where that is clearly faster, from one run of each after the warm-up;
    # the timed region then runs that schedule only.
    cal = {name: timed(name, n_cal)[0] for name in ("lookahead", "lookahead3")}
    sched = "lookahead3" if cal["lookahead3"] < 0.97 * cal["lookahead"] else "lookahead"
    other = "lookahead" if sched == "lookahead3" else "lookahead3"

    # ----------------------------------------------------- timed region --
    ms_total, first = timed(sched, steps)
    ms_step = ms_total / steps
    sel = [batch_at(first + k) for k in range(steps)]
    L_sel = [b["L"] for b in sel]
    U_sel = [int(b["nu"].item()) for b in sel]          # distinct rows each step updated
    new_rows = float(np.mean([int(b["nn"].item()) for b in sel]))   # rows each step's find inserted

    ms_by = {sched: round(ms_step, 4)}
    # The segmented-update kernel's launch time, from a second lookahead run
    # in which the library brackets every launch of that kernel with HIP
    # events on its stream (timing events add work to the stream, so the
    # headline run above goes without them)
    rse.trace_start(rse.K_SEG_UPDATE)
    ms_traced, first_tr = timed(sched, n_ref)
    n_seg, seg_ms = rse.trace_stop()
    t_seg = seg_ms / max(n_seg, 1)
    ms_by[sched + "_traced"] = round(ms_traced / n_ref, 4)
    sel_tr = [batch_at(first_tr + k) for k in range(n_ref)]
    phase = None
    rse.trace_start(rse.K_FWD)
    ms_by["serial"] = round(timed("serial", n_ref)[0] / n_ref, 4)
    if full_schedules:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_ref)]
        ms_by["overlap"] = round(timed("overlap", n_ref, evs)[0] / n_ref, 4)
        phase = {k: round(float(np.mean([e[a].elapsed_time(e[a + 1]) for e in evs])), 4)
                 for a, k in enumerate(("find", "fwd", "bwd_update"))}
        ms_by["pipelined"] = round(timed("pipelined", n_ref)[0] / n_ref, 4)
    n_fwd, fwd_ms = rse.trace_stop()
    fwd_ms_kernel = fwd_ms / max(n_fwd, 1)
    # the other lookahead, outside the forward's traced runs (as before it was added)
    ms_by[other] = round(timed(other, n_ref)[0] / n_ref, 4)
    idm_st, _ = idm.status()
    live_rows, st = blk.status()
    assert idm_st == 0 and st == 0, (idm_st, st)

    rb = blk.row_bytes
    L_avg, U_avg = float(np.mean(L_sel)), float(np.mean(U_sel))
    comp = float(np.mean([compulsory_bytes(cfg, L, U, new_rows, rb) for L, U in zip(L_sel, U_sel)]))
    logical = float(np.mean([logical_bytes(cfg, L, U, new_rows, rb) for L, U in zip(L_sel, U_sel)]))
    step_gbs = comp / (ms_step * 1e-3) / 1e9
    # roofline of the segmented-update kernel: algorithmic bytes per launch =
    # sorted (row, gradient-row) pairs read (8 B per lookup) + one gradient
    # row per lookup (dim * 4 B) + each touched row (weights + state) read
    # and written once
    L_tr = [b["L"] for b in sel_tr]
    U_tr = [int(b["nu"].item()) for b in sel_tr]
    seg_bytes = float(np.mean([L * 8 + L * D * 4 + U * rb * 2 for L, U in zip(L_tr, U_tr)]))
    # the same kernel by compulsory bytes: each bag's gradient row read once
    seg_comp = float(np.mean([L * 8 + T * B * D * 4 + U * rb * 2 for L, U in zip(L_tr, U_tr)]))
    seg_gbs = seg_bytes / (t_seg * 1e-3) / 1e9
    TB = T * B
    w_bytes = D * (2 if cfg.wdtype == synth.BF16 else 4)
    fwd_bytes = float(np.mean([L * 8 + (TB + 1) * 8 + U * w_bytes + TB * D * 4 for L, U in zip(L_sel, U_sel)]))
    sha = kernel_sources_sha()
    roofline = {"bound": "hbm", "kernel": f"k_seg_work<{D},{'bf16' if cfg.wdtype else 'f32'}>",
                "achieved": round(seg_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(seg_gbs / PEAK_HBM_GBS, 4), "traffic": read_traffic(n, sha),
                "algorithmic_bytes_per_launch": int(seg_bytes), "avg_launch_ms": round(t_seg, 4),
                "launches_timed": n_seg,
                "compulsory_bytes_per_launch": int(seg_comp),
                "compulsory_frac": round(seg_comp / (t_seg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    fwd_roof = {"kernel": "embedding_bag_fwd", "achieved": round(fwd_bytes / (fwd_ms_kernel * 1e-3) / 1e9, 1),
                "unit": "GB/s", "algorithmic_bytes_per_launch": int(fwd_bytes),
                "avg_launch_ms": round(float(fwd_ms_kernel), 4), "launches_timed": n_fwd}
    res = {
        "workload": f"{cfg.name}: {T} tables x batch {B}, dim {D}, {live_rows} live rows, map load {map_load}",
        "lookups_per_s": round(L_avg / (ms_step * 1e-3), 1),
        "updated_rows_per_s": round(U_avg / (ms_step * 1e-3), 1),
        "ms_per_step": round(ms_step, 4),
        "steps": steps, "warmup": warmup,
        "lookups_per_step": L_avg, "unique_rows_per_step": U_avg, "new_rows_per_step": round(new_rows, 1),
        "live_rows": live_rows, "map_load": map_load,
        "step_compulsory_bytes": int(comp),
        "step_hbm_gbs": round(step_gbs, 1),
        "step_frac_of_peak": round(step_gbs / PEAK_HBM_GBS, 4),
        "step_logical_bytes": int(logical),
        "step_logical_gbs": round(logical / (ms_step * 1e-3) / 1e9, 1),
        "schedule": sched,
        "schedule_calibration_ms": {k: round(v / n_cal, 4) for k, v in cal.items()},
        "ms_per_step_by_schedule": ms_by,
        "host_enqueue_ms_per_step": {k: round(v, 4) for k, v in host_ms.items()},
        "roofline": roofline,
        "fwd_roofline": fwd_roof,
        "kernel_sources_sha": sha,
        "setup_s": round(time.time() - t0, 1),
    }
    if phase:
        res["overlap_phase_ms"] = phase
    if full_schedules:
        res["interaction"] = bench_interaction(rse, out, steps)
        res["feature_transform"] = bench_features(rse, T, B, dev, steps)
    res["rehash"] = bench_rehash(rse, idm, blk, lambda: find(batch_at(cursor[0])), dev)
    # release the workload's device memory before the next one
    del batches, find_ws, ws2, out, idm, blk
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def bench_features(rse, T, B, dev, steps):
    """The fused feature transform at the workload's shape (T tables x B
    lookups): tables cycle through hash-then-mod of int64 ids, bucketize of
    float64 values over 1000 boundaries, mod of raw ids and a hashed float,
    all in one launch; average of `steps` launches timed with events on the
    stream the kernel runs on.  Algorithmic bytes per launch: 8 B raw value
    read and 8 B id written per lookup."""
    import torch

    rng = np.random.default_rng(7)
    progs, cols = [], []
    for t in range(T):
        k = t % 4
        if k == 0:
            progs.append((rse.FT_INT64, [(rse.FT_HASH, 1000 + t), (rse.FT_MOD, 1 << 24)]))
            cols.append(rng.integers(-(2**63), 2**63 - 1, B, dtype=np.int64))
        elif k == 1:
            progs.append((rse.FT_FLOAT64, [(rse.FT_BUCKETIZE, np.sort(rng.standard_normal(1000) * 3))]))
            cols.append((rng.standard_normal(B) * 3).view(np.int64))
        elif k == 2:
            progs.append((rse.FT_INT64, [(rse.FT_MOD, 1_000_003)]))
            cols.append(rng.integers(-(2**62), 2**62, B, dtype=np.int64))
        else:
            progs.append((rse.FT_FLOAT64, [(rse.FT_HASH, 5), (rse.FT_MOD, 1 << 20)]))
            cols.append(rng.standard_normal(B).view(np.int64))
    ft = rse.FeatureTransform(progs, device=dev)
    raw = torch.from_numpy(np.concatenate(cols)).to(dev)
    bounds = torch.arange(0, (T + 1) * B, B, dtype=torch.int64, device=dev)
    ids = torch.empty_like(raw)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        rse.feature_transform(ft, raw, bounds, out=ids)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        rse.feature_transform(ft, raw, bounds, out=ids)
    e1.record(stream)
    torch.cuda.synchronize()
    assert ft.status() == 0
    ms = e0.elapsed_time(e1) / steps
    nbytes = T * B * 16
    n_ops = sum(len(ops) for _, ops in progs)
    return {"lookups": T * B, "tables": T, "operations": n_ops, "launches": 1, "ms": round(ms, 4),
            "ids_per_s": round(T * B / (ms * 1e-3), 1), "algorithmic_bytes": nbytes,
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def bench_rehash(rse, idm, blk, find_next, dev):
    """The map's rehash at the workload's full size, into a second region of
    the same size: a resize (every key copied) and an eviction (age tracking
    on, one batch found at clock 1; the rehash with minimum clock 1 keeps that
    batch's keys, drops the rest and rebuilds the free list).  Each is the
    average of 3 launches after one warm-up launch, timed with events on the
    stream the kernels run on.  Algorithmic bytes: source slots read and
    destination slots cleared (16 B each), kept keys written (16 B), one bit
    per row of bitmap cleared and read twice, plus for the eviction one
    4-byte stamp per live key and one 4-byte free-list entry per freed row."""
    import torch

    stream = torch.cuda.current_stream()
    S = sum(-(-s // 8) * 8 for s in idm.slots_per_table) + idm.n_tables
    cap = blk.capacity
    live = sum(idm.status()[1])
    dst = rse.IdMap(idm.slots_per_table, idm.max_load, idm.merged, idm.hash_seed + 1, dev)

    def run(min_clock, reps=3):
        idm.rehash_into(dst, blk, min_clock)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            idm.rehash_into(dst, blk, min_clock)
        e1.record(stream)
        torch.cuda.synchronize()
        st, kept = dst.status()
        assert st == 0, st
        return e0.elapsed_time(e1) / reps, sum(kept)

    ms_r, kept_r = run(0)
    assert kept_r == live
    bytes_r = 16 * (2 * S + live) + 3 * cap // 8
    idm.track_age(cap)
    blk.enable_free_list()
    idm.set_clock(1)
    find_next()
    ms_e, kept_e = run(1)
    head, free = blk.free_list()
    n_free = int(free.numel())
    bytes_e = 16 * (2 * S + kept_e) + 4 * live + 3 * cap // 8 + 4 * n_free
    out = {"slots": S, "live_keys": live, "rows_capacity": cap,
           "resize_ms": round(ms_r, 4), "resize_gbs": round(bytes_r / (ms_r * 1e-3) / 1e9, 1),
           "resize_frac_of_peak": round(bytes_r / (ms_r * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "evict_ms": round(ms_e, 4), "evict_kept_keys": kept_e, "evict_freed_rows": n_free,
           "evict_gbs": round(bytes_e / (ms_e * 1e-3) / 1e9, 1),
           "evict_frac_of_peak": round(bytes_e / (ms_e * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "resize_algorithmic_bytes": int(bytes_r), "evict_algorithmic_bytes": int(bytes_e)}
    log(f"  rehash: resize {ms_r:.3f} ms ({out['resize_gbs']} GB/s), evict {ms_e:.3f} ms "
        f"({out['evict_gbs']} GB/s), kept {kept_e} of {live}, freed {n_free}")
    del dst
    return out


def bench_interaction(rse, pooled, steps):
    """The DLRM dot interaction on the workload's pooled output [B, T, d]
    (plus a dense vector [B, d]): forward and backward, timed with HIP events
    on the stream they run on, with their algorithmic bytes (every input read
    once, every output written once) and fp64 multiply-adds."""
    import torch

    B, T, D = pooled.shape
    F, P = T + 1, (T + 1) * T // 2
    dense = torch.randn((B, D), device=pooled.device)
    dout = torch.randn((B, D + P), device=pooled.device)
    out = torch.empty((B, D + P), device=pooled.device)
    for _ in range(2):
        rse.dlrm_interaction_fwd(dense, pooled, out)
        rse.dlrm_interaction_bwd(dense, pooled, dout)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(steps):
        rse.dlrm_interaction_fwd(dense, pooled, out)
    ev[1].record(stream)
    for _ in range(steps):
        rse.dlrm_interaction_bwd(dense, pooled, dout)
    ev[2].record(stream)
    torch.cuda.synchronize()
    t_f = ev[0].elapsed_time(ev[1]) / steps
    t_b = ev[1].elapsed_time(ev[2]) / steps
    fwd_bytes = B * F * D * 4 + B * (D + P) * 4
    bwd_bytes = B * F * D * 4 + B * (D + P) * 4 + B * F * D * 4
    return {"shape": f"batch {B}, {T} tables + dense, dim {D}: out [B, {D + P}]",
            "fwd_ms": round(t_f, 4), "bwd_ms": round(t_b, 4),
            "fwd_gbs": round(fwd_bytes / (t_f * 1e-3) / 1e9, 1), "bwd_gbs": round(bwd_bytes / (t_b * 1e-3) / 1e9, 1),
            "fwd_frac_of_hbm_peak": round(fwd_bytes / (t_f * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bwd_frac_of_hbm_peak": round(bwd_bytes / (t_b * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "fwd_fp64_tflops": round(2 * B * P * D / (t_f * 1e-3) / 1e12, 2),
            "bwd_fp64_tflops": round(2 * B * F * F * D / (t_b * 1e-3) / 1e12, 2)}


# ------------------------------------------------------- CPU baseline ------
# The oracle (plain single-threaded C++) on a bounded sample of each
# workload, a few seconds to a few tens of seconds each.
CPU_SAMPLE = {
    1: dict(overrides={}, steps=10, what="all 10 steps of the workload, tables starting empty"),
    2: dict(overrides={}, steps=2, what="2 full steps after inserting all {keys} keys"),
    3: dict(overrides={"cardinality": ("fixed", 500_000)}, steps=2,
            what="2 full-batch steps on a twin with 5e5 keys per table ({keys} keys)"),
    4: dict(overrides={"cardinality": ("fixed", 2_000_000), "batch": 16384}, steps=1,
            what="1 step of 16384 bags x 50 on a twin with 2e6 live keys"),
    5: dict(overrides={"cardinality": ("fixed", 100_000), "batch": 4096}, steps=1,
            what="1 step of 4096 x 100 bags (Poisson(20)) on a twin with 1e5 keys per table ({keys} keys)"),
}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(n: int) -> dict:
    """The oracle on the workload's bounded sample: keys inserted (untimed),
    then whole steps (find + forward + backward with update) timed; lookups
    and updated rows per second."""
    import oracle
    import synth

    spec = CPU_SAMPLE[n]
    cfg = synth.config(n, **spec["overrides"])
    wl = synth.Workload(cfg)
    t0 = time.time()
    orc = oracle.OracleTable(cfg.dim, cfg.wdtype, cfg.optim, cfg.n_tables, cfg.merged, seed=cfg.seed,
                             lr=cfg.lr, eps=cfg.eps, beta1=cfg.beta1, beta2=cfg.beta2)
    for ids, bounds in wl.prepopulation(chunk=1 << 24):
        orc.find_or_insert(ids, bounds, 1)
    prep = time.time() - t0
    tot_L, tot_U, tot_t = 0, 0, 0.0
    for k in range(spec["steps"]):
        ids, bo = wl.batch_inputs(k)
        g = wl.grad(k) if cfg.grad == "normal" else None
        s = time.perf_counter()
        ro, _ = orc.find_or_insert(ids, bo, cfg.batch)
        out = orc.fwd(ro, bo, cfg.batch, cfg.pooling)
        if g is None:
            g = (2.0 * out).astype(np.float32)
        tot_U += orc.bwd_update(ro, bo, cfg.batch, g, cfg.pooling)
        tot_t += time.perf_counter() - s
        tot_L += len(ids)
    del orc
    return {"value": round(tot_L / tot_t, 1), "unit": "lookups/s", "cores": 1, "kind": "oracle",
            "updated_rows_per_s": round(tot_U / tot_t, 1),
            "sample": spec["what"].format(keys=int(wl.card.sum())) + f": {tot_L} lookups in {tot_t:.2f}s timed "
                      f"(key insertion {prep:.1f}s, untimed)",
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.ceilings:
        ceilings()
        return
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    headline = args.config or 2
    order = [headline] if args.config else [2, 1, 3, 4, 5]
    results = {}
    w0 = time.time()
    for n in order:
        t = time.time()
        is_head = n == headline
        steps = args.steps if is_head else min(args.steps, args.other_steps)
        try:
            results[n] = run_workload(n, args, full_schedules=is_head, steps=steps, warmup=args.warmup)
        except Exception as e:      # one workload failing must not hide the others
            if is_head:
                raise
            results[n] = {"error": f"{type(e).__name__}: {e}"}
            gc.collect()
            torch.cuda.empty_cache()
        log(f"[{n}] done in {time.time() - t:.1f}s: "
            f"{results[n].get('ms_per_step')} ms/step, {results[n].get('lookups_per_s')} lookups/s")
    if not args.no_cpu_baseline:
        for n in order:
            t = time.time()
            results[n]["cpu_baseline"] = cpu_baseline(n)
            log(f"[{n}] oracle baseline in {time.time() - t:.1f}s: {results[n]['cpu_baseline']['value']} lookups/s")

    h = results[headline]
    cfg_keys = {k: h[k] for k in ("lookups_per_step", "unique_rows_per_step", "live_rows", "map_load")}
    res = {
        "metric": "embedding lookups/sec (fwd+bwd+update), 1 MI355X",
        "value": h["lookups_per_s"],
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": h["warmup"],
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 storage, f64 accumulate" if headline != 5 else "bf16 storage, f64 accumulate",
        "data": "synthetic (seeded Zipf or uniform lookups over random 63/64/56-bit keys, N(0,1) grads)",
        "config": {"workload": h["workload"], **cfg_keys},
        "updated_rows_per_s": h["updated_rows_per_s"],
        "step_compulsory_bytes": h["step_compulsory_bytes"],
        "step_hbm_gbs": h["step_hbm_gbs"],
        "step_frac_of_peak": h["step_frac_of_peak"],
        "roofline": h["roofline"],
        "cpu_baseline": h.get("cpu_baseline"),
        "schedule": ("fwd + bwd apply of batch i (stream 1) || bwd prepare of batch i+1, then find of batch i+2 "
                     "(stream 2)" if h["schedule"] == "lookahead" else
                     "fwd + bwd apply of batch i (stream 1) || bwd prepare of batch i+1 (stream 2) || find of batch "
                     "i+2 (stream 3)"),
        "workloads": {str(k): v for k, v in results.items()},
        "wall_s": round(time.time() - w0, 1),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
