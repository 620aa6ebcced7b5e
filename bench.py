"""Benchmark: one training step of the sparse-embedding hot path on one MI355X.

A step = idmap_find_or_insert -> embedding_bag_fwd -> embedding_bag_bwd_update
over one batch of the click-log workload: 26 one-hot tables, dim 128 fp32,
batch 65536, per-table cardinality log-uniform in [10, 4e7] (55.8M live rows
for the seed used), Zipf(1.1) lookups over random 63-bit keys, Adagrad (lr
0.01, eps 1e-8) with fp32 accumulator rows, N(0,1) upstream gradients.
Inputs are synthetic, seeded, and resident in HBM before timing starts.

Prints one JSON line: lookups/s (the metric), plus updated rows/s, the step's
compulsory HBM bytes per second against the 8 TB/s peak, a roofline entry for
the dominant kernel (timed live with HIP events on the library's stream) and
the CPU oracle timed on the host.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=2, help="workload number (2 = click-log, the headline)")
    p.add_argument("--batches", type=int, default=4, help="distinct batches cycled through")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-steps", type=int, default=2)
    p.add_argument("--map-load", type=float, default=0.5)
    p.add_argument("--serial-bwd", action="store_true",
                   help="report the serial schedule (find, fwd, bwd update on one stream) as the value instead "
                        "of the lookahead one")
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


def logical_bytes(cfg, L, U, row_bytes):
    """Bytes the step moves with no reuse across lookups: the compulsory
    bytes plus, for every lookup beyond the first of its row, the forward's
    row-weight gather and one map slot."""
    import synth

    w_bytes = cfg.dim * (2 if cfg.wdtype == synth.BF16 else 4)
    return compulsory_bytes(cfg, L, U, 0, row_bytes) + (L - U) * (w_bytes + 16)


def compulsory_bytes(cfg, L, U, n_new, row_bytes):
    """Bytes the step must move at least once: ids, bag offsets, one map slot
    per distinct key, read+write of every touched row (weights + state), the
    pooled output write and the upstream-gradient read, new-row init."""
    TB = cfg.n_tables * cfg.batch
    return (L * 8 + (TB + 1) * 8 + U * 16 + U * row_bytes * 2 + TB * cfg.dim * 4 * 2
            + n_new * row_bytes)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    import recommender_sparse_embedding_amd as rse
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.config(args.config)
    wl = synth.Workload(cfg)
    T, B, D = cfg.n_tables, cfg.batch, cfg.dim
    t0 = time.time()

    # ---------------------------------------------------------- setup ----
    total_keys = int(wl.card.sum())
    if cfg.merged:
        slots = [int(total_keys / args.map_load) + 1024]
    else:
        slots = [int(c / args.map_load) + 1024 for c in wl.card]
    idm = rse.IdMap(slots, max_load=0.9, merged=cfg.merged, hash_seed=12345, device=dev)
    chunk_log2 = 20
    blk = rse.EmbeddingBlocks(D, cfg.wdtype, cfg.optim, chunk_log2, max_chunks=4096, seed=cfg.seed,
                              device=dev)
    # rows the run can add: the whole universe when tables start empty (the
    # lookups draw from it), else the never-seen keys of every find the run
    # makes (warmup and timed steps of each schedule, plus look-ahead finds)
    max_bag = {"fixed": cfg.bag[1], "uniform": cfg.bag[-1], "poisson": 3 * cfg.bag[1]}[cfg.bag[0]]
    n_finds = 5 * (args.warmup + 2) + 5 * (args.steps + 2)   # five schedules, each primed
    if not cfg.prepopulate:
        headroom = total_keys
    else:
        headroom = int(cfg.fresh_frac * cfg.n_bags * max_bag * n_finds)
    headroom += 1 << chunk_log2
    blk.grow(-(-((total_keys if cfg.prepopulate else 0) + headroom) // (1 << chunk_log2)))
    opt = rse.Optim(cfg.optim, cfg.lr, cfg.eps, cfg.beta1, cfg.beta2)
    n_new = torch.zeros(1, dtype=torch.int64, device=dev)
    pre_ws = idm.workspace(1 << 24)
    for ids, bounds in wl.prepopulation(chunk=1 << 24):
        t_ids = torch.from_numpy(ids).to(dev)
        ro = torch.empty_like(t_ids)
        rse.idmap_find_or_insert(idm, blk, t_ids, torch.from_numpy(bounds).to(dev), 1, T, ro, n_new,
                                 ws=pre_ws)
    torch.cuda.synchronize()
    used, st = blk.status()
    assert st == 0 and used == (total_keys if cfg.prepopulate else 0), (used, st)
    log(f"prepopulated {total_keys} keys in {time.time() - t0:.1f}s")

    batches = []
    for k in range(args.batches):
        ids, bo = wl.batch_inputs(k)
        # distinct (table, key) pairs = rows the step updates (all keys are live)
        tab = np.repeat(np.arange(T), np.diff(bo[::B]))
        U = len(np.unique(np.stack([tab, ids], 1), axis=0)) if len(ids) else 0
        g = torch.from_numpy(wl.grad(k)).to(dev) if cfg.grad == "normal" else None
        batches.append(dict(ids=torch.from_numpy(ids).to(dev), bo=torch.from_numpy(bo).to(dev),
                            grad=g, L=len(ids), U=U, ro=torch.empty(len(ids), dtype=torch.int64, device=dev)))
    L_max = max(b["L"] for b in batches)
    find_ws = idm.workspace(L_max)
    bwd_ws = rse.bwd_workspace(L_max, T, B, D, dev)
    out = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    n_u = torch.zeros(1, dtype=torch.int64, device=dev)
    log(f"staged {len(batches)} batches, setup {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()
    # second stream (default priority) for the work that does not wait for
    # the previous phase: the backward's sort, and the next batch's find
    side = torch.cuda.Stream(device=dev)
    ws2 = [bwd_ws, rse.bwd_workspace(L_max, T, B, D, dev)]
    step_no = [0]

    def grad_of(b):
        return b["grad"] if b["grad"] is not None else 2.0 * out

    def step_serial(b):
        rse.idmap_find_or_insert(idm, blk, b["ids"], b["bo"], B, T, b["ro"], n_new, ws=find_ws)
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        step_no[0] += 1
        rse.embedding_bag_bwd_update(blk, b["ro"], b["bo"], T, B, cfg.pooling, grad_of(b), opt, step_no[0], n_u,
                                     ws=bwd_ws)

    def step_overlap(b, ev=None):
        """find; then the forward (stream 1) and the backward's sort (stream
        2) together; then the apply."""
        if ev:
            ev[0].record(stream)
        rse.idmap_find_or_insert(idm, blk, b["ids"], b["bo"], B, T, b["ro"], n_new, ws=find_ws)
        if ev:
            ev[1].record(stream)
        found = torch.cuda.Event()
        found.record(stream)
        side.wait_event(found)
        plan = rse.embedding_bag_bwd_prepare(blk, b["ro"], b["bo"], T, B, bwd_ws, stream=side)
        srt = torch.cuda.Event()
        srt.record(side)
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        if ev:
            ev[2].record(stream)
        g = grad_of(b)
        step_no[0] += 1
        stream.wait_event(srt)
        rse.embedding_bag_bwd_apply(blk, plan, b["bo"], T, B, cfg.pooling, g, opt, step_no[0], n_u, bwd_ws)
        if ev:
            ev[3].record(stream)

    # Pipelined steps: the find and sort of batch i+1 (stream 2) run while
    # batch i's forward and apply run (stream 1).  The find of batch i+1 only
    # touches the map, rows it creates and its own outputs, none of which
    # batch i's apply reads or writes; the forward of batch i+1 waits for
    # both.  Sort workspaces alternate; a sort waits for the apply that last
    # used its workspace.
    applied = [torch.cuda.Event(), torch.cuda.Event()]
    fronted = [torch.cuda.Event(), torch.cuda.Event()]
    plans = [None, None]

    def front(i, b):
        side.wait_event(applied[i % 2])
        rse.idmap_find_or_insert(idm, blk, b["ids"], b["bo"], B, T, b["ro"], n_new, ws=find_ws, stream=side)
        plans[i % 2] = rse.embedding_bag_bwd_prepare(blk, b["ro"], b["bo"], T, B, ws2[i % 2], stream=side)
        fronted[i % 2].record(side)

    def back(i, b):
        stream.wait_event(fronted[i % 2])
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        g = grad_of(b)
        step_no[0] += 1
        rse.embedding_bag_bwd_apply(blk, plans[i % 2], b["bo"], T, B, cfg.pooling, g, opt, step_no[0], n_u,
                                    ws2[i % 2])
        applied[i % 2].record(stream)

    # "staggered": stream 2 sorts batch i while stream 1 runs its forward,
    # then finds batch i+1 while stream 1 runs batch i's apply (the radix
    # passes slow the segmented update down when they share the GPU with it,
    # less so the forward).  Same per-step work and dependencies as above.
    found = [torch.cuda.Event(), torch.cuda.Event()]
    sorted_ = [torch.cuda.Event(), torch.cuda.Event()]

    def find_ahead(i, b):
        rse.idmap_find_or_insert(idm, blk, b["ids"], b["bo"], B, T, b["ro"], n_new, ws=find_ws, stream=side)
        found[i % 2].record(side)

    def staggered_step(i, b, b_next):
        side.wait_event(applied[(i + 1) % 2])         # apply(i-1) is done: stream 1 starts forward(i)
        plans[i % 2] = rse.embedding_bag_bwd_prepare(blk, b["ro"], b["bo"], T, B, ws2[i % 2], stream=side)
        sorted_[i % 2].record(side)
        find_ahead(i + 1, b_next)
        stream.wait_event(found[i % 2])
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        g = grad_of(b)
        step_no[0] += 1
        stream.wait_event(sorted_[i % 2])
        rse.embedding_bag_bwd_apply(blk, plans[i % 2], b["bo"], T, B, cfg.pooling, g, opt, step_no[0], n_u,
                                    ws2[i % 2])
        applied[i % 2].record(stream)

    # "lookahead": stream 2 runs one more batch ahead.  While stream 1 runs
    # batch i's forward and apply, stream 2 sorts batch i+1 (found during the
    # previous step) and then finds batch i+2.  The sort shares the GPU with
    # the forward and the find with the segmented update, and stream 1 never
    # waits for the tail of a sort.  The find of i+2 writes only the map, rows
    # it creates and batch i+2's offsets (a buffer last read by the forward
    # of batch i-2 when at least three batches cycle); finds still run in
    # batch order, so every result is that of the plain order.
    ready = [torch.cuda.Event() for _ in range(3)]        # find of batch k done: ready[k % 3]
    prepared = [torch.cuda.Event(), torch.cuda.Event()]   # prepare of batch k done: prepared[k % 2]

    def la_find(k):
        b = batch_at(k)
        rse.idmap_find_or_insert(idm, blk, b["ids"], b["bo"], B, T, b["ro"], n_new, ws=find_ws, stream=side)
        ready[k % 3].record(side)

    def la_prepare(k):
        side.wait_event(applied[k % 2])               # the apply that last used this workspace
        b = batch_at(k)
        plans[k % 2] = rse.embedding_bag_bwd_prepare(blk, b["ro"], b["bo"], T, B, ws2[k % 2], stream=side)
        prepared[k % 2].record(side)

    def la_step(i):
        la_prepare(i + 1)
        la_find(i + 2)
        b = batch_at(i)
        stream.wait_event(ready[i % 3])
        rse.embedding_bag_fwd(blk, b["ro"], b["bo"], T, B, cfg.pooling, out)
        g = grad_of(b)
        step_no[0] += 1
        stream.wait_event(prepared[i % 2])
        rse.embedding_bag_bwd_apply(blk, plans[i % 2], b["bo"], T, B, cfg.pooling, g, opt, step_no[0], n_u,
                                    ws2[i % 2])
        applied[i % 2].record(stream)

    def batch_at(k):
        return batches[k % len(batches)]

    host_ms = {}      # host time to enqueue one step, per schedule

    def timed(schedule, first, n, evs=None):
        """n steps over batches first.., timed between events on stream 1
        (every stream's work inside is waited for); returns ms."""
        torch.cuda.synchronize()
        if schedule == "pipelined":
            front(first, batch_at(first))
        if schedule == "staggered":
            find_ahead(first, batch_at(first))
        if schedule == "lookahead":
            la_find(first)
            la_prepare(first)
            la_find(first + 1)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        h0 = time.perf_counter()
        for k in range(n):
            i = first + k
            if schedule == "serial":
                step_serial(batch_at(i))
            elif schedule == "overlap":
                step_overlap(batch_at(i), evs[k] if evs else None)
            elif schedule == "staggered":
                staggered_step(i, batch_at(i), batch_at(i + 1))
            elif schedule == "lookahead":
                la_step(i)
            else:
                front(i + 1, batch_at(i + 1))      # the next batch: one find + sort per step
                back(i, batch_at(i))
        if schedule == "pipelined":
            stream.wait_event(fronted[(first + n) % 2])
        if schedule == "staggered":
            stream.wait_event(found[(first + n) % 2])
        if schedule == "lookahead":
            stream.wait_event(prepared[(first + n) % 2])
            stream.wait_event(ready[(first + n + 1) % 3])
        t1.record(stream)
        host_ms[schedule] = (time.perf_counter() - h0) * 1e3 / max(n, 1)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    schedule = "serial" if args.serial_bwd else ("lookahead" if len(batches) >= 3 else "overlap")
    for name in ("serial", "overlap", "staggered", "pipelined", schedule):
        timed(name, 0, args.warmup)
    used, st = blk.status()
    assert st == 0, st

    # ----------------------------------------------------- timed region --
    # The library brackets every launch of the segmented-update kernel (the
    # step's largest) with HIP events on its stream while the trace is on.
    rse.trace_start(rse.K_SEG_UPDATE)
    w0 = time.perf_counter()
    ms_total = timed(schedule, args.warmup, args.steps)
    wall = time.perf_counter() - w0
    n_seg, seg_ms = rse.trace_stop()
    ms_step = ms_total / args.steps
    t_seg = seg_ms / max(n_seg, 1)
    # the other schedules, and the phase split of the overlapped one, for reference
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    ms_overlap = timed("overlap", args.warmup, args.steps, evs) / args.steps
    t_find = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    t_fwd = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    t_bwd = np.mean([e[2].elapsed_time(e[3]) for e in evs])
    rse.trace_start(rse.K_FWD)
    ms_serial = timed("serial", args.warmup, args.steps) / args.steps
    ms_stag = timed("staggered", args.warmup, args.steps) / args.steps if len(batches) >= 2 else None
    ms_pipe = timed("pipelined", args.warmup, args.steps) / args.steps if len(batches) >= 2 else None
    n_fwd, fwd_ms = rse.trace_stop()
    t_fwd_kernel = fwd_ms / max(n_fwd, 1)
    idm_st, _ = idm.status()
    used, st = blk.status()
    assert idm_st == 0 and st == 0, (idm_st, st)
    live_rows = used

    sel = [batches[(args.warmup + k) % len(batches)] for k in range(args.steps)]
    L_avg = float(np.mean([b["L"] for b in sel]))
    U_avg = float(np.mean([b["U"] for b in sel]))
    rb = blk.row_bytes
    comp = float(np.mean([compulsory_bytes(cfg, b["L"], b["U"], 0, rb) for b in sel]))
    lookups_s = L_avg / (ms_step * 1e-3)
    rows_s = U_avg / (ms_step * 1e-3)
    step_gbs = comp / (ms_step * 1e-3) / 1e9
    logical = float(np.mean([logical_bytes(cfg, b["L"], b["U"], rb) for b in sel]))

    # roofline of the segmented-update kernel: algorithmic bytes per launch =
    # sorted (row, gradient-row) pairs read (8 B per lookup) + one gradient row
    # per lookup (dim * 4 B) + each touched row (weights + state) read and
    # written once
    seg_bytes = float(np.mean([b["L"] * 8 + b["L"] * D * 4 + b["U"] * rb * 2 for b in sel]))
    seg_gbs = seg_bytes / (t_seg * 1e-3) / 1e9
    TB = T * B
    w_bytes = D * (2 if cfg.wdtype == synth.BF16 else 4)
    fwd_bytes = float(np.mean([b["L"] * 8 + (TB + 1) * 8 + b["U"] * w_bytes + TB * D * 4 for b in sel]))
    traffic = read_traffic("seg_update_clicklog.txt", KERNEL_REV) if args.config == 2 else None
    roofline = {"bound": "hbm", "kernel": f"k_seg_work<{D},{'bf16' if cfg.wdtype else 'f32'}>",
                "achieved": round(seg_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(seg_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": int(seg_bytes), "avg_launch_ms": round(t_seg, 4),
                "launches_timed": n_seg}
    fwd_roof = {"kernel": "embedding_bag_fwd", "achieved": round(fwd_bytes / (t_fwd_kernel * 1e-3) / 1e9, 1),
                "unit": "GB/s", "algorithmic_bytes_per_launch": int(fwd_bytes),
                "avg_launch_ms": round(float(t_fwd_kernel), 4)}

    # --------------------------------------------------- CPU baseline -----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, wl, args.cpu_steps)

    res = {
        "metric": "embedding lookups/sec (fwd+bwd+update), 1 MI355X",
        "value": round(lookups_s, 1),
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 storage, f64 accumulate" if cfg.wdtype == synth.F32 else "bf16 storage, f64 accumulate",
        "data": "synthetic (seeded Zipf lookups over random 63-bit keys, N(0,1) grads)",
        "config": {"workload": f"{cfg.name}: {T} tables x batch {B}, dim {D}, "
                               f"{live_rows} live rows", "tables": T, "batch": B, "dim": D,
                   "lookups_per_step": L_avg, "unique_rows_per_step": U_avg, "live_rows": live_rows,
                   "map_load": args.map_load},
        "updated_rows_per_s": round(rows_s, 1),
        "step_compulsory_bytes": int(comp),
        "step_hbm_gbs": round(step_gbs, 1),
        "step_frac_of_peak": round(step_gbs / PEAK_HBM_GBS, 4),
        "step_logical_bytes": int(logical),
        "step_logical_gbs": round(logical / (ms_step * 1e-3) / 1e9, 1),
        "schedule": {"serial": "find; fwd; bwd update (one stream)",
                     "overlap": "find; fwd (stream 1) || bwd prepare = pairs + sort (stream 2); bwd apply",
                     "lookahead": "fwd + bwd apply of batch i (stream 1) || bwd prepare of batch i+1, then "
                                  "find of batch i+2 (stream 2)"}[schedule],
        "ms_per_step_by_schedule": {"serial": round(ms_serial, 4), "overlap": round(ms_overlap, 4),
                                    "staggered": round(ms_stag, 4) if ms_stag else None,
                                    "pipelined": round(ms_pipe, 4) if ms_pipe else None,
                                    "lookahead": round(ms_step, 4) if schedule == "lookahead" else None},
        "host_enqueue_ms_per_step": {k: round(v, 4) for k, v in host_ms.items()},
        "overlap_phase_ms": {"find": round(float(t_find), 4), "fwd": round(float(t_fwd), 4),
                             "bwd_update": round(float(t_bwd), 4)},
        "wall_s": round(wall, 4),
        "roofline": roofline,
        "fwd_roofline": fwd_roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


# identifies the kernel source the stored traffic counters were taken on
KERNEL_REV = "seg-v9"


def read_traffic(name, rev):
    """HBM bytes per launch from a committed counter summary (profiles/),
    or None if absent or taken on another kernel revision."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_rev") != rev or "hbm_bytes_per_launch" not in vals:
        return None
    return int(float(vals["hbm_bytes_per_launch"]))


def cpu_baseline(cfg, wl, steps):
    """The oracle, single-threaded, on the same workload: the full key
    universe inserted, then `steps` whole steps (find + forward + backward
    with update); lookups per second of the timed steps."""
    import oracle

    t0 = time.time()
    orc = oracle.OracleTable(cfg.dim, cfg.wdtype, cfg.optim, cfg.n_tables, cfg.merged, seed=cfg.seed,
                             lr=cfg.lr, eps=cfg.eps, beta1=cfg.beta1, beta2=cfg.beta2)
    for ids, bounds in wl.prepopulation(chunk=1 << 24):
        orc.find_or_insert(ids, bounds, 1)
    log(f"oracle prepopulated in {time.time() - t0:.1f}s")
    tot_L, tot_t = 0, 0.0
    for k in range(steps):
        ids, bo = wl.batch_inputs(k)
        g = wl.grad(k)
        s = time.perf_counter()
        ro, _ = orc.find_or_insert(ids, bo, cfg.batch)
        out = orc.fwd(ro, bo, cfg.batch, cfg.pooling)
        if cfg.grad != "normal":
            g = (2.0 * out).astype(np.float32)
        orc.bwd_update(ro, bo, cfg.batch, g, cfg.pooling)
        tot_t += time.perf_counter() - s
        tot_L += len(ids)
    return {"value": round(tot_L / tot_t, 1), "unit": "lookups/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full steps ({tot_L} lookups) after inserting all {int(wl.card.sum())} keys; "
                      f"{tot_t:.1f}s timed"}


if __name__ == "__main__":
    main()
