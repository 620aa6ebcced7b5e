"""HIP path vs the oracle at the workloads' full sizes, in the launch
configuration bench.py times (2^24-row chunks, the same kernels, the sort on
a second stream beside the forward).

The click-log and behaviour-sequence workloads are compared element by
element with the whole oracle. The 2e8-row and merged workloads are checked
through properties that hold at any size (a prepopulated key's row offset is
its insertion index; no new keys; the touched-row count) and through samples
that the oracle computes one by one: pooled outputs of sampled bags, updated
rows of sampled keys (a fresh oracle table fed exactly the lookups of those
keys, in lookup order: a row's update depends only on its key's initial
value and its own lookups), and sampled untouched rows against their initial
values.

In every workload, every row outside the step's batch is compared on the
device before and after the update (a copy of all chunks, or for the 154 GB
table a 64-bit fingerprint per row): no byte of such a row may change.
"""

from __future__ import annotations

import dataclasses
import gc

import numpy as np
import pytest
import torch

import synth
from harness import ChunkSnapshot, assert_close, assert_only_touched_changed, make_oracle, pooled_magnitude, rtol_for

pytestmark = pytest.mark.gpu

CHUNK_LOG2 = 24          # as bench.py allocates the tables


def _say(*a):
    print(*a, flush=True)


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class Full:
    """The library's objects for one workload at full size, as bench.py
    builds them, with every table's universe inserted."""

    def __init__(self, cfg: synth.Config, wl: synth.Workload, map_load: float, extra_keys: int = 0):
        import recommender_sparse_embedding_amd as rse

        self.rse = rse
        self.cfg = cfg
        self.dev = torch.device("cuda")
        total = int(wl.card.sum())
        if cfg.merged:
            slots = [int((total + extra_keys) / map_load) + 1024]
        else:
            slots = [int((int(c) + extra_keys) / map_load) + 1024 for c in wl.card]
        self.map = rse.IdMap(slots, max_load=0.9, merged=cfg.merged, hash_seed=12345, device=self.dev)
        self.blk = rse.EmbeddingBlocks(cfg.dim, cfg.wdtype, cfg.optim, CHUNK_LOG2, max_chunks=4096, seed=cfg.seed,
                                       device=self.dev)
        self.blk.grow(-(-(total + extra_keys + 1) // (1 << CHUNK_LOG2)))
        self.optim = rse.Optim(cfg.optim, cfg.lr, cfg.eps, cfg.beta1, cfg.beta2)
        n_new = torch.zeros(1, dtype=torch.int64, device=self.dev)
        ws = self.map.workspace(1 << 24)
        for ids, bounds in wl.prepopulation(chunk=1 << 24):
            t_ids = torch.from_numpy(ids).to(self.dev)
            ro = torch.empty_like(t_ids)
            rse.idmap_find_or_insert(self.map, self.blk, t_ids, torch.from_numpy(bounds).to(self.dev), 1,
                                     cfg.n_tables, ro, n_new, ws=ws)
        torch.cuda.synchronize()
        used, st = self.blk.status()
        assert st == 0 and used == total, (used, st)
        self.step_no = 0

    def step(self, ids: np.ndarray, bo: np.ndarray, G: np.ndarray):
        """find; the backward's prepare on a second stream beside the
        forward; apply.  Returns row offsets, n_new, pooled output, U, and a
        snapshot of every chunk taken after the find (before the update)."""
        rse, cfg, dev = self.rse, self.cfg, self.dev
        T, B, D = cfg.n_tables, cfg.batch, cfg.dim
        t_ids = torch.from_numpy(ids).to(dev)
        t_bo = torch.from_numpy(bo).to(dev)
        g = torch.from_numpy(G).to(dev)
        ro = torch.empty_like(t_ids)
        n_new = torch.zeros(1, dtype=torch.int64, device=dev)
        rse.idmap_find_or_insert(self.map, self.blk, t_ids, t_bo, B, T, ro, n_new, ws=self.map.workspace(len(ids)))
        snap = ChunkSnapshot(self.blk)
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream(device=dev)
        found = torch.cuda.Event()
        found.record(main)
        side.wait_event(found)
        bws = rse.bwd_workspace(len(ids), T, B, D, dev)
        for t in (ro, t_bo, bws):
            t.record_stream(side)
        plan = rse.embedding_bag_bwd_prepare(self.blk, ro, t_bo, T, B, bws, stream=side)
        srt = torch.cuda.Event()
        srt.record(side)
        out = torch.empty((B, T, D), dtype=torch.float32, device=dev)
        rse.embedding_bag_fwd(self.blk, ro, t_bo, T, B, cfg.pooling, out)
        # one-hot: the rows the forward read (before the update), [B, T, d]
        self.rows_read = None
        if cfg.bag == ("fixed", 1):
            w, _ = self.blk.read_rows(ro)
            self.rows_read = w.view(T, B, D).transpose(0, 1).contiguous()
        main.wait_event(srt)
        self.step_no += 1
        nu = torch.zeros(1, dtype=torch.int64, device=dev)
        rse.embedding_bag_bwd_apply(self.blk, plan, t_bo, T, B, cfg.pooling, g, self.optim, self.step_no, nu, bws)
        torch.cuda.synchronize()
        idm_st, _ = self.map.status()
        _, st = self.blk.status()
        assert idm_st == 0 and st == 0, (idm_st, st)
        return ro.cpu().numpy(), int(n_new.item()), out.cpu().numpy(), int(nu.item()), snap

    def rows(self, offs: np.ndarray):
        w, s = self.blk.read_rows(torch.from_numpy(np.ascontiguousarray(offs, np.int64)).to(self.dev))
        return w.cpu().numpy(), s.cpu().numpy()


def _compare_updated(w_g, s_g, w_prev, w_r, s_r, rtol, what):
    M = np.abs(w_prev.astype(np.float64)) + np.abs(w_r.astype(np.float64) - w_prev)
    assert_close(w_g, w_r, M, rtol, what + " weights")
    if s_r.size:
        assert_close(s_g, s_r, np.abs(s_r.astype(np.float64)) + 1e-30, 1e-5, what + " state")


def _whole_oracle_steps(cfg: synth.Config, steps: int, map_load: float, neighbours: bool = False):
    wl = synth.Workload(cfg)
    L_max = max(int(wl.batch_inputs(s)[1][-1]) for s in range(steps))
    extra = int(L_max * cfg.fresh_frac * 1.05 * steps) + 1024 if cfg.fresh_frac > 0 else 0
    _say(f"  {cfg.name}: {int(wl.card.sum())} rows, up to {L_max} lookups per step")
    gpu = Full(cfg, wl, map_load, extra_keys=extra)
    orc = make_oracle(cfg)
    for ids, bounds in wl.prepopulation(chunk=1 << 24):
        orc.find_or_insert(ids, bounds, 1)
    _say("  prepopulated both sides")
    rng = np.random.default_rng(11)
    rtol = rtol_for(cfg.wdtype)
    ever = np.zeros(0, np.int64)          # rows updated by any step so far
    for s in range(steps):
        ids, bo = wl.batch_inputs(s)
        G = wl.grad(s)
        ro_g, nn_g, out_g, nu_g, snap = gpu.step(ids, bo, G)
        ro_r, nn_r = orc.find_or_insert(ids, bo, cfg.batch)
        assert nn_g == nn_r, (nn_g, nn_r)
        assert np.array_equal(ro_g, ro_r), f"row offsets, step {s}"
        out_r = orc.fwd(ro_r, bo, cfg.batch, cfg.pooling)
        if cfg.bag == ("fixed", 1):
            # one-hot: the pooled row is the row the forward read, exactly (on
            # the device: the rows of every lookup, read back, in [B, T, d])
            assert torch.equal(torch.from_numpy(out_g).to(gpu.dev).view(torch.int32),
                               gpu.rows_read.view(torch.int32)), f"one-hot pooled rows differ from the rows read, step {s}"
            gpu.rows_read = None
            if s == 0:       # rows still hold their exact initial values
                assert np.array_equal(out_g.view(np.uint32), out_r.view(np.uint32)), f"one-hot pooled rows, step {s}"
        assert_close(out_g, out_r, pooled_magnitude(orc, ro_r, bo, cfg), rtol, f"pooled output, step {s}")
        last_out = out_g
        del out_g, out_r
        offs = np.unique(ro_r[ro_r >= 0])
        prev_w, _ = orc.get_rows(offs)
        n_rows = orc.n_rows
        U = orc.bwd_update(ro_r, bo, cfg.batch, G, cfg.pooling)
        assert nu_g == U == len(offs)
        w_g, s_g = gpu.rows(offs)
        w_r, s_r = orc.get_rows(offs)
        _compare_updated(w_g, s_g, prev_w, w_r, s_r, rtol, f"step {s}")
        ever = np.union1d(ever, offs)
        # every row outside the batch keeps its bytes (all rows, on the device)
        assert_only_touched_changed(snap, offs, f"step {s}")
        _say(f"  step {s}: every row outside the batch unchanged ({snap.mode} of all chunks)")
        del snap
        untouched = np.setdiff1d(rng.choice(n_rows, 40_000, replace=False), ever)[:20_000]
        w_g, s_g = gpu.rows(untouched)
        w_r, s_r = orc.get_rows(untouched)
        assert np.array_equal(w_g.view(np.uint32), w_r.view(np.uint32)), "never-touched rows changed"
        assert np.array_equal(s_g.view(np.uint32), s_r.view(np.uint32))
        _say(f"  step {s}: {len(ids)} lookups, {U} rows updated, all equal to the oracle")
    if neighbours:
        _interaction_full_size(last_out)
        del last_out
        _eviction_full_size(gpu, orc, wl, steps)


def _interaction_full_size(pooled: np.ndarray):
    """The DLRM interaction on the step's pooled output at its full shape
    (the launch the bench times), sampled samples against the oracle."""
    import recommender_sparse_embedding_amd as rse
    from oracle import interaction as ointer

    B, T, D = pooled.shape
    rng = np.random.default_rng(5)
    dense = rng.standard_normal((B, D)).astype(np.float32)
    t_dense, t_pooled = torch.from_numpy(dense).cuda(), torch.from_numpy(pooled).cuda()
    out = rse.dlrm_interaction_fwd(t_dense, t_pooled)
    dout = rng.standard_normal(tuple(out.shape)).astype(np.float32)
    dd, dp = rse.dlrm_interaction_bwd(t_dense, t_pooled, torch.from_numpy(dout).cuda())
    sel = np.sort(rng.choice(B, 512, replace=False))
    ref, mag = ointer.interaction_fwd(dense[sel], pooled[sel])
    assert_close(out.cpu().numpy()[sel], ref, mag, 1e-5, "interaction forward, sampled samples")
    rdd, rdp, mdd, mdp = ointer.interaction_bwd(dense[sel], pooled[sel], dout[sel])
    assert_close(dd.cpu().numpy()[sel], rdd, mdd, 1e-5, "interaction dense gradient, sampled samples")
    assert_close(dp.cpu().numpy()[sel], rdp, mdp, 1e-5, "interaction pooled gradient, sampled samples")
    _say(f"  interaction [{B}, {T}, {D}]: 512 sampled samples equal to the oracle")


def _eviction_full_size(gpu, orc, wl, step: int):
    """Eviction at full size: age tracking on, one batch at clock 1, the
    rehash with minimum clock 1 keeps that batch's keys; the map's entries
    and the rebuilt free list (every other row, ascending) equal the
    oracle's, and evicted keys are absent."""
    rse, cfg, dev = gpu.rse, gpu.cfg, gpu.dev
    gpu.map.track_age(gpu.blk.capacity)
    gpu.blk.enable_free_list()
    orc.set_tracking(True)
    orc.set_recycling(True)
    gpu.map.set_clock(1)
    orc.set_clock(1)
    ids, bo = wl.batch_inputs(step)
    t_ids, t_bo = torch.from_numpy(ids).to(dev), torch.from_numpy(bo).to(dev)
    ro = torch.empty_like(t_ids)
    n_new = torch.zeros(1, dtype=torch.int64, device=dev)
    rse.idmap_find_or_insert(gpu.map, gpu.blk, t_ids, t_bo, cfg.batch, cfg.n_tables, ro, n_new,
                             ws=gpu.map.workspace(len(ids)))
    ro_r, _ = orc.find_or_insert(ids, bo, cfg.batch)
    assert np.array_equal(ro.cpu().numpy(), ro_r)
    gpu.map.evict(gpu.blk, 1)
    kept = orc.rehash(1)
    k, t, o, cnt = gpu.map.export(kept + 16)
    order = torch.argsort(o)
    kr, tr, orr = orc.entries()
    assert cnt == kept == len(kr)
    assert np.array_equal(o[order].cpu().numpy(), orr) and np.array_equal(k[order].cpu().numpy(), kr)
    assert np.array_equal(t[order].cpu().numpy(), tr)
    head, left = gpu.blk.free_list()
    left_r, head_r = orc.free_list()
    assert head == head_r == 0 and np.array_equal(left.cpu().numpy(), left_r)
    ids2, bo2 = wl.batch_inputs(step + 1)
    t_ids2, t_bo2 = torch.from_numpy(ids2).to(dev), torch.from_numpy(bo2).to(dev)
    ro2 = torch.empty_like(t_ids2)
    rse.idmap_find_or_insert(gpu.map, gpu.blk, t_ids2, t_bo2, cfg.batch, cfg.n_tables, ro2, n_new,
                             insert_missing=False, ws=gpu.map.workspace(len(ids2)))
    ro2_r, _ = orc.find_or_insert(ids2, bo2, cfg.batch, insert_missing=False)
    assert np.array_equal(ro2.cpu().numpy(), ro2_r) and (ro2_r < 0).any()
    _say(f"  eviction: {kept} keys kept, {len(left_r)} rows freed, equal to the oracle")


def test_click_log_full_size_whole_oracle():
    """26 one-hot tables, 55.8M live rows, batch 65,536, dim 128, Adagrad:
    every row offset, every pooled row and every updated row of two steps;
    then the interaction on the pooled output at its full shape (sampled)
    and an eviction of the full map (entries and free list exactly)."""
    _free()
    try:
        _whole_oracle_steps(synth.config(2), 2, map_load=0.5, neighbours=True)
    finally:
        _free()


def test_behaviour_sequence_full_size_whole_oracle():
    """4 tables x 5M rows, batch 8,192, bags U[1,100], mean pooling, Adam,
    1% never-seen ids per step (inserted during the step)."""
    _free()
    try:
        _whole_oracle_steps(synth.config(3), 2, map_load=0.5)
    finally:
        _free()


def _mini_batch(cfg, ids, table, lookup_bag, positions, G):
    """The lookups at `positions` (in index order) as their own batch: one
    lookup per bag, table-major, each bag carrying its original upstream
    gradient row.  Exact for sum pooling."""
    T = cfg.n_tables
    tab = table[positions]
    per = np.bincount(tab, minlength=T)
    Bm = max(1, int(per.max()))
    lens = np.zeros(T * Bm, np.int64)
    mids = np.empty(len(positions), np.int64)
    Gm = np.zeros((Bm, T, cfg.dim), np.float32)
    k = 0
    for t in range(T):
        pos_t = positions[tab == t]
        n = len(pos_t)
        lens[t * Bm: t * Bm + n] = 1
        mids[k:k + n] = ids[pos_t]
        j = lookup_bag[pos_t]                       # original bag j = t * B + b
        Gm[:n, t, :] = G[j - t * cfg.batch, t, :]
        k += n
    bo = np.zeros(T * Bm + 1, np.int64)
    np.cumsum(lens, out=bo[1:])
    return mids, bo, Gm, Bm


def _sampled_checks(cfg: synth.Config, map_load: float, n_rows_sample: int, n_bag_sample: int):
    wl = synth.Workload(cfg)
    T, B = cfg.n_tables, cfg.batch
    counters, table, bo = wl.batch_counters(0)
    ids, bo2 = wl.batch_inputs(0)
    assert np.array_equal(bo, bo2)
    G = wl.grad(0)
    _say(f"  {cfg.name}: {int(wl.card.sum())} rows, {len(ids)} lookups")
    gpu = Full(cfg, wl, map_load)
    _say("  prepopulated")
    ro_g, nn_g, out_g, nu_g, snap = gpu.step(ids, bo, G)
    rtol = rtol_for(cfg.wdtype)
    # properties at full size: offset = insertion index (tables inserted in
    # order, each in generation order), no new keys, touched-row count
    base = np.zeros(T, np.int64)
    np.cumsum(wl.card[:-1], out=base[1:])
    expect = base[table] + counters.astype(np.int64)
    assert nn_g == 0
    assert np.array_equal(ro_g, expect), "row offset != insertion index"
    rowid = expect
    assert nu_g == len(np.unique(rowid))
    _say("  offsets and counts hold")
    assert_only_touched_changed(snap, np.unique(rowid), "the step")
    _say(f"  every row outside the batch unchanged ({snap.mode} of all chunks)")
    del snap
    _free()
    lookup_bag = np.repeat(np.arange(T * B), np.diff(bo))
    rng = np.random.default_rng(5)
    # pooled outputs of sampled samples b (all tables): a fresh oracle
    # table holding just those bags
    bs = np.sort(rng.choice(B, n_bag_sample, replace=False))
    sel = [np.arange(bo[t * B + b], bo[t * B + b + 1]) for t in range(T) for b in bs]
    m_ids = ids[np.concatenate(sel)] if sel else ids[:0]
    m_lens = np.array([len(x) for x in sel], np.int64)
    m_bo = np.zeros(len(sel) + 1, np.int64)
    np.cumsum(m_lens, out=m_bo[1:])
    mcfg = dataclasses.replace(cfg, batch=len(bs))
    morc = make_oracle(mcfg)
    m_ro, _ = morc.find_or_insert(m_ids, m_bo, len(bs))
    m_out = morc.fwd(m_ro, m_bo, len(bs), cfg.pooling)
    assert_close(out_g[bs], m_out, pooled_magnitude(morc, m_ro, m_bo, mcfg), rtol, "sampled pooled outputs")
    _say(f"  {len(bs)} x {T} sampled pooled outputs match")
    # updated rows of sampled keys
    uniq = np.unique(rowid)
    pick = np.sort(rng.choice(uniq, min(n_rows_sample, len(uniq)), replace=False))
    positions = np.nonzero(np.isin(rowid, pick))[0]
    r_ids, r_bo, r_G, r_B = _mini_batch(cfg, ids, table, lookup_bag, positions, G)
    rcfg = dataclasses.replace(cfg, batch=r_B)
    rorc = make_oracle(rcfg)
    r_ro, _ = rorc.find_or_insert(r_ids, r_bo, r_B)
    offs_m = np.unique(r_ro)
    w_prev, _ = rorc.get_rows(offs_m)
    U = rorc.bwd_update(r_ro, r_bo, r_B, r_G, cfg.pooling)
    assert U == len(pick)
    # oracle offset -> GPU offset: the mini batch lists the sampled lookups
    # table by table, in index order
    order = np.concatenate([positions[table[positions] == t] for t in range(T)])
    gpu_off = np.empty(len(offs_m), np.int64)
    gpu_off[r_ro] = rowid[order]
    w_r, s_r = rorc.get_rows(offs_m)
    w_g, s_g = gpu.rows(gpu_off)
    _compare_updated(w_g, s_g, w_prev, w_r, s_r, rtol, "sampled updated rows")
    _say(f"  {len(pick)} sampled updated rows match ({len(positions)} lookups)")
    # sampled untouched rows keep their initial values exactly
    total = int(wl.card.sum())
    cand = np.setdiff1d(rng.choice(total, 4 * n_rows_sample, replace=False), uniq)[:n_rows_sample]
    t_of = np.searchsorted(base, cand, side="right") - 1
    u_ids = np.concatenate([wl.keys(t, (cand[t_of == t] - base[t]).astype(np.uint64)) for t in range(T)])
    u_tab = np.concatenate([np.full(int((t_of == t).sum()), t) for t in range(T)])
    u_off = np.concatenate([cand[t_of == t] for t in range(T)])
    u_bounds = np.zeros(T + 1, np.int64)
    np.cumsum(np.bincount(u_tab, minlength=T), out=u_bounds[1:])
    uorc = make_oracle(cfg)
    u_ro, _ = uorc.find_or_insert(u_ids, u_bounds, 1)
    w_r, s_r = uorc.get_rows(u_ro)
    w_g, s_g = gpu.rows(u_off)
    assert np.array_equal(w_g.view(np.uint32), w_r.view(np.uint32)), "untouched rows differ from their init"
    assert not s_g.any()
    _say(f"  {len(u_off)} sampled untouched rows hold their initial values")


def test_billion_scale_id_space_full_size_sampled():
    """1 table of 2e8 live int64 keys at map load 0.7 (153.6 GB of rows),
    batch 131,072 bags of 50 uniform lookups, dim 64, Adam."""
    _free()
    free, _ = torch.cuda.mem_get_info()
    if free < 170 * 2**30:
        pytest.skip(f"needs ~170 GiB of free device memory, {free / 2**30:.0f} GiB free")
    try:
        _sampled_checks(synth.config(4), map_load=0.7, n_rows_sample=512, n_bag_sample=256)
    finally:
        _free()


def test_merged_bf16_full_size_sampled():
    """100 merged tables x 1M keys (1e8 rows, bf16 weights + fp32 Adagrad
    state), batch 32,768, Poisson(20) bags: ~65.5M lookups per step."""
    _free()
    try:
        _sampled_checks(synth.config(5), map_load=0.5, n_rows_sample=512, n_bag_sample=32)
    finally:
        _free()
