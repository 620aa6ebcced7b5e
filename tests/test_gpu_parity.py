"""HIP path vs the CPU oracle, element by element, on seeded inputs.

Bar: bit-exact for row offsets, new-key counts, map contents, unique-row
counts and untouched rows; pooled outputs and updated rows within
1e-5 (fp32 storage) / 1e-2 (bf16 storage) of the oracle's magnitude bound.
"""

import numpy as np
import pytest
import torch

import synth
from harness import (ChunkSnapshot, GpuTables, assert_close, assert_never_touched_match_oracle,
                     assert_only_touched_changed, compare_rows, make_oracle, pooled_magnitude, rtol_for)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def run_steps(cfg, steps, prepop_chunk=None, max_new=None, split=False, rows_per_chunk_log2=14):
    """Free-running steps against the oracle: row offsets and new-key counts
    bit-exact, pooled outputs and updated rows within tolerance, the set of
    rows whose bytes change in each update a subset of the rows in the batch
    (every row compared on the device), and at the end every row never
    updated bit-identical to the oracle's."""
    wl = synth.Workload(cfg)
    orc = make_oracle(cfg)
    L_est = int(cfg.n_bags * (cfg.bag[2] if cfg.bag[0] == "uniform" else
                              cfg.bag[1] * 3 if cfg.bag[0] == "poisson" else cfg.bag[1]))
    max_rows = int(wl.card.sum() if cfg.prepopulate else 0) + (max_new or L_est * steps) + 1024
    extra = (max_new or L_est * steps) if (cfg.fresh_frac > 0 or not cfg.prepopulate) else 0
    gpu = GpuTables(cfg, wl.card, max_rows, extra_keys=extra, split=split,
                    rows_per_chunk_log2=rows_per_chunk_log2)
    rtol = rtol_for(cfg.wdtype)
    for ids, bounds in wl.prepopulation(prepop_chunk):
        ro_r, nn_r = orc.find_or_insert(ids, bounds, 1)
        ro_g, nn_g = gpu.find_or_insert(ids, bounds, 1)
        assert nn_g == nn_r
        assert np.array_equal(ro_g.cpu().numpy(), ro_r)
    ever = np.zeros(0, np.int64)
    for step in range(steps):
        _say(f"  step {step}")
        ids, bo = wl.batch_inputs(step)
        ro_r, nn_r = orc.find_or_insert(ids, bo, cfg.batch)
        ro_g, nn_g = gpu.find_or_insert(ids, bo, cfg.batch)
        assert nn_g == nn_r, (nn_g, nn_r)
        assert np.array_equal(ro_g.cpu().numpy(), ro_r), "row offsets"
        snap = ChunkSnapshot(gpu.blocks)
        gpu.prepare(ro_g, bo)
        out_g = gpu.fwd(ro_g, bo)
        out_r = orc.fwd(ro_r, bo, cfg.batch, cfg.pooling)
        assert_close(out_g.cpu().numpy(), out_r, pooled_magnitude(orc, ro_r, bo, cfg), rtol, "pooled output")
        if cfg.grad == "sumsq":           # loss = sum of squared pooled outputs
            G_r = (2.0 * out_r).astype(np.float32)
            G_g = 2.0 * out_g
        else:
            G_r = wl.grad(step)
            G_g = torch.from_numpy(G_r).to(gpu.dev)
        offs = np.unique(ro_r[ro_r >= 0])
        prev_w, _ = orc.get_rows(offs)
        U_r = orc.bwd_update(ro_r, bo, cfg.batch, G_r, cfg.pooling)
        U_g = gpu.bwd(ro_g, bo, G_g)
        assert U_g == U_r == len(offs)
        compare_rows(gpu, orc, prev_w, offs, rtol, f"step {step}")
        assert_only_touched_changed(snap, offs, f"step {step}")
        del snap
        ever = np.union1d(ever, offs)
    n_rest = assert_never_touched_match_oracle(gpu, orc, ever, f"after {steps} steps")
    _say(f"  {len(ever)} rows updated, {n_rest} never-updated rows bit-identical to the oracle")
    return gpu, orc


def test_toy_example():
    """10-row dim-4 table, ids {2,5,7}, loss sum(e^2), SGD 0.1."""
    cfg = synth.config(1, n_tables=1, batch=3, dim=4, bag=("fixed", 1), prepopulate=False)
    orc = make_oracle(cfg)
    gpu = GpuTables(cfg, [10], 64)
    keys = np.arange(10, dtype=np.int64)
    ro_g, n_g = gpu.find_or_insert(keys, np.array([0, 10]), 1)
    ro_r, n_r = orc.find_or_insert(keys, [0, 10])
    assert n_g == n_r == 10 and np.array_equal(ro_g.cpu().numpy(), ro_r)
    W0_g, _ = gpu.rows(np.arange(10))
    W0_r, _ = orc.get_rows(np.arange(10))
    assert np.array_equal(W0_g.view(np.uint32), W0_r.view(np.uint32)), "initial rows"
    ids = np.array([2, 5, 7], np.int64)
    bo = np.arange(4, dtype=np.int64)
    ro_g, _ = gpu.find_or_insert(ids, bo, 3)
    out = gpu.fwd(ro_g, bo)
    assert np.array_equal(out.cpu().numpy()[:, 0], W0_r[ids])
    assert gpu.bwd(ro_g, bo, 2.0 * out) == 3
    W1, _ = gpu.rows(np.arange(10))
    rest = [0, 1, 3, 4, 6, 8, 9]
    assert np.array_equal(W1[rest].view(np.uint32), W0_r[rest].view(np.uint32))
    ref = (W0_r[ids].astype(np.float64) - 0.1 * (2.0 * W0_r[ids].astype(np.float64))).astype(np.float32)
    assert np.array_equal(W1[ids], ref)


@pytest.mark.parametrize("merged", [False, True])
def test_idmap_edge_keys_bit_exact(merged):
    """Sentinel-valued key, extremes, the modulo-collision pair, duplicates,
    the same key in several tables; a crowded map (load 0.9)."""
    T = 3
    cfg = synth.config(1, n_tables=T, batch=1, dim=8, merged=merged, prepopulate=False)
    orc = make_oracle(cfg)
    rng = np.random.default_rng(0)
    hi = 2**56 if merged else 2**63
    special = [0, 1, 1180210, 721458, hi - 1]
    if not merged:
        special += [-(2**63), -1, 2**63 - 1, -(2**62)]
    n_per = 3000
    ids_t = []
    for t in range(T):
        base = rng.integers(0, hi, n_per - len(special) - 200, dtype=np.int64)
        dup = rng.choice(base, 200)
        x = np.concatenate([special, base, dup]).astype(np.int64)
        rng.shuffle(x)
        ids_t.append(x)
    ids = np.concatenate(ids_t)
    bounds = np.array([0, n_per, 2 * n_per, 3 * n_per], np.int64)
    gpu = GpuTables(cfg, [n_per] * T, 4 * T * n_per, load=0.85)
    ro_r, n_r = orc.find_or_insert(ids, bounds, 1)
    ro_g, n_g = gpu.find_or_insert(ids, bounds, 1)
    assert n_g == n_r
    assert np.array_equal(ro_g.cpu().numpy(), ro_r)
    # a second pass: everything hits; plus a few unseen keys without insert
    probe = np.concatenate([ids[:100], np.array([12345678901, 98765], np.int64), ids[-100:]])
    pb = np.array([0, 100, 102, 202], np.int64)
    r1, nn1 = orc.find_or_insert(probe, pb, 1, insert_missing=False)
    g1, ng1 = gpu.find_or_insert(probe, pb, 1, insert=False)
    assert nn1 == ng1 == 0 and np.array_equal(g1.cpu().numpy(), r1)
    assert (r1 == -1).sum() >= 1
    # map contents
    keys_r, tabs_r = orc.map_dump()
    k, tb, off, cnt = gpu.map.export(len(keys_r) + 10)
    assert cnt == len(keys_r)
    order = np.argsort(off.cpu().numpy())
    assert np.array_equal(off.cpu().numpy()[order], np.arange(len(keys_r)))
    assert np.array_equal(k.cpu().numpy()[order], keys_r)
    assert np.array_equal(tb.cpu().numpy()[order], tabs_r)
    # initial rows are the key-derived values
    offs = np.arange(0, len(keys_r), 7)
    w_g, _ = gpu.rows(offs)
    w_r, _ = orc.get_rows(offs)
    assert np.array_equal(w_g.view(np.uint32), w_r.view(np.uint32))


@pytest.mark.parametrize("dim,wdtype,pooling", [
    (4, 0, 0), (16, 0, 0), (32, 1, 0), (64, 0, 1), (128, 0, 0), (256, 0, 1), (8, 1, 1), (256, 1, 0)])
def test_forward_variants(dim, wdtype, pooling):
    """Short and long bags (both schedules), empty bags, duplicates."""
    for bag in (("uniform", 0, 6), ("uniform", 20, 140)):
        cfg = synth.config(1, n_tables=3, batch=300, dim=dim, wdtype=wdtype, pooling=pooling, bag=bag,
                           cardinality=("fixed", 500), prepopulate=True, zipf_a=1.1)
        run_steps(cfg, 1)


@pytest.mark.parametrize("dim,wdtype", [(4, 0), (16, 0), (32, 1), (64, 0), (128, 0), (128, 1), (256, 0)])
def test_forward_one_hot_chunks(dim, wdtype):
    """One-hot batches take the chunked kernel: chunks that are wholly
    one-hot (fast path), chunks holding an empty bag and a two-lookup bag,
    the ragged last chunk (per-bag path), and ids not in the map (offset -1,
    a zero row)."""
    cfg = synth.config(2, n_tables=3, batch=301, dim=dim, wdtype=wdtype, cardinality=("fixed", 400))
    wl = synth.Workload(cfg)
    orc = make_oracle(cfg)
    gpu = GpuTables(cfg, wl.card, int(wl.card.sum()) + 64)
    for ids, bounds in wl.prepopulation():
        orc.find_or_insert(ids, bounds, 1)
        gpu.find_or_insert(ids, bounds, 1)
    ids, bo = wl.batch_inputs(0)
    assert np.array_equal(bo, np.arange(cfg.n_bags + 1))
    bo = bo.copy()
    for j in (17, 100, 640):            # bag j empty, bag j + 1 takes its lookup
        bo[j + 1] = bo[j]
    ids = ids.copy()
    ids[[5, 200, 433]] = (1 << 62) + np.arange(3)          # never inserted
    ro_r, _ = orc.find_or_insert(ids, bo, cfg.batch, insert_missing=False)
    ro_g, _ = gpu.find_or_insert(ids, bo, cfg.batch, insert=False)
    assert np.array_equal(ro_g.cpu().numpy(), ro_r) and (ro_r == -1).sum() >= 3
    out_g = gpu.fwd(ro_g, bo).cpu().numpy()
    out_r = orc.fwd(ro_r, bo, cfg.batch, cfg.pooling)
    assert_close(out_g, out_r, pooled_magnitude(orc, ro_r, bo, cfg), rtol_for(wdtype), "one-hot pooled output")
    for j in (17, 100, 640):
        t, b = divmod(j, cfg.batch)
        assert not out_g[b, t].any(), "empty bag"


def test_forward_poisson_bags_per_bag_path():
    """Bag lengths Poisson(1): the one-hot kernel is chosen (mean <= 1.5) and
    most chunks fall back to the per-bag path."""
    cfg = synth.config(1, n_tables=4, batch=500, dim=64, bag=("poisson", 1.0), cardinality=("fixed", 2000),
                       prepopulate=True)
    run_steps(cfg, 2)


@pytest.mark.parametrize("optim", [0, 1, 2])
@pytest.mark.parametrize("wdtype", [0, 1])
def test_update_variants(optim, wdtype):
    """Every optimizer x storage type, hot keys with segments far beyond one
    piece, mean pooling for Adam."""
    cfg = synth.config(3, n_tables=2, batch=512, dim=32, wdtype=wdtype, optim=optim,
                       lr=[0.05, 0.01, 1e-3][optim], cardinality=("fixed", 20000), bag=("uniform", 1, 40),
                       fresh_frac=0.01, pooling=1 if optim == 2 else 0)
    run_steps(cfg, 3)


@pytest.mark.parametrize("optim", [0, 1, 2])
@pytest.mark.parametrize("wdtype", [0, 1])
@pytest.mark.parametrize("pooling", [0, 1])
def test_update_read_once_batches(optim, wdtype, pooling):
    """Batches with no more lookups than bags (bags of 0 or 1 lookups) take
    the update's streaming path (gradient rows and touched rows read and
    written with the nontemporal hint): every optimizer x storage type x
    pooling, with Zipf-hot rows whose segments span many pieces."""
    cfg = synth.config(2, n_tables=3, batch=4096, dim=32, wdtype=wdtype, optim=optim,
                       lr=[0.05, 0.01, 1e-3][optim], cardinality=("fixed", 3000), bag=("uniform", 0, 1),
                       pooling=pooling)
    run_steps(cfg, 2)


@pytest.mark.parametrize("which", ["one_hot", "short_bags", "long_bags"])
def test_global_chunk_table_path(which):
    """Blocks of more than 512 chunks (16-row chunks here) address rows
    through the chunk table in device memory instead of its LDS copy: find,
    insert and row init, the one-hot, group-per-bags and wave-per-bag
    forwards, and the update's one-lookup, short and long segments."""
    if which == "one_hot":      # one-hot forward, Adagrad dim 128
        cfg = synth.config(2, n_tables=4, batch=4096, cardinality=("fixed", 4000))
        gpu, _ = run_steps(cfg, 2, rows_per_chunk_log2=4, max_new=1024)
    elif which == "short_bags":  # bags U[1,8]: group-per-bags forward, SGD dim 16, tables start empty
        cfg = synth.config(1, n_tables=8, batch=1024, cardinality=("fixed", 2000))
        gpu, _ = run_steps(cfg, 3, rows_per_chunk_log2=4, max_new=16000)
    else:                        # bags U[1,100]: wave-per-bag forward, mean, Adam dim 64, fresh ids
        cfg = synth.config(3, n_tables=2, batch=256, cardinality=("fixed", 8000))
        gpu, _ = run_steps(cfg, 2, rows_per_chunk_log2=4, max_new=2048)
    assert len(gpu.blocks.chunks) > 512


def test_contiguous_chunks():
    """Chunks of 256 MiB or more, of rows that fill whole 128-byte lines,
    come from physically contiguous device allocations (outside torch's
    allocator) where the driver can place them: the same parity bar on a
    click-log twin whose 512 MiB chunks take that path, twice, and the second
    round returns all of its device memory when its blocks go (the first
    absorbs the runtime's one-time allocations: code objects, static
    scratch)."""
    import gc

    import recommender_sparse_embedding_amd as rse

    def settled_free():
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()      # torch's cached blocks are not counted
        return torch.cuda.mem_get_info()[0]

    cfg = synth.config(2, n_tables=8, batch=2048, cardinality=("loguniform", 10, 200_000))
    free = []
    for _ in range(2):
        torch_before = torch.cuda.memory_allocated()
        gpu, _ = run_steps(cfg, 2, rows_per_chunk_log2=19)
        chunk_bytes = gpu.blocks.rows_per_chunk * gpu.blocks.row_bytes
        assert chunk_bytes >= rse.CONTIGUOUS_MIN_BYTES and gpu.blocks.row_bytes % 128 == 0
        assert all(c.numel() == chunk_bytes for c in gpu.blocks.chunks)
        # the chunks are not torch allocations
        assert torch.cuda.memory_allocated() - torch_before < chunk_bytes
        n = len(gpu.blocks.chunks)
        del gpu
        free.append(settled_free())
    assert free[1] > free[0] - chunk_bytes // 4, f"{n} chunks of the second round not returned: {free}"


def test_config1_multi_hot_sgd_full():
    """8 tables, dim 16, batch 1024, bags U[1,8], Zipf(1.05) over 1e5 keys,
    sum-of-squares loss, SGD 0.1, tables start empty: 10 free-running steps."""
    run_steps(synth.config(1), 10)


def test_config2_click_log_twin():
    """26 one-hot tables, dim 128, Adagrad; batch 2048, cardinalities
    log-uniform in [10, 2e5]."""
    run_steps(synth.config(2, batch=2048, cardinality=("loguniform", 10, 200_000)), 3, prepop_chunk=100_000)


def test_config3_sequence_mean_adam_twin():
    run_steps(synth.config(3, batch=256, cardinality=("fixed", 50_000)), 3)


def test_config4_uniform_int64_twin():
    run_steps(synth.config(4, batch=1024, cardinality=("fixed", 200_000)), 2)


def test_config5_merged_bf16_twin():
    run_steps(synth.config(5, batch=128, cardinality=("fixed", 10_000)), 2)


@pytest.mark.parametrize("dim,wdtype,optim", [(128, synth.F32, synth.ADAGRAD), (32, synth.BF16, synth.ADAGRAD),
                                              (16, synth.F32, synth.SGD), (64, synth.F32, synth.ADAM)])
def test_long_segment_boundaries(dim, wdtype, optim):
    """Segments placed on purpose in the sorted order (rows are numbered in
    insertion order and the backward sorts by row): a segment whose head and
    end fall exactly on 64-lookup piece boundaries (and later ones on
    32-lookup boundaries, the piece length of narrow rows), segments of exactly 64
    lookups (the longest reduced by one group) and 65 (the shortest split
    into pieces), one-lookup and short segments between them, and hot rows
    spanning many pieces and more than one work-kernel window (8 pieces for
    dim 128 fp32, 16 for dim 64, 64 for dim 32 bf16 and dim 16).  Two steps
    with different lookup orders; pooled outputs, every row and the
    distinct-row count against the oracle."""
    counts = [64, 320, 64, 65, 1, 2, 63, 128, 129, 191, 1, 1, 9000, 130, 2 * 4096 + 64, 127, 3, 1, 640, 66,
              # from position 19,264 on: segments on 32-lookup piece boundaries
              # (the piece length of fp32 rows of dim 16 and less)
              12, 32, 33, 31, 96, 97, 1, 30, 65]
    K = len(counts)
    L = int(sum(counts))
    rng = np.random.default_rng(11)
    keys = rng.integers(0, 1 << 62, K, dtype=np.int64)
    assert len(np.unique(keys)) == K
    cfg = synth.config(2, n_tables=1, batch=L, dim=dim, wdtype=wdtype, optim=optim,
                       lr=0.1 if optim == synth.SGD else 0.01, cardinality=("fixed", K), seed=77)
    orc = make_oracle(cfg)
    gpu = GpuTables(cfg, [K], K + 1024)
    bounds = np.array([0, K], np.int64)
    ro_r, nn_r = orc.find_or_insert(keys, bounds, 1)
    ro_g, nn_g = gpu.find_or_insert(keys, bounds, 1)
    assert nn_g == nn_r == K
    assert np.array_equal(ro_g.cpu().numpy(), ro_r) and np.array_equal(ro_r, np.arange(K))
    bo = np.arange(L + 1, dtype=np.int64)
    rtol = rtol_for(wdtype)
    offs = np.arange(K, dtype=np.int64)
    for step in range(2):
        ids = keys[rng.permutation(np.repeat(np.arange(K), counts))]
        ro_r, _ = orc.find_or_insert(ids, bo, cfg.batch)
        ro_g, _ = gpu.find_or_insert(ids, bo, cfg.batch)
        assert np.array_equal(ro_g.cpu().numpy(), ro_r), f"row offsets, step {step}"
        out_g = gpu.fwd(ro_g, bo)
        out_r = orc.fwd(ro_r, bo, cfg.batch, cfg.pooling)
        assert_close(out_g.cpu().numpy(), out_r, pooled_magnitude(orc, ro_r, bo, cfg), rtol, "pooled output")
        G = rng.standard_normal((L, 1, dim)).astype(np.float32)
        prev_w, _ = orc.get_rows(offs)
        U_r = orc.bwd_update(ro_r, bo, cfg.batch, G, cfg.pooling)
        U_g = gpu.bwd(ro_g, bo, G)
        assert U_g == U_r == K
        compare_rows(gpu, orc, prev_w, offs, rtol, f"step {step}")


def test_run_to_run_bit_identical():
    cfg = synth.config(2, n_tables=4, batch=4096, cardinality=("fixed", 3000))
    res = []
    for _ in range(2):
        gpu, orc = run_steps(cfg, 2)
        w, s = gpu.rows(np.arange(orc.n_rows))
        res.append((w.view(np.uint32).copy(), s.view(np.uint32).copy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


# ------------------------------------------- backward in two halves ----
@pytest.mark.parametrize("which", ["click_log", "mean_adam_bf16"])
def test_split_backward_overlapping_forward(which):
    """embedding_bag_bwd_prepare on a side stream, concurrent with the
    forward; embedding_bag_bwd_apply after an event wait: same bar as the
    one-call update."""
    if which == "click_log":
        cfg = synth.config(2, batch=2048, cardinality=("loguniform", 10, 200_000))
        run_steps(cfg, 3, prepop_chunk=100_000, split=True)
    else:
        cfg = synth.config(3, n_tables=2, batch=512, dim=32, wdtype=1, optim=2, lr=1e-3,
                           cardinality=("fixed", 20000), bag=("uniform", 1, 40), fresh_frac=0.01, pooling=1)
        run_steps(cfg, 3, split=True)


@pytest.mark.parametrize("schedule", ["pipelined", "lookahead", "lookahead3"])
@pytest.mark.parametrize("which", ["click_log", "fresh_keys_adam"])
def test_pipelined_next_find_overlaps_apply(which, schedule):
    """Two-stream schedules.  pipelined: the find and sort of batch s+1 on a
    second stream run while batch s's forward and apply run on the first (the
    forward of s+1 waits for both).  lookahead: the second stream sorts batch
    s+1 (found a step earlier) and then finds batch s+2 while batch s runs.
    lookahead3: the same with the finds on a third stream, beside the sorts
    (a sort waits for its batch's find, the find of batch s+2 for the apply
    of batch s-1).  Every step matches the oracle run in plain order, including new keys
    inserted while earlier batches' rows are being updated."""
    if which == "click_log":
        cfg = synth.config(2, batch=2048, cardinality=("loguniform", 10, 200_000))
    else:
        cfg = synth.config(3, n_tables=2, batch=512, dim=32, cardinality=("fixed", 20000), bag=("uniform", 1, 40),
                           fresh_frac=0.05)
    steps = 4
    wl = synth.Workload(cfg)
    orc = make_oracle(cfg)
    L_max = max(len(wl.batch_inputs(s)[0]) for s in range(steps))
    gpu = GpuTables(cfg, wl.card, int(wl.card.sum()) + L_max * steps + 1024, extra_keys=L_max * steps)
    for ids, bounds in wl.prepopulation(100_000):
        orc.find_or_insert(ids, bounds, 1)
        gpu.find_or_insert(ids, bounds, 1)
    rse = gpu.rse
    dev = gpu.dev
    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(device=dev)
    finder = torch.cuda.Stream(device=dev) if schedule == "lookahead3" else side
    inputs = []
    for s in range(steps):
        ids, bo = wl.batch_inputs(s)
        inputs.append(dict(ids=torch.from_numpy(ids).to(dev), bo=torch.from_numpy(bo).to(dev),
                           ro=torch.empty(len(ids), dtype=torch.int64, device=dev),
                           out=torch.empty((cfg.batch, cfg.n_tables, cfg.dim), dtype=torch.float32, device=dev),
                           g=torch.from_numpy(wl.grad(s)).to(dev), nu=torch.zeros(1, dtype=torch.int64, device=dev)))
    torch.cuda.synchronize()
    ws = [rse.bwd_workspace(L_max, cfg.n_tables, cfg.batch, cfg.dim, dev) for _ in range(2)]
    fws = gpu.map.workspace(L_max)
    applied = [torch.cuda.Event(), torch.cuda.Event()]
    fronted = [torch.cuda.Event(), torch.cuda.Event()]
    plans = [None, None]
    n_new = torch.zeros(1, dtype=torch.int64, device=dev)

    found = [torch.cuda.Event() for _ in range(3)]

    def find(s):
        x = inputs[s]
        if schedule == "lookahead3":
            finder.wait_event(applied[(s - 1) % 2])     # the apply of batch s-3
        rse.idmap_find_or_insert(gpu.map, gpu.blocks, x["ids"], x["bo"], cfg.batch, cfg.n_tables, x["ro"], n_new,
                                 ws=fws, stream=finder)
        found[s % 3].record(finder)

    def prepare(s):
        x = inputs[s]
        side.wait_event(applied[s % 2])
        if schedule == "lookahead3":
            side.wait_event(found[s % 3])
        plans[s % 2] = rse.embedding_bag_bwd_prepare(gpu.blocks, x["ro"], x["bo"], cfg.n_tables, cfg.batch,
                                                     ws[s % 2], stream=side)
        fronted[s % 2].record(side)

    if schedule == "pipelined":
        find(0)
        prepare(0)
    else:
        find(0)
        prepare(0)
        find(1)
    for s in range(steps):
        if schedule == "pipelined":
            if s + 1 < steps:
                find(s + 1)
                prepare(s + 1)
        elif schedule == "lookahead":
            if s + 1 < steps:
                prepare(s + 1)
            if s + 2 < steps:
                find(s + 2)
        else:
            if s + 2 < steps:
                find(s + 2)
            if s + 1 < steps:
                prepare(s + 1)
        x = inputs[s]
        main.wait_event(found[s % 3])
        rse.embedding_bag_fwd(gpu.blocks, x["ro"], x["bo"], cfg.n_tables, cfg.batch, cfg.pooling, x["out"])
        main.wait_event(fronted[s % 2])
        rse.embedding_bag_bwd_apply(gpu.blocks, plans[s % 2], x["bo"], cfg.n_tables, cfg.batch, cfg.pooling,
                                    x["g"], gpu.optim, s + 1, x["nu"], ws[s % 2])
        applied[s % 2].record(main)
    torch.cuda.synchronize()
    touched = set()
    for s in range(steps):
        ids, bo = wl.batch_inputs(s)
        ro_r, _ = orc.find_or_insert(ids, bo, cfg.batch)
        assert np.array_equal(inputs[s]["ro"].cpu().numpy(), ro_r), f"row offsets, step {s}"
        out_r = orc.fwd(ro_r, bo, cfg.batch, cfg.pooling)
        assert_close(inputs[s]["out"].cpu().numpy(), out_r, pooled_magnitude(orc, ro_r, bo, cfg),
                     rtol_for(cfg.wdtype), f"pooled output, step {s}")
        U = orc.bwd_update(ro_r, bo, cfg.batch, wl.grad(s), cfg.pooling)
        assert int(inputs[s]["nu"].item()) == U
        touched |= set(np.unique(ro_r[ro_r >= 0]).tolist())
    offs = np.array(sorted(touched), dtype=np.int64)
    w_g, s_g = gpu.rows(offs)
    w_r, s_r = orc.get_rows(offs)
    assert_close(w_g, w_r, np.abs(w_r.astype(np.float64)) + 1e-3, rtol_for(cfg.wdtype), "rows after the steps")
    if s_r.size:
        assert_close(s_g, s_r, np.abs(s_r.astype(np.float64)) + 1e-30, 1e-5, "state after the steps")
    assert_never_touched_match_oracle(gpu, orc, offs, "after the pipelined steps")


def _small_split_setup(rows_per_chunk_log2=4, n_chunks=1):
    import recommender_sparse_embedding_amd as rse

    cfg = synth.config(1, n_tables=1, batch=12, dim=16, bag=("fixed", 1), prepopulate=False, optim=1,
                       lr=0.05)
    gpu = GpuTables(cfg, [1000], (1 << rows_per_chunk_log2) * n_chunks, rows_per_chunk_log2=rows_per_chunk_log2)
    return rse, cfg, gpu, make_oracle(cfg)


def test_plan_applied_twice_updates_twice():
    rse, cfg, gpu, orc = _small_split_setup()
    ids = np.array([3, 7, 3, 9, 11, 7, 3, 20, 21, 22, 3, 9], dtype=np.int64)
    bo = np.arange(13, dtype=np.int64)
    ro_r, _ = orc.find_or_insert(ids, bo, cfg.batch)
    ro_g, _ = gpu.find_or_insert(ids, bo, cfg.batch)
    assert np.array_equal(ro_g.cpu().numpy(), ro_r)
    G = np.random.default_rng(3).standard_normal((cfg.batch, 1, cfg.dim)).astype(np.float32)
    t_bo = torch.from_numpy(bo).cuda()
    ws = rse.bwd_workspace(len(ids), 1, cfg.batch, cfg.dim)
    plan = rse.embedding_bag_bwd_prepare(gpu.blocks, ro_g, t_bo, 1, cfg.batch, ws)
    for step in (1, 2):
        rse.embedding_bag_bwd_apply(gpu.blocks, plan, t_bo, 1, cfg.batch, cfg.pooling, torch.from_numpy(G).cuda(),
                                    gpu.optim, step, gpu.n_unique, ws)
        U = orc.bwd_update(ro_r, bo, cfg.batch, G, cfg.pooling)
        assert int(gpu.n_unique.item()) == U == 7
    offs = np.arange(orc.n_rows)
    w_g, s_g = gpu.rows(offs)
    w_r, s_r = orc.get_rows(offs)
    assert np.allclose(w_g, w_r, rtol=1e-6, atol=1e-7) and np.allclose(s_g, s_r, rtol=1e-6, atol=1e-7)


def test_blocks_grow_between_prepare_and_apply():
    """Lookups without a row sort under a key fixed at prepare time (2^5 - 1
    for 16 rows); after growing to 48 rows and inserting keys up to row 34,
    row 31 is real and must stay untouched by the apply."""
    rse, cfg, gpu, orc = _small_split_setup()
    base = np.arange(100, 110, dtype=np.int64)                   # rows 0..9
    orc.find_or_insert(base, np.array([0, 10]), 1)
    gpu.find_or_insert(base, np.array([0, 10]), 1)
    ids = np.array([100, 101, 555, 102, 100, 556, 103, 104, 557, 105, 100, 109], dtype=np.int64)
    bo = np.arange(13, dtype=np.int64)
    ro_r, _ = orc.find_or_insert(ids, bo, cfg.batch, insert_missing=False)
    ro_g, _ = gpu.find_or_insert(ids, bo, cfg.batch, insert=False)
    assert np.array_equal(ro_g.cpu().numpy(), ro_r) and (ro_r == -1).sum() == 3
    t_bo = torch.from_numpy(bo).cuda()
    ws = rse.bwd_workspace(len(ids), 1, cfg.batch, cfg.dim)
    plan = rse.embedding_bag_bwd_prepare(gpu.blocks, ro_g, t_bo, 1, cfg.batch, ws)
    assert plan.key_bits == 5 and plan.invalid == 31
    gpu.blocks.grow(2)
    more = np.arange(200, 225, dtype=np.int64)                   # rows 10..34
    orc.find_or_insert(more, np.array([0, 25]), 1)
    ro_m, n_m = gpu.find_or_insert(more, np.array([0, 25]), 1)
    assert n_m == 25 and int(ro_m[-1].item()) == 34
    G = np.random.default_rng(4).standard_normal((cfg.batch, 1, cfg.dim)).astype(np.float32)
    rse.embedding_bag_bwd_apply(gpu.blocks, plan, t_bo, 1, cfg.batch, cfg.pooling, torch.from_numpy(G).cuda(),
                                gpu.optim, 1, gpu.n_unique, ws)
    U = orc.bwd_update(ro_r, bo, cfg.batch, G, cfg.pooling)
    assert int(gpu.n_unique.item()) == U == 7
    offs = np.arange(35)
    w_g, s_g = gpu.rows(offs)
    w_r, s_r = orc.get_rows(offs)
    assert np.array_equal(w_g[10:].view(np.uint32), w_r[10:].view(np.uint32)), "rows inserted later changed"
    assert np.array_equal(s_g[10:].view(np.uint32), s_r[10:].view(np.uint32))
    assert np.allclose(w_g, w_r, rtol=1e-6, atol=1e-7) and np.allclose(s_g, s_r, rtol=1e-6, atol=1e-7)


def test_plan_mismatch_rejected():
    rse, cfg, gpu, orc = _small_split_setup()
    ids = np.arange(12, dtype=np.int64)
    bo = np.arange(13, dtype=np.int64)
    ro_g, _ = gpu.find_or_insert(ids, bo, cfg.batch)
    t_bo = torch.from_numpy(bo).cuda()
    ws = rse.bwd_workspace(len(ids), 1, cfg.batch, cfg.dim)
    plan = rse.embedding_bag_bwd_prepare(gpu.blocks, ro_g, t_bo, 1, cfg.batch, ws)
    G6 = torch.zeros((6, 1, cfg.dim), dtype=torch.float32, device="cuda")
    with pytest.raises(rse.RseError) as e:                     # 6 bags, the plan has 12
        rse.embedding_bag_bwd_apply(gpu.blocks, plan, torch.arange(7, device="cuda"), 1, 6, 0, G6, gpu.optim, 1,
                                    gpu.n_unique, ws)
    assert e.value.code == -1
    G = torch.zeros((cfg.batch, 1, cfg.dim), dtype=torch.float32, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(rse.RseError) as e:
        rse.embedding_bag_bwd_apply(gpu.blocks, plan, t_bo, 1, cfg.batch, 0, G, gpu.optim, 1, gpu.n_unique, small)
    assert e.value.code == -3
    del orc


def test_empty_batch_through_every_call():
    """A batch with no lookups at all (every bag empty): find writes no
    offsets and inserts nothing, the forward writes zeros, the backward
    (whole and in two halves) reports 0 distinct rows and changes no row."""
    import recommender_sparse_embedding_amd as rse

    cfg = synth.config(3, n_tables=3, batch=40, dim=16, cardinality=("fixed", 500), fresh_frac=0.0)
    wl = synth.Workload(cfg)
    gpu = GpuTables(cfg, wl.card, int(wl.card.sum()) + 1024)
    for ids, bounds in wl.prepopulation():
        gpu.find_or_insert(ids, bounds, 1)
    used0, _ = gpu.blocks.status()
    offs = np.arange(used0, dtype=np.int64)
    w0, s0 = gpu.rows(offs)
    ids = np.zeros(0, dtype=np.int64)
    bo = np.zeros(cfg.n_bags + 1, dtype=np.int64)
    ro, n_new = gpu.find_or_insert(ids, bo, cfg.batch)
    assert n_new == 0 and ro.numel() == 0
    out = gpu.fwd(ro, bo)
    assert out.shape == (cfg.batch, cfg.n_tables, cfg.dim) and not out.any()
    G = torch.ones((cfg.batch, cfg.n_tables, cfg.dim), dtype=torch.float32, device="cuda")
    gpu.n_unique.fill_(7)
    assert gpu.bwd(ro, bo, G) == 0
    t_bo = torch.from_numpy(bo).cuda()
    ws = rse.bwd_workspace(0, cfg.n_tables, cfg.batch, cfg.dim)
    plan = rse.embedding_bag_bwd_prepare(gpu.blocks, ro, t_bo, cfg.n_tables, cfg.batch, ws)
    gpu.n_unique.fill_(7)
    rse.embedding_bag_bwd_apply(gpu.blocks, plan, t_bo, cfg.n_tables, cfg.batch, cfg.pooling, G, gpu.optim, 2,
                                gpu.n_unique, ws)
    assert int(gpu.n_unique.item()) == 0
    used1, st = gpu.blocks.status()
    assert used1 == used0 and st == 0 and gpu.map.status()[0] == 0
    w1, s1 = gpu.rows(offs)
    assert np.array_equal(w0.view(np.uint32), w1.view(np.uint32))
    assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))


# ----------------------------------------------------------- failures ----
def test_need_grow_commits_nothing_and_retry_matches():
    cfg = synth.config(1, n_tables=1, batch=40, dim=16, bag=("fixed", 1), prepopulate=False)
    import recommender_sparse_embedding_amd as rse

    gpu = GpuTables(cfg, [1000], 16, rows_per_chunk_log2=4)     # one chunk of 16 rows
    orc = make_oracle(cfg)
    ids = np.arange(100, 140, dtype=np.int64)                   # 40 new keys > 16 rows
    ro, n = gpu.find_or_insert(ids, np.array([0, 40]), 1)
    assert n == 0 and np.all(ro.cpu().numpy() == -1)
    st, nkeys = gpu.map.status()
    assert st == -5 and nkeys == [0]
    assert gpu.map.export(100)[3] == 0
    gpu.blocks.grow(2)
    gpu.map.clear_status()
    ro, n = gpu.find_or_insert(ids, np.array([0, 40]), 1)
    ro_r, n_r = orc.find_or_insert(ids, [0, 40])
    assert n == n_r == 40 and np.array_equal(ro.cpu().numpy(), ro_r)
    assert gpu.map.status()[0] == 0
    w_g, _ = gpu.rows(np.arange(40))
    w_r, _ = orc.get_rows(np.arange(40))
    assert np.array_equal(w_g, w_r)


def test_idmap_full_commits_nothing():
    cfg = synth.config(1, n_tables=1, batch=1, dim=8, prepopulate=False)
    import recommender_sparse_embedding_amd as rse

    m = rse.IdMap([16], max_load=0.5, device="cuda")             # at most 8 keys
    b = rse.EmbeddingBlocks(8, 0, 0, 6, device="cuda").grow(1)
    n_new = torch.zeros(1, dtype=torch.int64, device="cuda")
    ids = torch.arange(10, dtype=torch.int64, device="cuda")
    ro = torch.empty_like(ids)
    rse.idmap_find_or_insert(m, b, ids, torch.tensor([0, 10], device="cuda"), 1, 1, ro, n_new)
    assert int(n_new.item()) == 0 and bool((ro == -1).all())
    assert m.status() == (-4, [0])
    assert b.status() == (0, 0)
    m.clear_status()
    rse.idmap_find_or_insert(m, b, ids[:6], torch.tensor([0, 6], device="cuda"), 1, 1, ro[:6], n_new)
    assert int(n_new.item()) == 6 and ro[:6].tolist() == list(range(6))
    assert m.status() == (0, [6]) and b.status() == (6, 0)
    del cfg


def test_bad_inputs_are_reported_not_faulted():
    import recommender_sparse_embedding_amd as rse

    # merged map: an id >= 2^56 is rejected, nothing inserted
    m = rse.IdMap([64], max_load=0.7, merged=True, device="cuda")
    b = rse.EmbeddingBlocks(8, 0, 0, 6, device="cuda").grow(1)
    n_new = torch.zeros(1, dtype=torch.int64, device="cuda")
    ids = torch.tensor([5, 2**56, 7], dtype=torch.int64, device="cuda")
    ro = torch.empty_like(ids)
    rse.idmap_find_or_insert(m, b, ids, torch.tensor([0, 3], device="cuda"), 1, 1, ro, n_new)
    assert int(n_new.item()) == 0 and m.status()[0] == -9 and bool((ro == -1).all())
    # forward with decreasing offsets and an out-of-range row: status, no fault
    m.clear_status()
    ro = torch.tensor([0, 1, 5000], dtype=torch.int64, device="cuda")
    rse.idmap_find_or_insert(m, b, ids[[0, 2]].contiguous(), torch.tensor([0, 2], device="cuda"), 1, 1,
                             ro[:2], n_new)
    out = torch.zeros((2, 1, 8), dtype=torch.float32, device="cuda")
    rse.embedding_bag_fwd(b, ro, torch.tensor([0, 3, 1], device="cuda"), 1, 2, 0, out)
    torch.cuda.synchronize()
    assert b.status()[1] == -9
    b.clear_status()
    rse.embedding_bag_fwd(b, ro, torch.tensor([0, 2, 3], device="cuda"), 1, 2, 0, out)
    assert b.status()[1] == -9                                  # row 5000 >= capacity 64
    b.clear_status()
    g = torch.ones((2, 1, 8), dtype=torch.float32, device="cuda")
    nu = torch.zeros(1, dtype=torch.int64, device="cuda")
    w0, _ = b.read_rows(torch.tensor([0, 1], device="cuda"))
    rse.embedding_bag_bwd_update(b, ro, torch.tensor([0, 2, 3], device="cuda"), 1, 2, 0, g,
                                 rse.Optim(0, 0.1), 1, nu)
    assert b.status()[1] == -9 and int(nu.item()) == 0
    w1, _ = b.read_rows(torch.tensor([0, 1], device="cuda"))
    assert torch.equal(w0, w1)                                  # nothing updated


def test_objects_alive_at_interpreter_exit_are_released_cleanly():
    """A process that ends while an IdMap and two EmbeddingBlocks (one with a
    torch chunk, one with a physically contiguous 256 MiB chunk) are still
    alive exits with status 0 and prints no error from their release."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import recommender_sparse_embedding_amd as rse\n"
            "m = rse.IdMap([64], max_load=0.7)\n"
            "b = rse.EmbeddingBlocks(16, rse.F32, rse.SGD, 6).grow(1)\n"
            "c = rse.EmbeddingBlocks(128, rse.F32, rse.ADAGRAD, 18).grow(1)\n"
            "assert c.chunks[0].numel() >= rse.CONTIGUOUS_MIN_BYTES\n"
            "print('alive', flush=True)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "alive" in r.stdout, r.stderr
    assert "Exception ignored" not in r.stderr and "Error" not in r.stderr.replace("amdgpu.ids", ""), r.stderr


def test_forward_offset_endpoints_checked_on_device():
    """bag_offsets[0] must be 0 and bag_offsets[n_bags] must equal n_ids:
    the forward reports either violation in the blocks' sticky status (every
    read stays within [0, n_ids]), for the one-hot and the multi-hot
    schedules alike."""
    import recommender_sparse_embedding_amd as rse

    b = rse.EmbeddingBlocks(8, 0, 0, 6, device="cuda").grow(1)
    m = rse.IdMap([64], max_load=0.7, device="cuda")
    n_new = torch.zeros(1, dtype=torch.int64, device="cuda")
    ids = torch.tensor([5, 6, 7], dtype=torch.int64, device="cuda")
    ro = torch.empty_like(ids)
    rse.idmap_find_or_insert(m, b, ids, torch.tensor([0, 3], device="cuda"), 1, 1, ro, n_new)
    out = torch.zeros((2, 1, 8), dtype=torch.float32, device="cuda")
    for bo in ([1, 2, 3], [0, 1, 2], [0, 2, 2], [1, 1, 3]):   # one-hot-like and multi-hot, bad ends
        b.clear_status()
        rse.embedding_bag_fwd(b, ro, torch.tensor(bo, device="cuda"), 1, 2, 0, out)
        assert b.status()[1] == -9, bo
    b.clear_status()
    rse.embedding_bag_fwd(b, ro, torch.tensor([0, 2, 3], device="cuda"), 1, 2, 0, out)
    assert b.status()[1] == 0
