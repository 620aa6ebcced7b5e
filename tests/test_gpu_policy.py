"""Feature admission, age tracking, eviction, row recycling and resize on the
GPU against the oracle ("RecIS：阿里开源推荐系统统一训练框架", "代码架构": the
hash-table hook for feature admission and eviction; "Embedding Engine": the
IDMap over EmbeddingBlocks).

Multi-step streams whose tables start empty and that keep meeting never-seen
ids: every step compares, bit for bit, the row offsets, the number of new
keys, the sketch counters, the row stamps; after every eviction the map's
entries and the free list; rows (recycled ones included) and pooled outputs
within the tolerance of the other parity tests."""

import numpy as np
import pytest
import torch

import synth
from harness import GpuTables, assert_close, compare_rows, make_oracle, pooled_magnitude, rtol_for

pytestmark = pytest.mark.gpu

INT64_MIN = -(2**63)


def _say(*a):
    print(*a, flush=True)


def _entries(m, n_max):
    k, t, o, cnt = m.export(n_max)
    order = torch.argsort(o)
    return k[order].cpu().numpy(), t[order].cpu().numpy(), o[order].cpu().numpy(), cnt


def _check_entries(gpu, orc, what):
    kr, tr, orr = orc.entries()
    kg, tg, og, cnt = _entries(gpu.map, len(kr) + 16)
    assert cnt == len(kr), f"{what}: {cnt} live keys, oracle {len(kr)}"
    assert np.array_equal(og, orr) and np.array_equal(kg, kr) and np.array_equal(tg, tr), what


def _check_free(gpu, orc, what):
    head, left = gpu.blocks.free_list()
    left_r, head_r = orc.free_list()
    assert head == head_r and np.array_equal(left.cpu().numpy(), left_r), what


def _check_policy_state(gpu, orc, what):
    if getattr(gpu.map, "sketch", None) is not None:
        assert np.array_equal(gpu.map.sketch.cpu().numpy().view(np.uint32), orc.sketch()), what + ": sketch"
    if getattr(gpu.map, "stamps", None) is not None:
        n = orc.n_rows
        assert np.array_equal(gpu.map.stamps[:n].cpu().numpy().view(np.uint32), orc.last_seen()), what + ": stamps"


def run_stream(cfg, steps, admit=None, evict_every=0, window=2, recycle=True, seed=5):
    """admit: (threshold, width, depth) or None."""
    wl = synth.Workload(cfg)
    orc = make_oracle(cfg)
    L = [len(wl.batch_inputs(s)[0]) for s in range(steps)]
    max_rows = int(wl.card.sum()) + sum(L) + 1024
    gpu = GpuTables(cfg, wl.card, max_rows, extra_keys=sum(L))
    gpu.map.track_age(gpu.blocks.capacity)
    orc.set_tracking(True)
    if admit:
        thr, width, depth = admit
        gpu.map.enable_admission(thr, width, depth, seed=seed)
        orc.set_admission(thr, width, depth, seed=seed)
    if recycle:
        gpu.blocks.enable_free_list()
        orc.set_recycling(True)
    for ids, bounds in wl.prepopulation():
        orc.find_or_insert(ids, bounds, 1)
        gpu.find_or_insert(ids, bounds, 1)
    n_evicted = n_recycled = 0
    for s in range(steps):
        clock = s + 1
        gpu.map.set_clock(clock)
        orc.set_clock(clock)
        ids, bo = wl.batch_inputs(s)
        free_before = orc.free_list()[0].size
        ro_g, nn_g = gpu.find_or_insert(ids, bo, cfg.batch)
        ro_r, nn_r = orc.find_or_insert(ids, bo, cfg.batch)
        n_recycled += free_before - orc.free_list()[0].size
        assert np.array_equal(ro_g.cpu().numpy(), ro_r), f"row offsets, step {s}"
        assert nn_g == nn_r, f"new keys, step {s}: {nn_g} vs {nn_r}"
        _check_policy_state(gpu, orc, f"step {s}")
        if recycle:
            _check_free(gpu, orc, f"free list after the lookups of step {s}")
        out_g = gpu.fwd(ro_g, bo)
        out_r = orc.fwd(ro_r, bo, cfg.batch, cfg.pooling)
        assert_close(out_g.cpu().numpy(), out_r, pooled_magnitude(orc, ro_r, bo, cfg), 1e-5, f"pooled, step {s}")
        offs = np.unique(ro_r[ro_r >= 0])
        prev_w, _ = orc.get_rows(offs)
        U_g = gpu.bwd(ro_g, bo, wl.grad(s))
        U_r = orc.bwd_update(ro_r, bo, cfg.batch, wl.grad(s), cfg.pooling)
        assert U_g == U_r
        compare_rows(gpu, orc, prev_w, offs, rtol_for(cfg.wdtype), f"rows, step {s}")
        if evict_every and (s + 1) % evict_every == 0:
            min_clock = clock - window + 1
            before = len(orc.entries()[0])
            gpu.map.evict(gpu.blocks, min_clock)
            kept = orc.rehash(min_clock)
            n_evicted += before - kept
            _check_entries(gpu, orc, f"map after eviction at step {s}")
            if recycle:
                _check_free(gpu, orc, f"free list after eviction at step {s}")
    used, st = gpu.blocks.status()
    assert st == 0 and used == orc.n_rows
    assert gpu.map.status()[0] == 0
    _check_entries(gpu, orc, "final map")
    return orc, gpu, n_evicted, n_recycled


@pytest.mark.parametrize("which", ["sequence_adam_mean", "merged_bf16_adagrad", "multi_hot_sgd"])
def test_admission_eviction_recycling_stream(which):
    if which == "sequence_adam_mean":
        # mean pooling, Adam, 5% never-seen ids per step, a narrow sketch
        # (collisions certain), eviction every 3 steps of keys idle for 2
        cfg = synth.config(3, n_tables=4, batch=1024, cardinality=("fixed", 20_000), fresh_frac=0.05,
                           prepopulate=False)
        args = dict(steps=8, admit=(2, 4096, 2), evict_every=3, window=2)
    elif which == "merged_bf16_adagrad":
        cfg = synth.config(5, n_tables=6, batch=256, cardinality=("fixed", 5_000), prepopulate=False)
        args = dict(steps=6, admit=(3, 1 << 16, 4), evict_every=2, window=2)
    else:
        cfg = synth.config(1, batch=512)
        args = dict(steps=7, admit=None, evict_every=2, window=1)
    orc, gpu, n_ev, n_rec = run_stream(cfg, **args)
    _say(f"  {which}: {orc.n_rows} rows, {n_ev} keys evicted, {n_rec} rows recycled")
    assert n_ev > 0 and n_rec > 0


def test_resize_when_full_then_continue():
    """A map far too small for the stream: a call that overflows commits
    nothing (IDMAP_FULL, no new keys); resizes into regions four times
    larger keep every entry, the same call is retried until it fits, and the
    stream continues in step with the oracle."""
    cfg = synth.config(1, batch=512)
    wl = synth.Workload(cfg)
    orc = make_oracle(cfg)
    gpu = GpuTables(cfg, wl.card, 200_000)
    gpu.map = gpu.rse.IdMap([64] * cfg.n_tables, max_load=0.7, device=gpu.dev)
    resized = 0
    for s in range(4):
        ids, bo = wl.batch_inputs(s)
        for _ in range(10):
            ro_g, nn_g = gpu.find_or_insert(ids, bo, cfg.batch)
            st, _ = gpu.map.status()
            if st == 0:
                break
            assert st == -4 and nn_g == 0                   # RSE_ERR_IDMAP_FULL, nothing inserted
            before = _entries(gpu.map, 1 << 20)
            gpu.map.clear_status()
            gpu.map.resize([4 * x for x in gpu.map.slots_per_table], gpu.blocks)
            after = _entries(gpu.map, 1 << 20)
            assert all(np.array_equal(x, y) for x, y in zip(before[:3], after[:3]))
            resized += 1
        assert gpu.map.status()[0] == 0
        ro_r, nn_r = orc.find_or_insert(ids, bo, cfg.batch)
        assert np.array_equal(ro_g.cpu().numpy(), ro_r) and nn_g == nn_r, f"step {s}"
        out = gpu.fwd(ro_g, bo)
        gpu.bwd(ro_g, bo, 2.0 * out)
        orc.bwd_update(ro_r, bo, cfg.batch, 2.0 * orc.fwd(ro_r, bo, cfg.batch, cfg.pooling), cfg.pooling)
    _say(f"  {resized} resizes, final slots per table {gpu.map.slots_per_table[0]}")
    assert resized >= 2
    _check_entries(gpu, orc, "after resizes")


def test_failed_rehash_changes_nothing():
    cfg = synth.config(1, batch=256)
    wl = synth.Workload(cfg)
    orc = make_oracle(cfg)
    gpu = GpuTables(cfg, wl.card, 100_000)
    gpu.map.track_age(gpu.blocks.capacity)
    orc.set_tracking(True)
    gpu.blocks.enable_free_list()
    orc.set_recycling(True)
    gpu.map.set_clock(1)
    orc.set_clock(1)
    ids, bo = wl.batch_inputs(0)
    gpu.find_or_insert(ids, bo, cfg.batch)
    orc.find_or_insert(ids, bo, cfg.batch)
    orc.rehash(0)
    gpu.map.evict(gpu.blocks, 0)                        # nothing evicted; free list rebuilt (empty)
    _check_free(gpu, orc, "free list")
    before = _entries(gpu.map, 1 << 20)
    with pytest.raises(gpu.rse.RseError):
        gpu.map.resize([16] * cfg.n_tables, gpu.blocks)  # far too small
    after = _entries(gpu.map, 1 << 20)
    assert all(np.array_equal(x, y) for x, y in zip(before[:3], after[:3]))
    _check_free(gpu, orc, "free list after the failed rehash")
    ids, bo = wl.batch_inputs(1)
    ro_g, _ = gpu.find_or_insert(ids, bo, cfg.batch)
    ro_r, _ = orc.find_or_insert(ids, bo, cfg.batch)
    assert np.array_equal(ro_g.cpu().numpy(), ro_r)


def test_side_key_eviction_and_admission_undo():
    """The empty-slot marker INT64_MIN as a key (held in the side slot) is
    stamped, evicted and re-admitted into its recycled row; a call that
    fails for lack of rows takes its sketch counts back."""
    import recommender_sparse_embedding_amd as rse
    import oracle

    dev = torch.device("cuda")
    m = rse.IdMap([256], max_load=0.7, device=dev)
    b = rse.EmbeddingBlocks(8, rse.F32, rse.ADAGRAD, rows_per_chunk_log2=4, seed=3, device=dev).grow(1)  # 16 rows
    m.track_age(16)
    m.enable_admission(2, 1024, 3, seed=9)
    b.enable_free_list()
    orc = oracle.OracleTable(8, oracle.W_F32, oracle.OPT_ADAGRAD, 1, False, seed=3)
    orc.set_tracking(True)
    orc.set_admission(2, 1024, 3, seed=9)
    orc.set_recycling(True)
    n_new = torch.zeros(1, dtype=torch.int64, device=dev)

    def call(ids, clock, expect_ok=True):
        m.set_clock(clock)
        t = torch.tensor(ids, dtype=torch.int64, device=dev)
        bo = torch.tensor([0, len(ids)], dtype=torch.int64, device=dev)
        ro = torch.empty_like(t)
        rse.idmap_find_or_insert(m, b, t, bo, 1, 1, ro, n_new)
        st, _ = m.status()
        if not expect_ok:
            assert st != 0 or b.status()[1] != 0 or int(n_new.item()) == 0
            return None
        orc.set_clock(clock)
        ro_r, nn_r = orc.find_or_insert(np.array(ids, np.int64), np.array([0, len(ids)]))
        assert st == 0 and np.array_equal(ro.cpu().numpy(), ro_r) and int(n_new.item()) == nn_r, (ids, ro, ro_r)
        assert np.array_equal(m.sketch.cpu().numpy().view(np.uint32), orc.sketch())
        assert np.array_equal(m.stamps[:orc.n_rows].cpu().numpy().view(np.uint32), orc.last_seen())
        return ro_r

    assert list(call([INT64_MIN, INT64_MIN, 5], 1)) == [0, 0, -1]
    assert list(call([5, 6, 6, 7], 2)) == [1, 2, 2, -1]
    call([6], 3)
    m.evict(b, 3)
    orc.rehash(3)
    _, left = b.free_list()
    assert list(left.cpu().numpy()) == list(orc.free_list()[0]) == [0, 1]
    assert list(call([INT64_MIN, 5], 4)) == [0, 1]          # both re-admitted into recycled rows, in order
    # 13 rows left; 14 distinct new keys seen twice each would need a 17th
    # row: the call fails and its counts are taken back
    sk_before = m.sketch.clone()
    big = [100 + i for i in range(14) for _ in range(2)]
    call(big, 5, expect_ok=False)
    assert torch.equal(m.sketch, sk_before)


def test_save_after_eviction_and_load_with_free_list(tmp_path):
    """The Saver writes only referenced rows; loading with free_list=True
    rebuilds the pending free list (the unreferenced rows below the row
    counter, ascending), and both runs continue with the same offsets and
    bit-identical rows."""
    import recommender_sparse_embedding_amd as rse

    cfg = synth.config(1, batch=512)
    orc, gpu, n_ev, _ = run_stream(cfg, steps=4, admit=None, evict_every=2, window=1)
    assert n_ev > 0
    path = str(tmp_path / "evicted.safetensors")
    rse.save(path, gpu.map, gpu.blocks, step=gpu.step)
    idm2, blk2, meta = rse.load(path, device="cuda", free_list=True)
    _, left_a = gpu.blocks.free_list()
    _, left_b = blk2.free_list()
    assert torch.equal(left_a, left_b) and left_b.numel() == orc.free_list()[0].size > 0
    ka = _entries(gpu.map, 1 << 20)
    kb = _entries(idm2, 1 << 20)
    assert all(np.array_equal(x, y) for x, y in zip(ka[:3], kb[:3]))
    wl = synth.Workload(cfg)
    ids, bo = wl.batch_inputs(10)
    ro_a, nn_a = gpu.find_or_insert(ids, bo, cfg.batch)
    t_ids, t_bo = torch.from_numpy(ids).cuda(), torch.from_numpy(bo).cuda()
    ro_b = torch.empty_like(t_ids)
    n_new = torch.zeros(1, dtype=torch.int64, device="cuda")
    rse.idmap_find_or_insert(idm2, blk2, t_ids, t_bo, cfg.batch, cfg.n_tables, ro_b, n_new)
    assert torch.equal(ro_a, ro_b) and nn_a == int(n_new.item())
    g = torch.from_numpy(wl.grad(10)).cuda()
    gpu.bwd(ro_a, bo, g)
    n_u = torch.zeros(1, dtype=torch.int64, device="cuda")
    rse.embedding_bag_bwd_update(blk2, ro_b, t_bo, cfg.n_tables, cfg.batch, cfg.pooling, g, gpu.optim,
                                 meta["step"] + 1, n_u)
    offs = torch.unique(ro_a[ro_a >= 0])
    wa, sa = gpu.blocks.read_rows(offs)
    wb, sb = blk2.read_rows(offs)
    assert torch.equal(wa.view(torch.int32), wb.view(torch.int32))


def test_admission_and_stamps_through_the_noalloc_find():
    """Admission and age tracking through idmap_find_or_insert_noalloc (its
    candidate lists live in the library's static scratch) equal the
    workspace find's, call after call."""
    import recommender_sparse_embedding_amd as rse

    dev = torch.device("cuda")
    rng = np.random.default_rng(31)
    objs = []
    for _ in range(2):
        m = rse.IdMap([1 << 16] * 2, max_load=0.7, hash_seed=4, device=dev)
        b = rse.EmbeddingBlocks(16, rse.F32, rse.SGD, rows_per_chunk_log2=14, seed=1, device=dev).grow(4)
        m.enable_admission(2, 2048, 3, seed=8)
        m.track_age(b.capacity)
        b.enable_free_list()
        objs.append((m, b))
    (m_a, b_a), (m_b, b_b) = objs
    n_new_a = torch.zeros(1, dtype=torch.int64, device=dev)
    n_new_b = torch.zeros(1, dtype=torch.int64, device=dev)
    for call, n in enumerate((40_000, 9_000, 25_000)):
        ids = rng.zipf(1.2, n).astype(np.int64) % 30_000
        bounds = np.array([0, n // 2, n], np.int64)
        t_ids, t_b = torch.from_numpy(ids).to(dev), torch.from_numpy(bounds).to(dev)
        ro_a, ro_b = torch.empty_like(t_ids), torch.empty_like(t_ids)
        for m in (m_a, m_b):
            m.set_clock(call + 1)
        rse.idmap_find_or_insert(m_a, b_a, t_ids, t_b, 1, 2, ro_a, n_new_a)
        rse.idmap_find_or_insert_noalloc(m_b, b_b, t_ids, t_b, 1, 2, ro_b, n_new_b)
        assert torch.equal(ro_a, ro_b) and int(n_new_a.item()) == int(n_new_b.item()), f"call {call}"
        assert torch.equal(m_a.sketch, m_b.sketch) and torch.equal(m_a.stamps, m_b.stamps)
        assert int((ro_a < 0).sum()) > 0                       # some keys not admitted yet
        if call == 1:
            m_a.evict(b_a, 2)
            m_b.evict(b_b, 2)
    assert m_a.status() == m_b.status() and m_a.status()[0] == 0


def test_stamps_carried_over_when_reattached_after_grow():
    import recommender_sparse_embedding_amd as rse

    dev = torch.device("cuda")
    m = rse.IdMap([256], max_load=0.7, device=dev)
    b = rse.EmbeddingBlocks(8, rse.F32, rse.SGD, rows_per_chunk_log2=4, device=dev).grow(1)   # 16 rows
    m.track_age(b.capacity)
    m.set_clock(5)
    n_new = torch.zeros(1, dtype=torch.int64, device=dev)
    ids = torch.arange(10, dtype=torch.int64, device=dev)
    bo = torch.tensor([0, 10], dtype=torch.int64, device=dev)
    ro = torch.empty_like(ids)
    rse.idmap_find_or_insert(m, b, ids, bo, 1, 1, ro, n_new)
    b.grow(1)                                                   # 32 rows: the stamps no longer cover it
    with pytest.raises(rse.RseError):
        rse.idmap_find_or_insert(m, b, ids, bo, 1, 1, ro, n_new)
    m.track_age(b.capacity)
    m.set_clock(6)
    ids2 = torch.arange(5, 25, dtype=torch.int64, device=dev)
    bo2 = torch.tensor([0, 20], dtype=torch.int64, device=dev)
    ro2 = torch.empty_like(ids2)
    rse.idmap_find_or_insert(m, b, ids2, bo2, 1, 1, ro2, n_new)
    st = m.stamps.cpu().numpy()
    assert list(st[:5]) == [5] * 5 and list(st[5:25]) == [6] * 20 and not st[25:].any()


def test_degenerate_cases():
    """An empty map rehashed (free list of every row below the counter:
    none); a call whose every absent key is below the admission threshold
    (no new rows, free list untouched, -1 everywhere); an empty feature
    batch."""
    import recommender_sparse_embedding_amd as rse

    dev = torch.device("cuda")
    m = rse.IdMap([128, 128], max_load=0.7, device=dev)
    b = rse.EmbeddingBlocks(8, rse.F32, rse.SGD, rows_per_chunk_log2=4, device=dev).grow(1)
    b.enable_free_list()
    m.track_age(b.capacity)
    m.evict(b, 5)                                   # nothing to keep, nothing to free
    assert m.status() == (0, [0, 0]) and b.free_list()[1].numel() == 0 and b.status()[0] == 0
    m.enable_admission(1000, 64, 2)
    ids = torch.tensor([1, 2, 2, 3, 7, 7], dtype=torch.int64, device=dev)
    bo = torch.tensor([0, 3, 6], dtype=torch.int64, device=dev)
    ro = torch.empty_like(ids)
    n_new = torch.zeros(1, dtype=torch.int64, device=dev)
    rse.idmap_find_or_insert(m, b, ids, bo, 1, 2, ro, n_new)
    assert bool((ro == -1).all()) and int(n_new.item()) == 0 and b.status()[0] == 0
    assert int(m.sketch.view(-1)[:64].sum().item()) == 6          # each row of the sketch counted 6 lookups
    ft = rse.FeatureTransform([(rse.FT_INT64, [(rse.FT_MOD, 7)])] * 2, device=dev)
    out = rse.feature_transform(ft, torch.zeros(0, dtype=torch.int64, device=dev),
                                torch.zeros(3, dtype=torch.int64, device=dev))
    assert out.numel() == 0 and ft.status() == 0
