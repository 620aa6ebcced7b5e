"""Seeded input generators: determinism, key distinctness, Zipf shape."""

import numpy as np

import synth


def test_deterministic_and_layout():
    w1 = synth.Workload(synth.config(3, batch=64, cardinality=("fixed", 5000)))
    w2 = synth.Workload(synth.config(3, batch=64, cardinality=("fixed", 5000)))
    a_ids, a_bo = w1.batch_inputs(2)
    w1.batch_inputs(0)                       # call order must not matter
    b_ids, b_bo = w2.batch_inputs(2)
    assert np.array_equal(a_ids, b_ids) and np.array_equal(a_bo, b_bo)
    assert a_bo[0] == 0 and a_bo[-1] == len(a_ids) and np.all(np.diff(a_bo) >= 1)
    assert np.all(np.diff(a_bo) <= 100) and len(a_bo) == 4 * 64 + 1
    g = w1.grad(1)
    assert g.shape == (64, 4, 64) and g.dtype == np.float32
    assert np.array_equal(g, w2.grad(1))


def test_keys_distinct_and_in_range():
    for n, bits in ((2, 63), (4, 64), (5, 56)):
        w = synth.Workload(synth.config(n, cardinality=("fixed", 200_000)))
        u = w.universe(0)
        assert len(np.unique(u)) == len(u)
        if bits == 63:
            assert u.min() >= 0
        if bits == 56:
            assert u.min() >= 0 and u.max() < 2**56
        if bits == 64:
            assert u.min() < 0 < u.max()      # covers the whole signed range


def test_fresh_keys_never_seen():
    w = synth.Workload(synth.config(3, batch=256, cardinality=("fixed", 1000)))
    seen = set(w.universe(0).tolist())
    ids, bo = w.batch_inputs(0)
    t0 = ids[bo[0]:bo[256]]
    fresh = [k for k in t0.tolist() if k not in seen]
    assert len(fresh) == int(round(len(t0) * 0.01))
    ids1, bo1 = w.batch_inputs(1)
    fresh1 = [k for k in ids1[bo1[0]:bo1[256]].tolist() if k not in seen]
    assert not set(fresh) & set(fresh1)


def test_zipf_frequencies():
    w = synth.Workload(synth.config(1))
    rng = np.random.default_rng(0)
    n, a = 1000, 1.05
    r = w.zipf_ranks(n, 400_000, rng)
    assert r.min() >= 0 and r.max() < n
    freq = np.bincount(r, minlength=n) / len(r)
    p = np.arange(1, n + 1, dtype=np.float64) ** -a
    p /= p.sum()
    for k in (0, 1, 9, 99):
        assert abs(freq[k] - p[k]) < 5 * np.sqrt(p[k] / len(r)) + 1e-4


def test_loguniform_cardinalities():
    w = synth.Workload(synth.config(2))
    assert len(w.card) == 26 and w.card.min() >= 10 and w.card.max() <= 40_000_000


def test_prepopulation_pieces_cover_universe():
    w = synth.Workload(synth.config(2, batch=16, cardinality=("fixed", 1000)))
    whole = list(w.prepopulation())
    assert len(whole) == 1 and len(whole[0][0]) == 26 * 1000
    pieces = list(w.prepopulation(chunk=300))
    ids = np.concatenate([p[0] for p in pieces])
    assert np.array_equal(ids, whole[0][0])
    for pid, b in pieces:
        assert b[0] == 0 and b[-1] == len(pid)


def test_batch_counters_describe_the_same_batch():
    """batch_counters gives each lookup's table and generation counter: the
    keys they map to are batch_inputs' ids, and prepopulated counters index
    the universe (the insertion order)."""
    for n, kw in ((2, dict(batch=64, cardinality=("fixed", 1000))), (3, dict(batch=32)),
                  (5, dict(batch=16, n_tables=5, cardinality=("fixed", 1000)))):
        cfg = synth.config(n, **kw)
        wl = synth.Workload(cfg)
        ids, bo = wl.batch_inputs(2)
        counters, table, bo2 = wl.batch_counters(2)
        assert np.array_equal(bo, bo2)
        assert np.all(np.diff(table) >= 0)                      # table-major
        keys = np.concatenate([wl.keys(t, counters[table == t]) for t in range(cfg.n_tables)])
        assert np.array_equal(keys, ids)
        old = counters < wl.card[table]
        for t in range(cfg.n_tables):
            m = old & (table == t)
            assert np.array_equal(wl.universe(t)[counters[m].astype(np.int64)], ids[m])
