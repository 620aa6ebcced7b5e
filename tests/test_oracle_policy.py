"""Pins of the oracle's feature admission, age tracking, eviction and row
recycling ("RecIS：阿里开源推荐系统统一训练框架", "代码架构": a hook on the hash
table for feature admission and eviction; the policies are definitions
stated in the oracle's header).

Each pin checks the oracle against something it does not compute itself:
the closed form of a one-counter sketch, exact per-key counts (a sketch
wide enough to have no collisions must agree with them), the count-min
invariants, last-seen clocks and free lists derived with Python sets and
dicts from the stream the test itself generates, and the initial value of a
row (pinned to its closed form in test_oracle_pins)."""

import numpy as np
import pytest

import oracle

INT64_MIN = -(2**63)


def _bounds(per_table):
    """Table-major bounds (stride 1) from per-table id lists."""
    ids = np.concatenate([np.asarray(x, np.int64) for x in per_table]) if per_table else np.zeros(0, np.int64)
    b = np.zeros(len(per_table) + 1, np.int64)
    b[1:] = np.cumsum([len(x) for x in per_table])
    return ids, b


def _find(orc, per_table, insert=True):
    ids, b = _bounds(per_table)
    return orc.find_or_insert(ids, b, 1, insert)


def test_one_counter_sketch_is_a_global_count():
    """Width 1: every key shares each row's single counter, so the estimate
    is the number of absent-key lookups counted so far, for any depth."""
    for depth in (1, 3):
        orc = oracle.OracleTable(4, n_tables=1)
        orc.set_admission(5, width=1, depth=depth)
        ro, n = _find(orc, [[1, 2, 1]])                 # 3 counted: below 5
        assert n == 0 and list(ro) == [-1, -1, -1] and orc.n_rows == 0
        ro, n = _find(orc, [[3, 1]])                    # 5 counted: both admitted, first-sight order
        assert n == 2 and list(ro) == [0, 1]
        ro, n = _find(orc, [[1, 9, 9]])                 # 1 present (not counted); 9 twice -> 7
        assert n == 1 and list(ro) == [1, 2, 2]
        assert list(orc.sketch()) == [7] * depth
        ro, n = _find(orc, [[11]], insert=False)        # a lookup without insert counts nothing
        assert list(ro) == [-1] and list(orc.sketch()) == [7] * depth


def test_threshold_one_or_zero_is_admission_off():
    for thr in (0, 1):
        orc = oracle.OracleTable(4, n_tables=1)
        orc.set_admission(thr, width=64, depth=2)
        ro, n = _find(orc, [[4, 5, 4]])
        assert list(ro) == [0, 1, 0] and n == 2 and orc.sketch().size == 0


def _stream(seed, n_tables, n_calls, per_call, n_ids):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_calls):
        out.append([list((rng.zipf(1.3, per_call) % n_ids).astype(np.int64)) for _ in range(n_tables)])
    return out


def test_wide_sketch_matches_exact_counts():
    """A sketch far wider than the number of keys has no collisions here, so
    admission must follow the exact rule: a key absent at the start of a call
    is admitted once its count of absent lookups (this call's included)
    reaches the threshold; new keys get offsets in first-sight order."""
    T, thr = 3, 3
    orc = oracle.OracleTable(4, n_tables=T)
    orc.set_admission(thr, width=1 << 22, depth=4, seed=77)
    count, present, n_rows = {}, {}, 0
    for call in _stream(5, T, 6, 300, 4000):
        for t, ids in enumerate(call):
            for x in ids:
                if (t, x) not in present:
                    count[(t, x)] = count.get((t, x), 0) + 1
        want = []
        for t, ids in enumerate(call):
            for x in ids:
                if (t, x) in present:
                    want.append(present[(t, x)])
                elif count[(t, x)] >= thr:
                    present[(t, x)] = n_rows
                    n_rows += 1
                    want.append(present[(t, x)])
                else:
                    want.append(-1)
        ro, _ = _find(orc, call)
        assert list(ro) == want
        # the estimates of every counted key equal the exact counts
        for (t, x), c in list(count.items())[:200]:
            assert orc.estimate(x, t) == c
    assert orc.n_rows == n_rows


def test_count_min_invariants_on_a_narrow_sketch():
    """Width 16: collisions are certain, yet each row's counters sum to the
    number of counted lookups and no estimate is below the exact count."""
    T, depth, width = 2, 3, 16
    orc = oracle.OracleTable(4, n_tables=T)
    orc.set_admission(1000, width=width, depth=depth, seed=3)   # nothing admitted: every lookup counts
    count, total = {}, 0
    for call in _stream(9, T, 4, 200, 500):
        for t, ids in enumerate(call):
            for x in ids:
                count[(t, x)] = count.get((t, x), 0) + 1
                total += 1
        ro, n = _find(orc, call)
        assert n == 0 and (ro == -1).all()
    sk = orc.sketch().reshape(depth, width).astype(np.int64)
    assert (sk.sum(axis=1) == total).all()
    for (t, x), c in count.items():
        e = orc.estimate(x, t)
        assert c <= e <= total
    # the sketch of a table is not the sketch of another: map index is hashed
    assert any(orc.estimate(x, 0) != orc.estimate(x, 1) for x in range(50))


def test_stamps_are_the_clock_of_the_last_lookup():
    orc = oracle.OracleTable(4, n_tables=1)
    orc.set_tracking(True)
    last = {}
    for clock, ids in enumerate([[1, 2, 3], [2, 4], [1], [5, 2]], start=1):
        orc.set_clock(clock)
        ro, _ = _find(orc, [ids])
        for x in ids:
            last[x] = clock
        _find(orc, [[6]], insert=False)                  # a miss without insert stamps nothing
    keys, _, offs = orc.entries()
    ls = orc.last_seen()
    assert {int(k): int(ls[o]) for k, o in zip(keys, offs)} == last


@pytest.mark.parametrize("merged", [False, True])
def test_eviction_keeps_offsets_and_recycles_ascending(merged):
    T = 3
    orc = oracle.OracleTable(8, optim=oracle.OPT_ADAGRAD, n_tables=T, merged=merged, seed=11)
    orc.set_tracking(True)
    orc.set_recycling(True)
    last, where = {}, {}
    calls = _stream(21, T, 5, 40, 60)
    for clock, call in enumerate(calls, start=1):
        orc.set_clock(clock)
        ro, _ = _find(orc, call)
        q = 0
        for t, ids in enumerate(call):
            for x in ids:
                k = (t, int(x))
                last[k] = clock
                where[k] = int(ro[q])
                q += 1
    n_rows = orc.n_rows
    assert n_rows == len(where)
    min_clock = 4
    kept = orc.rehash(min_clock)
    survivors = {k for k, c in last.items() if c >= min_clock}
    assert kept == len(survivors)
    keys, tabs, offs = orc.entries()
    got = {}
    for k, tb, o in zip(keys, tabs, offs):
        t = int(k) >> 56 if merged else int(tb)
        x = int(k) & ((1 << 56) - 1) if merged else int(k)
        got[(t, x)] = int(o)
    assert got == {k: where[k] for k in survivors}                   # offsets unchanged
    free, done = orc.free_list()
    assert done == 0 and list(free) == sorted(set(range(n_rows)) - set(got.values()))
    # evicted keys are absent to a lookup without insert
    gone = sorted(set(last) - survivors)[:10]
    per = [[x for (t, x) in gone if t == tt] for tt in range(T)]
    ro, _ = _find(orc, per, insert=False)
    assert (ro == -1).all()
    # new keys take the free rows in order, then new rows; their rows start
    # from the new key's initial value and zero state
    fresh = [[10_000 + i for i in range(len(free) // T + 2)] for _ in range(T)]
    ro, n = _find(orc, fresh)
    n_fresh = sum(len(x) for x in fresh)
    assert n == n_fresh
    expect = list(free) + list(range(n_rows, n_rows + max(0, n_fresh - len(free))))
    assert list(ro) == expect[:n_fresh]
    w, st = orc.get_rows(ro)
    q = 0
    for t, ids in enumerate(fresh):
        for x in ids:
            key = ((t << 56) | x) if merged else x
            m = 0 if merged else t
            assert [oracle.init_value(key, m, c, 11) for c in range(8)] == list(w[q].astype(np.float64))
            q += 1
    assert not st.any()
    assert orc.free_list()[0].size == max(0, len(free) - n_fresh)


def test_recycled_row_trains_like_a_fresh_row():
    """A key given a recycled row (after its previous owner was trained) and
    the same key inserted into an empty table train identically."""
    a = oracle.OracleTable(4, optim=oracle.OPT_ADAGRAD, n_tables=1, seed=2, lr=0.1)
    a.set_tracking(True)
    a.set_recycling(True)
    a.set_clock(1)
    ro, _ = _find(a, [[100, 200]])
    g = np.full((2, 1, 4), 0.5, np.float32)
    a.bwd_update(ro, np.array([0, 1, 2]), 2, g)
    a.set_clock(2)
    _find(a, [[200]])
    assert a.rehash(2) == 1                              # key 100 (row 0) evicted
    ro_a, _ = _find(a, [[300]])
    assert list(ro_a) == [0]
    b = oracle.OracleTable(4, optim=oracle.OPT_ADAGRAD, n_tables=1, seed=2, lr=0.1)
    ro_b, _ = _find(b, [[300]])
    g1 = np.array([[[0.25, -1.0, 2.0, 0.0]]], np.float32)
    a.bwd_update(ro_a, np.array([0, 1]), 1, g1)
    b.bwd_update(ro_b, np.array([0, 1]), 1, g1)
    wa, sa = a.get_rows(ro_a)
    wb, sb = b.get_rows(ro_b)
    assert np.array_equal(wa, wb) and np.array_equal(sa, sb)
    w200, _ = a.get_rows(np.array([1]))
    assert not np.array_equal(w200, wb)


def test_rehash_without_eviction_keeps_every_key():
    orc = oracle.OracleTable(4, n_tables=2)
    orc.set_recycling(True)
    _find(orc, [[1, 2, 3], [1, 4]])
    before = orc.entries()
    assert orc.rehash(5) == 5                            # tracking off: min_clock has no effect
    after = orc.entries()
    assert all(np.array_equal(x, y) for x, y in zip(before, after))
    assert orc.free_list()[0].size == 0
    orc.set_tracking(True)                               # stamps restart at 0
    assert orc.rehash(0) == 5 and orc.rehash(1) == 0
    assert list(orc.free_list()[0]) == [0, 1, 2, 3, 4]


def test_side_key_is_evicted_and_readmitted():
    orc = oracle.OracleTable(4, n_tables=1)
    orc.set_tracking(True)
    orc.set_recycling(True)
    orc.set_clock(1)
    ro, _ = _find(orc, [[INT64_MIN, 7]])
    assert list(ro) == [0, 1]
    orc.set_clock(2)
    _find(orc, [[7]])
    orc.rehash(2)
    ro, _ = _find(orc, [[INT64_MIN]], insert=False)
    assert list(ro) == [-1]
    ro, n = _find(orc, [[INT64_MIN]])
    assert list(ro) == [0] and n == 1


def test_admission_with_recycling_and_eviction_together():
    """A key evicted and seen again is absent, counted again, and -- its old
    counts still in the sketch -- admitted at once, into a recycled row."""
    orc = oracle.OracleTable(4, n_tables=1)
    orc.set_admission(2, width=1 << 16, depth=2)
    orc.set_tracking(True)
    orc.set_recycling(True)
    orc.set_clock(1)
    assert list(_find(orc, [[8, 8, 9]])[0]) == [0, 0, -1]   # 8 counted twice; 9 once
    orc.set_clock(2)
    assert list(_find(orc, [[9, 10]])[0]) == [1, -1]
    orc.set_clock(3)
    _find(orc, [[9]])
    orc.rehash(3)                                        # 8 (row 0) evicted
    assert list(orc.free_list()[0]) == [0]
    orc.set_clock(4)
    ro, n = _find(orc, [[8, 10]])                        # 8: estimate 3 -> row 0; 10: 2 -> new row 2
    assert list(ro) == [0, 2] and n == 2
