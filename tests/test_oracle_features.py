"""Pins of the feature-transform oracle ("RecIS：阿里开源推荐系统统一训练框架",
"Feature Engine": Hash, Mod, Bucketize): XXH64 against the xxhash library,
Mod against Python's integer `%` and the page's modulo example, Bucketize
against numpy.searchsorted, and whole programs against those references
composed element by element."""

import os

import numpy as np
import pytest
import xxhash

from oracle import features as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EDGE_INTS = np.array([0, 1, -1, 2**63 - 1, -(2**63), 562, 721458, 1180210], np.int64)


def _xxh_lib(x: int, seed: int) -> int:
    return xxhash.xxh64_intdigest(int(x).to_bytes(8, "little", signed=True), seed=seed)


@pytest.mark.parametrize("seed", [0, 1, 12345, 2**64 - 1, 2**63 + 7])
def test_xxh64_matches_the_library(seed):
    rng = np.random.default_rng(seed % 1000)
    v = np.concatenate([EDGE_INTS, rng.integers(-(2**63), 2**63 - 1, 500, dtype=np.int64)])
    got = F.xxh64_u64(v.view(np.uint64), seed)
    ref = np.array([_xxh_lib(x, seed) for x in v.tolist()], np.uint64)
    assert np.array_equal(got, ref)


def test_mod_is_python_floor_mod_and_the_pages_example():
    vals = {}
    with open(os.path.join(GOLDEN, "modulo_collision.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    r = F.floor_mod(np.array([vals["id_a"], vals["id_b"]], np.int64), vals["slice_len"])
    assert list(r) == [vals["residue"], vals["residue"]]
    rng = np.random.default_rng(3)
    v = np.concatenate([EDGE_INTS, rng.integers(-(2**63), 2**63 - 1, 300, dtype=np.int64)])
    for m in (1, 2, 7, 65536, 2**40 + 3, 2**63 - 1):
        got = F.floor_mod(v, m)
        assert [int(x) for x in got] == [x % m for x in v.tolist()]
        assert (got >= 0).all() and (got < m).all()


def test_bucketize_is_searchsorted_right():
    rng = np.random.default_rng(5)
    b = np.sort(rng.standard_normal(37))
    b = np.concatenate([b[:10], b[9:10], b[10:]])            # a repeated boundary
    x = np.concatenate([rng.standard_normal(400) * 2, b, [np.inf, -np.inf, np.nan, 0.0, -0.0]])
    got = F.bucketize(x, b)
    ref = np.searchsorted(b, x, side="right")                 # numpy sorts NaN last
    assert np.array_equal(got, ref)
    assert got[-3] == len(b) and got[-4] == 0
    assert np.array_equal(F.bucketize(x, np.zeros(0)), np.zeros(x.size, np.int64))


def test_programs_compose_the_ops_in_order():
    rng = np.random.default_rng(11)
    ints = rng.integers(-(2**40), 2**40, 200, dtype=np.int64)
    floats = rng.standard_normal(150) * 10
    floats[::17] = np.nan
    bnd = np.linspace(-20, 20, 33)
    progs = [
        F.Program(F.INT64, [(F.HASH, 7), (F.MOD, 1000)]),
        F.Program(F.FLOAT64, [(F.BUCKETIZE, bnd), (F.MOD, 5)]),
        F.Program(F.INT64, []),
        F.Program(F.FLOAT64, [(F.HASH, 99)]),
        F.Program(F.INT64, [(F.MOD, 97), (F.HASH, 3), (F.MOD, 11)]),
    ]
    cols = [ints[:80], floats[:100].view(np.int64), ints[80:130], floats[100:].view(np.int64), ints[130:]]
    raw = np.concatenate(cols)
    bounds = np.concatenate([[0], np.cumsum([len(c) for c in cols])])
    out = F.transform(raw, bounds, progs)

    def signed(u):
        return u - 2**64 if u >= 2**63 else u

    ref = []
    ref += [signed(_xxh_lib(x, 7)) % 1000 for x in cols[0].tolist()]
    ref += [int(k) % 5 for k in np.searchsorted(bnd, cols[1].view(np.float64), side="right")]
    ref += cols[2].tolist()
    ref += [signed(_xxh_lib(x, 99)) for x in cols[3].tolist()]
    ref += [signed(_xxh_lib(x % 97, 3)) % 11 for x in cols[4].tolist()]
    assert out.tolist() == ref


def test_invalid_programs_are_rejected():
    b = np.array([0.0, 1.0])
    assert not F.Program(F.FLOAT64, []).valid()                         # ends as a float
    assert not F.Program(F.FLOAT64, [(F.MOD, 3)]).valid()               # mod of a float
    assert not F.Program(F.INT64, [(F.BUCKETIZE, b)]).valid()           # bucketize of an int
    assert not F.Program(F.FLOAT64, [(F.BUCKETIZE, b[::-1])]).valid()   # boundaries descending
    assert not F.Program(F.INT64, [(F.MOD, 0)]).valid()
    assert not F.Program(F.INT64, [(F.MOD, 2)] * 5).valid()             # more than four ops
    assert F.Program(F.FLOAT64, [(F.BUCKETIZE, b), (F.HASH, 1), (F.MOD, 2)]).valid()
    with pytest.raises(ValueError):
        F.transform(np.zeros(2, np.int64), np.array([0, 2]), [F.Program(F.FLOAT64, [])])
