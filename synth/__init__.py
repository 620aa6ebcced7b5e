"""Seeded synthetic inputs for the sparse-embedding training step.

This module only draws inputs: key universes, Zipf-distributed lookups, bag
lengths and upstream gradients.  It holds none of the method's arithmetic
(no hashing into the ID map, no pooling, no optimizer) and imports neither the
HIP library nor the oracle; both are fed from here.

Workloads (the shapes the pages' examples and problem statement describe):

1. multi-hot: 8 tables, dim 16 fp32, batch 1024, bags of U[1,8] ids, sum
   pooling, Zipf(1.05) over 1e5 keys per table, loss = sum of squared pooled
   outputs, SGD lr 0.1, tables start empty.
2. click-log: 26 one-hot tables, dim 128 fp32, batch 65536, per-table
   cardinality log-uniform in [10, 4e7], Zipf(1.1), Adagrad lr 0.01 eps 1e-8,
   N(0,1) upstream gradients.
3. behaviour sequence: 4 tables, dim 64 fp32, batch 8192, bags of U[1,100],
   mean pooling, Zipf(1.2) over 5e6 keys, 1% of each step's lookups are
   never-seen keys, Adam (0.9, 0.999).
4. billion-scale ID space: 1 table of 2e8 live keys uniform over all int64
   values, dim 64 fp32 + Adam, batch 131072 x 50 ids, sum pooling, map at
   load 0.7.
5. merged tables: 100 tables of dim 32 merged into one map keyed by
   (table << 56) | id, bf16 weights, fp32 Adagrad state, batch 32768, bags of
   Poisson(20) ids, Zipf(1.05) over 1e6 keys per table.

Keys: table t's key universe is ``keymix(counter)`` for counters 0..n-1,
where ``keymix`` is a seeded bijection of the key space (odd multipliers and
xor-shifts), so keys are distinct by construction and look uniform.  Fresh
keys use counters past n.  Popularity rank r maps to counter ``perm[r]`` for a
seeded permutation, so hot keys are scattered over insertion order.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

SUM, MEAN = 0, 1
SGD, ADAGRAD, ADAM = 0, 1, 2
F32, BF16 = 0, 1

_M64 = (1 << 64) - 1
FRESH_STRIDE = 1 << 28   # counters reserved per step for never-seen keys


@dataclasses.dataclass
class Config:
    name: str
    n_tables: int
    batch: int
    dim: int
    wdtype: int            # F32 | BF16
    pooling: int           # SUM | MEAN
    optim: int             # SGD | ADAGRAD | ADAM
    lr: float
    eps: float = 1e-8
    beta1: float = 0.9
    beta2: float = 0.999
    zipf_a: float = 1.05
    key_bits: int = 63     # 63: [0, 2^63); 64: all int64 values; 56: merged ids
    merged: bool = False
    bag: tuple = ("fixed", 1)   # ("uniform", lo, hi) | ("fixed", n) | ("poisson", mean)
    cardinality: tuple = ("fixed", 100000)  # ("fixed", n) | ("loguniform", lo, hi)
    query: str = "zipf"    # "zipf" | "uniform"
    fresh_frac: float = 0.0
    prepopulate: bool = True
    grad: str = "normal"   # "normal" | "sumsq" (G = 2 * out, from the caller)
    seed: int = 0

    @property
    def n_bags(self):
        return self.n_tables * self.batch


def config(n: int, **overrides) -> Config:
    """The five named workloads, optionally resized (e.g. batch=...)."""
    base = {
        1: Config("multi-hot sum, SGD", n_tables=8, batch=1024, dim=16, wdtype=F32, pooling=SUM,
                  optim=SGD, lr=0.1, zipf_a=1.05, bag=("uniform", 1, 8),
                  cardinality=("fixed", 100_000), prepopulate=False, grad="sumsq", seed=1001),
        2: Config("click-log one-hot, Adagrad", n_tables=26, batch=65536, dim=128, wdtype=F32,
                  pooling=SUM, optim=ADAGRAD, lr=0.01, eps=1e-8, zipf_a=1.1, bag=("fixed", 1),
                  cardinality=("loguniform", 10, 40_000_000), seed=1002),
        3: Config("behaviour sequence mean, Adam", n_tables=4, batch=8192, dim=64, wdtype=F32,
                  pooling=MEAN, optim=ADAM, lr=1e-3, eps=1e-8, zipf_a=1.2, bag=("uniform", 1, 100),
                  cardinality=("fixed", 5_000_000), fresh_frac=0.01, seed=1003),
        4: Config("billion-scale ID space, Adam", n_tables=1, batch=131072, dim=64, wdtype=F32,
                  pooling=SUM, optim=ADAM, lr=1e-3, eps=1e-8, key_bits=64, bag=("fixed", 50),
                  cardinality=("fixed", 200_000_000), query="uniform", seed=1004),
        5: Config("merged tables bf16, Adagrad", n_tables=100, batch=32768, dim=32, wdtype=BF16,
                  pooling=SUM, optim=ADAGRAD, lr=0.01, eps=1e-8, zipf_a=1.05, key_bits=56,
                  merged=True, bag=("poisson", 20), cardinality=("fixed", 1_000_000), seed=1005),
    }[n]
    return dataclasses.replace(base, **overrides)


# ---------------------------------------------------------------- keys ----
def _keymix(counter: np.ndarray, salt: int, bits: int) -> np.ndarray:
    """Seeded bijection on [0, 2^bits): odd multiplies and xor-shifts."""
    mask = np.uint64(_M64 if bits == 64 else (1 << bits) - 1)
    x = (counter.astype(np.uint64) ^ np.uint64(salt & int(mask))) & mask
    with np.errstate(over="ignore"):
        x = (x * np.uint64(0xD1342543DE82EF95)) & mask
        x ^= x >> np.uint64(bits // 2 + 1)
        x = (x * np.uint64(0xAEF17502108EF2D9)) & mask
        x ^= x >> np.uint64(bits // 2 - 3)
        x = (x * np.uint64(0x9FB21C651E98DF25)) & mask
        x ^= x >> np.uint64(bits // 3)
    return x.view(np.int64)


def _rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


class Workload:
    """Deterministic inputs of one configuration.

    ``batch_inputs(step)`` gives the lookups of one step in the table-major CSR
    layout: bag ``j = t * batch + b`` spans ``ids[bag_offsets[j]:bag_offsets[j+1]]``.
    """

    def __init__(self, cfg: Config):
        self.cfg = cfg
        r = _rng(cfg.seed, 0)
        kind = cfg.cardinality[0]
        if kind == "fixed":
            self.card = np.full(cfg.n_tables, cfg.cardinality[1], np.int64)
        else:
            lo, hi = cfg.cardinality[1], cfg.cardinality[2]
            self.card = np.rint(np.exp(r.uniform(math.log(lo), math.log(hi), cfg.n_tables))).astype(np.int64)
        self._salt = [int(s) for s in _rng(cfg.seed, 1).integers(0, 2**63, cfg.n_tables)]
        self._perm = {}
        self._cdf = {}

    # -- key universes
    def keys(self, t: int, counters: np.ndarray) -> np.ndarray:
        return _keymix(np.asarray(counters, np.uint64), self._salt[t], self.cfg.key_bits)

    def universe(self, t: int) -> np.ndarray:
        """Table t's live keys in generation (insertion) order."""
        return self.keys(t, np.arange(self.card[t], dtype=np.uint64))

    def prepopulation(self, chunk: int | None = None):
        """Pieces (ids, table_bounds) that insert every table's universe once,
        table by table in generation order; table t's ids of a piece are
        ``ids[bounds[t]:bounds[t+1]]``.  Empty if tables start empty.  With
        ``chunk``, no piece holds more than ``chunk`` ids."""
        cfg = self.cfg
        if not cfg.prepopulate:
            return
        T = cfg.n_tables
        if chunk is None:
            ids = np.concatenate([self.universe(t) for t in range(T)])
            bounds = np.zeros(T + 1, np.int64)
            np.cumsum(self.card, out=bounds[1:])
            yield ids, bounds
            return
        for t in range(T):
            for a in range(0, int(self.card[t]), chunk):
                b = min(a + chunk, int(self.card[t]))
                ids = self.keys(t, np.arange(a, b, dtype=np.uint64))
                bounds = np.zeros(T + 1, np.int64)
                bounds[t + 1:] = b - a
                yield ids, bounds

    def _rank_perm(self, t):
        if t not in self._perm:
            self._perm[t] = _rng(self.cfg.seed, 2, t).permutation(int(self.card[t])).astype(np.uint64)
        return self._perm[t]

    def _zipf_cdf(self, n):
        key = (n, self.cfg.zipf_a)
        if key not in self._cdf:
            ranks = np.arange(1, n + 1, dtype=np.float64)
            pmf = ranks ** (-self.cfg.zipf_a)
            cdf = np.cumsum(pmf)
            cdf /= cdf[-1]
            self._cdf[key] = cdf
        return self._cdf[key]

    def zipf_ranks(self, n_keys: int, count: int, rng: np.random.Generator) -> np.ndarray:
        """Finite Zipf: rank r in 1..n_keys with P(r) proportional to r^-a,
        returned 0-based, by inverse CDF."""
        cdf = self._zipf_cdf(int(n_keys))
        u = rng.random(count)
        return np.minimum(np.searchsorted(cdf, u, side="right"), n_keys - 1)

    def bag_lengths(self, rng: np.random.Generator) -> np.ndarray:
        cfg = self.cfg
        kind = cfg.bag[0]
        n = cfg.n_bags
        if kind == "fixed":
            return np.full(n, cfg.bag[1], np.int64)
        if kind == "uniform":
            return rng.integers(cfg.bag[1], cfg.bag[2] + 1, n).astype(np.int64)
        if kind == "poisson":
            return rng.poisson(cfg.bag[1], n).astype(np.int64)
        raise ValueError(kind)

    def batch_inputs(self, step: int):
        """ids int64[L], bag_offsets int64[T*B+1] for one step (step >= 0)."""
        ids, _, bo = self._batch(step, as_counters=False)
        return ids, bo

    def batch_counters(self, step: int):
        """The same step as generation counters: (counters uint64[L], table
        int32[L], bag_offsets).  Lookup i's id is keys(table[i], counters[i]);
        a prepopulated key's counter is its insertion index within its table."""
        counters, table, bo = self._batch(step, as_counters=True)
        return counters, table, bo

    def _batch(self, step: int, as_counters: bool):
        cfg = self.cfg
        r = _rng(cfg.seed, 3, step)
        lens = self.bag_lengths(r)
        bo = np.zeros(cfg.n_bags + 1, np.int64)
        np.cumsum(lens, out=bo[1:])
        ids = np.empty(int(bo[-1]), np.uint64 if as_counters else np.int64)
        table = np.empty(int(bo[-1]), np.int32) if as_counters else None
        for t in range(cfg.n_tables):
            a, b = int(bo[t * cfg.batch]), int(bo[(t + 1) * cfg.batch])
            n = b - a
            if n == 0:
                continue
            if cfg.query == "uniform":
                counters = r.integers(0, int(self.card[t]), n).astype(np.uint64)
            else:
                counters = self._rank_perm(t)[self.zipf_ranks(int(self.card[t]), n, r)]
            if cfg.fresh_frac > 0:
                # never-seen keys: counters past the universe, a disjoint
                # range per step
                n_fresh = int(round(n * cfg.fresh_frac))
                pos = r.choice(n, n_fresh, replace=False)
                start = int(self.card[t]) + step * FRESH_STRIDE
                counters[pos] = np.arange(start, start + n_fresh, dtype=np.uint64)
            if as_counters:
                ids[a:b] = counters
                table[a:b] = t
            else:
                ids[a:b] = self.keys(t, counters)
        return ids, table, bo

    def grad(self, step: int, dtype=np.float32) -> np.ndarray:
        """Upstream gradient N(0,1), layout [batch, n_tables, dim]."""
        cfg = self.cfg
        r = _rng(cfg.seed, 4, step)
        return r.standard_normal((cfg.batch, cfg.n_tables, cfg.dim), dtype=np.float32)
