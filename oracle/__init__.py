"""CPU oracle for the sparse-embedding training step (test infrastructure).

This package is the checker, not the product.  Only the test suite, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import it.  It shares no code with the HIP library: the arithmetic lives
in ``rse_oracle.cpp`` (plain single-threaded C++), compiled with g++ and loaded
here through ctypes.

Semantics followed (by page and section of the source pages):

* "阿里 RecIS：搜广推训练的背景与难点": lookups read only the indexed rows,
  backward touches only those rows; the nn.Embedding(10,4) SGD toy.
* "RecIS：阿里开源推荐系统统一训练框架", "Embedding Engine": ID -> offset map
  over growable blocks of parameters plus optimizer state; same-attribute
  tables merged into one map.
* "DLRM模型的核心价值与工业落地挑战" section 2.1: EmbeddingBag sum pooling of
  variable-length bags.
* "DLRM — Meta 把工业推荐模型拆成 4 个标准积木", "踩过的坑" 4: sparse optimizer
  updates only the rows seen in the batch.
* "RecIS：阿里开源推荐系统统一训练框架", "代码架构": a hook on the hash table
  for feature admission and eviction.  The pages give no policy; the ones
  defined here (count-min admission threshold, eviction by last-seen clock,
  recycled rows handed out in ascending order) are stated in rse_oracle.cpp.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rse_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
# RSE_ORACLE_LIB selects another build of the same source (the sanitizer
# build, loaded by a process that preloads the sanitizer runtimes)
_LIB_OVERRIDE = os.environ.get("RSE_ORACLE_LIB")

W_F32, W_BF16 = 0, 1
OPT_SGD, OPT_ADAGRAD, OPT_ADAM = 0, 1, 2
POOL_SUM, POOL_MEAN = 0, 1

_lib = None


def build(sanitize: bool = False) -> str:
    """Compile the oracle with g++ (always rebuilds). Returns the .so path.
    sanitize=True builds liboracle_san.so with AddressSanitizer and
    UndefinedBehaviorSanitizer (host code only)."""
    out = _SAN_LIB if sanitize else _LIB
    tmp = out + ".tmp"
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    cmd = ["g++", *flags, "-std=c++17", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, u64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
    lib.orc_create.restype = P
    lib.orc_create.argtypes = [i32, i32, i32, i32, i32, u64, f64, f64, f64, f64]
    lib.orc_destroy.argtypes = [P]
    lib.orc_find_or_insert.restype = ctypes.c_int
    lib.orc_find_or_insert.argtypes = [P, P, i64, P, i64, i32, i32, P, P]
    lib.orc_fwd.restype = ctypes.c_int
    lib.orc_fwd.argtypes = [P, P, P, i32, i64, i32, P]
    lib.orc_bwd_update.restype = ctypes.c_int
    lib.orc_bwd_update.argtypes = [P, P, P, i32, i64, i32, P, P]
    lib.orc_n_rows.restype = i64
    lib.orc_n_rows.argtypes = [P]
    lib.orc_step.restype = i64
    lib.orc_step.argtypes = [P]
    lib.orc_get_rows.restype = ctypes.c_int
    lib.orc_get_rows.argtypes = [P, P, i64, P, P]
    lib.orc_map_dump.restype = ctypes.c_int
    lib.orc_map_dump.argtypes = [P, P, P]
    lib.orc_touched.restype = i64
    lib.orc_touched.argtypes = [P, P, P]
    lib.orc_last_grad.restype = ctypes.c_int
    lib.orc_last_grad.argtypes = [P, i64, P]
    lib.orc_import.restype = ctypes.c_int
    lib.orc_import.argtypes = [P, P, P, P, P, P, i64, i64, i64]
    u32 = ctypes.c_uint32
    lib.orc_set_tracking.restype = ctypes.c_int
    lib.orc_set_tracking.argtypes = [P, i32]
    lib.orc_set_clock.restype = ctypes.c_int
    lib.orc_set_clock.argtypes = [P, u32]
    lib.orc_set_admission.restype = ctypes.c_int
    lib.orc_set_admission.argtypes = [P, i32, i64, u32, u64]
    lib.orc_set_recycling.restype = ctypes.c_int
    lib.orc_set_recycling.argtypes = [P, i32]
    lib.orc_rehash.restype = i64
    lib.orc_rehash.argtypes = [P, u32]
    lib.orc_entries.restype = i64
    lib.orc_entries.argtypes = [P, P, P, P]
    lib.orc_sketch.restype = i64
    lib.orc_sketch.argtypes = [P, P]
    lib.orc_estimate.restype = u32
    lib.orc_estimate.argtypes = [P, i64, i32]
    lib.orc_last_seen.restype = ctypes.c_int
    lib.orc_last_seen.argtypes = [P, P]
    lib.orc_free_list.restype = i64
    lib.orc_free_list.argtypes = [P, P, P]
    lib.orc_init_value.restype = f64
    lib.orc_init_value.argtypes = [u64, i32, i32, u64, i32]
    lib.orc_splitmix64_mix.restype = u64
    lib.orc_splitmix64_mix.argtypes = [u64]
    lib.orc_round_bf16.restype = ctypes.c_uint16
    lib.orc_round_bf16.argtypes = [f64]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def init_value(key: int, table: int, c: int, seed: int, wdtype: int = W_F32) -> float:
    """Initial value of column c of a new row with this key (exact)."""
    return _load().orc_init_value(ctypes.c_uint64(key & (2**64 - 1)), table, c, seed, wdtype)


def splitmix64_mix(z: int) -> int:
    return int(_load().orc_splitmix64_mix(ctypes.c_uint64(z & (2**64 - 1))))


def round_bf16_bits(x: float) -> int:
    """bf16 bit pattern nearest to the double x (ties to even)."""
    return int(_load().orc_round_bf16(float(x)))


class OracleTable:
    """One group of tables sharing dim, storage type and optimizer.

    ``n_tables`` logical tables, each with its own ID map (``merged=False``)
    or one map keyed by ``(table << 56) | id`` (``merged=True``); one shared
    row-offset space.
    """

    def __init__(self, dim, wdtype=W_F32, optim=OPT_SGD, n_tables=1, merged=False, seed=0,
                 lr=0.1, eps=1e-8, beta1=0.9, beta2=0.999):
        lib = _load()
        self.dim, self.wdtype, self.optim = dim, wdtype, optim
        self.n_tables, self.merged = n_tables, bool(merged)
        self._h = lib.orc_create(dim, wdtype, optim, n_tables, int(merged), seed, lr, eps, beta1, beta2)
        if not self._h:
            raise ValueError("oracle: bad table arguments")
        self._lib = lib

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.orc_destroy(h)

    @property
    def state_per_elem(self):
        return {OPT_SGD: 0, OPT_ADAGRAD: 1, OPT_ADAM: 2}[self.optim]

    @property
    def n_rows(self) -> int:
        return int(self._lib.orc_n_rows(self._h))

    @property
    def step(self) -> int:
        return int(self._lib.orc_step(self._h))

    def find_or_insert(self, ids, bounds, stride=1, insert_missing=True):
        """Table t's lookups are ids[bounds[t*stride]:bounds[(t+1)*stride]];
        pass the bag offsets with stride=batch for a training batch."""
        ids = _c(ids, np.int64)
        bo = _c(bounds, np.int64)
        row_off = np.empty(ids.shape[0], np.int64)
        n_new = np.zeros(1, np.int64)
        rc = self._lib.orc_find_or_insert(self._h, _p(ids), ids.shape[0], _p(bo), int(stride),
                                          self.n_tables, int(insert_missing), _p(row_off), _p(n_new))
        if rc != 0:
            raise ValueError("oracle find_or_insert: bad arguments")
        return row_off, int(n_new[0])

    def fwd(self, row_off, bag_offsets, batch, pooling=POOL_SUM):
        ro = _c(row_off, np.int64)
        bo = _c(bag_offsets, np.int64)
        out = np.empty((batch, self.n_tables, self.dim), np.float32)
        self._lib.orc_fwd(self._h, _p(ro), _p(bo), self.n_tables, batch, pooling, _p(out))
        return out

    def bwd_update(self, row_off, bag_offsets, batch, grad, pooling=POOL_SUM):
        ro = _c(row_off, np.int64)
        bo = _c(bag_offsets, np.int64)
        g = _c(grad, np.float32)
        assert g.size == batch * self.n_tables * self.dim
        n_u = np.zeros(1, np.int64)
        self._lib.orc_bwd_update(self._h, _p(ro), _p(bo), self.n_tables, batch, pooling, _p(g), _p(n_u))
        return int(n_u[0])

    def get_rows(self, offs):
        offs = _c(offs, np.int64)
        n = offs.shape[0]
        w = np.empty((n, self.dim), np.float32)
        k = self.state_per_elem
        st = np.empty((n, k * self.dim), np.float32)
        rc = self._lib.orc_get_rows(self._h, _p(offs), n, _p(w), _p(st) if k else None)
        if rc != 0:
            raise IndexError("oracle get_rows: offset out of range")
        return w, st

    def map_dump(self):
        n = self.n_rows
        keys = np.empty(n, np.int64)
        tabs = np.empty(n, np.int32)
        self._lib.orc_map_dump(self._h, _p(keys), _p(tabs))
        return keys, tabs

    def export_state(self):
        """(keys, map index, offsets, weights [n, dim], state [n, k*dim], step)
        of every row, in offset order."""
        keys, tabs = self.map_dump()
        offs = np.arange(self.n_rows, dtype=np.int64)
        w, st = self.get_rows(offs)
        return keys, tabs, offs, w, st, self.step

    def import_state(self, keys, tables, offs, w, state, step):
        """Replace the table's maps, rows and step by a saved state (the
        inverse of export_state; every row 0..n-1 listed once)."""
        keys = _c(keys, np.int64)
        tabs = _c(tables, np.int32)
        offs = _c(offs, np.int64)
        w = _c(w, np.float32)
        st = _c(state, np.float32) if self.state_per_elem else None
        n = keys.shape[0]
        rc = self._lib.orc_import(self._h, _p(keys), _p(tabs), _p(offs), _p(w), _p(st) if st is not None else None,
                                  n, n, int(step))
        if rc != 0:
            raise ValueError("oracle import_state: bad state")

    def touched(self):
        n = int(self._lib.orc_touched(self._h, None, None))
        offs = np.empty(n, np.int64)
        cnt = np.empty(n, np.int64)
        self._lib.orc_touched(self._h, _p(offs), _p(cnt))
        return offs, cnt

    def last_grad(self, off):
        g = np.empty(self.dim, np.float64)
        if self._lib.orc_last_grad(self._h, int(off), _p(g)) != 0:
            raise KeyError(off)
        return g

    # -------------------------------------- admission, age and eviction --
    def set_tracking(self, on=True):
        """Lookups stamp their rows with the clock; all stamps restart at 0."""
        self._lib.orc_set_tracking(self._h, int(bool(on)))

    def set_clock(self, clock: int):
        self._lib.orc_set_clock(self._h, int(clock))

    def set_admission(self, threshold: int, width: int = 0, depth: int = 0, seed: int = 0):
        """Count-min admission with a fresh sketch; threshold <= 1 turns it off."""
        if self._lib.orc_set_admission(self._h, int(depth), int(width), int(threshold),
                                       ctypes.c_uint64(seed & (2**64 - 1))) != 0:
            raise ValueError("oracle set_admission: bad sketch shape")

    def set_recycling(self, on=True):
        self._lib.orc_set_recycling(self._h, int(bool(on)))

    def rehash(self, min_clock: int = 0) -> int:
        """Evict keys last seen before min_clock (with tracking on) and, with
        recycling on, rebuild the free list. Returns the number of keys kept."""
        return int(self._lib.orc_rehash(self._h, int(min_clock)))

    def entries(self):
        """Live (key, map index, offset) entries, sorted by offset."""
        n = int(self._lib.orc_entries(self._h, None, None, None))
        keys = np.empty(n, np.int64)
        tabs = np.empty(n, np.int32)
        offs = np.empty(n, np.int64)
        self._lib.orc_entries(self._h, _p(keys), _p(tabs), _p(offs))
        o = np.argsort(offs, kind="stable")
        return keys[o], tabs[o], offs[o]

    def sketch(self):
        n = int(self._lib.orc_sketch(self._h, None))
        out = np.empty(n, np.uint32)
        if n:
            self._lib.orc_sketch(self._h, _p(out))
        return out

    def estimate(self, key: int, table: int = 0) -> int:
        return int(self._lib.orc_estimate(self._h, int(key), int(table)))

    def last_seen(self):
        out = np.empty(self.n_rows, np.uint32)
        if out.size:
            self._lib.orc_last_seen(self._h, _p(out))
        return out

    def free_list(self):
        """(rows not yet handed out, in order; number already handed out)."""
        n = int(self._lib.orc_free_list(self._h, None, None))
        out = np.empty(n, np.int64)
        done = np.zeros(1, np.int64)
        self._lib.orc_free_list(self._h, _p(out) if n else None, _p(done))
        return out, int(done[0])
