"""MI355X sparse-embedding training hot path: Python binding of librse.so.

Every step of the path runs in the HIP library (include/rse.h); this module
only marshals arguments: torch tensors provide device memory and the current
HIP stream (large chunks of rows are physically contiguous HIP allocations,
seen by torch as tensors).  The functions keep the C ABI's names:

    idmap_find_or_insert, embedding_bag_fwd, embedding_bag_bwd_update, blocks_grow

and embedding_bag_bwd_update's two halves, embedding_bag_bwd_prepare (sort;
may overlap the forward on another stream) and embedding_bag_bwd_apply.

``IdMap`` and ``EmbeddingBlocks`` own the caller-side device memory of the two
library objects.  Importing this package loads librse.so and fails if it is
missing (there is no CPU fallback).
"""

from __future__ import annotations

import ctypes
import os
import weakref
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import RseBwdPlan, RseError, RseOptim, check

F32, BF16 = 0, 1
SGD, ADAGRAD, ADAM = 0, 1, 2
SUM, MEAN = 0, 1
MAX_TABLES = 1024
MAX_MERGED_TABLES = 128

lib = _lib.load()


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t: torch.Tensor, dtype, name):
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name}: expected a contiguous {dtype} CUDA tensor, got {t.dtype} "
                        f"on {t.device} (contiguous={t.is_contiguous()})")


def _bytes(n: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    t = torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


# Large chunks of rows whose size is a multiple of 128 bytes are allocated
# physically contiguous (hipExtMallocWithFlags with
# hipDeviceMallocContiguous), which the GPU maps with its largest page
# fragments.  Click-log step, 57 GB table of 1 KB rows in 16 GB chunks, 7
# processes each on two GPUs: 0.541-0.569 ms (mean 0.556) with torch's
# allocations, 0.536-0.548 ms (mean 0.541) with contiguous ones (on other
# GPUs some processes still ran at the slower 0.555-0.568).  Rows that straddle
# 128-byte lines stay on torch's memory: the merged-table update (192-byte
# rows) wrote 4.3 GB per launch into contiguous chunks against 2.7 GB into
# torch's, and ran 3% longer.  Where the driver cannot place a chunk, torch
# allocates it.
_HIP_DEVICE_MALLOC_CONTIGUOUS = 0x4
CONTIGUOUS_MIN_BYTES = 1 << 28
_hip_rt = None


def _hip():
    """The HIP runtime torch has loaded: the libamdhip64 already mapped into
    this process, opened by its path (the same library instance, never a
    second runtime)."""
    global _hip_rt
    if _hip_rt is None:
        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                name = line.rstrip().split(" ")[-1]
                if os.path.basename(name).startswith("libamdhip64.so"):
                    path = name
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        h = ctypes.CDLL(path)
        h.hipExtMallocWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        h.hipExtMallocWithFlags.restype = ctypes.c_int
        h.hipFree.argtypes = [ctypes.c_void_p]
        h.hipFree.restype = ctypes.c_int
        h.hipGetLastError.argtypes = []
        h.hipGetLastError.restype = ctypes.c_int
        h.hipGetDevice.argtypes = [ctypes.POINTER(ctypes.c_int)]
        h.hipGetDevice.restype = ctypes.c_int
        h.hipSetDevice.argtypes = [ctypes.c_int]
        h.hipSetDevice.restype = ctypes.c_int
        _hip_rt = h
    return _hip_rt


def _free_contiguous(ptr: int, index: int):
    """hipFree on the allocation's device (HIP calls only, so that it also
    runs at interpreter exit)."""
    h = _hip()
    cur = ctypes.c_int(index)
    h.hipGetDevice(ctypes.byref(cur))
    h.hipSetDevice(index)
    h.hipFree(ctypes.c_void_p(ptr))
    h.hipSetDevice(cur.value)


class _ContiguousAlloc:
    """One hipExtMallocWithFlags allocation, seen by torch as a uint8 tensor
    through __cuda_array_interface__; the tensor keeps this owner alive, and
    the memory is freed with the last reference, or at interpreter exit
    (weakref.finalize runs before modules are torn down)."""

    def __init__(self, nbytes: int, device: torch.device):
        self.nbytes, self.device, self.ptr = int(nbytes), device, None
        p = ctypes.c_void_p()
        with torch.cuda.device(device):
            rc = _hip().hipExtMallocWithFlags(ctypes.byref(p), self.nbytes, _HIP_DEVICE_MALLOC_CONTIGUOUS)
            if rc != 0 or not p.value:
                _hip().hipGetLastError()      # leave no error for the library's next launch check
                raise MemoryError(f"hipExtMallocWithFlags({self.nbytes}, contiguous) returned {rc}")
        self.ptr = p.value
        index = device.index if device.index is not None else torch.cuda.current_device()
        self._free = weakref.finalize(self, _free_contiguous, p.value, index)

    @property
    def __cuda_array_interface__(self):
        return {"shape": (self.nbytes,), "typestr": "|u1", "data": (self.ptr, False), "version": 2}


def _chunk_bytes(n: int, row_bytes: int, device) -> torch.Tensor:
    """Device memory of a chunk: physically contiguous when large and its
    rows fill whole 128-byte lines (torch's allocator otherwise, or if that
    fails)."""
    device = torch.device(device)
    if n >= CONTIGUOUS_MIN_BYTES and row_bytes % 128 == 0 and device.type == "cuda":
        try:
            owner = _ContiguousAlloc(n, device)
        except MemoryError:
            return _bytes(n, device)
        t = torch.as_tensor(owner, device=device)
        assert t.data_ptr() == owner.ptr and t.numel() == n and t.data_ptr() % 256 == 0
        return t
    return _bytes(n, device)


def status_str(code: int) -> str:
    return lib.rse_status_str(code).decode()


def row_bytes(dim: int, w_dtype: int, optim: int) -> int:
    out = ctypes.c_int64()
    check(lib.rse_blocks_row_bytes(dim, w_dtype, optim, ctypes.byref(out)), "rse_blocks_row_bytes")
    return out.value


@dataclass
class Optim:
    """Optimizer of a blocks object (kind = SGD | ADAGRAD | ADAM)."""

    kind: int
    lr: float
    eps: float = 1e-8
    beta1: float = 0.9
    beta2: float = 0.999

    def struct(self, step: int) -> RseOptim:
        return RseOptim(self.kind, 0, self.lr, self.eps, self.beta1, self.beta2, int(step))


# ------------------------------------------------------------------ blocks --
class EmbeddingBlocks:
    """Chunked rows of weights + optimizer state (library object + memory)."""

    def __init__(self, dim: int, w_dtype: int = F32, optim: int = SGD, rows_per_chunk_log2: int = 20,
                 max_chunks: int = 1024, seed: int = 0, device="cuda", stream=None):
        self.dim, self.w_dtype, self.optim = dim, w_dtype, optim
        self.rows_per_chunk_log2, self.max_chunks, self.seed = rows_per_chunk_log2, max_chunks, seed
        self.rows_per_chunk = 1 << rows_per_chunk_log2
        self.row_bytes = row_bytes(dim, w_dtype, optim)
        self.device = torch.device(device)
        sz = ctypes.c_size_t()
        check(lib.rse_blocks_meta_size(max_chunks, ctypes.byref(sz)), "rse_blocks_meta_size")
        self.meta = _bytes(sz.value, self.device)
        h = ctypes.c_void_p()
        check(lib.rse_blocks_create(ctypes.byref(h), _ptr(self.meta), sz.value, dim, w_dtype, optim,
                                    rows_per_chunk_log2, max_chunks, seed, _stream(stream)),
              "rse_blocks_create")
        self.handle = h
        self.chunks: list[torch.Tensor] = []
        # the handle holds host memory only; freed when the object goes, or
        # at interpreter exit (before module globals are torn down)
        self._finalizer = weakref.finalize(self, lib.rse_blocks_destroy, h)

    @property
    def state_per_elem(self) -> int:
        return {SGD: 0, ADAGRAD: 1, ADAM: 2}[self.optim]

    @property
    def capacity(self) -> int:
        cap = ctypes.c_int64()
        check(lib.rse_blocks_capacity(self.handle, ctypes.byref(cap), None, None), "rse_blocks_capacity")
        return cap.value

    def grow(self, n_chunks: int = 1, stream=None):
        """Allocate n_chunks chunks and register them (blocks_grow).  Chunks of
        CONTIGUOUS_MIN_BYTES or more, of rows that are a multiple of 128 bytes,
        are physically contiguous allocations where the driver can place
        them; the rest come from torch."""
        for _ in range(n_chunks):
            chunk = _chunk_bytes(self.rows_per_chunk * self.row_bytes, self.row_bytes, self.device)
            blocks_grow(self, chunk, stream)
        return self

    def status(self, stream=None):
        """(rows_used, sticky status); synchronises the stream."""
        used, st = ctypes.c_int64(), ctypes.c_int32()
        check(lib.rse_blocks_status(self.handle, ctypes.byref(used), ctypes.byref(st), _stream(stream)),
              "rse_blocks_status")
        return used.value, st.value

    def clear_status(self, stream=None):
        check(lib.rse_blocks_clear_status(self.handle, _stream(stream)), "rse_blocks_clear_status")

    def write_rows(self, offs: torch.Tensor, w: torch.Tensor, state: torch.Tensor | None = None, stream=None):
        """Inverse of read_rows: rows `offs` (int64 CUDA) get weights w [n, dim]
        (fp32) and state [n, k*dim] (fp32; None for SGD)."""
        _need(offs, torch.int64, "offs")
        _need(w, torch.float32, "w")
        n = offs.numel()
        if w.numel() != n * self.dim:
            raise ValueError("w must hold n * dim floats")
        k = self.state_per_elem
        if k:
            _need(state, torch.float32, "state")
            if state.numel() != n * k * self.dim:
                raise ValueError("state must hold n * k * dim floats")
        check(lib.rse_blocks_write_rows(self.handle, _ptr(offs), n, _ptr(w), _ptr(state) if k else None,
                                        _stream(stream)), "rse_blocks_write_rows")

    def set_rows_used(self, rows_used: int, stream=None):
        check(lib.rse_blocks_set_rows_used(self.handle, int(rows_used), _stream(stream)), "rse_blocks_set_rows_used")

    def enable_free_list(self, capacity: int | None = None, stream=None):
        """Attach an (empty) free list of recycled rows for `capacity` rows
        (default: the current capacity); a map rehash fills it."""
        cap = self.capacity if capacity is None else int(capacity)
        self.free_rows = torch.zeros(max(cap, 1), dtype=torch.int32, device=self.device)   # uint32 entries
        check(lib.rse_blocks_set_free_list(self.handle, _ptr(self.free_rows), cap, _stream(stream)),
              "rse_blocks_set_free_list")
        return self

    def disable_free_list(self, stream=None):
        check(lib.rse_blocks_set_free_list(self.handle, None, 0, _stream(stream)), "rse_blocks_set_free_list")
        self.free_rows = None

    def free_list(self, stream=None):
        """(rows already handed out, rows left as an int64 tensor, in order);
        synchronises the stream."""
        head, count = ctypes.c_int64(), ctypes.c_int64()
        check(lib.rse_blocks_free_status(self.handle, ctypes.byref(head), ctypes.byref(count), _stream(stream)),
              "rse_blocks_free_status")
        rows = getattr(self, "free_rows", None)
        if rows is None or count.value == 0:
            return head.value, torch.zeros(0, dtype=torch.int64, device=self.device)
        left = rows[head.value:head.value + count.value].to(torch.int64) & 0xFFFFFFFF
        return head.value, left

    def read_rows(self, offs: torch.Tensor, stream=None):
        """Weights (widened to fp32) and state of rows `offs` (int64 CUDA)."""
        _need(offs, torch.int64, "offs")
        n = offs.numel()
        w = torch.empty((n, self.dim), dtype=torch.float32, device=self.device)
        k = self.state_per_elem
        st = torch.empty((n, k * self.dim), dtype=torch.float32, device=self.device)
        check(lib.rse_blocks_read_rows(self.handle, _ptr(offs), n, _ptr(w), _ptr(st) if k else None,
                                       _stream(stream)), "rse_blocks_read_rows")
        return w, st


def blocks_grow(blocks: EmbeddingBlocks, chunk: torch.Tensor, stream=None):
    """Register one caller-allocated chunk (uint8 CUDA tensor)."""
    _need(chunk, torch.uint8, "chunk")
    check(lib.blocks_grow(blocks.handle, _ptr(chunk), chunk.numel(), _stream(stream)), "blocks_grow")
    blocks.chunks.append(chunk)


# ------------------------------------------------------------------- idmap --
class IdMap:
    """Open-addressing ID -> row map (library object + slot memory)."""

    def __init__(self, slots_per_table, max_load: float = 0.7, merged: bool = False,
                 hash_seed: int = 0, device="cuda", stream=None):
        slots = [int(s) for s in slots_per_table]
        self.slots_per_table, self.max_load, self.hash_seed = slots, float(max_load), int(hash_seed)
        self.n_tables = len(slots)
        self.merged = bool(merged)
        self.device = torch.device(device)
        arr = (ctypes.c_int64 * len(slots))(*slots)
        sz = ctypes.c_size_t()
        check(lib.rse_idmap_mem_size(len(slots), arr, ctypes.byref(sz)), "rse_idmap_mem_size")
        # torch's memory: with a physically contiguous map (tried) the
        # click-log step was in its slower mode in about half of the runs
        self.mem = _bytes(sz.value, self.device)
        h = ctypes.c_void_p()
        check(lib.rse_idmap_create(ctypes.byref(h), _ptr(self.mem), sz.value, len(slots), arr, max_load,
                                   int(merged), hash_seed, _stream(stream)), "rse_idmap_create")
        self.handle = h
        self._ws = None
        self._finalizer = weakref.finalize(self, lib.rse_idmap_destroy, h)

    def workspace(self, n_ids: int) -> torch.Tensor:
        sz = ctypes.c_size_t()
        check(lib.rse_idmap_workspace_size(n_ids, ctypes.byref(sz)), "rse_idmap_workspace_size")
        if self._ws is None or self._ws.numel() < sz.value:
            self._ws = _bytes(sz.value, self.device)
        return self._ws

    def status(self, stream=None):
        """(sticky status, per-table key counts); synchronises the stream."""
        st = ctypes.c_int32()
        keys = (ctypes.c_int64 * self.n_tables)()
        check(lib.rse_idmap_status(self.handle, ctypes.byref(st), keys, _stream(stream)), "rse_idmap_status")
        return st.value, list(keys)

    def clear_status(self, stream=None):
        check(lib.rse_idmap_clear_status(self.handle, _stream(stream)), "rse_idmap_clear_status")

    def import_entries(self, keys: torch.Tensor, tables: torch.Tensor, offs: torch.Tensor, stream=None):
        """Insert saved (key, table, offset) entries (int64 / int32 / int64 CUDA)."""
        _need(keys, torch.int64, "keys")
        _need(tables, torch.int32, "tables")
        _need(offs, torch.int64, "offs")
        n = keys.numel()
        if tables.numel() != n or offs.numel() != n:
            raise ValueError("keys, tables and offs must have the same length")
        check(lib.rse_idmap_import(self.handle, _ptr(keys), _ptr(tables), _ptr(offs), n, _stream(stream)),
              "rse_idmap_import")

    # ---------------------------------- admission, age, eviction, resize --
    def track_age(self, n_rows: int, stream=None):
        """Attach per-row stamps for rows [0, n_rows); lookups write the clock
        into them (n_rows must cover the blocks' capacity: after the blocks
        grow, call again with the new capacity).  Stamps already attached are
        carried over; new rows start at 0."""
        old = getattr(self, "stamps", None)
        new = torch.zeros(max(int(n_rows), 1), dtype=torch.int32, device=self.device)   # uint32
        if old is not None:                     # copied on the current stream
            k = min(old.numel(), new.numel())
            new[:k].copy_(old[:k])
        self.stamps = new
        check(lib.rse_idmap_set_stamps(self.handle, _ptr(self.stamps), int(n_rows)), "rse_idmap_set_stamps")
        return self

    def set_clock(self, clock: int):
        check(lib.rse_idmap_set_clock(self.handle, int(clock) & 0xFFFFFFFF), "rse_idmap_set_clock")

    def enable_admission(self, threshold: int, width: int, depth: int = 4, seed: int = 0, stream=None):
        """Count-min admission: an absent key is inserted once its estimated
        count of absent lookups reaches `threshold` (<= 1 turns it off)."""
        if threshold <= 1:
            self.sketch = None
            check(lib.rse_idmap_set_admission(self.handle, None, 0, 0, int(threshold), 0, _stream(stream)),
                  "rse_idmap_set_admission")
            return self
        self.sketch = torch.empty(int(depth) * int(width), dtype=torch.int32, device=self.device)   # uint32
        self.sketch_shape = (int(depth), int(width))
        check(lib.rse_idmap_set_admission(self.handle, _ptr(self.sketch), int(depth), int(width), int(threshold),
                                          int(seed) & (2**64 - 1), _stream(stream)), "rse_idmap_set_admission")
        return self

    def rehash_into(self, dst: "IdMap", blocks: EmbeddingBlocks, min_clock: int = 0, stream=None):
        """Copy this map's keys into `dst` (same tables, any size), evicting
        keys last seen before min_clock when stamps are attached; rebuilds
        the blocks' free list if one is attached.  Stream-ordered: read
        dst.status() for the outcome."""
        sz = ctypes.c_size_t()
        check(lib.rse_idmap_rehash_workspace_size(self.handle, blocks.handle, ctypes.byref(sz)),
              "rse_idmap_rehash_workspace_size")
        ws = _bytes(sz.value, self.device)
        check(lib.rse_idmap_rehash(dst.handle, self.handle, blocks.handle, int(min_clock) & 0xFFFFFFFF, _ptr(ws),
                                   sz.value, _stream(stream)), "rse_idmap_rehash")
        dst._ws_keep = ws            # the stream may still be reading it
        for name in ("stamps", "sketch", "sketch_shape"):
            if hasattr(self, name):
                setattr(dst, name, getattr(self, name))

    def _replace_with(self, other: "IdMap"):
        """Take over other's library object and memory (other gets ours)."""
        self._finalizer.detach()
        other._finalizer.detach()
        self.handle, other.handle = other.handle, self.handle
        self.mem, other.mem = other.mem, self.mem
        self.slots_per_table, other.slots_per_table = other.slots_per_table, self.slots_per_table
        self._finalizer = weakref.finalize(self, lib.rse_idmap_destroy, self.handle)
        other._finalizer = weakref.finalize(other, lib.rse_idmap_destroy, other.handle)

    def _rebuild(self, slots_per_table, blocks, min_clock, stream):
        dst = IdMap(slots_per_table, self.max_load, self.merged, self.hash_seed, self.device, stream)
        self.rehash_into(dst, blocks, min_clock, stream)
        st, _ = dst.status(stream)
        if st != 0:
            raise RseError("rse_idmap_rehash", st)
        self._replace_with(dst)
        return self

    def evict(self, blocks: EmbeddingBlocks, min_clock: int, stream=None):
        """Drop keys last seen before min_clock (rows go to the free list, if
        any); the map keeps its size.  Synchronises the stream."""
        return self._rebuild(self.slots_per_table, blocks, min_clock, stream)

    def resize(self, slots_per_table, blocks: EmbeddingBlocks, stream=None):
        """Rehash every key into new slot regions of the given sizes (offsets
        unchanged).  Synchronises the stream."""
        return self._rebuild([int(x) for x in slots_per_table], blocks, 0, stream)

    def export(self, capacity: int, stream=None):
        """Live entries (keys int64, table int32, offsets int64), any order."""
        keys = torch.empty(max(capacity, 1), dtype=torch.int64, device=self.device)
        tabs = torch.empty(max(capacity, 1), dtype=torch.int32, device=self.device)
        offs = torch.empty(max(capacity, 1), dtype=torch.int64, device=self.device)
        cnt = torch.empty(1, dtype=torch.int64, device=self.device)
        check(lib.rse_idmap_export(self.handle, _ptr(keys), _ptr(tabs), _ptr(offs), capacity, _ptr(cnt),
                                   _stream(stream)), "rse_idmap_export")
        n = min(int(cnt.item()), capacity)
        return keys[:n], tabs[:n], offs[:n], int(cnt.item())


def idmap_find_or_insert(idmap: IdMap, blocks: EmbeddingBlocks, ids: torch.Tensor, bounds: torch.Tensor,
                         stride: int, n_tables: int, row_off: torch.Tensor, n_new: torch.Tensor,
                         insert_missing: bool = True, ws: torch.Tensor | None = None, stream=None):
    """Table t's lookups are ids[bounds[t*stride] : bounds[(t+1)*stride]]."""
    # sizes first: the kernels write row_off[i] for every lookup i and read
    # bounds[t * stride] for t <= n_tables
    if row_off.numel() != ids.numel():
        raise ValueError(f"row_off must hold one offset per id ({ids.numel()}), got {row_off.numel()}")
    if stride <= 0 or n_tables <= 0:
        raise ValueError("stride and n_tables must be positive")
    if bounds.numel() < n_tables * stride + 1:
        raise ValueError(f"bounds must hold at least n_tables * stride + 1 = {n_tables * stride + 1} entries, "
                         f"got {bounds.numel()}")
    if n_new.numel() < 1:
        raise ValueError("n_new must hold one int64")
    _need(ids, torch.int64, "ids")
    _need(bounds, torch.int64, "bounds")
    _need(row_off, torch.int64, "row_off")
    _need(n_new, torch.int64, "n_new")
    n = ids.numel()
    if ws is None:
        ws = idmap.workspace(n)
    check(lib.idmap_find_or_insert(idmap.handle, blocks.handle, _ptr(ids), n, _ptr(bounds), stride,
                                   n_tables, int(bool(insert_missing)), _ptr(row_off), _ptr(n_new),
                                   _ptr(ws), ws.numel(), _stream(stream)), "idmap_find_or_insert")


NOALLOC_MAX_IDS = 2097152


def idmap_find_or_insert_noalloc(idmap: IdMap, blocks: EmbeddingBlocks, ids: torch.Tensor, bounds: torch.Tensor,
                                 stride: int, n_tables: int, row_off: torch.Tensor, n_new: torch.Tensor,
                                 insert_missing: bool = True, stream=None):
    """idmap_find_or_insert over the library's static per-GPU scratch (no
    workspace, no allocation); at most NOALLOC_MAX_IDS lookups, and calls on
    one GPU must not overlap."""
    if row_off.numel() != ids.numel():
        raise ValueError(f"row_off must hold one offset per id ({ids.numel()}), got {row_off.numel()}")
    if stride <= 0 or n_tables <= 0:
        raise ValueError("stride and n_tables must be positive")
    if bounds.numel() < n_tables * stride + 1:
        raise ValueError(f"bounds must hold at least n_tables * stride + 1 = {n_tables * stride + 1} entries, "
                         f"got {bounds.numel()}")
    _need(ids, torch.int64, "ids")
    _need(bounds, torch.int64, "bounds")
    _need(row_off, torch.int64, "row_off")
    _need(n_new, torch.int64, "n_new")
    check(lib.idmap_find_or_insert_noalloc(idmap.handle, blocks.handle, _ptr(ids), ids.numel(), _ptr(bounds),
                                           stride, n_tables, int(bool(insert_missing)), _ptr(row_off),
                                           _ptr(n_new), _stream(stream)), "idmap_find_or_insert_noalloc")


def embedding_bag_fwd(blocks: EmbeddingBlocks, row_off: torch.Tensor, bag_offsets: torch.Tensor,
                      n_tables: int, batch: int, pooling: int, out: torch.Tensor, stream=None):
    """out [batch, n_tables, dim] fp32 = pooled rows of each bag."""
    if out.numel() != batch * n_tables * blocks.dim:
        raise ValueError("out must hold batch * n_tables * dim floats")
    if bag_offsets.numel() != n_tables * batch + 1:
        raise ValueError("bag_offsets must hold n_tables * batch + 1 entries")
    _need(row_off, torch.int64, "row_off")
    _need(bag_offsets, torch.int64, "bag_offsets")
    _need(out, torch.float32, "out")
    check(lib.embedding_bag_fwd(blocks.handle, _ptr(row_off), row_off.numel(), _ptr(bag_offsets),
                                n_tables, batch, pooling, _ptr(out), _stream(stream)), "embedding_bag_fwd")


def bwd_workspace(n_ids: int, n_tables: int, batch: int, dim: int, device="cuda") -> torch.Tensor:
    sz = ctypes.c_size_t()
    check(lib.rse_bwd_workspace_size(n_ids, n_tables, batch, dim, ctypes.byref(sz)), "rse_bwd_workspace_size")
    return _bytes(sz.value, device)


def embedding_bag_bwd_update(blocks: EmbeddingBlocks, row_off: torch.Tensor, bag_offsets: torch.Tensor,
                             n_tables: int, batch: int, pooling: int, grad: torch.Tensor, optim: Optim,
                             step: int, n_unique: torch.Tensor, ws: torch.Tensor | None = None,
                             stream=None):
    """Merge duplicate-row gradients and update the touched rows in place."""
    _need(row_off, torch.int64, "row_off")
    _need(bag_offsets, torch.int64, "bag_offsets")
    _need(grad, torch.float32, "grad")
    _need(n_unique, torch.int64, "n_unique")
    if grad.numel() != batch * n_tables * blocks.dim:
        raise ValueError("grad must hold batch * n_tables * dim floats")
    if bag_offsets.numel() != n_tables * batch + 1:
        raise ValueError("bag_offsets must hold n_tables * batch + 1 entries")
    if ws is None:
        ws = bwd_workspace(row_off.numel(), n_tables, batch, blocks.dim, blocks.device)
    o = optim.struct(step)
    check(lib.embedding_bag_bwd_update(blocks.handle, _ptr(row_off), row_off.numel(), _ptr(bag_offsets),
                                       n_tables, batch, pooling, _ptr(grad), ctypes.byref(o), _ptr(n_unique),
                                       _ptr(ws), ws.numel(), _stream(stream)), "embedding_bag_bwd_update")


def embedding_bag_bwd_prepare(blocks: EmbeddingBlocks, row_off: torch.Tensor, bag_offsets: torch.Tensor,
                              n_tables: int, batch: int, ws: torch.Tensor, stream=None):
    """First half of embedding_bag_bwd_update: validates the offsets and sorts
    the lookups by row into ws.  Needs no gradient, so it may run on another
    stream while the forward runs.  Returns the plan for
    embedding_bag_bwd_apply."""
    _need(row_off, torch.int64, "row_off")
    _need(bag_offsets, torch.int64, "bag_offsets")
    if bag_offsets.numel() != n_tables * batch + 1:
        raise ValueError("bag_offsets must hold n_tables * batch + 1 entries")
    plan = RseBwdPlan()
    check(lib.embedding_bag_bwd_prepare(blocks.handle, _ptr(row_off), row_off.numel(), _ptr(bag_offsets),
                                        n_tables, batch, _ptr(ws), ws.numel(), ctypes.byref(plan),
                                        _stream(stream)), "embedding_bag_bwd_prepare")
    return plan


def embedding_bag_bwd_apply(blocks: EmbeddingBlocks, plan, bag_offsets: torch.Tensor, n_tables: int,
                            batch: int, pooling: int, grad: torch.Tensor, optim: Optim, step: int,
                            n_unique: torch.Tensor, ws: torch.Tensor, stream=None):
    """Second half of embedding_bag_bwd_update: reduces grad over the lookups
    sorted by embedding_bag_bwd_prepare (same ws) and updates the rows."""
    _need(bag_offsets, torch.int64, "bag_offsets")
    _need(grad, torch.float32, "grad")
    _need(n_unique, torch.int64, "n_unique")
    if grad.numel() != batch * n_tables * blocks.dim:
        raise ValueError("grad must hold batch * n_tables * dim floats")
    o = optim.struct(step)
    check(lib.embedding_bag_bwd_apply(blocks.handle, ctypes.byref(plan), _ptr(bag_offsets), n_tables, batch,
                                      pooling, _ptr(grad), ctypes.byref(o), _ptr(n_unique), _ptr(ws),
                                      ws.numel(), _stream(stream)), "embedding_bag_bwd_apply")


# ------------------------------------------------- DLRM dot interaction --
# ------------------------------------------------------ feature transforms --
FT_INT64, FT_FLOAT64 = 0, 1
FT_IDENTITY, FT_HASH, FT_MOD, FT_BUCKETIZE = 0, 1, 2, 3


class FeatureTransform:
    """Per-table programs of Hash / Mod / Bucketize, applied to every table's
    raw values in one launch.  `programs`: one (input_kind, ops) per table,
    ops a list of (FT_HASH, seed) | (FT_MOD, m) | (FT_BUCKETIZE, boundaries)."""

    def __init__(self, programs, device="cuda", stream=None):
        import numpy as np

        self.device = torch.device(device)
        n = len(programs)
        progs = (_lib.RseFeatureProgram * n)()
        bnd = []
        for t, (kind, ops) in enumerate(programs):
            if len(ops) > 4:
                raise ValueError(f"table {t}: at most 4 operations")
            progs[t].input = int(kind)
            progs[t].n_ops = len(ops)
            for k, (op, arg) in enumerate(ops):
                progs[t].ops[k].kind = int(op)
                if op == FT_BUCKETIZE:
                    b = np.asarray(arg, np.float64).ravel()
                    progs[t].ops[k].arg = len(bnd)
                    progs[t].ops[k].n_boundaries = b.size
                    bnd.extend(b.tolist())
                elif op == FT_HASH:
                    seed = int(arg) & (2**64 - 1)
                    progs[t].ops[k].arg = seed - 2**64 if seed >= 2**63 else seed
                else:
                    progs[t].ops[k].arg = int(arg)
        self.n_tables = n
        b_arr = (ctypes.c_double * max(len(bnd), 1))(*bnd)
        sz = ctypes.c_size_t()
        check(lib.rse_features_mem_size(n, len(bnd), ctypes.byref(sz)), "rse_features_mem_size")
        self.mem = _bytes(sz.value, self.device)
        h = ctypes.c_void_p()
        check(lib.rse_features_create(ctypes.byref(h), _ptr(self.mem), sz.value, progs, n, b_arr, len(bnd),
                                      _stream(stream)), "rse_features_create")
        self.handle = h
        self._finalizer = weakref.finalize(self, lib.rse_features_destroy, h)

    def status(self, stream=None) -> int:
        st = ctypes.c_int32()
        check(lib.rse_features_status(self.handle, ctypes.byref(st), _stream(stream)), "rse_features_status")
        return st.value


def feature_transform(ft: FeatureTransform, raw: torch.Tensor, bounds: torch.Tensor, stride: int = 1,
                      out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """ids (int64) of every lookup from its raw 64-bit value (int64 tensor;
    float64 features passed as their bits, e.g. x.view(torch.int64))."""
    _need(raw, torch.int64, "raw")
    _need(bounds, torch.int64, "bounds")
    n = raw.numel()
    if bounds.numel() < ft.n_tables * stride + 1:
        raise ValueError("bounds must hold n_tables * stride + 1 entries")
    if out is None:
        out = torch.empty_like(raw)
    _need(out, torch.int64, "out")
    if out.numel() != n:
        raise ValueError("out must have one id per raw value")
    check(lib.feature_transform(ft.handle, _ptr(raw), n, _ptr(bounds), int(stride), _ptr(out), _stream(stream)),
          "feature_transform")
    return out


def dlrm_interaction_fwd(dense: torch.Tensor, pooled: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """dense [B, d], pooled [B, T, d] fp32 CUDA -> [B, d + (T+1)T/2]: the dense
    vector, then the dot products of every pair of (dense, table 0..T-1) in
    row-major upper-triangle order."""
    B, T, d = pooled.shape
    if dense.shape != (B, d):
        raise ValueError("dense must be [B, d] for pooled [B, T, d]")
    P = (T + 1) * T // 2
    if out is None:
        out = torch.empty((B, d + P), dtype=torch.float32, device=pooled.device)
    if out.numel() != B * (d + P):
        raise ValueError("out must hold B * (d + (T+1)T/2) floats")
    _need(dense, torch.float32, "dense")
    _need(pooled, torch.float32, "pooled")
    _need(out, torch.float32, "out")
    check(lib.dlrm_interaction_fwd(_ptr(dense), _ptr(pooled), B, T, d, _ptr(out), _stream(stream)),
          "dlrm_interaction_fwd")
    return out


def dlrm_interaction_bwd(dense: torch.Tensor, pooled: torch.Tensor, dout: torch.Tensor, stream=None):
    """Gradients (ddense [B, d], dpooled [B, T, d]) of dlrm_interaction_fwd for
    the upstream gradient dout [B, d + (T+1)T/2]."""
    B, T, d = pooled.shape
    if dense.shape != (B, d) or dout.numel() != B * (d + (T + 1) * T // 2):
        raise ValueError("shapes of dense / dout do not match pooled [B, T, d]")
    _need(dense, torch.float32, "dense")
    _need(pooled, torch.float32, "pooled")
    _need(dout, torch.float32, "dout")
    ddense = torch.empty_like(dense)
    dpooled = torch.empty_like(pooled)
    check(lib.dlrm_interaction_bwd(_ptr(dense), _ptr(pooled), _ptr(dout), B, T, d, _ptr(ddense), _ptr(dpooled),
                                   _stream(stream)), "dlrm_interaction_bwd")
    return ddense, dpooled


# ----------------------------------------------------------------- trace --
K_PROBE, K_FWD, K_SORT_SCATTER, K_SEG_UPDATE, K_COMBINE, K_INTERACT = 1, 2, 3, 4, 5, 6


def trace_start(kernel: int):
    """Record HIP events around every launch of `kernel` (a K_* id)."""
    check(lib.rse_trace_start(kernel), "rse_trace_start")


def trace_stop():
    """(launches, total ms) of the traced kernel since trace_start."""
    n, ms = ctypes.c_int64(), ctypes.c_double()
    check(lib.rse_trace_stop(ctypes.byref(n), ctypes.byref(ms)), "rse_trace_stop")
    return n.value, ms.value


__all__ = [
    "F32", "BF16", "SGD", "ADAGRAD", "ADAM", "SUM", "MEAN", "Optim", "EmbeddingBlocks", "IdMap",
    "RseError", "blocks_grow", "idmap_find_or_insert", "idmap_find_or_insert_noalloc", "embedding_bag_fwd", "embedding_bag_bwd_update",
    "embedding_bag_bwd_prepare", "embedding_bag_bwd_apply",
    "bwd_workspace", "row_bytes", "status_str", "lib", "trace_start", "trace_stop", "K_PROBE", "K_FWD",
    "K_SORT_SCATTER", "K_SEG_UPDATE", "K_COMBINE", "K_INTERACT", "save", "load", "dlrm_interaction_fwd",
    "dlrm_interaction_bwd",
]

from .saver import load, save  # noqa: E402  (the Saver uses the classes above)
