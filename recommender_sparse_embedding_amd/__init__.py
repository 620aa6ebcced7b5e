"""MI355X sparse-embedding training hot path: Python binding of librse.so.

Every step of the path runs in the HIP library (include/rse.h); this module
only marshals arguments: torch tensors provide device memory and the current
HIP stream.  The functions keep the C ABI's names:

    idmap_find_or_insert, embedding_bag_fwd, embedding_bag_bwd_update, blocks_grow

and embedding_bag_bwd_update's two halves, embedding_bag_bwd_prepare (sort;
may overlap the forward on another stream) and embedding_bag_bwd_apply.

``IdMap`` and ``EmbeddingBlocks`` own the caller-side device memory of the two
library objects.  Importing this package loads librse.so and fails if it is
missing (there is no CPU fallback).
"""

from __future__ import annotations

import ctypes
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

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            lib.rse_blocks_destroy(h)
            self.handle = None

    @property
    def state_per_elem(self) -> int:
        return {SGD: 0, ADAGRAD: 1, ADAM: 2}[self.optim]

    @property
    def capacity(self) -> int:
        cap = ctypes.c_int64()
        check(lib.rse_blocks_capacity(self.handle, ctypes.byref(cap), None, None), "rse_blocks_capacity")
        return cap.value

    def grow(self, n_chunks: int = 1, stream=None):
        """Allocate n_chunks chunks with torch and register them (blocks_grow)."""
        for _ in range(n_chunks):
            chunk = _bytes(self.rows_per_chunk * self.row_bytes, self.device)
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
        self.n_tables = len(slots)
        self.merged = bool(merged)
        self.device = torch.device(device)
        arr = (ctypes.c_int64 * len(slots))(*slots)
        sz = ctypes.c_size_t()
        check(lib.rse_idmap_mem_size(len(slots), arr, ctypes.byref(sz)), "rse_idmap_mem_size")
        self.mem = _bytes(sz.value, self.device)
        h = ctypes.c_void_p()
        check(lib.rse_idmap_create(ctypes.byref(h), _ptr(self.mem), sz.value, len(slots), arr, max_load,
                                   int(merged), hash_seed, _stream(stream)), "rse_idmap_create")
        self.handle = h
        self._ws = None

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            lib.rse_idmap_destroy(h)
            self.handle = None

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


def embedding_bag_fwd(blocks: EmbeddingBlocks, row_off: torch.Tensor, bag_offsets: torch.Tensor,
                      n_tables: int, batch: int, pooling: int, out: torch.Tensor, stream=None):
    """out [batch, n_tables, dim] fp32 = pooled rows of each bag."""
    _need(row_off, torch.int64, "row_off")
    _need(bag_offsets, torch.int64, "bag_offsets")
    _need(out, torch.float32, "out")
    if out.numel() != batch * n_tables * blocks.dim:
        raise ValueError("out must hold batch * n_tables * dim floats")
    if bag_offsets.numel() != n_tables * batch + 1:
        raise ValueError("bag_offsets must hold n_tables * batch + 1 entries")
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


# ----------------------------------------------------------------- trace --
K_PROBE, K_FWD, K_SORT_SCATTER, K_SEG_UPDATE, K_COMBINE = 1, 2, 3, 4, 5


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
    "RseError", "blocks_grow", "idmap_find_or_insert", "embedding_bag_fwd", "embedding_bag_bwd_update",
    "embedding_bag_bwd_prepare", "embedding_bag_bwd_apply",
    "bwd_workspace", "row_bytes", "status_str", "lib", "trace_start", "trace_stop", "K_PROBE", "K_FWD",
    "K_SORT_SCATTER", "K_SEG_UPDATE", "K_COMBINE",
]
