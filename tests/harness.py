"""Side-by-side driver for parity tests: the HIP path (through the Python
binding of the C ABI) and the CPU oracle, fed the same seeded inputs."""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import synth


def rtol_for(wdtype):
    return 1e-5 if wdtype == synth.F32 else 1e-2


class GpuTables:
    """The library's objects for one table group, sized for `max_rows`."""

    def __init__(self, cfg: synth.Config, card, max_rows: int, rows_per_chunk_log2: int = 14,
                 load: float = 0.7, device="cuda", extra_keys=0, split: bool = False):
        import recommender_sparse_embedding_amd as rse

        self.rse = rse
        self.cfg = cfg
        self.dev = torch.device(device)
        if cfg.merged:
            slots = [int(math.ceil((int(np.sum(card)) + extra_keys + 16) / load)) + 64]
        else:
            slots = [int(math.ceil((int(c) + extra_keys + 16) / load)) + 64 for c in card]
        self.map = rse.IdMap(slots, max_load=min(0.95, load + 0.05), merged=cfg.merged,
                             hash_seed=cfg.seed + 77, device=self.dev)
        self.blocks = rse.EmbeddingBlocks(cfg.dim, cfg.wdtype, cfg.optim, rows_per_chunk_log2,
                                          max_chunks=4096, seed=cfg.seed, device=self.dev)
        n_chunks = max(1, -(-max_rows // (1 << rows_per_chunk_log2)))
        self.blocks.grow(n_chunks)
        self.optim = rse.Optim(cfg.optim, cfg.lr, cfg.eps, cfg.beta1, cfg.beta2)
        self.step = 0
        self.n_new = torch.zeros(1, dtype=torch.int64, device=self.dev)
        self.n_unique = torch.zeros(1, dtype=torch.int64, device=self.dev)
        # split: the backward's sort (prepare) runs on a side stream while the
        # forward runs; the apply waits for it on the main stream
        self.split = split
        self.side = torch.cuda.Stream(device=self.dev) if split else None
        self.plan = None

    def find_or_insert(self, ids, bounds, stride, insert=True):
        t_ids = torch.from_numpy(np.ascontiguousarray(ids)).to(self.dev)
        t_b = torch.from_numpy(np.ascontiguousarray(bounds)).to(self.dev)
        ro = torch.empty_like(t_ids)
        self.rse.idmap_find_or_insert(self.map, self.blocks, t_ids, t_b, stride, self.cfg.n_tables, ro,
                                      self.n_new, insert_missing=insert)
        return ro, int(self.n_new.item())

    def fwd(self, ro, bo):
        cfg = self.cfg
        t_bo = torch.from_numpy(bo).to(self.dev)
        out = torch.empty((cfg.batch, cfg.n_tables, cfg.dim), dtype=torch.float32, device=self.dev)
        self.rse.embedding_bag_fwd(self.blocks, ro, t_bo, cfg.n_tables, cfg.batch, cfg.pooling, out)
        return out

    def prepare(self, ro, bo):
        """Split mode: start the backward's sort on the side stream (after
        the work queued so far on the main stream)."""
        if not self.split:
            return
        cfg = self.cfg
        main = torch.cuda.current_stream(self.dev)
        t_bo = torch.from_numpy(bo).to(self.dev)
        self.ws = self.rse.bwd_workspace(ro.numel(), cfg.n_tables, cfg.batch, cfg.dim, self.dev)
        ev = torch.cuda.Event()
        ev.record(main)
        self.side.wait_event(ev)
        for t in (ro, t_bo, self.ws):
            t.record_stream(self.side)
        self.plan = self.rse.embedding_bag_bwd_prepare(self.blocks, ro, t_bo, cfg.n_tables, cfg.batch, self.ws,
                                                       stream=self.side)
        self.prepared = torch.cuda.Event()
        self.prepared.record(self.side)

    def bwd(self, ro, bo, grad):
        cfg = self.cfg
        self.step += 1
        t_bo = torch.from_numpy(bo).to(self.dev)
        g = grad if isinstance(grad, torch.Tensor) else torch.from_numpy(grad).to(self.dev)
        if self.split:
            torch.cuda.current_stream(self.dev).wait_event(self.prepared)
            self.rse.embedding_bag_bwd_apply(self.blocks, self.plan, t_bo, cfg.n_tables, cfg.batch, cfg.pooling,
                                             g.contiguous(), self.optim, self.step, self.n_unique, self.ws)
        else:
            self.rse.embedding_bag_bwd_update(self.blocks, ro, t_bo, cfg.n_tables, cfg.batch, cfg.pooling,
                                              g.contiguous(), self.optim, self.step, self.n_unique)
        return int(self.n_unique.item())

    def rows(self, offs):
        w, s = self.blocks.read_rows(torch.from_numpy(np.ascontiguousarray(offs, np.int64)).to(self.dev))
        return w.cpu().numpy(), s.cpu().numpy()


def make_oracle(cfg: synth.Config):
    return oracle.OracleTable(cfg.dim, cfg.wdtype, cfg.optim, cfg.n_tables, cfg.merged, seed=cfg.seed,
                              lr=cfg.lr, eps=cfg.eps, beta1=cfg.beta1, beta2=cfg.beta2)


def pooled_magnitude(orc, row_off, bo, cfg):
    """Sum of |row| per bag (divided by length for mean): the scale of the
    forward's rounding error."""
    valid = row_off >= 0
    offs = np.unique(row_off[valid])
    if len(offs) == 0:
        return np.zeros((cfg.batch, cfg.n_tables, cfg.dim))
    w, _ = orc.get_rows(offs)
    idx = np.searchsorted(offs, np.where(valid, row_off, offs[0]))
    a = np.abs(w[idx].astype(np.float64)) * valid[:, None]
    lens = np.diff(bo)
    bag = np.repeat(np.arange(cfg.n_bags), lens)
    M = np.zeros((cfg.n_bags, cfg.dim))
    np.add.at(M, bag, a)
    if cfg.pooling == synth.MEAN:
        M /= np.maximum(lens, 1)[:, None]
    return M.reshape(cfg.n_tables, cfg.batch, cfg.dim).transpose(1, 0, 2)


def assert_close(got, ref, M, rtol, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    tol = rtol * M + 1e-30
    bad = err > tol
    if bad.any():
        k = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements beyond {rtol} x magnitude; "
                             f"first at {tuple(k)}: got {got[tuple(k)]!r} ref {ref[tuple(k)]!r} M {M[tuple(k)]!r}")


def compare_rows(gpu: GpuTables, orc, prev_w, offs, rtol, what):
    """Rows after an update: |gpu - ref| <= rtol * (|w_prev| + |delta|);
    optimizer state likewise against its own scale."""
    w_g, s_g = gpu.rows(offs)
    w_r, s_r = orc.get_rows(offs)
    M = np.abs(prev_w.astype(np.float64)) + np.abs(w_r.astype(np.float64) - prev_w)
    assert_close(w_g, w_r, M, rtol, what + " weights")
    if s_r.size:
        assert_close(s_g, s_r, np.abs(s_r.astype(np.float64)) + 1e-30, 1e-5, what + " state")
    return w_g, w_r


class ChunkSnapshot:
    """State of every chunk of a blocks object, kept on the device;
    changed_rows() lists (ascending, global row numbers) the rows whose
    bytes differ from it, weights and state alike.  Bytes of a chunk past
    its last row must not change either.

    mode "copy" keeps a clone of the chunks and compares bytes exactly;
    mode "fingerprint" (for tables too large to hold twice) keeps one 64-bit
    linear hash per row, sum of the row's 8-byte words times fixed random
    odd multipliers mod 2^64: a changed row keeps its fingerprint only if the
    change lies in the kernel of that map, about 2^-64 for a random change.
    "auto" copies when the device has room for a second copy."""

    def __init__(self, blocks, mode="auto"):
        self.blocks = blocks
        R, rb = blocks.rows_per_chunk, blocks.row_bytes
        total = sum(c.numel() for c in blocks.chunks)
        if mode == "auto":
            free, _ = torch.cuda.mem_get_info()
            mode = "copy" if total + (8 << 30) < free else "fingerprint"
        self.mode = mode
        if mode == "copy":
            self.copies = [c.clone() for c in blocks.chunks]
        else:
            g = torch.Generator().manual_seed(12345)
            w = torch.randint(-(2**62), 2**62, (rb // 8,), generator=g, dtype=torch.int64) * 2 + 1
            self.w = w.to(blocks.chunks[0].device)
            self.copies = [self._fp(c) for c in blocks.chunks]

    def _fp(self, c):
        R, rb = self.blocks.rows_per_chunk, self.blocks.row_bytes
        n = R * rb
        rows = c[:n].view(torch.int64).view(R, rb // 8)
        fp = (rows * self.w).sum(dim=1)
        tail = c[n:].clone() if c.numel() > n else None
        return fp, tail

    def changed_rows(self) -> np.ndarray:
        R, rb = self.blocks.rows_per_chunk, self.blocks.row_bytes
        n = R * rb
        out = []
        for k, (cur, old) in enumerate(zip(self.blocks.chunks, self.copies)):
            if self.mode == "copy":
                a = cur[:n].view(torch.int32).view(R, rb // 4)
                b = old[:n].view(torch.int32).view(R, rb // 4)
                diff = (a != b).any(dim=1)
                tail_ok = cur.numel() <= n or torch.equal(cur[n:], old[n:])
            else:
                fp, tail = self._fp(cur)
                diff = fp != old[0]
                tail_ok = tail is None or torch.equal(tail, old[1])
            assert tail_ok, f"bytes past the last row of chunk {k} changed"
            ch = torch.nonzero(diff).flatten()
            if ch.numel():
                out.append(ch.cpu().numpy().astype(np.int64) + k * R)
        return np.concatenate(out) if out else np.zeros(0, np.int64)


def assert_only_touched_changed(snap: ChunkSnapshot, touched: np.ndarray, what: str):
    """Every row outside `touched` keeps its bits exactly."""
    changed = snap.changed_rows()
    stray = np.setdiff1d(changed, touched)
    assert stray.size == 0, f"{what}: {stray.size} rows outside the batch changed, first {stray[:8]}"


def assert_never_touched_match_oracle(gpu, orc, ever_touched: np.ndarray, what: str, batch_rows=1 << 18):
    """Rows never updated hold the oracle's values bit for bit (their key-
    derived initial weights and zero state)."""
    n = orc.n_rows
    rest = np.setdiff1d(np.arange(n, dtype=np.int64), ever_touched)
    for a in range(0, len(rest), batch_rows):
        part = rest[a:a + batch_rows]
        w_g, s_g = gpu.rows(part)
        w_r, s_r = orc.get_rows(part)
        assert np.array_equal(w_g.view(np.uint32), w_r.view(np.uint32)), f"{what}: untouched weights differ"
        assert np.array_equal(s_g.view(np.uint32), s_r.view(np.uint32)), f"{what}: untouched state differs"
    return len(rest)
