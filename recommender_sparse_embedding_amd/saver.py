"""Saver: the sparse state of one table group as a SafeTensors file
("RecIS：阿里开源推荐系统统一训练框架", "Saver": the sparse parameters are
exported and imported so that training resumes where it stopped).

The file holds, in row-offset order, every live entry of the ID map and its
row:

    keys     int64 [n]            feature ID (merged maps: (t << 56) | id)
    tables   int32 [n]            map table (0 for a merged map)
    offsets  int64 [n]            row offset
    weights  float32 or bfloat16 [n, dim]   the row's weights, in storage type
    state    float32 [n, k*dim]   Adagrad accumulator / Adam m then v

and, as string metadata, what recreates the objects: the blocks' dim, weight
type, optimizer, chunk size, chunk-table size and init seed, the map's slot
counts per table, max load, merged flag and hash seed, the row counter, the
optimizer step and a format tag.  Rows below the row counter that no key
references (rows freed by an eviction and not yet reused) are not written:
the free list they form is, at any time, exactly those rows in ascending
order, so load(free_list=True) rebuilds it with a rehash.  Every step runs
in the library (map export / import, row read / write, rehash); this module
only moves tensors between the device and the file.
"""

from __future__ import annotations

import json

import torch
from safetensors import safe_open
from safetensors.torch import save_file

FORMAT = "rse-sparse-state-1"


def save(path: str, idmap, blocks, step: int = 0, extra: dict | None = None, stream=None) -> dict:
    """Write the state of (idmap, blocks) and the optimizer step to `path`.
    Returns the metadata written."""
    from . import BF16, RseError

    rows_used, st = blocks.status(stream)
    map_st, n_keys = idmap.status(stream)
    if st != 0 or map_st != 0:
        raise RseError("save: objects carry a sticky error status", st or map_st)
    total = int(sum(n_keys))
    keys, tabs, offs, cnt = idmap.export(total, stream)
    if cnt != total or cnt > rows_used:
        raise ValueError(f"save: {cnt} map entries, {total} counted keys, {rows_used} rows in use")
    order = torch.argsort(offs)
    keys, tabs, offs = keys[order].contiguous(), tabs[order].contiguous(), offs[order].contiguous()
    w, state = blocks.read_rows(offs, stream)
    if blocks.w_dtype == BF16:
        w = w.to(torch.bfloat16)          # exact: the rows hold bf16 values
    tensors = {"keys": keys.cpu(), "tables": tabs.cpu(), "offsets": offs.cpu(), "weights": w.cpu(),
               "state": state.cpu()}
    meta = {
        "format": FORMAT, "dim": blocks.dim, "w_dtype": blocks.w_dtype, "optim": blocks.optim,
        "rows_per_chunk_log2": blocks.rows_per_chunk_log2, "max_chunks": blocks.max_chunks,
        "init_seed": blocks.seed, "slots_per_table": idmap.slots_per_table, "max_load": idmap.max_load,
        "merged": int(idmap.merged), "hash_seed": idmap.hash_seed, "rows_used": int(rows_used),
        "step": int(step), "extra": extra or {},
    }
    save_file(tensors, path, metadata={k: json.dumps(v) for k, v in meta.items()})
    return meta


def load(path: str, device="cuda", extra_rows: int = 0, free_list: bool = False, stream=None):
    """Recreate (idmap, blocks) from a file written by save(), with room for
    `extra_rows` more rows.  free_list=True attaches a free list to the
    blocks and rebuilds it (the rows below the row counter that no key
    references, ascending), as the saved run's free list held them.
    Returns (idmap, blocks, metadata); metadata["step"] is the optimizer
    step to continue from."""
    from . import EmbeddingBlocks, IdMap, RseError

    with safe_open(path, framework="pt") as f:
        meta = {k: json.loads(v) for k, v in f.metadata().items()}
        if meta.get("format") != FORMAT:
            raise ValueError(f"{path}: not a {FORMAT} file")
        t = {k: f.get_tensor(k) for k in ("keys", "tables", "offsets", "weights", "state")}
    dev = torch.device(device)
    idm = IdMap(meta["slots_per_table"], max_load=meta["max_load"], merged=bool(meta["merged"]),
                hash_seed=meta["hash_seed"], device=dev, stream=stream)
    blk = EmbeddingBlocks(meta["dim"], meta["w_dtype"], meta["optim"], meta["rows_per_chunk_log2"],
                          max_chunks=meta["max_chunks"], seed=meta["init_seed"], device=dev, stream=stream)
    rows = meta["rows_used"] + int(extra_rows)
    blk.grow(max(1, -(-rows // blk.rows_per_chunk)), stream)
    keys, tabs, offs = (t[k].to(dev) for k in ("keys", "tables", "offsets"))
    w = t["weights"].to(dev, torch.float32).contiguous()
    state = t["state"].to(dev).contiguous()
    idm.import_entries(keys, tabs, offs, stream)
    blk.write_rows(offs, w, state if blk.state_per_elem else None, stream)
    blk.set_rows_used(meta["rows_used"], stream)
    map_st, _ = idm.status(stream)
    _, st = blk.status(stream)
    if map_st != 0 or st != 0:
        raise RseError("load: restoring the state failed", map_st or st)
    if free_list:
        blk.enable_free_list(stream=stream)
        idm.evict(blk, 0, stream)          # nothing evicted: rebuilds the free list
    return idm, blk, meta
