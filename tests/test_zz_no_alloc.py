"""idmap_find_or_insert_noalloc (static per-GPU scratch, no workspace)
against idmap_find_or_insert (caller workspace), called through the C ABI:
two calls in a row on twin maps and blocks, the second with a smaller input,
must give identical row offsets, new-key counts, map contents and initial
rows.  A call beyond RSE_NOALLOC_MAX_IDS is refused before any work."""

import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _ids(rng, n_tables, per_table, universe):
    """Table-major lookups drawn with repeats from each table's universe."""
    parts = [rng.choice(universe[t], per_table[t]) for t in range(n_tables)]
    bounds = np.zeros(n_tables + 1, np.int64)
    np.cumsum(per_table, out=bounds[1:])
    return np.concatenate(parts).astype(np.int64), bounds


def test_noalloc_find_matches_workspace_find_on_two_calls():
    import recommender_sparse_embedding_amd as rse

    lib = rse.lib
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    T = 3
    rng = np.random.default_rng(2024)
    universe = [rng.integers(-(2**63), 2**63 - 1, 400_000, dtype=np.int64) for _ in range(T)]
    objs = []
    for _ in range(2):
        m = rse.IdMap([1 << 20] * T, max_load=0.8, hash_seed=9, device=dev)
        b = rse.EmbeddingBlocks(32, rse.BF16, rse.ADAGRAD, rows_per_chunk_log2=18, seed=3, device=dev).grow(6)
        objs.append((m, b))
    (m_ws, b_ws), (m_na, b_na) = objs
    ws = m_ws.workspace(1_200_000)

    # call 1: 1.2M lookups; call 2: 90k lookups, old and new keys mixed
    for call, per_table in enumerate(([500_000, 300_000, 400_000], [40_000, 20_000, 30_000])):
        ids, bounds = _ids(rng, T, per_table, universe)
        n = len(ids)
        _say(f"  call {call}: {n} lookups")
        t_ids = torch.from_numpy(ids).to(dev)
        t_b = torch.from_numpy(bounds).to(dev)
        ro_ws = torch.full((n,), -7, dtype=torch.int64, device=dev)
        ro_na = torch.full((n,), -7, dtype=torch.int64, device=dev)
        nn_ws = torch.zeros(1, dtype=torch.int64, device=dev)
        nn_na = torch.full((1,), -7, dtype=torch.int64, device=dev)
        rc = lib.idmap_find_or_insert(m_ws.handle, b_ws.handle, t_ids.data_ptr(), n, t_b.data_ptr(), 1, T, 1,
                                      ro_ws.data_ptr(), nn_ws.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        assert rc == 0, rse.status_str(rc)
        rc = lib.idmap_find_or_insert_noalloc(m_na.handle, b_na.handle, t_ids.data_ptr(), n, t_b.data_ptr(), 1,
                                              T, 1, ro_na.data_ptr(), nn_na.data_ptr(), stream)
        assert rc == 0, rse.status_str(rc)
        torch.cuda.synchronize()
        assert int(nn_na.item()) == int(nn_ws.item()) > 0
        assert torch.equal(ro_na, ro_ws), f"row offsets differ on call {call}"
        assert m_na.status() == m_ws.status() and m_na.status()[0] == 0
        assert b_na.status() == b_ws.status()
        cap = sum(m_ws.status()[1]) + 16
        k1, t1, o1, c1 = m_ws.export(cap)
        k2, t2, o2, c2 = m_na.export(cap)
        assert c1 == c2
        a = np.lexsort((k1.cpu().numpy(), t1.cpu().numpy()))
        b = np.lexsort((k2.cpu().numpy(), t2.cpu().numpy()))
        for x, y in ((k1, k2), (t1, t2), (o1, o2)):
            assert np.array_equal(x.cpu().numpy()[a], y.cpu().numpy()[b]), f"map contents differ on call {call}"
        used = b_ws.status()[0]
        offs = torch.arange(used, device=dev)
        w1, s1 = b_ws.read_rows(offs)
        w2, s2 = b_na.read_rows(offs)
        assert torch.equal(w1.view(torch.int32), w2.view(torch.int32)) and torch.equal(s1, s2)
        _say(f"  call {call}: {int(nn_na.item())} new keys, {used} rows, identical")

    # beyond the limit: refused on the host, nothing enqueued
    big = rse.NOALLOC_MAX_IDS + 1
    rc = lib.idmap_find_or_insert_noalloc(m_na.handle, b_na.handle, t_ids.data_ptr(), big, t_b.data_ptr(), 1, T, 1,
                                          ro_na.data_ptr(), nn_na.data_ptr(), stream)
    assert rc == -3
    torch.cuda.synchronize()
    assert m_na.status()[0] == 0
