"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against what the pages print (worked examples
under tests/golden/), closed forms, or an independent library routine
(PyTorch CPU nn.Embedding / EmbeddingBag / SGD / Adagrad / Adam / SparseAdam),
so that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.
"""

import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            out[k] = v
    return out


def _ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(np.maximum(x, np.float32(1e-30))).astype(np.float64)


def _within_ulps(a, b, n=1):
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    tol = n * np.maximum(_ulp32(a), _ulp32(b))
    return np.all(np.abs(a - b) <= tol)


def _one_hot_offsets(n):
    return np.arange(n + 1, dtype=np.int64)


# ------------------------------------------------------------------ toy ----
def test_toy_sgd_example(oracle_mod):
    """The nn.Embedding(10,4) / ids {2,5,7} / sum(e^2) / SGD lr 0.1 toy."""
    g = _golden("toy_sgd.txt")
    n, d = int(g["num_embeddings"][0]), int(g["embedding_dim"][0])
    ids = np.array([int(x) for x in g["ids"]], np.int64)
    lr = float(g["lr"][0])
    T = oracle_mod.OracleTable(d, optim=oracle_mod.OPT_SGD, lr=lr, seed=7)
    # the table holds ids 0..9; inserting them in order gives offsets 0..9
    off0, n_new = T.find_or_insert(np.arange(n), [0, n])
    assert n_new == n and np.array_equal(off0, np.arange(n))
    W0, _ = T.get_rows(np.arange(n))

    row_off, n_new = T.find_or_insert(ids, [0, len(ids)])
    assert n_new == 0 and np.array_equal(row_off, ids)
    bo = _one_hot_offsets(len(ids))
    out = T.fwd(row_off, bo, batch=len(ids))
    assert out.shape == (len(ids), 1, d)
    assert np.array_equal(out[:, 0, :], W0[ids])            # one row per lookup

    # the same step in PyTorch, as printed on the page
    emb = torch.nn.Embedding(n, d)
    with torch.no_grad():
        emb.weight.copy_(torch.from_numpy(W0))
    opt = torch.optim.SGD(emb.parameters(), lr=lr)
    vecs = emb(torch.from_numpy(ids))
    loss = (vecs ** 2).sum()
    opt.zero_grad()
    loss.backward()
    tgrad = emb.weight.grad.detach().numpy().copy()
    opt.step()
    tW = emb.weight.detach().numpy()

    G = (2.0 * out).astype(np.float32)                       # d sum(out^2) / d out
    U = T.bwd_update(row_off, bo, len(ids), G)
    assert U == len(ids)
    factor = float(g["grad_factor"][0])
    for o in ids:
        gr = T.last_grad(o)
        assert np.array_equal(gr, factor * W0[o].astype(np.float64))   # exactly 2e
        assert np.array_equal(gr.astype(np.float32), tgrad[o])
    untouched = [int(x) for x in g["untouched_rows"]]
    assert np.all(tgrad[untouched] == 0)
    W1, _ = T.get_rows(np.arange(n))
    assert np.array_equal(W1[untouched].view(np.uint32), W0[untouched].view(np.uint32))
    tf = float(g["touched_factor"][0])
    assert _within_ulps(W1[ids], (tf * W0[ids].astype(np.float64)).astype(np.float32), 2)
    assert _within_ulps(W1[ids], tW[ids], 1)
    assert np.array_equal(tW[untouched], W1[untouched])


# ------------------------------------------------------ DLRM shapes -------
def test_dlrm_forward_shape_walkthrough(oracle_mod):
    """Batch 4, d 4, three one-hot fields: pooled output [B, T, d] feeds the
    page's stack -> pairwise dot -> upper triangle -> concat shapes."""
    g = _golden("dlrm_shapes.txt")
    B, d, F, Din = (int(g[k][0]) for k in ("batch", "dim", "fields", "dense_in"))
    rng = np.random.default_rng(3)
    T = oracle_mod.OracleTable(d, n_tables=F, seed=11)
    cats = [rng.integers(0, 200, B) for _ in range(F)]     # e.g. 200 countries
    ids = np.concatenate(cats).astype(np.int64)
    bo = _one_hot_offsets(F * B)
    row_off, _ = T.find_or_insert(ids, bo, stride=B)
    out = T.fwd(row_off, bo, batch=B)
    assert list(out.shape) == [B, F, d]
    for t in range(F):
        rows, _ = T.get_rows(row_off[t * B:(t + 1) * B])
        assert np.array_equal(out[:, t, :], rows)            # one-hot pooling = row lookup

    torch.manual_seed(0)
    dense = torch.randn(B, Din)
    assert list(dense.shape) == eval(g["dense"][0])
    bottom = torch.nn.Linear(Din, d)(dense)
    assert list(bottom.shape) == eval(g["bottom_mlp"][0])
    lookups = [torch.from_numpy(out[:, t, :]) for t in range(F)]
    assert all(list(x.shape) == eval(g["lookup"][0]) for x in lookups)
    X = torch.stack([bottom] + lookups, dim=1)
    assert list(X.shape) == eval(g["stacked"][0])
    Z = torch.bmm(X, X.transpose(1, 2).contiguous())
    assert list(Z.shape) == eval(g["dots"][0])
    iu = torch.triu_indices(F + 1, F + 1, offset=1)
    tri = Z[:, iu[0], iu[1]]
    assert list(tri.shape) == eval(g["upper_triangle"][0])
    cat = torch.cat([bottom, tri], dim=1)
    assert list(cat.shape) == eval(g["concat"][0])
    top = torch.nn.Linear(cat.shape[1], 1)(cat)
    assert list(top.shape) == eval(g["top_mlp"][0])
    # pair (0, t+1) of the triangle is the dot of the dense vector with field t
    for t in range(F):
        k = [i for i in range(iu.shape[1]) if iu[0, i] == 0 and iu[1, i] == t + 1][0]
        ref = (bottom * lookups[t]).sum(1)
        assert torch.allclose(tri[:, k], ref, rtol=1e-6, atol=1e-7)


# -------------------------------------------------- modulo collision ------
def test_modulo_collision_pair_gets_distinct_rows(oracle_mod):
    g = _golden("modulo_collision.txt")
    sl, cards = int(g["slice_len"][0]), int(g["cards"][0])
    a, b, res = int(g["id_a"][0]), int(g["id_b"][0]), int(g["residue"][0])
    assert sl // cards == int(g["per_card"][0])
    assert a % sl == res and b % sl == res          # the collision the page describes
    assert b % (sl - 1) != res                       # the page's "% 65535" is a typo
    T = oracle_mod.OracleTable(4, optim=oracle_mod.OPT_SGD, lr=0.1, seed=5)
    ro, n_new = T.find_or_insert(np.array([a, b, a, b], np.int64), [0, 4])
    assert n_new == 2 and ro[0] != ro[1] and ro[2] == ro[0] and ro[3] == ro[1]
    W0, _ = T.get_rows(ro[:2])
    assert not np.array_equal(W0[0], W0[1])
    # one bag per id; the rows must move independently, each by its own grad
    bo = _one_hot_offsets(2)
    G = np.array([[[1.0, 2.0, 3.0, 4.0]], [[-4.0, 0.5, 0.0, 8.0]]], np.float32)
    T.bwd_update(ro[:2], bo, 2, G)
    W1, _ = T.get_rows(ro[:2])
    for k in range(2):
        ref = (W0[k].astype(np.float64) - 0.1 * G[k, 0].astype(np.float64)).astype(np.float32)
        assert np.array_equal(W1[k], ref)


# --------------------------------------------- brute force vs PyTorch ----
def _random_batch(rng, n_tables, batch, universe, max_len):
    lens = rng.integers(0, max_len + 1, n_tables * batch)
    lens[0] = 0                                   # an empty bag
    bo = np.zeros(n_tables * batch + 1, np.int64)
    np.cumsum(lens, out=bo[1:])
    ids = np.empty(bo[-1], np.int64)
    for j in range(n_tables * batch):
        ids[bo[j]:bo[j + 1]] = rng.choice(universe, bo[j + 1] - bo[j], replace=True)
    if len(ids) > 2:
        ids[bo[1] + 1:bo[1] + 2] = ids[bo[1]:bo[1] + 1]   # a duplicate inside a bag
    return ids, bo


def _torch_pooled(W, row_off, bo, n_tables, batch, mean):
    """EmbeddingBag over the dense matrix W (index = oracle offset), float64,
    reshaped to [batch, n_tables, d]."""
    idx = torch.from_numpy(row_off)
    offs = torch.from_numpy(bo[:-1].copy())
    out = torch.nn.functional.embedding_bag(idx, W, offs, mode="mean" if mean else "sum",
                                            include_last_offset=False)
    d = W.shape[1]
    return out.reshape(n_tables, batch, d).permute(1, 0, 2)


def _torch_step(optim, rows64, state, grad64, lr, eps, b1, b2, step):
    """One step of torch.optim on the touched rows only (float64)."""
    p = torch.nn.Parameter(rows64.clone())
    if optim == 0:
        opt = torch.optim.SGD([p], lr=lr)
    elif optim == 1:
        opt = torch.optim.Adagrad([p], lr=lr, eps=eps, initial_accumulator_value=0.0, foreach=False)
        opt.state[p]["sum"] = state[0].clone()
        opt.state[p]["step"] = torch.tensor(float(step - 1), dtype=torch.float64)
    else:
        opt = torch.optim.Adam([p], lr=lr, betas=(b1, b2), eps=eps, foreach=False)
        opt.state[p]["exp_avg"] = state[0].clone()
        opt.state[p]["exp_avg_sq"] = state[1].clone()
        opt.state[p]["step"] = torch.tensor(float(step - 1), dtype=torch.float64)
    p.grad = grad64
    opt.step()
    if optim == 0:
        new_state = []
    elif optim == 1:
        new_state = [opt.state[p]["sum"]]
    else:
        new_state = [opt.state[p]["exp_avg"], opt.state[p]["exp_avg_sq"]]
    return p.detach(), new_state


@pytest.mark.parametrize("optim", [0, 1, 2])
@pytest.mark.parametrize("mean", [False, True])
@pytest.mark.parametrize("wdtype", [0, 1])
def test_bruteforce_against_torch(oracle_mod, optim, mean, wdtype):
    """Tiny universes: forward against EmbeddingBag, merged gradient against
    autograd, and each optimizer step against torch.optim in float64 rounded
    once to the storage type."""
    rng = np.random.default_rng(100 + optim * 4 + int(mean) * 2 + wdtype)
    d, n_tables, batch = 8, 2, 6
    lr = [0.1, 0.01, 1e-3][optim]
    eps, b1, b2 = 1e-8, 0.9, 0.999
    T = oracle_mod.OracleTable(d, wdtype=wdtype, optim=optim, n_tables=n_tables, lr=lr, eps=eps,
                               beta1=b1, beta2=b2, seed=21)
    k = T.state_per_elem
    universe = rng.choice(2**40, 12, replace=False).astype(np.int64)   # same keys in both tables
    for step in range(1, 5):
        ids, bo = _random_batch(rng, n_tables, batch, universe, 5)
        row_off, _ = T.find_or_insert(ids, bo, stride=batch)
        n = T.n_rows
        W, S = T.get_rows(np.arange(n))
        W64 = torch.from_numpy(W.astype(np.float64))
        # per-table maps: the same key in two tables is two rows
        keys, tabs = T.map_dump()
        assert len(set(zip(keys.tolist(), tabs.tolist()))) == n

        out = T.fwd(row_off, bo, batch, pooling=int(mean))
        Wt = W64.clone().requires_grad_(True)
        ref = _torch_pooled(Wt, row_off, bo, n_tables, batch, mean)
        assert _within_ulps(out, ref.detach().numpy().astype(np.float32), 1)
        # empty bag pools to zero
        assert np.all(out[0, 0] == 0)

        G = rng.standard_normal((batch, n_tables, d)).astype(np.float32)
        (ref * torch.from_numpy(G.astype(np.float64))).sum().backward()
        U = T.bwd_update(row_off, bo, batch, G, pooling=int(mean))
        touched, counts = T.touched()
        assert U == len(touched)
        assert np.array_equal(np.sort(np.unique(row_off[row_off >= 0])), touched)
        assert np.array_equal(counts, np.bincount(row_off, minlength=n)[touched])
        gref = Wt.grad.numpy()
        for o in touched:
            assert np.allclose(T.last_grad(o), gref[o], rtol=1e-12, atol=1e-14)
        untouched = np.setdiff1d(np.arange(n), touched)

        # one optimizer step in torch on exactly the touched rows
        st = [torch.from_numpy(S[touched, q * d:(q + 1) * d].astype(np.float64)) for q in range(k)]
        new_w, new_st = _torch_step(optim, W64[touched], st, torch.from_numpy(gref[touched]),
                                    lr, eps, b1, b2, step)
        W1, S1 = T.get_rows(np.arange(n))
        # The oracle feeds the fp32-rounded state into the weight update;
        # torch keeps it in float64.  That moves the step by at most a few
        # parts in 2^24 of its size, on top of the final rounding.
        ref = new_w.numpy()
        delta = np.abs(ref - W64[touched].numpy())
        got = W1[touched].astype(np.float64)
        if wdtype == 0:
            assert np.all(np.abs(got - ref) <= _ulp32(ref) + delta * 2.0**-21)
        else:
            assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0**-8 + delta * 2.0**-21 + 1e-38)
        for q in range(k):
            assert _within_ulps(S1[touched, q * d:(q + 1) * d], new_st[q].numpy().astype(np.float32), 1)
        assert np.array_equal(W1[untouched].view(np.uint32), W[untouched].view(np.uint32))
        if k:
            assert np.array_equal(S1[untouched].view(np.uint32), S[untouched].view(np.uint32))


def test_lazy_adam_against_sparse_adam(oracle_mod):
    """Multi-step lazy Adam: rows not in a batch keep m and v (SparseAdam).
    SparseAdam places eps inside the bias-corrected step (eps / sqrt(1-b2^t)
    in the oracle's form), so the match is to 1e-6 relative, not bitwise."""
    rng = np.random.default_rng(9)
    d, n_keys = 4, 10
    T = oracle_mod.OracleTable(d, optim=oracle_mod.OPT_ADAM, lr=1e-2, seed=3)
    T.find_or_insert(np.arange(n_keys), [0, n_keys])
    W0, _ = T.get_rows(np.arange(n_keys))
    emb = torch.nn.Embedding(n_keys, d, sparse=True).double()
    with torch.no_grad():
        emb.weight.copy_(torch.from_numpy(W0.astype(np.float64)))
    opt = torch.optim.SparseAdam(emb.parameters(), lr=1e-2, betas=(0.9, 0.999), eps=1e-8)
    for step in range(6):
        ids = rng.choice(n_keys, 5, replace=False).astype(np.int64)   # rows skipped per step
        ro, _ = T.find_or_insert(ids, [0, len(ids)])
        G = rng.standard_normal((len(ids), 1, d)).astype(np.float32)
        T.bwd_update(ro, _one_hot_offsets(len(ids)), len(ids), G)
        opt.zero_grad()
        (emb(torch.from_numpy(ids)) * torch.from_numpy(G[:, 0].astype(np.float64))).sum().backward()
        opt.step()
    W, _ = T.get_rows(np.arange(n_keys))
    ref = emb.weight.detach().numpy()
    assert np.allclose(W, ref, rtol=1e-6, atol=1e-7)
    # a dense Adam would have moved every row on every step: make sure the
    # comparison can tell (rows skipped in a step keep their value)
    assert not np.allclose(W, W0, atol=1e-4)


# --------------------------------------------------------- closed forms ---
def test_first_step_closed_forms(oracle_mod):
    """First Adagrad and Adam steps from zero state reduce to
    w - lr * g / (|g| + eps) (Adam up to fp32 storage of m and v)."""
    rng = np.random.default_rng(4)
    d = 8
    for optim, lr, tol in ((oracle_mod.OPT_ADAGRAD, 0.01, 0), (oracle_mod.OPT_ADAM, 1e-3, 1e-9)):
        T = oracle_mod.OracleTable(d, optim=optim, lr=lr, eps=1e-8, seed=1)
        ro, _ = T.find_or_insert(np.array([3, 4, 3], np.int64), [0, 3])
        W0, _ = T.get_rows(ro[:2])
        G = rng.standard_normal((3, 1, d)).astype(np.float32)
        T.bwd_update(ro, _one_hot_offsets(3), 3, G)
        g = np.stack([T.last_grad(ro[0]), T.last_grad(ro[1])])
        assert np.array_equal(g[0], G[0, 0].astype(np.float64) + G[2, 0].astype(np.float64))
        ref = W0.astype(np.float64) - lr * g / (np.abs(g) + 1e-8)
        W1, S1 = T.get_rows(ro[:2])
        if tol == 0:
            assert _within_ulps(W1, ref.astype(np.float32), 1)
            assert np.array_equal(S1, (g * g).astype(np.float32))       # a = g^2
        else:
            assert np.all(np.abs(W1 - ref) <= 1e-6 * lr + _ulp32(ref))
            assert np.array_equal(S1[:, :d], (0.1 * g).astype(np.float32))
            assert np.array_equal(S1[:, d:], (0.001 * g * g).astype(np.float32))


def test_pooling_special_cases(oracle_mod):
    """Mean of identical rows is the row; an empty bag gives 0 and no
    gradient; a duplicate id in a sum bag counts twice."""
    d = 4
    T = oracle_mod.OracleTable(d, optim=oracle_mod.OPT_SGD, lr=0.5, seed=2)
    ids = np.array([9, 9, 9, 5, 5], np.int64)
    bo = np.array([0, 3, 3, 5], np.int64)       # bags: [9,9,9], [], [5,5]
    ro, _ = T.find_or_insert(ids, bo, stride=3)
    w9, _ = T.get_rows([ro[0]])
    w5, _ = T.get_rows([ro[3]])
    mean = T.fwd(ro, bo, 3, pooling=oracle_mod.POOL_MEAN)
    assert np.array_equal(mean[0, 0], w9[0])
    assert np.all(mean[1, 0] == 0)
    sm = T.fwd(ro, bo, 3, pooling=oracle_mod.POOL_SUM)
    assert np.array_equal(sm[2, 0], (2.0 * w5[0].astype(np.float64)).astype(np.float32))
    G = np.ones((3, 1, d), np.float32)
    U = T.bwd_update(ro, bo, 3, G, pooling=oracle_mod.POOL_MEAN)
    offs, cnt = T.touched()
    assert U == 2 and list(cnt) == [3, 2]
    assert np.allclose(T.last_grad(ro[0]), 3 * (1.0 / 3.0))
    assert np.array_equal(T.last_grad(ro[3]), np.full(d, 1.0))


def test_missing_keys_without_insert(oracle_mod):
    d = 4
    T = oracle_mod.OracleTable(d, seed=2)
    T.find_or_insert(np.array([1, 2], np.int64), [0, 2])
    ro, n_new = T.find_or_insert(np.array([2, 3, 1], np.int64), [0, 3], insert_missing=False)
    assert n_new == 0 and list(ro) == [1, -1, 0] and T.n_rows == 2
    out = T.fwd(ro, np.array([0, 3], np.int64), 1)
    w, _ = T.get_rows([0, 1])
    assert np.array_equal(out[0, 0], (w[0].astype(np.float64) + w[1]).astype(np.float32))


def test_merged_keys(oracle_mod):
    """Merged mode: one map keyed by (table << 56) | id; ids must be < 2^56."""
    T = oracle_mod.OracleTable(4, n_tables=3, merged=True, seed=2)
    ids = np.array([7, 7, 7, 8], np.int64)
    bounds = np.array([0, 1, 2, 4], np.int64)
    ro, n_new = T.find_or_insert(ids, bounds)
    assert n_new == 4 and len(set(ro.tolist())) == 4
    keys, tabs = T.map_dump()
    assert list(keys) == [7, (1 << 56) | 7, (2 << 56) | 7, (2 << 56) | 8]
    assert np.all(tabs == 0)
    with pytest.raises(ValueError):
        T.find_or_insert(np.array([1 << 56], np.int64), [0, 1, 1, 1])


def test_offsets_first_sight_and_stable(oracle_mod):
    """New keys get 0, 1, 2, ... in first-sight order; offsets never move."""
    T = oracle_mod.OracleTable(4, n_tables=2, seed=2)
    ro, n = T.find_or_insert(np.array([50, 40, 50, 40, 60], np.int64), [0, 3, 5], 1)
    assert n == 4 and list(ro) == [0, 1, 0, 2, 3]
    ro2, n2 = T.find_or_insert(np.array([40, 70, 60, 40, 80], np.int64), [0, 2, 5], 1)
    assert n2 == 2 and list(ro2) == [1, 4, 3, 2, 5]
    keys, tabs = T.map_dump()
    assert list(keys) == [50, 40, 40, 60, 70, 80] and list(tabs) == [0, 0, 1, 1, 0, 1]


# ------------------------------------------------------------- init -------
def test_init_hash_matches_published_splitmix64(oracle_mod):
    G = 0x9E3779B97F4A7C15
    with open(os.path.join(GOLDEN, "splitmix64_seed0.txt")) as f:
        rows = [line.split() for line in f if line.strip() and not line.startswith("#")]
    for k, v in rows:
        assert oracle_mod.splitmix64_mix((int(k) * G) % 2**64) == int(v, 16)


def test_init_values_exact_and_spread(oracle_mod):
    keys = np.random.default_rng(0).integers(0, 2**63, 400)
    v32 = np.array([[oracle_mod.init_value(int(k), 0, c, 123, 0) for c in range(4)] for k in keys])
    vbf = np.array([[oracle_mod.init_value(int(k), 0, c, 123, 1) for c in range(4)] for k in keys])
    assert np.all(v32 >= -1 / 16) and np.all(v32 < 1 / 16)
    assert np.all(np.abs(v32) == np.abs(v32).astype(np.float32))           # exact in fp32
    assert np.all((v32 * 2.0**27) == np.round(v32 * 2.0**27))
    assert np.all((vbf * 2.0**11) == np.round(vbf * 2.0**11))             # 8-bit grid
    bits = torch.from_numpy(vbf.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(bits, vbf.astype(np.float32))                    # exact in bf16
    assert abs(v32.mean()) < 0.01 and 0.03 < v32.std() < 0.04             # U(-1/16,1/16): sd 0.036
    assert len(np.unique(v32[:, 0])) > 390
    # the table index and the seed change the row
    assert oracle_mod.init_value(5, 0, 0, 1, 0) != oracle_mod.init_value(5, 1, 0, 1, 0)
    assert oracle_mod.init_value(5, 0, 0, 1, 0) != oracle_mod.init_value(5, 0, 0, 2, 0)


# ------------------------------------------------------------ bf16 --------
def test_bf16_rounding_matches_torch_and_avoids_double_rounding(oracle_mod):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(2000).astype(np.float32),
                        (rng.standard_normal(200) * 1e-39).astype(np.float32),   # subnormals
                        np.array([3.0e38, -3.0e38, 0.0, -0.0], np.float32)])
    # exact ties: an 8-bit value plus half a bf16 ulp
    base = rng.integers(128, 256, 200).astype(np.float64) * 2.0 ** rng.integers(-20, 20, 200)
    ties = (base + base / 256.0).astype(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle_mod.round_bf16_bits(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)
    # a double just above a tie rounds up; going through fp32 first would
    # land on the tie and round to even (down)
    t = 1.0 + 2.0**-8 + 2.0**-40
    assert oracle_mod.round_bf16_bits(t) == 0x3F81
    assert torch.tensor(np.float32(t)).to(torch.bfloat16).view(torch.int16).item() == 0x3F80


# ------------------------------------------------------------- saver ----
def test_resume_from_exported_state_equals_uninterrupted_run(oracle_mod):
    """"RecIS", "Saver": exporting the sparse state (keys, offsets, rows,
    optimizer state, step) after some steps and importing it into a fresh
    table must continue exactly as the uninterrupted run: same offsets for
    old and new keys, same pooled outputs, same rows bit for bit.  Covers
    Adam (step-dependent bias correction), mean pooling and fresh ids, and a
    merged bf16 Adagrad table."""
    import synth

    for cfg in (synth.config(3, n_tables=2, batch=64, cardinality=("fixed", 500), fresh_frac=0.05),
                synth.config(5, n_tables=3, batch=16, cardinality=("fixed", 300))):
        wl = synth.Workload(cfg)

        def table():
            return oracle_mod.OracleTable(cfg.dim, cfg.wdtype, cfg.optim, cfg.n_tables, cfg.merged, seed=cfg.seed,
                                          lr=cfg.lr, eps=cfg.eps, beta1=cfg.beta1, beta2=cfg.beta2)

        a = table()
        for ids, bounds in wl.prepopulation():
            a.find_or_insert(ids, bounds, 1)

        def step(t, s):
            ids, bo = wl.batch_inputs(s)
            ro, nn = t.find_or_insert(ids, bo, cfg.batch)
            out = t.fwd(ro, bo, cfg.batch, cfg.pooling)
            U = t.bwd_update(ro, bo, cfg.batch, wl.grad(s), cfg.pooling)
            return ro, nn, out, U

        for s in range(2):
            step(a, s)
        b = table()
        b.import_state(*a.export_state())
        assert b.step == a.step == 2 and b.n_rows == a.n_rows
        for s in range(2, 4):
            ra, rb = step(a, s), step(b, s)
            assert np.array_equal(ra[0], rb[0]) and ra[1] == rb[1] and ra[3] == rb[3]
            assert np.array_equal(ra[2].view(np.uint32), rb[2].view(np.uint32))
        ka, ta, oa, wa, sa, _ = a.export_state()
        kb, tb, ob, wb, sb, _ = b.export_state()
        assert np.array_equal(ka, kb) and np.array_equal(ta, tb)
        assert np.array_equal(wa.view(np.uint32), wb.view(np.uint32)) and np.array_equal(sa.view(np.uint32),
                                                                                       sb.view(np.uint32))


def test_import_state_rejects_inconsistent_states(oracle_mod):
    t = oracle_mod.OracleTable(4, optim=oracle_mod.OPT_SGD)
    w = np.zeros((2, 4), np.float32)
    st = np.zeros((2, 0), np.float32)
    with pytest.raises(ValueError):          # the same key twice
        t.import_state(np.array([7, 7]), np.array([0, 0], np.int32), np.array([0, 1]), w, st, 0)
    with pytest.raises(ValueError):          # row 1 listed twice, row 0 missing
        t.import_state(np.array([7, 8]), np.array([0, 0], np.int32), np.array([1, 1]), w, st, 0)
    t.import_state(np.array([7, 8]), np.array([0, 0], np.int32), np.array([1, 0]), w, st, 3)
    assert t.n_rows == 2 and t.step == 3
    ro, nn = t.find_or_insert(np.array([8, 7, 9]), [0, 3])
    assert ro.tolist() == [0, 1, 2] and nn == 1


# ------------------------------------------------------ dot interaction ----
def _interaction():
    from oracle import interaction
    return interaction


def test_interaction_shapes_from_the_page():
    """Batch 4, d 4, three fields: pooled [4,3,4] plus the dense vector give
    6 pairs ([4,6]) and [4,10] after the concatenation."""
    g = _golden("dlrm_shapes.txt")
    B, d, F = (int(g[k][0]) for k in ("batch", "dim", "fields"))
    rng = np.random.default_rng(1)
    dense = rng.standard_normal((B, d))
    pooled = rng.standard_normal((B, F, d))
    out, _ = _interaction().interaction_fwd(dense, pooled)
    assert list(out.shape) == eval(g["concat"][0])
    assert out.shape[1] - d == eval(g["upper_triangle"][0])[1]
    assert np.array_equal(out[:, :d], dense)


def test_interaction_pairs_are_the_dots_listed():
    """Every pair of the stacked vectors (dense first, then the fields in
    table order) is one dot product; pair (0, t+1) is dense . field t."""
    rng = np.random.default_rng(2)
    B, T, d = 3, 5, 7
    dense = rng.standard_normal((B, d))
    pooled = rng.standard_normal((B, T, d))
    out, _ = _interaction().interaction_fwd(dense, pooled)
    vecs = [dense] + [pooled[:, t, :] for t in range(T)]
    p = d
    for i in range(T + 1):
        for j in range(i + 1, T + 1):
            for b in range(B):
                assert abs(out[b, p] - sum(vecs[i][b, k] * vecs[j][b, k] for k in range(d))) < 1e-12
            p += 1
    assert p == d + (T + 1) * T // 2


def test_interaction_backward_matches_torch_autograd():
    """The oracle's backward against torch autograd (float64) of the same
    forward built from torch ops (bmm, triu_indices, cat)."""
    rng = np.random.default_rng(3)
    B, T, d = 4, 6, 8
    dense = torch.tensor(rng.standard_normal((B, d)), requires_grad=True)
    pooled = torch.tensor(rng.standard_normal((B, T, d)), requires_grad=True)
    X = torch.cat([dense[:, None, :], pooled], dim=1)
    Z = torch.bmm(X, X.transpose(1, 2).contiguous())
    iu = torch.triu_indices(T + 1, T + 1, offset=1)
    out = torch.cat([dense, Z[:, iu[0], iu[1]]], dim=1)
    dout = torch.tensor(rng.standard_normal(tuple(out.shape)))
    out.backward(dout)
    dd, dp, _, _ = _interaction().interaction_bwd(dense.detach().numpy(), pooled.detach().numpy(), dout.numpy())
    o, _ = _interaction().interaction_fwd(dense.detach().numpy(), pooled.detach().numpy())
    assert np.allclose(o, out.detach().numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(dd, dense.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dp, pooled.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_interaction_backward_matches_finite_differences():
    rng = np.random.default_rng(4)
    B, T, d = 2, 3, 4
    dense = rng.standard_normal((B, d))
    pooled = rng.standard_normal((B, T, d))
    inter = _interaction()
    out, _ = inter.interaction_fwd(dense, pooled)
    dout = rng.standard_normal(out.shape)
    dd, dp, _, _ = inter.interaction_bwd(dense, pooled, dout)
    h = 1e-6

    def loss(de, po):
        return float((inter.interaction_fwd(de, po)[0] * dout).sum())

    for b in range(B):
        for k in range(d):
            e = np.zeros_like(dense)
            e[b, k] = h
            assert abs((loss(dense + e, pooled) - loss(dense - e, pooled)) / (2 * h) - dd[b, k]) < 1e-6
            for t in range(T):
                e = np.zeros_like(pooled)
                e[b, t, k] = h
                assert abs((loss(dense, pooled + e) - loss(dense, pooled - e)) / (2 * h) - dp[b, t, k]) < 1e-6


def test_interaction_field_permutation_permutes_pairs():
    """Swapping two fields swaps the pairs that involve them; pairs of the
    other vectors are unchanged."""
    rng = np.random.default_rng(5)
    B, T, d = 2, 4, 3
    dense = rng.standard_normal((B, d))
    pooled = rng.standard_normal((B, T, d))
    inter = _interaction()
    a, _ = inter.interaction_fwd(dense, pooled)
    sw = pooled[:, [0, 2, 1, 3], :]
    b_, _ = inter.interaction_fwd(dense, sw)
    F = T + 1

    def p(i, j):
        i, j = min(i, j), max(i, j)
        return d + i * F - i * (i + 1) // 2 + (j - i - 1)

    perm = {0: 0, 1: 1, 2: 3, 3: 2, 4: 4}          # vector index after the swap of fields 1 and 2
    for i in range(F):
        for j in range(i + 1, F):
            assert np.allclose(a[:, p(i, j)], b_[:, p(perm[i], perm[j])])
