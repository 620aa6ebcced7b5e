"""DLRM dot interaction on the GPU against the oracle ("DLRM — Meta 把工业推荐
模型拆成 4 个标准积木", "案例 3"): forward and backward element by element
within 1e-5 of each element's magnitude bound, at the workloads' shapes
(click-log 26 tables x dim 128, 100 merged tables x dim 32, the page's
batch 4 / dim 4 / 3 fields, ragged batches), and chained with the pooled
forward and the sparse update."""

import numpy as np
import pytest
import torch

import synth
from harness import GpuTables, assert_close, make_oracle, pooled_magnitude
from oracle import interaction as ointer

pytestmark = pytest.mark.gpu

RTOL = 1e-5


@pytest.mark.parametrize("B,T,d", [(4, 3, 4), (300, 3, 4), (1000, 26, 128), (257, 100, 32), (513, 8, 16),
                                   (77, 4, 64), (33, 1, 256), (5, 15, 8)])
def test_interaction_matches_oracle(B, T, d):
    import recommender_sparse_embedding_amd as rse

    rng = np.random.default_rng(B * 1000 + T * 10 + d)
    dense = rng.standard_normal((B, d)).astype(np.float32)
    pooled = rng.standard_normal((B, T, d)).astype(np.float32)
    t_dense, t_pooled = torch.from_numpy(dense).cuda(), torch.from_numpy(pooled).cuda()
    out = rse.dlrm_interaction_fwd(t_dense, t_pooled)
    ref, mag = ointer.interaction_fwd(dense, pooled)
    assert out.shape == (B, d + (T + 1) * T // 2)
    assert_close(out.cpu().numpy(), ref, mag, RTOL, "interaction forward")
    assert torch.equal(out[:, :d], t_dense)
    dout = rng.standard_normal(tuple(out.shape)).astype(np.float32)
    dd, dp = rse.dlrm_interaction_bwd(t_dense, t_pooled, torch.from_numpy(dout).cuda())
    rdd, rdp, mdd, mdp = ointer.interaction_bwd(dense, pooled, dout)
    assert_close(dd.cpu().numpy(), rdd, mdd, RTOL, "interaction dense gradient")
    assert_close(dp.cpu().numpy(), rdp, mdp, RTOL, "interaction pooled gradient")


def test_interaction_empty_batch_and_limits():
    import recommender_sparse_embedding_amd as rse

    e = torch.empty((0, 8), device="cuda")
    out = rse.dlrm_interaction_fwd(e, torch.empty((0, 3, 8), device="cuda"))
    assert out.shape == (0, 8 + 6)
    big = torch.zeros((2, 200, 128), device="cuda")      # 201 x 129 floats + 201^2 > 64 KiB
    with pytest.raises(rse.RseError) as ex:
        rse.dlrm_interaction_fwd(torch.zeros((2, 128), device="cuda"), big)
    assert ex.value.code == -2


def test_interaction_chained_with_lookup_and_update():
    """ids -> pooled forward -> interaction -> (upstream gradient of the
    interaction output) -> interaction backward -> sparse update, against the
    oracle's chain: pooled outputs, interaction outputs, the pooled-output
    gradient and the updated rows."""
    import recommender_sparse_embedding_amd as rse

    cfg = synth.config(2, n_tables=6, batch=512, dim=32, cardinality=("fixed", 3000))
    wl = synth.Workload(cfg)
    orc = make_oracle(cfg)
    gpu = GpuTables(cfg, wl.card, int(wl.card.sum()) + 64)
    for ids, bounds in wl.prepopulation():
        orc.find_or_insert(ids, bounds, 1)
        gpu.find_or_insert(ids, bounds, 1)
    ids, bo = wl.batch_inputs(0)
    ro_r, _ = orc.find_or_insert(ids, bo, cfg.batch)
    ro_g, _ = gpu.find_or_insert(ids, bo, cfg.batch)
    assert np.array_equal(ro_g.cpu().numpy(), ro_r)
    pooled_g = gpu.fwd(ro_g, bo)
    pooled_r = orc.fwd(ro_r, bo, cfg.batch, cfg.pooling)
    assert_close(pooled_g.cpu().numpy(), pooled_r, pooled_magnitude(orc, ro_r, bo, cfg), RTOL, "pooled")
    rng = np.random.default_rng(9)
    dense = rng.standard_normal((cfg.batch, cfg.dim)).astype(np.float32)
    out_g = rse.dlrm_interaction_fwd(torch.from_numpy(dense).cuda(), pooled_g)
    out_r, mag = ointer.interaction_fwd(dense, pooled_r)
    assert_close(out_g.cpu().numpy(), out_r, mag, RTOL, "interaction output")
    dout = rng.standard_normal(tuple(out_g.shape)).astype(np.float32)
    _, dp_g = rse.dlrm_interaction_bwd(torch.from_numpy(dense).cuda(), pooled_g, torch.from_numpy(dout).cuda())
    _, dp_r, _, mdp = ointer.interaction_bwd(dense, pooled_r, dout)
    assert_close(dp_g.cpu().numpy(), dp_r, mdp, RTOL, "pooled-output gradient")
    offs = np.unique(ro_r)
    prev, _ = orc.get_rows(offs)
    U_r = orc.bwd_update(ro_r, bo, cfg.batch, dp_r.astype(np.float32), cfg.pooling)
    U_g = gpu.bwd(ro_g, bo, dp_g)
    assert U_g == U_r
    w_g, _ = gpu.rows(offs)
    w_r, _ = orc.get_rows(offs)
    # rows: the update's own bound plus the gradient's difference carried
    # through one Adagrad step (at most lr per element)
    M = np.abs(prev.astype(np.float64)) + np.abs(w_r.astype(np.float64) - prev) + cfg.lr * 1e-3
    assert_close(w_g, w_r, M, RTOL, "updated rows")
