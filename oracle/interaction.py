"""Oracle of the DLRM pairwise dot interaction (test infrastructure only:
imported by the tests, never by the library or its binding).

"DLRM — Meta 把工业推荐模型拆成 4 个标准积木", "核心思想" item 3 and "案例 3":
the dense vector and the N pooled embeddings of each sample are stacked
(dense first), every pair is dotted, the strict upper triangle of the
resulting F x F matrix is kept (row-major: (0,1), (0,2), ..., (1,2), ...) and
concatenated after the dense vector.  Plain numpy in float64; the batched
product X X^T is the one library step.
"""

from __future__ import annotations

import numpy as np


def _stack(dense, pooled):
    dense = np.asarray(dense, np.float64)
    pooled = np.asarray(pooled, np.float64)
    B, T, d = pooled.shape
    assert dense.shape == (B, d)
    return np.concatenate([dense[:, None, :], pooled], axis=1), T, d


def interaction_fwd(dense, pooled):
    """out [B, d + F(F-1)/2] (float64) and the magnitude bound of each output
    element (|dense| for the copied part, sum_k |x_ik x_jk| for a pair)."""
    X, T, d = _stack(dense, pooled)
    F = T + 1
    Z = np.matmul(X, np.transpose(X, (0, 2, 1)))
    A = np.abs(X)
    M = np.matmul(A, np.transpose(A, (0, 2, 1)))
    iu = np.triu_indices(F, k=1)
    out = np.concatenate([X[:, 0, :], Z[:, iu[0], iu[1]]], axis=1)
    mag = np.concatenate([A[:, 0, :], M[:, iu[0], iu[1]]], axis=1)
    return out, mag


def interaction_bwd(dense, pooled, dout):
    """(ddense [B, d], dpooled [B, T, d]) in float64, and their magnitude
    bounds: with G the symmetric matrix of the pair gradients (zero
    diagonal), dX = G X; ddense = dout[:, :d] + dX[:, 0]."""
    X, T, d = _stack(dense, pooled)
    F = T + 1
    dout = np.asarray(dout, np.float64)
    B = X.shape[0]
    iu = np.triu_indices(F, k=1)
    G = np.zeros((B, F, F))
    G[:, iu[0], iu[1]] = dout[:, d:]
    G = G + np.transpose(G, (0, 2, 1))
    dX = np.matmul(G, X)
    dM = np.matmul(np.abs(G), np.abs(X))
    ddense = dout[:, :d] + dX[:, 0, :]
    mdense = np.abs(dout[:, :d]) + dM[:, 0, :]
    return ddense, dX[:, 1:, :], mdense, dM[:, 1:, :]
