"""A pruned weight's column never reaches the sum.

The product sums kept weights only (y[r] = sum over kept c of W[r][c] x[c],
"Method", item (1): only the kept weights are stored and the mask names their
columns), and the oracle skips every pruned entry.  So x may hold Inf or NaN
at a column that every row pruned, and the result is still the finite sum of
the kept terms.  This pins the traversals that take kept columns only: the
2:4 chunk path and the sparse matrix cores, the fixed-step and direct kernels
at other densities, and the unstructured kernel, whose steps past a lane's
count read a zeroed pad slot of x.  The decompressed-tile matrix-core path
(N:M other than 2:4 at batch >= 5) shares one dense x tile between rows and
multiplies the tile's stored zeros, so it is left out: there Inf or NaN at a
pruned column gives NaN, as a dense product of the zero-filled matrix would.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_gemv_memory_amd import native, synth

from test_gpu_parity import DEV, TOL, f64, gpu_pack, rel_l2, t16

pytestmark = pytest.mark.gpu

INF, NINF, NAN = 0x7C00, 0xFC00, 0x7E00  # binary16 patterns


def prune_columns(keep, cols_j, m):
    """Move every kept entry at a column of cols_j to a pruned column of the
    same group (one column of cols_j per group), so no row keeps them."""
    keep = keep.copy()
    for j in cols_j:
        g0 = j - j % m
        for r in np.nonzero(keep[:, j])[0]:
            free = [c for c in range(g0, g0 + m) if keep[r, c] == 0]
            keep[r, j], keep[r, free[0]] = 0, 1
    return keep


def poisoned_x(batch, cols, cols_j, seed):
    X = synth.activations(batch, cols, seed=seed, dtype="f16").copy()
    for i, j in enumerate(cols_j):
        X[:, j] = (INF, NINF, NAN)[i % 3]
    return X


@pytest.mark.parametrize("n,m,batch", [(2, 4, 1), (2, 4, 4), (2, 4, 8), (4, 8, 1), (8, 16, 1),
                                       (1, 4, 1), (3, 4, 8), (3, 8, 3), (5, 16, 2), (7, 8, 1)])
def test_nonfinite_x_at_pruned_columns(n, m, batch):
    rows, cols = 96, 2112
    W = synth.weights(rows, cols, seed=n + m, dtype="f16")
    cols_j = [5, 70, 1001, 2111 - (2111 % m)]
    keep = prune_columns(synth.random_mask(rows, cols, n, m, seed=m), cols_j, m)
    assert keep[:, cols_j].sum() == 0
    X = poisoned_x(batch, cols, cols_j, seed=batch)
    values, bits = gpu_pack(W, keep, n, m, "f16")
    Y = f64(native.nm_spmm_small(values, bits, t16(X, "f16"), n, m))
    want = oracle.masked_gemv(W, keep, X, False)
    assert np.isfinite(want).all()
    assert np.isfinite(Y).all()
    for b in range(batch):
        assert rel_l2(Y[b], want[b]) <= TOL


@pytest.mark.parametrize("batch", [1, 8])
def test_nonfinite_x_at_pruned_columns_unstructured(batch):
    rows, cols = 96, 4160
    W = synth.weights(rows, cols, seed=3, dtype="f16")
    keep = synth.topk_row_mask(W, 0.5).copy()
    cols_j = [0, 31, 2048, 4159]
    keep[:, cols_j] = 0
    X = poisoned_x(batch, cols, cols_j, seed=batch + 1)
    values, bits, offs = native.nm_pack_bitmask(t16(W, "f16"), torch.from_numpy(keep).to(DEV))
    Y = f64(native.nm_spmm_bitmask(values, bits, offs, t16(X, "f16")))
    want = oracle.masked_gemv(W, keep, X, False)
    assert np.isfinite(Y).all()
    for b in range(batch):
        assert rel_l2(Y[b], want[b]) <= TOL
