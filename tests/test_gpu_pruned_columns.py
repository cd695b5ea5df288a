"""A pruned weight's column never reaches the sum.

The product sums kept weights only (y[r] = sum over kept c of W[r][c] x[c],
"Method", item (1): only the kept weights are stored and the mask names their
columns), and the oracle skips every pruned entry.  So x may hold Inf or NaN
at a column that every row pruned, and the result is still the finite sum of
the kept terms.  This pins every traversal under its default launch: the 2:4
chunk path and the sparse matrix cores, the 4:8 pair table (whose zero
selectors never read a pruned column's x), the fixed-step scan, the
decompressed-tile matrix-core kinds (4:8, 8:16, 16:32 at batch >= 5, whose
tile product falls back to a kept-column sum for a block whose x is not
finite), the direct and window kernels at other densities, and the
unstructured kernel, whose steps past a lane's count read a zeroed pad slot
of x.  Where Inf or NaN sits at a kept column, the row's result is Inf or NaN
exactly where the oracle's is (same sign for Inf).
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_gemv_memory_amd import native, synth

from test_gpu_parity import DEV, TOL, f64, gpu_pack, rel_l2, t16

pytestmark = pytest.mark.gpu

INF, NINF, NAN = 0x7C00, 0xFC00, 0x7E00  # binary16 patterns

# (n, m, batch) on every kernel the default launch picks: 2:4 chunk path
# (batch 1), its form with x plain per token (batch 4 on this small shape) and
# the sparse matrix cores (batch 8); the 4:8 pair table (batch 1) and the
# scan (8:16, 16:32 at batch 1, 8:16 at batch 2); the decompressed
# tile (4:8 at 5 and 8, 8:16 and 16:32 at 8); other densities
CASES = [(2, 4, 1), (2, 4, 4), (2, 4, 8), (4, 8, 1), (8, 16, 1), (16, 32, 1), (8, 16, 2),
         (4, 8, 5), (4, 8, 8), (8, 16, 8), (16, 32, 8), (1, 4, 1), (3, 4, 8), (3, 8, 3),
         (5, 16, 2), (7, 8, 1)]


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


def default_kernel(rows, cols, batch, n, m):
    return native.nm_default_launch(rows, cols, batch, n, m).kernel


@pytest.mark.parametrize("n,m,batch", CASES)
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


def test_cases_cover_every_kernel():
    """The decompressed-tile kinds are among the cases (4:8 at batch 5, and
    8:16 / 16:32 at batch 8 take the matrix cores by default), and so are the
    sparse matrix cores (2:4 at batch 8) and the VALU 2:4 kernel with x stored
    plainly per token (2:4 at batch 4 on this small shape)."""
    for n, m, batch in [(4, 8, 5), (4, 8, 8), (8, 16, 8), (16, 32, 8), (2, 4, 8)]:
        assert default_kernel(96, 2112, batch, n, m) == native.NM_KERNEL_MFMA
    for n, m, batch in [(2, 4, 1), (2, 4, 4), (4, 8, 1), (8, 16, 1), (16, 32, 1), (8, 16, 2)]:
        assert default_kernel(96, 2112, batch, n, m) == native.NM_KERNEL_VALU


def same_class(got, want):
    """Element by element: NaN where the oracle is NaN, the oracle's Inf where
    it is infinite, finite elsewhere."""
    nan_w, inf_w = np.isnan(want), np.isinf(want)
    assert np.array_equal(np.isnan(got), nan_w)
    assert np.array_equal(np.isinf(got), inf_w)
    assert np.array_equal(got[inf_w], want[inf_w])


@pytest.mark.parametrize("n,m,batch", CASES)
def test_nonfinite_x_at_kept_columns(n, m, batch):
    """Inf / -Inf / NaN in x at columns some rows keep and others prune: the
    rows that keep one are Inf or NaN as the oracle's fp64 sum is; every other
    row is finite and matches."""
    rows, cols = 96, 2112
    W = synth.weights(rows, cols, seed=2 * n + m, dtype="f16")
    keep = synth.random_mask(rows, cols, n, m, seed=m + 1)
    cols_j = [5, 70, 1001, 2111 - (2111 % m)]
    # each poisoned column kept by a few rows only
    for i, j in enumerate(cols_j):
        kept_rows = np.nonzero(keep[:, j])[0]
        keep = prune_columns_rows(keep, j, kept_rows[3 + i:], m)
    X = poisoned_x(batch, cols, cols_j, seed=batch + 10)
    values, bits = gpu_pack(W, keep, n, m, "f16")
    Y = f64(native.nm_spmm_small(values, bits, t16(X, "f16"), n, m))
    want = oracle.masked_gemv(W, keep, X, False)
    assert (~np.isfinite(want)).any() and np.isfinite(want).any()
    same_class(Y, want)
    fin = np.isfinite(want)
    for b in range(batch):
        assert rel_l2(Y[b][fin[b]], want[b][fin[b]]) <= TOL


def prune_columns_rows(keep, j, rows_r, m):
    """prune_columns for column j in the given rows only."""
    keep = keep.copy()
    g0 = j - j % m
    for r in rows_r:
        free = [c for c in range(g0, g0 + m) if keep[r, c] == 0]
        keep[r, j], keep[r, free[0]] = 0, 1
    return keep


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
