"""Parity of the N:M product at densities other than 50% with the CPU oracle.

Every aligned 32-bit mask word of an N:M row with M | 32 holds exactly
32N/M set bits ("Method", item (2), whose fixed-count argument the pages make
at 50%), so the packed format and the fixed-step traversal carry over; these
patterns run on the generic window kernel.  Bars as in test_gpu_parity: pack
bit-exact; fp32 output within rel-L2 1e-3 of the oracle's fp64 result, and
bit-exact on integer-valued inputs; 16-bit output the fp32 sum rounded to
nearest-even.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_gemv_memory_amd import native, synth

from test_gpu_parity import (DEV, TOL, check_16bit_output, f64, gpu_pack, inputs, rel_l2, t16,
                             u16, u32)

pytestmark = pytest.mark.gpu

# 1:4, 3:4, 1:8, 3:8 and 2:16, 6:16, 8:32, 24:32 take the direct kernel (4, 2 and
# 1 independent scan chains per word); the others the window kernel
DENSITIES = [(1, 4), (3, 4), (1, 8), (3, 8), (7, 8), (5, 16), (1, 32), (31, 32),
             (2, 16), (6, 16), (8, 32), (24, 32)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", DENSITIES)
@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (37, 320), (130, 1056), (64, 4096)])
@pytest.mark.parametrize("mask", ["topn", "random"])
def test_pack_other_densities_bit_exact(rows, cols, n, m, dtype, mask):
    W, keep, _ = inputs(rows, cols, n, m, dtype, 1, seed=rows * 5 + cols + n, mask=mask)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    st, ov, ob = oracle.pack(W, keep, n, m)
    assert st == oracle.OK
    assert values.shape == (rows, cols * n // m)
    assert np.array_equal(u16(values), ov)
    assert np.array_equal(u32(bits), ob)


def test_pack_other_densities_rejects_wrong_count():
    W, keep, _ = inputs(8, 128, 1, 4, "f16", 1, seed=3)
    with pytest.raises(native.NMError) as e:
        gpu_pack(W, keep, 3, 4, "f16")  # a 1:4 mask is not a 3:4 mask
    assert e.value.status == native.NM_ERR_MASK


# ragged shapes: window tails (cols not a multiple of 2048 = 64 words),
# odd row counts, a single word per row
SHAPES = [(1, 32), (5, 96), (67, 1056), (130, 2080), (257, 4160)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", DENSITIES)
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_product_other_densities_matches_oracle(rows, cols, n, m, dtype):
    batch = 3
    W, keep, X = inputs(rows, cols, n, m, dtype, batch, seed=rows + cols + 3 * n + m)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16")
    y1 = native.nm_spmv(values, bits, t16(X[0], dtype), n, m)
    assert rel_l2(f64(y1)[None], want[:1]) <= TOL
    Y = native.nm_spmm_small(values, bits, t16(X, dtype), n, m)
    for b in range(batch):
        assert rel_l2(f64(Y[b]), want[b]) <= TOL


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,m", [(1, 4), (3, 4), (3, 8), (5, 16)])
def test_product_other_densities_every_batch(batch, n, m):
    rows, cols = 203, 4160
    W, keep, X = inputs(rows, cols, n, m, "f16", batch, seed=batch * 11 + n)
    values, bits = gpu_pack(W, keep, n, m, "f16")
    want = oracle.masked_gemv(W, keep, X, False)
    Y = native.nm_spmm_small(values, bits, t16(X, "f16"), n, m)
    for b in range(batch):
        assert rel_l2(f64(Y[b]), want[b]) <= TOL


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", [(1, 4), (3, 4), (7, 8), (1, 32), (31, 32)])
def test_integer_inputs_bit_exact_other_densities(n, m, dtype):
    """W, x in {-3..3}: every partial sum is an integer far below 2**24, so the
    fp32 result equals the oracle exactly in any summation order."""
    rows, cols, batch = 97, 2112, 4
    rng = np.random.default_rng(n * 100 + m)
    W = synth.f32_to_16_bits(rng.integers(-3, 4, size=(rows, cols)).astype(np.float32), dtype)
    X = synth.f32_to_16_bits(rng.integers(-3, 4, size=(batch, cols)).astype(np.float32), dtype)
    keep = synth.random_mask(rows, cols, n, m, seed=n + m)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16")
    Y = native.nm_spmm_small(values, bits, t16(X, dtype), n, m)
    assert np.array_equal(f64(Y), want)


@pytest.mark.parametrize("n,m", [(1, 4), (3, 8), (5, 16)])
def test_one_hot_x_picks_the_kept_weight(n, m):
    """x = e_j: y[r] = W[r][j] if column j of row r is kept, else 0 -- pins the
    bit <-> column mapping and the value offsets w * 32N/M end to end."""
    rows, cols = 64, 2112
    W, keep, _ = inputs(rows, cols, n, m, "f16", 1, seed=7 + n)
    values, bits = gpu_pack(W, keep, n, m, "f16")
    for j in (0, 31, 32, 1000, 2047, 2048, 2111):
        x = np.zeros((1, cols), dtype=np.uint16)
        x[0, j] = 0x3C00  # 1.0
        y = f64(native.nm_spmv(values, bits, t16(x[0], "f16"), n, m))
        want = np.where(keep[:, j] != 0, W[:, j].view(np.float16).astype(np.float64), 0.0)
        assert np.array_equal(y, want)


@pytest.mark.parametrize("n,m", [(1, 4), (3, 4), (3, 8), (5, 16)])
@pytest.mark.parametrize("seg,threads,rpw", [(2048, 256, 1), (4096, 128, 3), (6144, 512, 2),
                                             (32, 64, 1), (8320, 512, 64)])
def test_launch_shapes_and_x_segments(n, m, seg, threads, rpw):
    """x staged in several segments (seg < cols; segments that end inside a
    load batch, a one-word segment), several rows per wave, other workgroup
    sizes: the same sums, on the direct kernel (1:4, 3:4, 3:8) and the window
    kernel (5:16)."""
    rows, cols, batch = 149, 8320, 2
    W, keep, X = inputs(rows, cols, n, m, "bf16", batch, seed=seg + rpw)
    values, bits = gpu_pack(W, keep, n, m, "bf16")
    want = oracle.masked_gemv(W, keep, X, True)
    cfg = native.LaunchCfg(threads, rpw, seg, native.NM_KERNEL_VALU)
    Y = native.nm_spmm_small(values, bits, t16(X, "bf16"), n, m, cfg=cfg)
    for b in range(batch):
        assert rel_l2(f64(Y[b]), want[b]) <= TOL


@pytest.mark.parametrize("n,m", [(1, 4), (3, 4), (1, 8), (3, 8), (5, 16)])
@pytest.mark.parametrize("batch", [5, 8])
def test_default_x_segments_at_large_k(n, m, batch):
    """K = 14336 at batch 5-8: all of x does not fit the LDS budget, so the
    library's own launch stages it in segments."""
    rows, cols = 67, 14336
    W, keep, X = inputs(rows, cols, n, m, "f16", batch, seed=batch + 7 * n + m)
    values, bits = gpu_pack(W, keep, n, m, "f16")
    want = oracle.masked_gemv(W, keep, X, False)
    Y = native.nm_spmm_small(values, bits, t16(X, "f16"), n, m)
    for b in range(batch):
        assert rel_l2(f64(Y[b]), want[b]) <= TOL


def test_launch_shape_rejections_other_densities():
    W, keep, X = inputs(16, 1024, 1, 4, "f16", 1, seed=1)
    values, bits = gpu_pack(W, keep, 1, 4, "f16")
    x = t16(X[0], "f16")
    for cfg in [(256, 1, 0, native.NM_KERNEL_MFMA), (96, 1, 1024, 0), (256, 65, 1024, 0),
                (256, 1, 48, 0), (1024, 1, 1 << 20, 0)]:
        with pytest.raises(native.NMError):
            native.nm_spmv(values, bits, x, 1, 4, cfg=native.LaunchCfg(*cfg))
    # the 50%-only entry points reject these densities
    with pytest.raises(native.NMError) as e:
        native.nm_spmm_swiglu(values, bits, x[None], 1, 4)
    assert e.value.status == native.NM_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", [(1, 4), (3, 4), (5, 16)])
def test_16bit_output_other_densities(n, m, dtype):
    rows, cols, batch = 130, 2080, 2
    W, keep, X = inputs(rows, cols, n, m, dtype, batch, seed=n * 3 + m)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    Xd = t16(X, dtype)
    Y32 = native.nm_spmm_small(values, bits, Xd, n, m)
    Y16 = native.nm_spmm_small(values, bits, Xd, n, m, out_dtype=Xd.dtype)
    check_16bit_output(Y16, Y32, W, keep, X, n, m, dtype)


def test_empty_and_degenerate_other_densities():
    # rows == 0: nothing launched; cols == 0: every sum is empty
    v = torch.empty((0, 0), dtype=torch.float16, device=DEV)
    b = torch.empty((0, 0), dtype=torch.int32, device=DEV)
    y = native.nm_spmv(v, b, torch.empty((0,), dtype=torch.float16, device=DEV), 1, 4)
    assert y.numel() == 0
    v = torch.empty((5, 0), dtype=torch.float16, device=DEV)
    b = torch.empty((5, 0), dtype=torch.int32, device=DEV)
    Y = native.nm_spmm_small(v, b, torch.empty((2, 0), dtype=torch.float16, device=DEV), 3, 4)
    assert torch.equal(Y.cpu(), torch.zeros((2, 5)))


def test_values_without_padding_are_refused():
    """The 16-byte loads of the last window may reach the packed-size padding:
    a copy of the values without it is refused before any launch."""
    W, keep, X = inputs(3, 64, 5, 16, "f16", 1, seed=2)
    values, bits = gpu_pack(W, keep, 5, 16, "f16")
    with pytest.raises(ValueError):
        native.nm_spmv(values.clone(), bits, t16(X[0], "f16"), 5, 16)
    y = native.nm_spmv(native.clone_packed(values), bits, t16(X[0], "f16"), 5, 16)
    assert rel_l2(f64(y)[None], oracle.masked_gemv(W, keep, X, False)) <= TOL


# Full-size layers at other densities, in the launch shape the library picks,
# checked on sampled rows that the oracle computes one by one.
@pytest.mark.parametrize("rows,cols,n,m,dtype", [(14336, 4096, 1, 4, "f16"),
                                                 (14336, 4096, 3, 4, "f16"),
                                                 (4096, 14336, 1, 8, "bf16"),
                                                 (2048, 28672, 3, 8, "f16")])
@pytest.mark.parametrize("batch", [1, 8])
def test_full_size_sampled_rows_other_densities(rows, cols, n, m, dtype, batch):
    W, keep, X = inputs(rows, cols, n, m, dtype, batch, seed=rows + n)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    Y = native.nm_spmm_small(values, bits, t16(X, dtype), n, m)
    idx = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(5).integers(0, rows, 60)]))
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16", rows_idx=idx)
    got = f64(Y)[:, idx]
    for b in range(batch):
        assert rel_l2(got[b], want[b]) <= TOL
