"""Parity of the unstructured bitmask path with the CPU oracle.

Any keep mask (the pages evaluate 50% unstructured pruning for quality,
"Experiments"): a word's count varies, so the values of window t of row r
start at offs[r * nwr + t] (64-word windows).  Bars: values, bits and the
offsets exact (the offsets against the oracle's row starts plus the set bits
of the row's earlier words); fp32 output within rel-L2 1e-3 of the oracle,
bit-exact on integer-valued inputs.
"""

import numpy as np
import pytest
import torch

import oracle
from sparse_gemv_memory_amd import native, synth

from test_gpu_parity import DEV, TOL, f64, rel_l2, t16, u16, u32

pytestmark = pytest.mark.gpu


def masks(kind, rows, cols, W, seed):
    rng = np.random.default_rng(seed)
    if kind == "half":
        return synth.topk_row_mask(W, 0.5)
    if kind == "random":
        return (rng.random((rows, cols)) < rng.random((rows, 1))).astype(np.uint8)  # row densities vary
    keep = (rng.random((rows, cols)) < 0.5).astype(np.uint8)
    keep[0] = 0
    if rows > 1:
        keep[1] = 1
    if rows > 2:
        keep[2, :] = 0
        keep[2, cols - 1] = 1
    return keep


def expected_offs(bits, row_ptr, cols):
    rows = bits.shape[0]
    nwr = (cols // 32 + 63) // 64
    pop = np.unpackbits(bits.view(np.uint8).reshape(rows, -1, 4), axis=-1).sum(axis=-1)
    offs = np.zeros(rows * nwr + 1, dtype=np.int64)
    for r in range(rows):
        for t in range(nwr):
            offs[r * nwr + t] = row_ptr[r] + pop[r, :64 * t].sum()
    offs[-1] = row_ptr[-1]
    return offs


SHAPES = [(1, 32), (5, 96), (37, 2080), (130, 4160), (64, 8192)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("kind", ["half", "random", "edges"])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_pack_bitmask_exact(rows, cols, kind, dtype):
    W = synth.weights(rows, cols, seed=rows + cols, dtype=dtype)
    keep = masks(kind, rows, cols, W, seed=cols)
    values, bits, offs = native.nm_pack_bitmask(t16(W, dtype), torch.from_numpy(keep).to(DEV))
    st, ov, ob, orp = oracle.pack_bitmask(W, keep)
    assert st == oracle.OK
    assert np.array_equal(u16(values), ov)
    assert np.array_equal(u32(bits), ob)
    assert np.array_equal(offs.cpu().numpy(), expected_offs(ob, orp, cols))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("kind", ["half", "random", "edges"])
@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("batch", [1, 2, 3, 5, 8])
def test_bitmask_product_matches_oracle(rows, cols, kind, dtype, batch):
    W = synth.weights(rows, cols, seed=rows * 3 + cols, dtype=dtype)
    keep = masks(kind, rows, cols, W, seed=rows)
    X = synth.activations(batch, cols, seed=cols + batch, dtype=dtype)
    values, bits, offs = native.nm_pack_bitmask(t16(W, dtype), torch.from_numpy(keep).to(DEV))
    Y = native.nm_spmm_bitmask(values, bits, offs, t16(X, dtype))
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16")
    for b in range(batch):
        if np.linalg.norm(want[b]) == 0:
            assert np.array_equal(f64(Y[b]), want[b])
        else:
            assert rel_l2(f64(Y[b]), want[b]) <= TOL


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bitmask_integer_inputs_bit_exact(dtype):
    rows, cols, batch = 97, 6208, 4
    rng = np.random.default_rng(5)
    W = synth.f32_to_16_bits(rng.integers(-3, 4, size=(rows, cols)).astype(np.float32), dtype)
    X = synth.f32_to_16_bits(rng.integers(-3, 4, size=(batch, cols)).astype(np.float32), dtype)
    keep = masks("random", rows, cols, W, seed=9)
    values, bits, offs = native.nm_pack_bitmask(t16(W, dtype), torch.from_numpy(keep).to(DEV))
    Y = native.nm_spmm_bitmask(values, bits, offs, t16(X, dtype))
    assert np.array_equal(f64(Y), oracle.masked_gemv(W, keep, X, dtype == "bf16"))


def clustered_mask(rows, cols, seed):
    """Rows whose kept columns come in a few short runs separated by long
    empty stretches (a group's 8 values then span many words), with a dense
    row, an empty row and rows of one kept column among them."""
    rng = np.random.default_rng(seed)
    keep = np.zeros((rows, cols), np.uint8)
    for r in range(rows):
        for _ in range(int(rng.integers(0, 6))):
            c0 = int(rng.integers(0, cols))
            keep[r, c0:c0 + int(rng.integers(1, 12))] = 1
    keep[0] = 1
    if rows > 1:
        keep[1] = 0
    if rows > 2:
        keep[2] = 0
        keep[2, int(rng.integers(0, cols))] = 1
    return keep


@pytest.mark.parametrize("kind", ["half", "random", "clustered", "dense"])
@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 64), (37, 2080), (300, 4096), (64, 14336),
                                       (5, 32768)])
def test_bitmask_batch1_integer_exact(rows, cols, kind):
    """Batch 1: exact on integer inputs for per-row halves, row densities
    from 0 to 1, short runs of kept columns between long empty stretches,
    nearly full rows (windows read from global memory), empty rows and single
    kept columns, K from 32 to 32768."""
    rng = np.random.default_rng(rows + cols)
    W = synth.f32_to_16_bits(rng.integers(-3, 4, size=(rows, cols)).astype(np.float32), "f16")
    x = synth.f32_to_16_bits(rng.integers(-3, 4, size=(1, cols)).astype(np.float32), "f16")
    if kind == "clustered":
        keep = clustered_mask(rows, cols, seed=cols)
    elif kind == "dense":
        keep = (rng.random((rows, cols)) < 0.97).astype(np.uint8)
    else:
        keep = masks(kind, rows, cols, W, seed=rows)
    values, bits, offs = native.nm_pack_bitmask(t16(W, "f16"), torch.from_numpy(keep).to(DEV))
    Y = native.nm_spmm_bitmask(values, bits, offs, t16(x, "f16"))
    assert np.array_equal(f64(Y), oracle.masked_gemv(W, keep, x, False))


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_bitmask_windows_around_buffer_size_integer_exact(batch):
    """Windows of 1490 to 1570 kept values beside full and empty ones.  The
    copy of a window holds 1528 to 1536 values, depending on where the
    window's first value falls in its 16-byte group; a denser window is read
    by the lanes from global memory.  Both ways are exact on integer inputs,
    in one launch, and so are the rows around them."""
    rows, cols = 48, 4160  # three windows per row, the last of two words
    rng = np.random.default_rng(17 + batch)
    W = synth.f32_to_16_bits(rng.integers(-3, 4, size=(rows, cols)).astype(np.float32), "f16")
    X = synth.f32_to_16_bits(rng.integers(-3, 4, size=(batch, cols)).astype(np.float32), "f16")
    keep = np.zeros((rows, cols), np.uint8)
    counts = []
    for r in range(rows):
        for t in range(2):
            cnt = 1490 + (r * 7 + t * 13) % 81
            keep[r, 2048 * t + rng.choice(2048, cnt, replace=False)] = 1
            counts.append(cnt)
        keep[r, 4096:] = rng.random(64) < 0.5
    keep[0] = 1
    keep[1] = 0
    assert min(counts) < 1528 and max(counts) > 1536
    values, bits, offs = native.nm_pack_bitmask(t16(W, "f16"), torch.from_numpy(keep).to(DEV))
    Y = native.nm_spmm_bitmask(values, bits, offs, t16(X, "f16"))
    assert np.array_equal(f64(Y), oracle.masked_gemv(W, keep, X, False))


@pytest.mark.parametrize("batch", [1, 4])
def test_bitmask_words_disagreeing_with_offsets_stay_in_their_rows(batch):
    """Mask words with more or fewer set bits than the offsets give their
    window (the header leaves those rows unspecified): every other row is
    still exact on integer inputs, and the call succeeds."""
    rows, cols = 40, 4096
    rng = np.random.default_rng(23 + batch)
    W = synth.f32_to_16_bits(rng.integers(-3, 4, size=(rows, cols)).astype(np.float32), "f16")
    X = synth.f32_to_16_bits(rng.integers(-3, 4, size=(batch, cols)).astype(np.float32), "f16")
    keep = synth.topk_row_mask(W, 0.5)
    values, bits, offs = native.nm_pack_bitmask(t16(W, "f16"), torch.from_numpy(keep).to(DEV))
    bad = [5, 17, 23]
    b = bits.view(rows, cols // 32)
    b[5, :] = -1          # every word full: 4096 set bits against 2048 values
    b[17, 64:] = -1       # the second window full
    b[23, ::3] = 0        # fewer set bits than values
    Y = f64(native.nm_spmm_bitmask(values, bits, offs, t16(X, "f16")))
    torch.cuda.synchronize()
    good = np.array([r for r in range(rows) if r not in bad])
    want = oracle.masked_gemv(W, keep, X, False)
    assert np.array_equal(Y[:, good], want[:, good])


def test_bitmask_one_hot_x():
    rows, cols = 48, 4160
    W = synth.weights(rows, cols, seed=11)
    keep = synth.topk_row_mask(W, 0.5)
    values, bits, offs = native.nm_pack_bitmask(t16(W, "f16"), torch.from_numpy(keep).to(DEV))
    for j in (0, 31, 2047, 2048, 4159):
        x = np.zeros((cols,), dtype=np.uint16)
        x[j] = 0x3C00
        y = f64(native.nm_spmm_bitmask(values, bits, offs, t16(x, "f16")))
        want = np.where(keep[:, j] != 0, W[:, j].view(np.float16).astype(np.float64), 0.0)
        assert np.array_equal(y, want)


def test_bitmask_all_zero_and_empty():
    W = synth.weights(4, 64, seed=1)
    keep = np.zeros((4, 64), np.uint8)
    values, bits, offs = native.nm_pack_bitmask(t16(W, "f16"), torch.from_numpy(keep).to(DEV))
    assert values.numel() == 0 and int(offs[-1]) == 0
    Y = native.nm_spmm_bitmask(values, bits, offs, t16(synth.activations(2, 64, seed=1), "f16"))
    assert torch.equal(Y.cpu(), torch.zeros((2, 4)))


@pytest.mark.parametrize("rows,cols", [(14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_bitmask_full_size_sampled_rows(rows, cols, batch):
    # the library's launches: three 4-wave workgroups per CU (batch 1), two
    # (batch 2), 8-wave workgroups with x whole or in segments (batch 4-8)
    W = synth.weights(rows, cols, seed=rows)
    keep = synth.topk_row_mask(W, 0.5)
    X = synth.activations(batch, cols, seed=rows)
    values, bits, offs = native.nm_pack_bitmask(t16(W, "f16"), torch.from_numpy(keep).to(DEV))
    assert int(offs[-1]) == rows * cols // 2
    Y = native.nm_spmm_bitmask(values, bits, offs, t16(X, "f16"))
    idx = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(3).integers(0, rows, 60)]))
    want = oracle.masked_gemv(W, keep, X, False, rows_idx=idx)
    got = f64(Y)[:, idx]
    for b in range(batch):
        assert rel_l2(got[b], want[b]) <= TOL
