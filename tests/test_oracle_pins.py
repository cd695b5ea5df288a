"""Pins for the CPU oracle: facts that do not come from the oracle itself.

Each test names the passage of the pages (SparseDecoding, arXiv 2610.12327) or
the mathematical fact it checks.  A plausible mistake in the oracle -- a wrong
bit order, a dropped term, a transposed operand, a mis-decoded exponent --
fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from sparse_gemv_memory_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- binary16 / bfloat16 decoding ---------------------------------------------

def test_decode_f16_all_patterns_match_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode16(bits, is_bf16=False)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero survives
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_decode_bf16_all_patterns_match_float32_top_half():
    bits = np.arange(1 << 16, dtype=np.uint32)
    got = oracle.decode16(bits.astype(np.uint16), is_bf16=True)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_decode_known_values():
    # closed forms: 1.0, -2.0, smallest subnormal, largest finite
    f16 = np.array([0x3C00, 0xC000, 0x0001, 0x7BFF], dtype=np.uint16)
    assert list(oracle.decode16(f16, False)) == [1.0, -2.0, 2.0 ** -24, 65504.0]
    bf = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F], dtype=np.uint16)
    assert list(oracle.decode16(bf, True)) == [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127]


# ---- pack / unpack ------------------------------------------------------------

def _brute_pack(W, keep):
    """Pack from the list of kept columns (a second, independent formulation)."""
    rows, cols = W.shape
    vals, words = [], []
    for r in range(rows):
        kept = [c for c in range(cols) if keep[r, c]]
        vals.append([int(W[r, c]) for c in sorted(kept)])
        words.append([sum(1 << (c - 32 * w) for c in kept if c // 32 == w) for w in range(cols // 32)])
    return np.array(vals, dtype=np.uint16), np.array(words, dtype=np.uint32)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16), (16, 32)])
def test_pack_matches_brute_force(n, m):
    rows, cols = 5, 96
    W = synth.weights(rows, cols, seed=7)
    keep = synth.random_mask(rows, cols, n, m, seed=11)
    st, values, bits = oracle.pack(W, keep, n, m)
    assert st == oracle.OK
    bv, bb = _brute_pack(W, keep)
    assert np.array_equal(values, bv)
    assert np.array_equal(bits, bb)


def test_pack_exhaustive_2of4_words():
    """Every one of the 6**8 aligned 2:4 words, as the rows of one matrix.

    With W[r, c] = c the packed values of a row are its kept column indices,
    which pins the bit <-> column mapping (bit b of word w is column 32w+b)
    and the increasing-column value order ("Method", item (1))."""
    nibbles = np.array([0b0011, 0b0101, 0b0110, 0b1001, 0b1010, 0b1100], dtype=np.uint32)
    idx = np.arange(6 ** 8, dtype=np.int64)
    word = np.zeros(idx.shape, dtype=np.uint32)
    for g in range(8):
        word |= nibbles[(idx // 6 ** g) % 6] << np.uint32(4 * g)
    keep = ((word[:, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.uint8)
    W = np.broadcast_to(np.arange(32, dtype=np.uint16), keep.shape).copy()
    st, values, bits = oracle.pack(W, keep, 2, 4)
    assert st == oracle.OK
    assert np.array_equal(bits[:, 0], word)
    assert len(np.unique(bits[:, 0])) == 6 ** 8
    expect = np.nonzero(keep)[1].reshape(-1, 16).astype(np.uint16)
    assert np.array_equal(values, expect)
    # 16 set bits in every aligned word ("Method", item (2))
    assert np.all(np.unpackbits(bits.view(np.uint8), axis=1).sum(axis=1) == 16)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16), (16, 32)])
def test_every_word_has_16_set_bits(n, m):
    W = synth.weights(64, 256, seed=3)
    keep = synth.topn_mask(W, n, m)
    st, values, bits = oracle.pack(W, keep, n, m)
    assert st == oracle.OK
    pop = np.unpackbits(bits.view(np.uint8).reshape(bits.shape + (4,)), axis=-1).sum(axis=-1)
    assert np.all(pop == 16)


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16), (16, 32)])
def test_unpack_inverts_pack(n, m):
    W = synth.weights(33, 160, seed=5, dtype="bf16")
    keep = synth.random_mask(33, 160, n, m, seed=6)
    st, values, bits = oracle.pack(W, keep, n, m)
    assert st == oracle.OK
    st, W2, k2 = oracle.unpack(values, bits, 160, n, m)
    assert st == oracle.OK
    assert np.array_equal(k2, keep)
    assert np.array_equal(W2, np.where(keep != 0, W, 0).astype(np.uint16))


def test_pack_moves_raw_patterns():
    """Kept -0.0, subnormals, inf and NaN patterns survive unchanged (the mask
    decides what is kept, not the value)."""
    W = np.array([[0x8000, 0x0001, 0x7C00, 0x7E01] * 8], dtype=np.uint16)
    keep = np.array([[1, 1, 0, 0, 0, 0, 1, 1] * 4], dtype=np.uint8)
    st, values, bits = oracle.pack(W, keep, 2, 4)
    assert st == oracle.OK
    assert list(values[0, :4]) == [0x8000, 0x0001, 0x7C00, 0x7E01]
    assert bits[0, 0] == 0xC3C3C3C3


def test_pack_rejects_bad_inputs():
    W = synth.weights(2, 64, seed=1)
    keep = synth.random_mask(2, 64, 2, 4, seed=2)
    bad = keep.copy()
    bad[1, 5] ^= 1  # one group now holds 1 or 3
    assert oracle.pack(W, bad, 2, 4)[0] == oracle.ERR_MASK
    assert oracle.count_bad_groups(bad, 2, 4) == 1
    # patterns outside 0 < N < M, M in {4, 8, 16, 32}
    for n, m in [(0, 4), (4, 4), (2, 6), (3, 12), (32, 64)]:
        assert oracle.pack(W, keep, n, m)[0] == oracle.ERR_UNSUPPORTED
    # a valid 2:4 mask is not a valid 1:4 or 3:4 mask
    assert oracle.pack(W, keep, 1, 4)[0] == oracle.ERR_MASK
    assert oracle.pack(W, keep, 3, 4)[0] == oracle.ERR_MASK
    assert oracle.pack(W[:, :48], keep[:, :48], 2, 4)[0] == oracle.ERR_SHAPE


def test_sizes_match_worked_slice_on_the_pages():
    """The explainer's 32-column fp16 slice: 256 value bits + one 32-bit word
    = 288 bits against 512 dense; 2 metadata bits per kept weight."""
    g = json.load(open(os.path.join(GOLDEN, "p4_bit_count.json")))
    m2 = json.load(open(os.path.join(GOLDEN, "p2_metadata_bits.json")))
    W = synth.weights(1, g["cols"], seed=0)
    keep = synth.topn_mask(W, 2, 4)
    st, values, bits = oracle.pack(W, keep, 2, 4)
    assert st == oracle.OK
    assert values.size == g["kept"]
    assert values.nbytes * 8 == g["kept_value_bits"]
    assert bits.nbytes * 8 == g["bitmask_metadata_bits"]
    assert values.nbytes * 8 + bits.nbytes * 8 == g["bitmask_slice_bits"]
    assert W.nbytes * 8 == g["dense_slice_bits"]
    assert g["kept"] * 32 + values.nbytes * 8 == g["int32_index_slice_bits"]
    per_nz = bits.nbytes * 8 / values.size
    assert per_nz == g["bitmask_bits_per_kept_weight"] == m2["bitmask_bits_per_nonzero"]
    assert m2["int32_index_bits_per_nonzero"] / per_nz == m2["reduction_vs_int32"]
    assert m2["uint8_offset_bits_per_nonzero"] / per_nz == m2["reduction_vs_uint8"]
    assert abs(g["bitmask_slice_bits"] / g["dense_slice_bits"] - g["bitmask_fraction_of_dense_approx"]) < 0.01


def test_packed_size_is_pattern_independent():
    """All 50% patterns keep the same bytes per row ("Experiments", Table 3
    paragraph: identical memory traffic per row)."""
    W = synth.weights(8, 256, seed=9)
    sizes = set()
    for n, m in [(2, 4), (4, 8), (8, 16), (16, 32)]:
        st, values, bits = oracle.pack(W, synth.topn_mask(W, n, m), n, m)
        assert st == oracle.OK
        sizes.add((values.nbytes, bits.nbytes))
    assert sizes == {(8 * 128 * 2, 8 * 8 * 4)}


# ---- densities other than 50% (N:M with M | 32, any 0 < N < M) ------------------

OTHER_DENSITIES = [(1, 4), (3, 4), (1, 8), (3, 8), (7, 8), (5, 16), (1, 32), (31, 32)]


@pytest.mark.parametrize("n,m", OTHER_DENSITIES)
def test_pack_other_densities_match_brute_force(n, m):
    rows, cols = 6, 160
    W = synth.weights(rows, cols, seed=17)
    keep = synth.random_mask(rows, cols, n, m, seed=19)
    st, values, bits = oracle.pack(W, keep, n, m)
    assert st == oracle.OK
    bv, bb = _brute_pack(W, keep)
    assert values.shape == (rows, cols * n // m)
    assert np.array_equal(values, bv)
    assert np.array_equal(bits, bb)


@pytest.mark.parametrize("n,m", OTHER_DENSITIES)
def test_every_word_has_32n_over_m_set_bits(n, m):
    """Fixed count per aligned word at any N:M with M | 32, so word w's values
    start at w * 32N/M of the row ("Method", item (2), generalised)."""
    W = synth.weights(16, 256, seed=23)
    keep = synth.topn_mask(W, n, m)
    st, values, bits = oracle.pack(W, keep, n, m)
    assert st == oracle.OK
    pop = np.unpackbits(bits.view(np.uint8).reshape(bits.shape + (4,)), axis=-1).sum(axis=-1)
    p = 32 * n // m
    assert np.all(pop == p)
    # with W[r, c] = c the values of word w are its kept columns, at w * p
    Wc = np.broadcast_to(np.arange(256, dtype=np.uint16), keep.shape).copy()
    st, vc, _ = oracle.pack(Wc, keep, n, m)
    assert st == oracle.OK
    for w in range(256 // 32):
        cols = np.nonzero(keep[0, 32 * w:32 * w + 32])[0] + 32 * w
        assert np.array_equal(vc[0, w * p:(w + 1) * p], cols.astype(np.uint16))


@pytest.mark.parametrize("n,m", OTHER_DENSITIES)
def test_unpack_inverts_pack_other_densities(n, m):
    W = synth.weights(9, 96, seed=29, dtype="bf16")
    keep = synth.random_mask(9, 96, n, m, seed=31)
    st, values, bits = oracle.pack(W, keep, n, m)
    assert st == oracle.OK
    st, W2, k2 = oracle.unpack(values, bits, 96, n, m)
    assert st == oracle.OK
    assert np.array_equal(k2, keep)
    assert np.array_equal(W2, np.where(keep != 0, W, 0).astype(np.uint16))


def test_packed_size_scales_with_density():
    """Values take K*N/M 16-bit words per row, the mask K/32 words whatever
    the density: 16*N/M + 1 bits per column in all."""
    W = synth.weights(4, 512, seed=37)
    for n, m in OTHER_DENSITIES + [(2, 4)]:
        st, values, bits = oracle.pack(W, synth.topn_mask(W, n, m), n, m)
        assert st == oracle.OK
        assert values.nbytes == 4 * 512 * n // m * 2
        assert bits.nbytes == 4 * 512 // 8


@pytest.mark.parametrize("n,m", [(1, 4), (3, 4), (5, 16)])
def test_masked_gemv_from_packed_form_other_densities(n, m):
    """The product read back from the packed form, walked word by word with
    the lowest-set-bit scan in pure Python, equals the oracle's dense masked
    product (a second formulation of the same sum)."""
    rows, cols = 5, 96
    W = synth.weights(rows, cols, seed=41)
    keep = synth.topn_mask(W, n, m)
    x = synth.activations(2, cols, seed=43)
    st, values, bits = oracle.pack(W, keep, n, m)
    assert st == oracle.OK
    vf = _f64(values, False)
    xf = _f64(x, False)
    p = 32 * n // m
    y = np.zeros((2, rows))
    for r in range(rows):
        for w in range(cols // 32):
            word, j = int(bits[r, w]), 0
            while word:
                c = (word & -word).bit_length() - 1
                word &= word - 1
                y[:, r] += vf[r, w * p + j] * xf[:, 32 * w + c]
                j += 1
            assert j == p
    assert np.allclose(oracle.masked_gemv(W, keep, x, False), y, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n,m", [(1, 4), (3, 4), (3, 8)])
def test_topn_mask_other_densities_brute_force(n, m):
    """The harness mask at other densities: per group the n largest |w|,
    ties to the lower column, against a sort of every group."""
    W = synth.weights(3, 64, seed=47)
    W[0, :m] = W[0, 0]  # a group of equal magnitudes
    keep = synth.topn_mask(W, n, m)
    mag = (W & 0x7FFF).astype(np.int64)
    for r in range(3):
        for g in range(64 // m):
            idx = sorted(range(m), key=lambda j: (-mag[r, g * m + j], j))[:n]
            want = np.zeros(m, np.uint8)
            want[idx] = 1
            assert np.array_equal(keep[r, g * m:(g + 1) * m], want)


# ---- unstructured bitmasks (any keep mask, row offsets) -------------------------

def _brute_pack_bitmask(W, keep):
    """Rows' kept values concatenated, from the list of kept columns."""
    rows, cols = W.shape
    vals, ptr = [], [0]
    for r in range(rows):
        kept = [c for c in range(cols) if keep[r, c]]
        vals += [int(W[r, c]) for c in kept]
        ptr.append(len(vals))
    words = [[sum(1 << b for b in range(32) if keep[r, 32 * w + b]) for w in range(cols // 32)]
             for r in range(rows)]
    return (np.array(vals, dtype=np.uint16), np.array(words, dtype=np.uint32),
            np.array(ptr, dtype=np.int64))


@pytest.mark.parametrize("rows,cols", [(1, 32), (5, 96), (9, 160)])
def test_pack_bitmask_matches_brute_force(rows, cols):
    W = synth.weights(rows, cols, seed=53)
    rng = np.random.default_rng(rows + cols)
    keep = (rng.random((rows, cols)) < 0.5).astype(np.uint8)
    keep[0, :] = 0            # an empty row
    if rows > 1:
        keep[1, :] = 1        # a full row
    st, values, bits, row_ptr = oracle.pack_bitmask(W, keep)
    assert st == oracle.OK
    bv, bb, bp = _brute_pack_bitmask(W, keep)
    assert np.array_equal(values, bv)
    assert np.array_equal(bits, bb)
    assert np.array_equal(row_ptr, bp)


def test_pack_bitmask_offsets_are_prefix_popcounts():
    """Word w of row r starts at row_ptr[r] plus the set bits of the row's
    words before w (the per-word prefix offsets the format needs once the
    count per word varies)."""
    W = np.broadcast_to(np.arange(256, dtype=np.uint16), (6, 256)).copy()
    keep = synth.topk_row_mask(synth.weights(6, 256, seed=59), 0.5)
    st, values, bits, row_ptr = oracle.pack_bitmask(W, keep)
    assert st == oracle.OK
    assert np.array_equal(np.diff(row_ptr), keep.sum(axis=1))
    for r in range(6):
        off = row_ptr[r]
        for w in range(8):
            word = int(bits[r, w])
            cols = [32 * w + b for b in range(32) if word >> b & 1]
            assert list(values[off:off + len(cols)]) == cols
            off += len(cols)
        assert off == row_ptr[r + 1]


def test_unpack_bitmask_inverts_pack():
    W = synth.weights(7, 128, seed=61, dtype="bf16")
    keep = synth.topk_row_mask(W, 0.5)
    st, values, bits, row_ptr = oracle.pack_bitmask(W, keep)
    assert st == oracle.OK
    st, W2, k2 = oracle.unpack_bitmask(values, bits, row_ptr, 128)
    assert st == oracle.OK
    assert np.array_equal(k2, keep)
    assert np.array_equal(W2, np.where(keep != 0, W, 0).astype(np.uint16))


def test_pack_bitmask_of_an_nm_mask_is_the_nm_pack():
    """An N:M mask is a special unstructured mask: the same values and words,
    rows at stride K*N/M."""
    W = synth.weights(5, 128, seed=67)
    keep = synth.topn_mask(W, 2, 4)
    st, values, bits, row_ptr = oracle.pack_bitmask(W, keep)
    st2, v2, b2 = oracle.pack(W, keep, 2, 4)
    assert st == st2 == oracle.OK
    assert np.array_equal(values, v2.reshape(-1))
    assert np.array_equal(bits, b2)
    assert np.array_equal(row_ptr, np.arange(6) * 64)


def test_topk_row_mask_keeps_the_larger_half_per_row():
    W = synth.weights(4, 64, seed=71)
    W[0, :] = W[0, 0]  # all ties: the lower columns win
    keep = synth.topk_row_mask(W, 0.5)
    assert np.all(keep.sum(axis=1) == 32)
    assert np.array_equal(keep[0], np.r_[np.ones(32), np.zeros(32)].astype(np.uint8))
    mag = (W & 0x7FFF).astype(np.int64)
    for r in range(1, 4):
        order = sorted(range(64), key=lambda c: (-mag[r, c], c))[:32]
        want = np.zeros(64, np.uint8)
        want[order] = 1
        assert np.array_equal(keep[r], want)


def test_masked_gemv_from_bitmask_form():
    """The product re-walked from the unstructured packed form equals the
    dense masked product."""
    rows, cols = 6, 96
    W = synth.weights(rows, cols, seed=73)
    keep = synth.topk_row_mask(W, 0.5)
    x = synth.activations(2, cols, seed=73)
    st, values, bits, row_ptr = oracle.pack_bitmask(W, keep)
    vf, xf = _f64(values, False), _f64(x, False)
    y = np.zeros((2, rows))
    for r in range(rows):
        j = row_ptr[r]
        for w in range(cols // 32):
            word = int(bits[r, w])
            while word:
                c = (word & -word).bit_length() - 1
                word &= word - 1
                y[:, r] += vf[j] * xf[:, 32 * w + c]
                j += 1
    assert np.allclose(oracle.masked_gemv(W, keep, x, False), y, rtol=1e-12, atol=1e-12)


# ---- the product ----------------------------------------------------------------

def _f64(bits, bf16):
    if bf16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", [(2, 4), (16, 32)])
def test_masked_gemv_matches_numpy_matmul(dtype, n, m):
    rows, cols, batch = 37, 320, 3
    W = synth.weights(rows, cols, seed=1, dtype=dtype)
    keep = synth.topn_mask(W, n, m)
    x = synth.activations(batch, cols, seed=1, dtype=dtype)
    bf = dtype == "bf16"
    y = oracle.masked_gemv(W, keep, x, bf)
    ref = _f64(x, bf) @ (_f64(W, bf) * keep).T
    assert y.shape == (batch, rows)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)
    # dense product (keep=None) is the unmasked matmul
    yd = oracle.masked_gemv(W, None, x, bf)
    assert np.allclose(yd, _f64(x, bf) @ _f64(W, bf).T, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_masked_gemv_integer_inputs_exact(dtype):
    rows, cols, batch = 50, 512, 4
    W = synth.integer_weights(rows, cols, seed=2, dtype=dtype)
    xi = np.random.default_rng(3).integers(-4, 5, size=(batch, cols))
    x = synth.f32_to_16_bits(xi.astype(np.float32), dtype)
    keep = synth.random_mask(rows, cols, 2, 4, seed=4)
    Wi = np.rint(_f64(W, dtype == "bf16")).astype(np.int64)
    exact = xi @ (Wi * keep).T
    y = oracle.masked_gemv(W, keep, x, dtype == "bf16")
    assert np.array_equal(y, exact.astype(np.float64))


def test_masked_gemv_one_hot_picks_a_column():
    rows, cols = 20, 128
    W = synth.weights(rows, cols, seed=8)
    keep = synth.topn_mask(W, 2, 4)
    Wf = _f64(W, False)
    for j in (0, 1, 31, 32, 77, 127):
        x = np.zeros(cols, dtype=np.float16)
        x[j] = 1.0
        y = oracle.masked_gemv(W, keep, x.view(np.uint16), False)
        assert np.array_equal(y, Wf[:, j] * keep[:, j])


def test_masked_gemv_all_ones_sums_kept_values():
    rows, cols = 16, 256
    W = synth.weights(rows, cols, seed=12)
    keep = synth.topn_mask(W, 4, 8)
    st, values, bits = oracle.pack(W, keep, 4, 8)
    x = np.ones(cols, dtype=np.float16).view(np.uint16)
    y = oracle.masked_gemv(W, keep, x, False)
    ref = np.array([np.sum(values[r].view(np.float16).astype(np.float64)) for r in range(rows)])
    assert np.allclose(y, ref, rtol=1e-13, atol=0)


def test_masked_gemv_row_sampling_matches_full():
    W = synth.weights(64, 128, seed=13)
    keep = synth.topn_mask(W, 2, 4)
    x = synth.activations(2, 128, seed=13)
    full = oracle.masked_gemv(W, keep, x, False, threads=4)
    idx = np.array([63, 0, 17, 17, 5])
    part = oracle.masked_gemv(W, keep, x, False, rows_idx=idx)
    assert np.array_equal(part, full[:, idx])


def test_masked_gemv_empty_cols_is_zero():
    W = np.zeros((3, 0), dtype=np.uint16)
    x = np.zeros((1, 0), dtype=np.uint16)
    y = oracle.masked_gemv(W, np.zeros((3, 0), np.uint8), x, False)
    assert np.array_equal(y, np.zeros((1, 3)))


# ---- silu(gate) * up around the product -------------------------------------------

def test_silu_closed_forms():
    """silu(z) = z * sigmoid(z): 0 at 0, sigmoid(1) = e / (1 + e) at 1, and
    z itself (to fp64 precision) for large z."""
    h = oracle.silu_mul(np.array([0.0, 1.0, 40.0, -40.0]), np.ones(4))
    assert h[0] == 0.0
    assert abs(h[1] - math.e / (1.0 + math.e)) <= 1e-16
    assert h[2] == 40.0
    assert abs(h[3]) < 1e-15 and h[3] < 0


def test_silu_odd_part_is_identity():
    """silu(z) - silu(-z) = z (sigmoid(z) + sigmoid(-z) = 1): catches a wrong
    sign in the exponent or a swapped operand."""
    z = np.random.default_rng(3).normal(0.0, 4.0, size=1000)
    d = oracle.silu_mul(z, np.ones_like(z)) - oracle.silu_mul(-z, np.ones_like(z))
    assert np.allclose(d, z, rtol=1e-13, atol=1e-13)


def test_silu_mul_is_linear_in_up():
    rng = np.random.default_rng(4)
    g, u = rng.normal(size=200), rng.normal(size=200)
    assert np.allclose(oracle.silu_mul(g, u), oracle.silu_mul(g, np.ones_like(g)) * u,
                       rtol=1e-15, atol=0)


def test_swiglu_gemv_matches_brute_force():
    """Tiny row-interleaved gate/up matrix, small integers: pure-Python sums
    and math.exp against the oracle."""
    rng = np.random.default_rng(5)
    rows, cols, batch = 6, 32, 2
    W = synth.f32_to_16_bits(rng.integers(-3, 4, size=(rows, cols)).astype(np.float32), "f16")
    keep = synth.random_mask(rows, cols, 2, 4, seed=6)
    X = synth.f32_to_16_bits(rng.integers(-3, 4, size=(batch, cols)).astype(np.float32), "f16")
    Wf = W.view(np.float16).astype(float)
    Xf = X.view(np.float16).astype(float)
    got = oracle.swiglu_gemv(W, keep, X, False)
    assert got.shape == (batch, rows // 2)
    for b in range(batch):
        for r in range(rows // 2):
            g = sum(Wf[2 * r, c] * Xf[b, c] for c in range(cols) if keep[2 * r, c])
            u = sum(Wf[2 * r + 1, c] * Xf[b, c] for c in range(cols) if keep[2 * r + 1, c])
            want = g / (1.0 + math.exp(-g)) * u
            assert abs(got[b, r] - want) <= 1e-12 * max(1.0, abs(want))


# ---- the layer Hessian -------------------------------------------------------------

def _x16(a, dtype="f16"):
    return synth.f32_to_16_bits(np.asarray(a, dtype=np.float32), dtype)


def test_hessian_matches_brute_force():
    rng = np.random.default_rng(21)
    xf = rng.integers(-3, 4, size=(5, 3)).astype(np.float32)
    H = oracle.hessian(_x16(xf), scale=2.0)
    for i in range(5):
        for j in range(5):
            want = 2.0 * sum(float(xf[i, t]) * float(xf[j, t]) for t in range(3))
            assert H[i, j] == want


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_hessian_matches_numpy_matmul(dtype):
    rng = np.random.default_rng(22)
    X = _x16(rng.normal(size=(40, 23)), dtype)
    xd = oracle.decode16(X, dtype == "bf16")
    H = oracle.hessian(X, scale=2.0, is_bf16=dtype == "bf16")
    assert np.allclose(H, 2.0 * xd @ xd.T, rtol=1e-13, atol=1e-12)


def test_hessian_one_hot_columns():
    """Column t = e_{i_t}: H = scale * sum_t e_{i_t} e_{i_t}^T (counts on the
    diagonal)."""
    d, idx = 7, [0, 3, 3, 6]
    xf = np.zeros((d, len(idx)), dtype=np.float32)
    for t, i in enumerate(idx):
        xf[i, t] = 1.0
    H = oracle.hessian(_x16(xf), scale=2.0)
    want = np.zeros((d, d))
    for i in idx:
        want[i, i] += 2.0
    assert np.array_equal(H, want)


def test_hessian_is_symmetric_psd_with_trace_identity():
    rng = np.random.default_rng(23)
    X = _x16(rng.normal(size=(30, 50)))
    xd = oracle.decode16(X, False)
    H = oracle.hessian(X, scale=2.0)
    assert np.array_equal(H, H.T)
    assert np.linalg.eigvalsh(H).min() >= -1e-9
    assert abs(np.trace(H) - 2.0 * float((xd ** 2).sum())) <= 1e-9 * np.trace(H)


def test_hessian_reads_only_the_first_ntok_columns():
    rng = np.random.default_rng(24)
    X = _x16(rng.normal(size=(9, 16)))
    Xg = X.copy()
    Xg[:, 11:] = _x16(rng.normal(size=(9, 5)) * 100)
    assert np.array_equal(oracle.hessian(X, ntok=11), oracle.hessian(Xg, ntok=11))
    assert np.array_equal(oracle.hessian(X, ntok=0), np.zeros((9, 9)))


# ---- N:M mask selection -------------------------------------------------------------

SEL_PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]


def _topn_by_sort(score, n, m):
    """Keep the n largest of each m-group, lower column first among equals, by
    a stable sort of the negated scores (a library routine, not the oracle's
    one-at-a-time choice)."""
    rows, cols = score.shape
    keep = np.zeros((rows, cols), dtype=np.uint8)
    for r in range(rows):
        for g in range(0, cols, m):
            order = np.argsort(-score[r, g:g + m], kind="stable")[:n]
            keep[r, g + order] = 1
    return keep


@pytest.mark.parametrize("n,m", SEL_PATTERNS)
def test_select_nm_minimizes_reconstruction_error_for_orthogonal_activations(n, m):
    """Eq. (1) without the weight update: with X = diag(a) Had (rows of a
    Hadamard matrix, exactly orthogonal in fp16), ||W X - (W o K) X||_F^2 over
    each group's C(m, n) choices is smallest at the selected mask when
    s = diag(2 X X^T).  The error is the direct matrix product, not a score."""
    import scipy.linalg
    rng = np.random.default_rng(31)
    rows, cols, ntok = 3, 2 * m, 64 if 2 * m <= 64 else 2 * m
    had = scipy.linalg.hadamard(ntok)[:cols].astype(np.float32)
    a = rng.integers(1, 9, size=cols).astype(np.float32) / 4.0
    X = _x16(a[:, None] * had)
    xd = oracle.decode16(X, False)
    H = oracle.hessian(X, scale=2.0)
    assert np.array_equal(H, np.diag(np.diag(H)))  # orthogonal rows
    W = _x16(rng.normal(size=(rows, cols)))
    wd = oracle.decode16(W, False)
    keep = oracle.select_nm(W, np.diag(H).astype(np.float32), n, m, False)
    assert oracle.count_bad_groups(keep, n, m) == 0

    def err(k):
        return float((((wd * (1 - k)) @ xd) ** 2).sum())

    base = err(keep)
    checks = 0
    for r in range(rows):
        for g in range(0, cols, m):
            for kept in itertools.combinations(range(m), n):
                if m > 8 and checks > 4000:
                    break
                k = keep.astype(np.float64).copy()
                k[r, g:g + m] = 0
                k[r, [g + e for e in kept]] = 1
                assert err(k) >= base * (1 - 1e-12)
                checks += 1
    assert checks > 0


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", SEL_PATTERNS)
def test_select_nm_unit_column_weight_is_magnitude_pruning(n, m, dtype):
    """s = 1: keep the n largest |w| per group (w^2 is exact in fp32 for
    16-bit inputs); integer weights make ties common and the lower column
    wins them."""
    rng = np.random.default_rng(32)
    W = _x16(rng.integers(-4, 5, size=(6, 4 * m)), dtype)
    wd = oracle.decode16(W, dtype == "bf16")
    keep = oracle.select_nm(W, np.ones(4 * m, np.float32), n, m, dtype == "bf16")
    assert np.array_equal(keep, _topn_by_sort(np.abs(wd), n, m))


@pytest.mark.parametrize("n,m", SEL_PATTERNS)
def test_select_nm_equal_magnitudes_follow_column_weight(n, m):
    rng = np.random.default_rng(33)
    W = _x16(np.where(rng.random((5, 2 * m)) < 0.5, -1.0, 1.0))
    s = rng.integers(0, 6, size=2 * m).astype(np.float32)
    keep = oracle.select_nm(W, s, n, m, False)
    assert np.array_equal(keep, _topn_by_sort(np.broadcast_to(s, (5, 2 * m)), n, m))


def test_select_nm_matches_wanda_order_from_activation_norms():
    """s = diag(2 X X^T) ranks by |w| * ||x_c||, the norm taken directly from
    X in fp64; groups whose n-th and (n+1)-th scores are within 1e-5 of each
    other are skipped (fp32 against fp64)."""
    rng = np.random.default_rng(34)
    n, m, rows, cols = 2, 4, 40, 64
    X = _x16(rng.normal(size=(cols, 30)) * rng.uniform(0.2, 3.0, size=(cols, 1)))
    W = _x16(rng.normal(size=(rows, cols)))
    H = oracle.hessian(X, scale=2.0)
    keep = oracle.select_nm(W, np.diag(H).astype(np.float32), n, m, False)
    wanda = np.abs(oracle.decode16(W, False)) * np.linalg.norm(oracle.decode16(X, False), axis=1)
    want = _topn_by_sort(wanda, n, m)
    compared = 0
    for r in range(rows):
        for g in range(0, cols, m):
            srt = np.sort(wanda[r, g:g + m])[::-1]
            if srt[n - 1] - srt[n] <= 1e-5 * srt[n - 1]:
                continue
            assert np.array_equal(keep[r, g:g + m], want[r, g:g + m])
            compared += 1
    assert compared > rows * cols // m * 0.9


def test_select_nm_invariants():
    rng = np.random.default_rng(35)
    n, m, d = 4, 8, 64
    W = _x16(rng.normal(size=(12, d)))
    s = rng.uniform(0.1, 5.0, size=d).astype(np.float32)
    keep = oracle.select_nm(W, s, n, m, False)
    assert oracle.count_bad_groups(keep, n, m) == 0
    assert int(keep.sum()) == 12 * d // 2
    # the sign of a weight does not matter
    assert np.array_equal(oracle.select_nm(W ^ np.uint16(0x8000), s, n, m, False), keep)
    # a power-of-two scale of s does not change the order
    assert np.array_equal(oracle.select_nm(W, s * 4, n, m, False), keep)
    # reading s as the diagonal of a matrix (stride d + 1)
    S = np.diag(s).astype(np.float32) + rng.normal(size=(d, d)).astype(np.float32) * 9
    np.fill_diagonal(S, s)
    assert np.array_equal(oracle.select_nm(W, S, n, m, False, cstride=d + 1), keep)
    # permuting the columns of a group (with s) permutes its selection
    perm = np.concatenate([g + rng.permutation(m) for g in range(0, d, m)])
    assert np.array_equal(oracle.select_nm(W[:, perm], s[perm], n, m, False), keep[:, perm])


def test_select_nm_nan_scores_rank_last():
    nan16 = 0x7E00
    W = _x16([[1.0, 3.0, 2.0, 4.0, 1.0, 0.0, 1.0, 1.0]])
    W[0, 3] = nan16  # NaN weight
    s = np.array([1, 1, 1, 1, 1, np.inf, 1, 1], np.float32)  # 0 * inf = NaN
    keep = oracle.select_nm(W, s, 2, 4, False)
    assert keep.tolist() == [[0, 1, 1, 0, 1, 0, 1, 0]]
    Wn = np.full((1, 4), nan16, np.uint16)
    assert oracle.select_nm(Wn, np.ones(4, np.float32), 2, 4, False).tolist() == [[1, 1, 0, 0]]


def test_select_nm_rejects_bad_pattern_and_shape():
    W = _x16(np.ones((2, 8)))
    with pytest.raises(ValueError):
        oracle.select_nm(W, np.ones(8, np.float32), 1, 4, False)
    with pytest.raises(ValueError):
        oracle.select_nm(_x16(np.ones((2, 6))), np.ones(6, np.float32), 2, 4, False)
