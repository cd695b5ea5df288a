"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars:
* nm_pack: values and bits bit-exact;
* products with fp32 output: rel-L2 <= 1e-3 against the oracle's fp64 result
  (per matrix and batch); with integer-valued inputs every partial sum is an
  exact integer below 2**24, so the fp32 output must equal the oracle exactly;
* products with 16-bit output: within 1 ulp of the fp64 result rounded to
  nearest-even.
Full-size workloads are checked on sampled rows that the oracle computes one by
one, with the launch shape the benchmark uses (the library default).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_gemv_memory_amd import native, synth, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-3
PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def t16(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(TDT[dtype]).to(DEV)


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u32(t):
    return t.contiguous().cpu().numpy().view(np.uint32)


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(got, want):
    d = np.linalg.norm(want)
    return np.linalg.norm(got - want) / d if d > 0 else np.linalg.norm(got)


def inputs(rows, cols, n, m, dtype, batch, seed, mask="topn"):
    W = synth.weights(rows, cols, seed=seed, dtype=dtype)
    keep = synth.topn_mask(W, n, m) if mask == "topn" else synth.random_mask(rows, cols, n, m, seed + 1)
    X = synth.activations(batch, cols, seed=seed, dtype=dtype)
    return W, keep, X


def gpu_pack(W, keep, n, m, dtype):
    return native.nm_pack(t16(W, dtype), torch.from_numpy(keep).to(DEV), n, m)


def round16_f64(a, dtype):
    """fp64 -> nearest-even 16-bit pattern (binary16 via numpy; bfloat16 by
    rounding the significand to 8 bits)."""
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    mant, ex = np.frexp(a)
    q = np.rint(mant * 256.0)  # 8 significant bits, ties to even
    r = np.ldexp(q, ex - 8).astype(np.float32)  # exact in fp32
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def ordered16(bits):
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_16bit_output(Y16, Y32, W, keep, X, n, m, dtype):
    """A 16-bit output is the kernel's fp32 sum rounded to nearest-even: it
    must equal the fp32 output of the same launch so rounded, bit for bit, and
    that fp32 sum must lie within the worst-case bound of fp32 summation of
    its kept products, |s32 - s64| <= gamma_k * sum |w x| with
    gamma_k = k u / (1 - k u), u = 2**-24, k = kept weights per row (products
    of 16-bit values are exact in fp32, so only the additions round).  Where
    cancellation leaves |y| far below sum |w x| this is the bar that holds for
    every summation order; 1 ulp of the 16-bit result does not."""
    bf = dtype == "bf16"
    assert np.array_equal(u16(Y16), round16_f64(f64(Y32), dtype))
    want = oracle.masked_gemv(W, keep, X, bf)
    mag = oracle.masked_gemv(W & 0x7FFF, keep, X & 0x7FFF, bf)
    k = W.shape[1] * n // m
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    assert np.all(np.abs(f64(Y32) - want) <= gamma * mag)
    # and where the result is not dominated by cancellation, within 1 ulp
    big = np.abs(want) >= 0.1 * mag
    diff = np.abs(ordered16(u16(Y16)) - ordered16(round16_f64(want, dtype)))
    assert diff[big].max(initial=0) <= 1


# ---- pack -------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (37, 320), (130, 1056), (64, 4096)])
@pytest.mark.parametrize("mask", ["topn", "random"])
def test_pack_bit_exact(rows, cols, n, m, dtype, mask):
    W, keep, _ = inputs(rows, cols, n, m, dtype, 1, seed=rows * 7 + cols, mask=mask)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    st, ov, ob = oracle.pack(W, keep, n, m)
    assert st == oracle.OK
    assert np.array_equal(u16(values), ov)
    assert np.array_equal(u32(bits), ob)


def test_pack_exhaustive_2of4_words():
    """All 6**8 aligned 2:4 words; with W[r, c] = c the packed values of a row
    are its kept column numbers."""
    nib = np.array([0b0011, 0b0101, 0b0110, 0b1001, 0b1010, 0b1100], dtype=np.uint32)
    idx = np.arange(6 ** 8, dtype=np.int64)
    word = np.zeros(idx.shape, dtype=np.uint32)
    for g in range(8):
        word |= nib[(idx // 6 ** g) % 6] << np.uint32(4 * g)
    keep = ((word[:, None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.uint8)
    W = np.broadcast_to(np.arange(32, dtype=np.uint16), keep.shape).copy()
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    st, ov, ob = oracle.pack(W, keep, 2, 4)
    assert st == oracle.OK
    assert np.array_equal(u32(bits)[:, 0], word)
    assert np.array_equal(u16(values), ov)


def test_pack_keeps_raw_patterns():
    W = np.array([[0x8000, 0x0001, 0x7C00, 0x7E01] * 8] * 3, dtype=np.uint16)
    keep = np.array([[1, 1, 0, 0, 0, 0, 1, 1] * 4] * 3, dtype=np.uint8)
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    assert list(u16(values)[0, :4]) == [0x8000, 0x0001, 0x7C00, 0x7E01]
    assert np.all(u32(bits) == 0xC3C3C3C3)


@pytest.mark.parametrize("n,m", PATTERNS)
def test_pack_rejects_invalid_mask_without_writing_outside(n, m):
    rows, cols = 9, 160
    W, keep, _ = inputs(rows, cols, n, m, "f16", 1, seed=3, mask="random")
    keep[4, 37] ^= 1  # one group now keeps n-1 or n+1
    guard = 4096
    vbuf = torch.full((guard + rows * cols // 2 + guard,), 0x5A5A, dtype=torch.int32, device=DEV)
    bbuf = torch.full((guard + rows * cols // 32 + guard,), 0x5A5A, dtype=torch.int32, device=DEV)
    vptr = vbuf.data_ptr() + guard * 4
    bptr = bbuf.data_ptr() + guard * 4
    Wd = t16(W, "f16")
    kd = torch.from_numpy(keep).to(DEV)
    st = native.lib().nm_pack(Wd.data_ptr(), kd.data_ptr(), rows, cols, n, m, native.NM_F16,
                              vptr, bptr, torch.cuda.current_stream().cuda_stream)
    assert st == native.NM_ERR_MASK
    v = vbuf.cpu().numpy()
    b = bbuf.cpu().numpy()
    nv = rows * cols // 2 * 2 // 4  # int32 slots covered by the values
    assert np.all(v[:guard] == 0x5A5A) and np.all(v[guard + nv:] == 0x5A5A)
    assert np.all(b[:guard] == 0x5A5A) and np.all(b[guard + rows * cols // 32:] == 0x5A5A)
    with pytest.raises(native.NMError):
        gpu_pack(W, keep, n, m, "f16")


# ---- products ---------------------------------------------------------------

SHAPES = [(1, 32), (5, 96), (37, 320), (129, 1056), (300, 4096), (70, 14336)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_spmv_matches_oracle(rows, cols, n, m, dtype):
    W, keep, X = inputs(rows, cols, n, m, dtype, 1, seed=rows + cols + m)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    y = native.nm_spmv(values, bits, t16(X[0], dtype), n, m)
    want = oracle.masked_gemv(W, keep, X[0], dtype == "bf16")
    assert rel_l2(f64(y), want) <= TOL


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,m", [(2, 4), (16, 32)])
def test_spmm_small_matches_oracle(batch, n, m, dtype):
    rows, cols = 203, 2080  # 65 words: ragged against every load batch
    W, keep, X = inputs(rows, cols, n, m, dtype, batch, seed=batch)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    Y = native.nm_spmm_small(values, bits, t16(X, dtype), n, m)
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16")
    for b in range(batch):
        assert rel_l2(f64(Y[b]), want[b]) <= TOL


VALU = native.NM_KERNEL_VALU
MFMA = native.NM_KERNEL_MFMA
# (threads_per_wg, rows_per_wave, seg_cols, kernel)
CFGS = [(64, 1, 32, VALU), (64, 4, 96, VALU), (128, 2, 1024, VALU), (256, 1, 0, VALU),
        (256, 4, 64, VALU), (512, 2, 2080, VALU), (1024, 1, 160, VALU), (1024, 4, 0, VALU),
        (64, 3, 0, VALU), (256, 7, 0, VALU), (128, 64, 0, VALU), (256, 3, 0, VALU), (256, 6, 0, VALU)]


@pytest.mark.parametrize("cfg", CFGS)
@pytest.mark.parametrize("batch", [1, 3, 8])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16), (16, 32)])
def test_launch_shapes_integer_exact(cfg, batch, n, m):
    """Every launch shape (threads, rows per wave, LDS segment) gives the exact
    result on integer inputs, including segments that split K raggedly."""
    rows, cols = 257, 2080
    W = synth.integer_weights(rows, cols, seed=5)
    keep = synth.random_mask(rows, cols, n, m, seed=6)
    xi = np.random.default_rng(7).integers(-4, 5, size=(batch, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, n, m, "f16")
    Y = native.nm_spmm_small(values, bits, t16(X, "f16"), n, m, cfg=cfg)
    want = oracle.masked_gemv(W, keep, X, False)
    assert np.array_equal(f64(Y), want)


@pytest.mark.parametrize("cols", [4160, 8224])
@pytest.mark.parametrize("batch", [1, 2, 8])
@pytest.mark.parametrize("n,m", [(2, 4), (16, 32)])
def test_rows_pipeline_several_batches_per_row(cols, batch, n, m):
    """Rows longer than one load batch (256 chunks), ragged against it, walked
    by waves owning 1..7 rows: the two-stage pipeline crosses row and batch
    boundaries in every phase."""
    rows = 203
    W = synth.integer_weights(rows, cols, seed=61)
    keep = synth.random_mask(rows, cols, n, m, seed=62)
    xi = np.random.default_rng(63).integers(-4, 5, size=(batch, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, n, m, "f16")
    want = oracle.masked_gemv(W, keep, X, False)
    for cfg in ((64, 1, 0, VALU), (64, 3, 0, VALU), (256, 5, 0, VALU), (256, 7, 0, VALU),
                (1024, 2, 0, VALU)):
        Y = native.nm_spmm_small(values, bits, t16(X, "f16"), n, m, cfg=cfg)
        assert np.array_equal(f64(Y), want), cfg


@pytest.mark.parametrize("cols", [1024, 2048, 5120, 7168, 14336, 25600])
@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (16, 32)])
def test_batch1_load_batch_sizes_exact(cols, n, m):
    """The batch-1 kernel sizes its load batches (4 or 5 chunks per lane, full
    or ragged last batch for these K); every size, crossed with several rows
    per wave, gives the exact result on integer inputs."""
    rows = 131
    W = synth.integer_weights(rows, cols, seed=71)
    keep = synth.random_mask(rows, cols, n, m, seed=72)
    xi = np.random.default_rng(73).integers(-4, 5, size=(1, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, n, m, "f16")
    want = oracle.masked_gemv(W, keep, X, False)
    # x staged by 4 or 8 groups per thread before the weight loads, with and
    # without the staging loop for the rest (64..512 threads)
    for cfg in (None, (64, 1, 0, VALU), (128, 3, 0, VALU), (256, 6, 0, VALU), (512, 1, 0, VALU)):
        y = native.nm_spmv(values, bits, t16(X[0], "f16"), n, m, cfg=cfg)
        assert np.array_equal(f64(y), want[0]), cfg


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", PATTERNS)
def test_integer_inputs_bit_exact(n, m, dtype):
    rows, cols = 311, 4096
    W = synth.integer_weights(rows, cols, seed=11, dtype=dtype)
    keep = synth.random_mask(rows, cols, n, m, seed=12)
    xi = np.random.default_rng(13).integers(-4, 5, size=(4, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, dtype)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16")
    y1 = native.nm_spmv(values, bits, t16(X[0], dtype), n, m)
    assert np.array_equal(f64(y1), want[0])
    Y = native.nm_spmm_small(values, bits, t16(X, dtype), n, m)
    assert np.array_equal(f64(Y), want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_24_batch1_malformed_mask_words_stay_in_their_row(dtype):
    """2:4 at batch 1 reads x by chunk, never at an address taken from the
    mask, so mask words without two set bits per nibble (0, all ones, three
    bits) only make their own row's sum undefined: every other row stays
    exact (integer inputs)."""
    rows, cols = 300, 4096
    W = synth.integer_weights(rows, cols, seed=21, dtype=dtype)
    keep = synth.random_mask(rows, cols, 2, 4, seed=22)
    xi = np.random.default_rng(23).integers(-4, 5, size=cols).astype(np.float32)
    X = synth.f32_to_16_bits(xi, dtype)
    values, bits = gpu_pack(W, keep, 2, 4, dtype)
    bad = [0, 7, 150, 299]
    b = bits.clone()
    for i, r in enumerate(bad):
        b[r, (37 * i) % b.shape[1]] = [0, -1, 0x77777777, 0x1][i]
    y = f64(native.nm_spmv(values, b, t16(X, dtype), 2, 4))
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16")
    good = np.setdiff1d(np.arange(rows), bad)
    assert np.array_equal(y[good], want[good])


@pytest.mark.parametrize("batch", [1, 2, 4])
@pytest.mark.parametrize("n,m", [(4, 8), (8, 16), (16, 32)])
def test_scan_patterns_malformed_mask_words_stay_in_their_row(n, m, batch):
    """Mask words that break the pattern (no set bit, all set, too few or
    too many in a group) only make their own row's sum undefined under the
    default launch: every other row stays exact on integer inputs."""
    rows, cols = 300, 4096
    W = synth.integer_weights(rows, cols, seed=31, dtype="bf16")
    keep = synth.random_mask(rows, cols, n, m, seed=32)
    xi = np.random.default_rng(33).integers(-4, 5, size=(batch, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "bf16")
    values, bits = gpu_pack(W, keep, n, m, "bf16")
    bad = [0, 7, 150, 299]
    b = bits.clone()
    for i, r in enumerate(bad):
        b[r, (37 * i) % b.shape[1]] = [0, -1, 0x77777777, 0x1][i]
    Y = f64(native.nm_spmm_small(values, b, t16(X, "bf16"), n, m))
    want = oracle.masked_gemv(W, keep, X, True)
    good = np.setdiff1d(np.arange(rows), bad)
    assert np.array_equal(Y[:, good], want[:, good])


@pytest.mark.parametrize("n,m", PATTERNS)
def test_one_hot_x_selects_a_column(n, m):
    """x = e_j gives y[r] = W[r, j] * keep[r, j] exactly: pins the bit ->
    column mapping end to end."""
    rows, cols = 64, 1024
    W, keep, _ = inputs(rows, cols, n, m, "f16", 1, seed=21)
    values, bits = gpu_pack(W, keep, n, m, "f16")
    Wf = W.view(np.float16).astype(np.float64)
    for j in (0, 1, 15, 16, 17, 31, 32, 511, 1000, 1023):
        x = np.zeros(cols, dtype=np.float16)
        x[j] = 1.0
        y = native.nm_spmv(values, bits, t16(x.view(np.uint16), "f16"), n, m)
        assert np.array_equal(f64(y), Wf[:, j] * keep[:, j])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("batch", [1, 4, 8])
def test_16bit_output_is_rounded_fp32_sum(batch, dtype):
    rows, cols, n, m = 515, 4096, 4, 8
    W, keep, X = inputs(rows, cols, n, m, dtype, batch, seed=31)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    Y16 = native.nm_spmm_small(values, bits, t16(X, dtype), n, m, out_dtype=TDT[dtype])
    Y32 = native.nm_spmm_small(values, bits, t16(X, dtype), n, m)
    check_16bit_output(Y16, Y32, W, keep, X, n, m, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("batch", [1, 2, 5, 8])
@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 320), (300, 4096)])
def test_dense_gemv_matches_oracle(rows, cols, batch, dtype):
    W = synth.weights(rows, cols, seed=41, dtype=dtype)
    X = synth.activations(batch, cols, seed=41, dtype=dtype)
    Y = native.nm_dense_gemv(t16(W, dtype), t16(X, dtype))
    want = oracle.masked_gemv(W, None, X, dtype == "bf16")
    for b in range(batch):
        assert rel_l2(f64(Y[b]), want[b]) <= TOL


@pytest.mark.parametrize("cols", [2080, 8224])
def test_dense_integer_exact(cols):
    """Dense kernels (all of x in LDS with any rows per wave, or K walked in
    segments) give the exact result on integer inputs."""
    rows = 129
    W = synth.integer_weights(rows, cols, seed=51)
    xi = np.random.default_rng(52).integers(-4, 5, size=(8, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    want = oracle.masked_gemv(W, None, X, False)
    for batch in (1, 3, 8):
        for cfg in (None, (64, 4, 96, VALU), (1024, 2, 1024, VALU), (64, 1, 0, VALU),
                    (256, 3, 0, VALU), (512, 7, 0, VALU)):
            Y = native.nm_dense_gemv(t16(W, "f16"), t16(X[:batch], "f16"), cfg=cfg)
            assert np.array_equal(f64(Y), want[:batch]), (batch, cfg)


# ---- 2:4 on the sparse matrix cores ------------------------------------------

# (waves x 64 threads, ring depth in blocks of 256 columns); every shape fits
# the LDS for every kind at batch 8
MFMA_CFGS = [(64, 2, 0, MFMA), (64, 4, 0, MFMA), (128, 3, 0, MFMA), (192, 4, 0, MFMA),
             (256, 2, 0, MFMA), (256, 3, 0, MFMA), (320, 2, 0, MFMA), (384, 2, 0, MFMA)]
MFMA_CFGS_24 = [(256, 4, 0, MFMA), (448, 2, 0, MFMA), (512, 2, 0, MFMA)]  # 2:4 only (smaller LDS)


@pytest.mark.parametrize("rows,cols", [(1, 64), (16, 128), (17, 192), (203, 4160), (257, 2112),
                                       (48, 14336)])
@pytest.mark.parametrize("batch", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("n,m", PATTERNS)
def test_mfma_integer_exact(rows, cols, batch, n, m):
    """The matrix-core kernel (2:4 on the sparse instruction, the other
    patterns through the decompressed tile), over ring depths 2..4 and 1..8
    waves splitting K (including more waves than 64-column steps, waves left
    with no steps, and ragged last blocks), gives the exact result on integer
    inputs; ragged row tiles and tokens beyond the batch are never stored."""
    W = synth.integer_weights(rows, cols, seed=81)
    keep = synth.random_mask(rows, cols, n, m, seed=82)
    xi = np.random.default_rng(83).integers(-4, 5, size=(batch, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, n, m, "f16")
    want = oracle.masked_gemv(W, keep, X, False)
    for cfg in MFMA_CFGS + (MFMA_CFGS_24 if (n, m) == (2, 4) else []):
        Y = native.nm_spmm_small(values, bits, t16(X, "f16"), n, m, cfg=cfg)
        assert np.array_equal(f64(Y), want), cfg


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("batch", [2, 4, 7, 8])
@pytest.mark.parametrize("out", ["f32", "16"])
@pytest.mark.parametrize("n,m", PATTERNS)
def test_mfma_matches_oracle(batch, dtype, out, n, m):
    rows, cols = 333, 4096
    W, keep, X = inputs(rows, cols, n, m, dtype, batch, seed=90 + batch)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16")
    cfg = (256, 2, 0, MFMA)
    Y = native.nm_spmm_small(values, bits, t16(X, dtype), n, m, cfg=cfg)
    for b in range(batch):
        assert rel_l2(f64(Y[b]), want[b]) <= TOL
    if out == "16":
        Y16 = native.nm_spmm_small(values, bits, t16(X, dtype), n, m, out_dtype=TDT[dtype], cfg=cfg)
        check_16bit_output(Y16, Y, W, keep, X, n, m, dtype)


@pytest.mark.parametrize("kernel", [VALU, MFMA])
def test_pruned_columns_never_read(kernel):
    """x holds inf and NaN at columns every row prunes: the sums run over kept
    columns only, so the outputs stay finite and equal the oracle's."""
    rows, cols, batch = 96, 1024, 4
    W = synth.integer_weights(rows, cols, seed=95)
    keep = np.zeros((rows, cols), dtype=np.uint8)
    keep[:, 0::4] = 1
    keep[:, 3::4] = 1
    xi = np.random.default_rng(96).integers(-4, 5, size=(batch, cols)).astype(np.float32)
    xi[:, 1::4] = np.inf
    xi[:, 2::4] = np.nan
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    want = oracle.masked_gemv(W, keep, X, False)
    assert np.all(np.isfinite(want))
    Y = native.nm_spmm_small(values, bits, t16(X, "f16"), 2, 4, cfg=(0, 0, 0, kernel))
    assert np.array_equal(f64(Y), want)


def test_mfma_rejected_where_it_cannot_run():
    rows, cols = 32, 96  # 96 % 64 != 0
    W, keep, X = inputs(rows, cols, 2, 4, "f16", 2, seed=97)
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    with pytest.raises(native.NMError) as e:
        native.nm_spmm_small(values, bits, t16(X, "f16"), 2, 4, cfg=(0, 0, 0, MFMA))
    assert e.value.status == native.NM_ERR_UNSUPPORTED
    W, keep, X = inputs(rows, 96, 16, 32, "f16", 2, seed=98)
    values, bits = gpu_pack(W, keep, 16, 32, "f16")
    with pytest.raises(native.NMError) as e:
        native.nm_spmm_small(values, bits, t16(X, "f16"), 16, 32, cfg=(0, 0, 0, MFMA))
    assert e.value.status == native.NM_ERR_UNSUPPORTED
    with pytest.raises(native.NMError) as e:
        native.nm_dense_gemv(t16(W, "f16"), t16(X, "f16"), cfg=(0, 0, 0, MFMA))
    assert e.value.status == native.NM_ERR_UNSUPPORTED
    W, keep, X = inputs(rows, 128, 2, 4, "f16", 2, seed=99)
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    for cfg in ((256, 5, 0, MFMA), (256, 1, 0, MFMA), (96, 2, 0, MFMA), (1024, 4, 0, MFMA),
                (256, 2, 0, 5)):
        # ring depth outside 2..4; 96 threads; 16 waves x 4 blocks exceed LDS; no kernel 5
        with pytest.raises(native.NMError) as e:
            native.nm_spmm_small(values, bits, t16(X, "f16"), 2, 4, cfg=cfg)
        assert e.value.status == native.NM_ERR_INVALID_ARG, cfg


def test_default_launch_picks_matrix_cores_for_small_batch():
    for n, m in PATTERNS:
        assert native.nm_default_launch(14336, 4096, 8, n, m).kernel == MFMA, (n, m)
        assert native.nm_default_launch(14336, 4096, 1, n, m).kernel == VALU, (n, m)
        # the decompressing kinds start at batch 5, 2:4 on the sparse
        # instruction at batch 3
        want4 = MFMA if (n, m) == (2, 4) else VALU
        assert native.nm_default_launch(14336, 4096, 4, n, m).kernel == want4, (n, m)
        assert native.nm_default_launch(8192, 8192, 4, n, m).kernel == want4, (n, m)
    assert native.nm_default_launch(14336, 4080 + 16, 8, 2, 4).kernel == MFMA
    assert native.nm_default_launch(14336, 4064, 8, 2, 4).kernel == VALU  # K % 64 != 0
    assert native.nm_default_launch(14336, 4096, 8, dense=True).kernel == VALU


def test_default_launch_2of4_small_batch_rule():
    """2:4 at batch 2 takes the VALU kernel (x plain per token) on every shape
    whose x fits in LDS, and at batch 3 and 4 on shapes of at most 1024 rows,
    where it measured faster than the matrix cores; every other shape at
    batch 3 and 4, every shape at batch 5..8, and batch 2 with x beyond the
    LDS take the matrix cores."""
    d = native.nm_default_launch
    for b in (2, 3, 4):
        for rows, cols in [(1024, 4096), (1024, 8192)]:
            assert d(rows, cols, b, 2, 4).kernel == VALU, (rows, cols, b)
    for rows, cols in [(4096, 4096), (14336, 4096), (25600, 5120), (28672, 8192), (8192, 28672),
                       (5120, 25600), (4096, 14336), (8192, 8192), (8192, 5120), (5120, 8192),
                       (6144, 4096)]:
        assert d(rows, cols, 2, 2, 4).kernel == VALU, (rows, cols)
    assert d(4096, 65536, 2, 2, 4).kernel == MFMA  # 2 x 128 KiB of x
    for b in (3, 4):
        for rows, cols in [(4096, 4096), (14336, 4096), (4096, 14336), (25600, 5120), (28672, 8192),
                           (8192, 28672)]:
            assert d(rows, cols, b, 2, 4).kernel == MFMA, (rows, cols, b)
    for b in (5, 8):
        for rows, cols in [(1024, 4096), (4096, 4096), (14336, 4096)]:
            assert d(rows, cols, b, 2, 4).kernel == MFMA, (rows, cols, b)


def test_default_launch_matrix_core_shape():
    """Waves per workgroup and ring depth of the 2:4 matrix-core kernel (256
    CUs, 160 KiB of LDS): four waves, halved while a wave would walk fewer
    than 32 steps of 64 columns and at least 1024 waves remain, and one wave
    where two would walk fewer than 64 steps on at least 1024 tiles; three
    blocks in the ring while 8 waves of such workgroups fit a CU, else two."""
    d = native.nm_default_launch
    want = {(14336, 4096, 4): (128, 3), (14336, 4096, 8): (128, 2), (4096, 4096, 8): (256, 2),
            (4096, 4096, 4): (256, 3), (8192, 5120, 8): (128, 2), (8192, 8192, 8): (256, 2),
            (4096, 14336, 4): (256, 3), (28672, 8192, 8): (256, 2), (6144, 4096, 8): (256, 2),
            (25600, 5120, 4): (64, 3), (25600, 5120, 8): (64, 2)}
    for (rows, cols, b), (threads, nb) in want.items():
        c = d(rows, cols, b, 2, 4)
        assert c.kernel == MFMA and (c.threads_per_wg, c.rows_per_wave) == (threads, nb), (rows, cols, b)


@pytest.mark.parametrize("batch", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("rows,cols", [(203, 4096), (130, 8192), (257, 2080), (64, 14336)])
def test_plain_x_batch_integer_exact(rows, cols, batch):
    """The VALU 2:4 kernel at batch 2..8 with x stored plainly per token (the
    chunk's pair selectors applied to every token's x): exact on integer
    inputs, for whole and ragged last load batches and several launch shapes."""
    W = synth.integer_weights(rows, cols, seed=101)
    keep = synth.random_mask(rows, cols, 2, 4, seed=102)
    xi = np.random.default_rng(103).integers(-4, 5, size=(batch, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    want = oracle.masked_gemv(W, keep, X, False)
    cfgs = [native.LaunchCfg(0, 0, 0, VALU), (64, 1, 0, VALU), (256, 4, 0, VALU), (512, 2, 0, VALU)]
    if native.nm_resolve_launch(rows, cols, batch, 2, 4, cfg=native.LaunchCfg(0, 0, 0, VALU)).seg_cols >= cols:
        # all of x in LDS (the row kernel): shapes the batch >= 2 rule picks on
        # larger layers (6, 7 or 14 rows a wave in 4-wave workgroups, 3 in
        # 8-wave ones), each with a ragged last workgroup here
        cfgs += [(256, 6, 0, VALU), (256, 7, 0, VALU), (256, 14, 0, VALU), (512, 3, 0, VALU)]
    for cfg in cfgs:
        Y = native.nm_spmm_small(values, bits, t16(X, "f16"), 2, 4, cfg=cfg)
        assert np.array_equal(f64(Y), want), cfg


@pytest.mark.parametrize("rows,cols", [(1024, 4096), (300, 2080), (77, 8192)])
def test_batch1_x_staging_paths_integer_exact(rows, cols):
    """The batch-1 2:4 row kernel copies x into LDS with direct-to-LDS loads
    when a workgroup holds at most 4 rows, and stages it through registers
    otherwise: both exact on integer inputs, for launch shapes on either side
    of that line, with whole and ragged load batches and with the split
    reduction."""
    W = synth.integer_weights(rows, cols, seed=111)
    keep = synth.random_mask(rows, cols, 2, 4, seed=112)
    xi = np.random.default_rng(113).integers(-4, 5, size=(1, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    want = oracle.masked_gemv(W, keep, X, False)
    cfgs = [(256, 1, 0, VALU), (64, 4, 0, VALU), (128, 2, 0, VALU),  # <= 4 rows: copies
            (256, 2, 0, VALU), (512, 4, 0, VALU), (1024, 1, 0, VALU)]  # more: registers
    if cols % 2048 == 0:
        cfgs += [(256, 1, 0, VALU, 2), (1024, 1, 0, VALU, 2)]  # split over 2 waves: 2 / 8 rows
    for cfg in cfgs:
        Y = native.nm_spmm_small(values, bits, t16(X, "f16"), 2, 4, cfg=native.LaunchCfg(*cfg))
        assert np.array_equal(f64(Y), want), cfg


def test_default_launch_shapes_follow_the_measured_rules():
    """Launch shapes the library picks on the 8B shapes (256 CUs), each the
    measured best of its sweep: 2:4 q|k|v 6144x4096 and q 4096x4096 as one
    4-wave workgroup per CU; 4:8 (x plain, pair table) takes the 2:4 shapes;
    the scan of 8:16 keeps 2
    rows per wave and 4-wave workgroups; at other densities, x of K = 14336 at
    batch 8 in two equal segments staged by 16-wave workgroups, and K = 4096
    whole with 4-wave workgroups."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the rules are pinned for 256 CUs")

    def shape(*a):
        c = native.nm_default_launch(*a)
        return c.threads_per_wg, c.rows_per_wave, c.seg_cols

    # 2:4 and 4:8 at batch 1, 12..24 rows per CU and K <= 8192: one 4-wave
    # workgroup per CU; the 8:16 / 16:32 scan at 24 rows per CU: two 4-wave
    # workgroups of 3 rows a wave
    assert shape(6144, 4096, 1, 2, 4) == (256, 6, 4096)
    assert shape(4096, 4096, 1, 2, 4) == (256, 4, 4096)
    assert shape(5120, 8192, 1, 2, 4) == (256, 5, 8192)
    assert shape(8192, 8192, 1, 2, 4) == (256, 4, 8192)
    assert shape(4096, 4096, 1, 4, 8) == shape(4096, 4096, 1, 2, 4)
    assert shape(6144, 4096, 1, 4, 8) == (256, 6, 4096)
    assert shape(6144, 4096, 1, 8, 16) == (256, 3, 4096)
    assert shape(6144, 4096, 1, 16, 32) == (256, 3, 4096)
    assert shape(4096, 14336, 1, 4, 8) == shape(4096, 14336, 1, 2, 4)
    assert shape(4096, 4096, 1, 8, 16) == (256, 2, 4096)
    assert shape(4096, 14336, 1, 8, 16) == (256, 2, 14336)
    assert shape(4096, 14336, 8, 1, 4) == (1024, 1, 7168)
    assert shape(14336, 4096, 8, 1, 4) == (256, 7, 4096)
    # 2:4 at batch 2: the CU's rows over one workgroup of 4 (K <= 4096) or 8
    # waves, two workgroups past 8 rows a wave, 4 rows a wave for the long-K
    # tall shapes
    assert shape(1024, 4096, 2, 2, 4) == (256, 1, 4096)
    assert shape(4096, 4096, 2, 2, 4) == (256, 4, 4096)
    assert shape(6144, 4096, 2, 2, 4) == (256, 6, 4096)
    assert shape(14336, 4096, 2, 2, 4) == (256, 7, 4096)
    assert shape(4096, 14336, 2, 2, 4) == (512, 2, 14336)
    assert shape(5120, 8192, 2, 2, 4) == (512, 3, 8192)
    assert shape(8192, 8192, 2, 2, 4) == (256, 4, 8192)
    assert shape(8192, 28672, 2, 2, 4) == (256, 8, 28672)
    assert shape(25600, 5120, 2, 2, 4) == (512, 7, 5120)


def test_forced_valu_shape_equals_the_automatic_valu_shape():
    """Forcing NM_KERNEL_VALU keeps the pattern's own launch rules: where the
    library's choice is already the VALU kernel (batch 1) the forced shape is
    the same, e.g. 2:4 at K = 14336 keeps one row per wave; at batch 2..8 a
    forced VALU launch gets the VALU shape of that pattern and batch."""
    V = native.LaunchCfg(0, 0, 0, VALU)
    for rows, cols in [(14336, 4096), (4096, 14336), (4096, 4096), (1024, 4096), (6144, 4096),
                       (8192, 8192), (28672, 8192), (5120, 25600), (96, 2112)]:
        for n, m in PATTERNS + [(1, 4), (3, 4), (3, 8)]:
            auto = native.nm_default_launch(rows, cols, 1, n, m)
            forced = native.nm_resolve_launch(rows, cols, 1, n, m, cfg=V)
            assert auto.kernel == VALU
            assert (forced.kernel, forced.threads_per_wg, forced.rows_per_wave, forced.seg_cols) == \
                (auto.kernel, auto.threads_per_wg, auto.rows_per_wave, auto.seg_cols), (rows, cols, n, m)
        for batch in (2, 4, 8):
            forced = native.nm_resolve_launch(rows, cols, batch, 2, 4, cfg=V)
            assert forced.kernel == VALU
    # no override: the resolved shape is the default one
    for b in (1, 2, 5, 8):
        a, r = native.nm_default_launch(4096, 4096, b, 4, 8), native.nm_resolve_launch(4096, 4096, b, 4, 8)
        assert (a.kernel, a.threads_per_wg, a.rows_per_wave, a.seg_cols) == \
            (r.kernel, r.threads_per_wg, r.rows_per_wave, r.seg_cols)


def test_zero_columns_give_zero_output_batch():
    for batch in (1, 2, 8):
        values = torch.empty((7, 0), dtype=torch.float16, device=DEV)
        bits = torch.empty((7, 0), dtype=torch.int32, device=DEV)
        X = torch.empty((batch, 0), dtype=torch.float16, device=DEV)
        Y = torch.full((batch, 7), 3.0, device=DEV)
        native.nm_spmm_small(values, bits, X, 2, 4, out=Y)
        assert torch.count_nonzero(Y).item() == 0


def test_zero_columns_give_zero_output():
    values = torch.empty((7, 0), dtype=torch.float16, device=DEV)
    bits = torch.empty((7, 0), dtype=torch.int32, device=DEV)
    x = torch.empty((0,), dtype=torch.float16, device=DEV)
    y = torch.full((7,), 3.0, device=DEV)
    native.nm_spmv(values, bits, x, 2, 4, out=y)
    assert torch.count_nonzero(y).item() == 0


# ---- full-size workloads, sampled rows ----------------------------------------

def _full_cases():
    cases = []
    for cfg_id in (1, 2, 3, 4):
        for mt, batches in workloads.config_matrices(cfg_id):
            cases.append(pytest.param(mt, batches, id=f"cfg{cfg_id}-{mt.name}-{mt.rows}x{mt.cols}"))
    # the 32-layer sweep: the first and the last layer
    sweep = workloads.config_matrices(5)
    for mt, batches in sweep[:7] + sweep[-7:]:
        cases.append(pytest.param(mt, batches, id=f"cfg5-seed{mt.seed}-{mt.name}"))
    return cases


SAMPLE_ROWS = 384


@pytest.mark.parametrize("mt,batches", _full_cases())
def test_full_size_sampled_rows(mt, batches):
    rng = np.random.default_rng(mt.seed + 99)
    W = synth.weights(mt.rows, mt.cols, seed=mt.seed, dtype=mt.dtype)
    keep = synth.topn_mask(W, mt.n, mt.m)
    Wd = t16(W, mt.dtype)
    values, bits = native.nm_pack(Wd, torch.from_numpy(keep).to(DEV), mt.n, mt.m)
    idx = np.sort(rng.choice(mt.rows, size=min(SAMPLE_ROWS, mt.rows), replace=False))
    # pack: bit-exact on the sampled rows, and 16 set bits in every word
    st, ov, ob = oracle.pack(W[idx], keep[idx], mt.n, mt.m)
    assert st == oracle.OK
    ti = torch.from_numpy(idx).to(DEV)
    assert np.array_equal(u16(values.index_select(0, ti)), ov)
    assert np.array_equal(u32(bits.index_select(0, ti)), ob)
    allbits = u32(bits)
    pop = np.unpackbits(allbits.view(np.uint8)).reshape(-1, 32).sum(axis=1)
    assert np.all(pop == 16)
    bf = mt.dtype == "bf16"
    for batch in batches:
        X = synth.activations(batch, mt.cols, seed=mt.seed, dtype=mt.dtype, outliers=mt.outliers)
        Xd = t16(X, mt.dtype)
        if batch == 1:
            Y = native.nm_spmv(values, bits, Xd[0], mt.n, mt.m).reshape(1, -1)
        else:
            Y = native.nm_spmm_small(values, bits, Xd, mt.n, mt.m)
        Ys = f64(Y.index_select(1, ti))
        want = oracle.masked_gemv(W, keep, X, bf, rows_idx=idx, threads=8)
        for b in range(batch):
            assert rel_l2(Ys[b], want[b]) <= TOL, (mt, batch, b)
        # the dense comparison kernel on the same sampled rows
        Yd = f64(native.nm_dense_gemv(Wd, Xd).index_select(1, ti))
        wd = oracle.masked_gemv(W, None, X, bf, rows_idx=idx, threads=8)
        for b in range(batch):
            assert rel_l2(Yd[b], wd[b]) <= TOL, (mt, batch, b)


# ---- fused gate/up product with the SwiGLU epilogue --------------------------------

def _swiglu_inputs(inter, cols, n, m, dtype, batch, seed):
    W = synth.weights(2 * inter, cols, seed=seed, dtype=dtype)  # rows 2r gate, 2r+1 up
    keep = synth.topn_mask(W, n, m)
    X = synth.activations(batch, cols, seed=seed, dtype=dtype)
    return W, keep, X


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("batch", [1, 2, 5, 8])
@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("cols", [2080, 2112])  # 2112: matrix-core eligible at batch >= 2 / 5
def test_swiglu_matches_oracle(cols, n, m, batch, dtype):
    inter = 203
    W, keep, X = _swiglu_inputs(inter, cols, n, m, dtype, batch, seed=100 + batch)
    values, bits = gpu_pack(W, keep, n, m, dtype)
    H = native.nm_spmm_swiglu(values, bits, t16(X, dtype), n, m)
    want = oracle.swiglu_gemv(W, keep, X, dtype == "bf16")
    assert H.shape == (batch, inter)
    for b in range(batch):
        assert rel_l2(f64(H[b]), want[b]) <= TOL


SWIGLU_CFGS = [(64, 2, 0, VALU), (256, 4, 0, VALU), (128, 6, 0, VALU), (512, 2, 0, VALU),
               (256, 2, 0, MFMA), (128, 3, 0, MFMA), (64, 2, 0, MFMA)]


@pytest.mark.parametrize("cfg", SWIGLU_CFGS)
@pytest.mark.parametrize("batch", [1, 3, 8])
@pytest.mark.parametrize("n,m", [(2, 4), (16, 32)])
def test_swiglu_epilogue_matches_separate_product(cfg, batch, n, m):
    """The epilogue equals silu(gate) * up applied on the host to the fp32
    sums of the same kernel without it (integer inputs: the sums are exact, so
    only the fp32 silu differs, within a few ulp), for ragged pair counts."""
    inter, cols = 77, 4160
    W = synth.integer_weights(2 * inter, cols, seed=110)
    keep = synth.random_mask(2 * inter, cols, n, m, seed=111)
    xi = np.random.default_rng(112).integers(-2, 3, size=(batch, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, n, m, "f16")
    Y = f64(native.nm_spmm_small(values, bits, t16(X, "f16"), n, m, cfg=cfg))
    assert np.array_equal(Y, oracle.masked_gemv(W, keep, X, False))
    H = f64(native.nm_spmm_swiglu(values, bits, t16(X, "f16"), n, m, cfg=cfg))
    g = Y[:, 0::2].astype(np.float32)
    u = Y[:, 1::2].astype(np.float32)
    with np.errstate(over="ignore"):  # exp(-g) = inf for very negative g: silu -> -0
        want = (g / (np.float32(1) + np.exp(-g))) * u
    assert np.allclose(H, want, rtol=1e-5, atol=1e-6 * np.abs(want).max())


def test_swiglu_16bit_output_is_rounded_fp32():
    inter, cols = 150, 2112
    for dtype in ("f16", "bf16"):
        for batch in (1, 4):
            W, keep, X = _swiglu_inputs(inter, cols, 2, 4, dtype, batch, seed=120)
            values, bits = gpu_pack(W, keep, 2, 4, dtype)
            H32 = native.nm_spmm_swiglu(values, bits, t16(X, dtype), 2, 4)
            H16 = native.nm_spmm_swiglu(values, bits, t16(X, dtype), 2, 4, out_dtype=TDT[dtype])
            assert np.array_equal(u16(H16), round16_f64(f64(H32), dtype)), (dtype, batch)


def test_swiglu_rejects_shapes_it_cannot_run():
    inter, cols = 32, 2112
    W, keep, X = _swiglu_inputs(inter, cols, 4, 8, "f16", 2, seed=130)
    values, bits = gpu_pack(W, keep, 4, 8, "f16")
    with pytest.raises(native.NMError) as e:  # odd rows per wave: pairs would straddle waves
        native.nm_spmm_swiglu(values, bits, t16(X, "f16"), 4, 8, cfg=(256, 3, 0, VALU))
    assert e.value.status == native.NM_ERR_INVALID_ARG
    with pytest.raises(native.NMError) as e:  # K walked in LDS segments: no epilogue there
        native.nm_spmm_swiglu(values, bits, t16(X, "f16"), 4, 8, cfg=(256, 2, 512, VALU))
    assert e.value.status == native.NM_ERR_UNSUPPORTED


def test_swiglu_zero_columns():
    for batch in (1, 6):
        values = torch.empty((8, 0), dtype=torch.float16, device=DEV)
        bits = torch.empty((8, 0), dtype=torch.int32, device=DEV)
        X = torch.empty((batch, 0), dtype=torch.float16, device=DEV)
        H = torch.full((batch, 4), 3.0, device=DEV)
        native.nm_spmm_swiglu(values, bits, X, 2, 4, out=H)
        assert torch.count_nonzero(H).item() == 0


# ---- the layer Hessian (calibration side) ------------------------------------------

def _hx(d, ld, seed, dtype="f16", ints=True):
    rng = np.random.default_rng(seed)
    xf = rng.integers(-3, 4, size=(d, ld)) if ints else rng.normal(size=(d, ld))
    return synth.f32_to_16_bits(xf.astype(np.float32), dtype)


@pytest.mark.parametrize("d", [1, 16, 100, 128, 129, 300])
@pytest.mark.parametrize("ntok", [1, 7, 8, 31, 32, 33, 100])
def test_hessian_integer_exact(d, ntok):
    """Integer activations: every sum is an exact integer in fp32, so
    H0 + 2 X X^T must match the oracle exactly, ragged tiles, ragged token
    chunks and columns past ntok (filled with other values) included."""
    ld = (ntok + 7) // 8 * 8 + 8
    X = _hx(d, ld, seed=d * 131 + ntok)
    H0 = np.random.default_rng(d + ntok).integers(-50, 50, size=(d, d)).astype(np.float32)
    H0 = H0 + H0.T  # a symmetric start
    H = torch.from_numpy(H0).to(DEV)
    native.nm_hessian_accumulate(H, t16(X, "f16"), ntok=ntok, scale=2.0)
    want = H0.astype(np.float64) + oracle.hessian(X, ntok=ntok, scale=2.0)
    got = H.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_hessian_matches_oracle(dtype):
    d, ntok = 520, 256
    X = _hx(d, ntok, seed=7, dtype=dtype, ints=False)
    H = torch.zeros((d, d), device=DEV)
    native.nm_hessian_accumulate(H, t16(X, dtype), scale=2.0)
    want = oracle.hessian(X, scale=2.0, is_bf16=dtype == "bf16", threads=8)
    got = H.cpu().numpy().astype(np.float64)
    assert rel_l2(got.ravel(), want.ravel()) <= 1e-6
    assert np.array_equal(got, got.T)


def test_hessian_accumulates_over_calls():
    """Two calls over the two halves of the columns equal one call over all
    of them (integer inputs, exact)."""
    d, ntok = 200, 96
    X = _hx(d, ntok, seed=9)
    Xa, Xb = np.ascontiguousarray(X[:, :48]), np.ascontiguousarray(X[:, 48:])
    H1 = torch.zeros((d, d), device=DEV)
    native.nm_hessian_accumulate(H1, t16(X, "f16"))
    H2 = torch.zeros((d, d), device=DEV)
    native.nm_hessian_accumulate(H2, t16(Xa, "f16"))
    native.nm_hessian_accumulate(H2, t16(Xb, "f16"))
    assert torch.equal(H1, H2)


def test_hessian_zero_tokens_leaves_h():
    H = torch.full((33, 33), 1.5, device=DEV)
    X = torch.zeros((33, 8), dtype=torch.float16, device=DEV)
    native.nm_hessian_accumulate(H, X, ntok=0)
    assert torch.all(H == 1.5).item()


# ---- N:M mask selection (calibration side) -----------------------------------------

def _sel_w(rows, cols, seed, dtype, kind="normal"):
    rng = np.random.default_rng(seed)
    if kind == "ints":
        a = rng.integers(-4, 5, size=(rows, cols))
    else:
        a = rng.normal(size=(rows, cols)) * 0.02
    return synth.f32_to_16_bits(a.astype(np.float32), dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("rows,cols,cstride", [(1, 32, 1), (37, 96, 1), (300, 4096, 3), (129, 2080, 1)])
def test_select_matches_oracle_bit_exact(rows, cols, cstride, n, m, dtype):
    """The keep-mask is an integer result decided in fp32 on both sides:
    bit-exact, ragged final block of lanes included."""
    W = _sel_w(rows, cols, seed=rows + cols + m, dtype=dtype)
    rng = np.random.default_rng(cols * 7 + m)
    colw = rng.uniform(0.0, 4.0, size=(cols - 1) * cstride + 1).astype(np.float32)
    keep = native.nm_select_nm(t16(W, dtype), torch.from_numpy(colw).to(DEV), n, m, cstride=cstride)
    want = oracle.select_nm(W, colw, n, m, dtype == "bf16", cstride=cstride)
    assert np.array_equal(keep.cpu().numpy(), want)


@pytest.mark.parametrize("n,m", PATTERNS)
def test_select_ties_and_nan_scores(n, m):
    """Integer weights and a few distinct column weights make equal scores
    common (lower column wins); NaN weights and 0 * inf rank last."""
    rows, cols = 64, 512
    W = _sel_w(rows, cols, seed=5 + m, dtype="f16", kind="ints")
    rng = np.random.default_rng(m)
    W[rng.random((rows, cols)) < 0.05] = 0x7E00  # NaN
    colw = rng.integers(0, 3, size=cols).astype(np.float32)
    colw[rng.random(cols) < 0.05] = np.inf
    keep = native.nm_select_nm(t16(W, "f16"), torch.from_numpy(colw).to(DEV), n, m)
    want = oracle.select_nm(W, colw, n, m, False)
    assert np.array_equal(keep.cpu().numpy(), want)
    assert oracle.count_bad_groups(want, n, m) == 0


def test_select_from_gpu_hessian_then_pack():
    """The calibration step end to end on the device: H = 2 X X^T from
    integer activations (exact in fp32), selection from its diagonal
    (cstride = d + 1), then nm_pack; values and bits equal the oracle's
    pack of the oracle's selection from the oracle's Hessian."""
    d, ntok, rows, n, m = 256, 40, 96, 2, 4
    X = _hx(d, ntok, seed=11)
    H = torch.zeros((d, d), device=DEV)
    native.nm_hessian_accumulate(H, t16(X, "f16"), scale=2.0)
    W = _sel_w(rows, d, seed=12, dtype="f16")
    Wt = t16(W, "f16")
    keep = native.nm_select_nm(Wt, H, n, m, cstride=d + 1)
    values, bits = native.nm_pack(Wt, keep, n, m)
    Hd = np.diag(oracle.hessian(X, scale=2.0)).astype(np.float32)
    want_keep = oracle.select_nm(W, Hd, n, m, False)
    st, want_v, want_b = oracle.pack(W, want_keep, n, m)
    assert st == oracle.OK
    assert np.array_equal(keep.cpu().numpy(), want_keep)
    assert np.array_equal(u16(values).ravel(), want_v.ravel())
    assert np.array_equal(u32(bits).ravel(), want_b.ravel())


def test_select_full_size_layer():
    """A 14336 x 4096 layer (the gate/up shape), fp16 2:4, against the
    oracle over every group."""
    rows, cols = 14336, 4096
    W = synth.weights(rows, cols, seed=77, dtype="f16")
    colw = np.random.default_rng(78).uniform(0.0, 4.0, size=cols).astype(np.float32)
    keep = native.nm_select_nm(t16(W, "f16"), torch.from_numpy(colw).to(DEV), 2, 4)
    want = oracle.select_nm(W, colw, 2, 4, False)
    assert np.array_equal(keep.cpu().numpy(), want)


def test_select_zero_sized_and_rejections():
    colw = torch.ones(64, device=DEV)
    k = native.nm_select_nm(torch.zeros((0, 64), dtype=torch.float16, device=DEV), colw, 2, 4)
    assert k.shape == (0, 64)
    with pytest.raises(native.NMError):
        native.nm_select_nm(torch.zeros((4, 48), dtype=torch.float16, device=DEV), colw, 2, 4)
    with pytest.raises(native.NMError):
        native.nm_select_nm(torch.zeros((4, 64), dtype=torch.float16, device=DEV), colw, 3, 4)
    with pytest.raises(ValueError):
        native.nm_select_nm(torch.zeros((4, 64), dtype=torch.float16, device=DEV), colw, 2, 4, cstride=2)


# ---- prefill-side product (2:4 on the sparse matrix cores, any batch) ----------------

# Tile shapes the launch picks on 256 compute units (row tiles, token tiles
# per wave, parts of K): (7, 1, 1) for the smallest shapes, (7, 1, 2) for
# 257 x 1024 x 130 and 640 x 2112 x 257, (7, 1, 4) for 512 x 4096 x 128,
# (7, 2, 1) for 7201 x 600, (8, 1, 1), (8, 2, 1) and (8, 4, 1) for 4096 rows
# at 1024, 2048 and 4096 tokens, (7, 4, 1) for 14336 rows at 1024 tokens,
# (8, 1, 4) for 1000 x 2048 x 1024, (7, 2, 4) for 4100 x 4096 x 256, (8, 2, 4)
# for 1000 x 4096 x 2048
PREFILL_SHAPES = [(1, 64, 1), (16, 128, 16), (300, 320, 17), (257, 1024, 130), (512, 4096, 128),
                  (100, 64, 300), (640, 2112, 257), (7201, 128, 600), (4096, 64, 1024),
                  (4096, 64, 2048), (4096, 64, 4096), (14336, 64, 1024), (1000, 2048, 1024),
                  (4100, 4096, 256), (1000, 4096, 2048)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("rows,cols,batch", PREFILL_SHAPES)
def test_prefill_integer_exact(rows, cols, batch, dtype):
    """Integer weights and activations: every partial sum is an exact integer
    in fp32, so the product must equal the oracle exactly, ragged row and
    token tiles and several K steps included."""
    W = synth.integer_weights(rows, cols, seed=rows + cols, dtype=dtype)
    keep = synth.random_mask(rows, cols, 2, 4, seed=batch)
    xi = np.random.default_rng(rows * batch).integers(-4, 5, size=(batch, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, dtype)
    values, bits = gpu_pack(W, keep, 2, 4, dtype)
    Y = native.nm_spmm_prefill(values, bits, t16(X, dtype))
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16", threads=8)
    assert np.array_equal(f64(Y), want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_matches_oracle(dtype):
    rows, cols, batch = 700, 1536, 200
    W, keep, X = inputs(rows, cols, 2, 4, dtype, batch, seed=31)
    values, bits = gpu_pack(W, keep, 2, 4, dtype)
    Y = f64(native.nm_spmm_prefill(values, bits, t16(X, dtype)))
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16", threads=8)
    for b in range(batch):
        assert rel_l2(Y[b], want[b]) <= TOL


@pytest.mark.parametrize("rows", [300, 257])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_16bit_output_is_rounded_fp32(dtype, rows):
    cols, batch = 512, 40
    W, keep, X = inputs(rows, cols, 2, 4, dtype, batch, seed=32)
    values, bits = gpu_pack(W, keep, 2, 4, dtype)
    Xt = t16(X, dtype)
    Y32 = native.nm_spmm_prefill(values, bits, Xt)
    Y16 = native.nm_spmm_prefill(values, bits, Xt, out_dtype=TDT[dtype])
    assert torch.equal(Y16, Y32.to(TDT[dtype]))


@pytest.mark.parametrize("batch", [1, 3, 8])
def test_prefill_agrees_with_decode_kernels(batch):
    rows, cols = 1000, 4096
    W, keep, X = inputs(rows, cols, 2, 4, "f16", batch, seed=33)
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    Xt = t16(X, "f16")
    a = f64(native.nm_spmm_prefill(values, bits, Xt))
    b = f64(native.nm_spmm_small(values, bits, Xt, 2, 4))
    for t in range(batch):
        assert rel_l2(a[t], b[t]) <= 1e-5


def test_prefill_full_size_sampled_rows():
    """14336 x 4096 (the gate/up shape) at 256 tokens, 384 rows against the
    oracle one by one."""
    rows, cols, batch = 14336, 4096, 256
    W = synth.weights(rows, cols, seed=41, dtype="f16")
    keep = synth.topn_mask(W, 2, 4)
    X = synth.activations(batch, cols, seed=42, dtype="f16")
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    Y = f64(native.nm_spmm_prefill(values, bits, t16(X, "f16")))
    idx = np.sort(np.random.default_rng(43).choice(rows, SAMPLE_ROWS, replace=False))
    idx[0], idx[-1] = 0, rows - 1
    want = oracle.masked_gemv(W, keep, X, False, rows_idx=idx, threads=8)
    got = Y[:, idx]
    for b in range(batch):
        assert rel_l2(got[b], want[b]) <= TOL


@pytest.mark.parametrize("rows,cols,batch", [(4096, 14336, 1024), (4100, 8192, 512)])
def test_prefill_split_k_sampled_rows_integer_exact(rows, cols, batch):
    """K in 4 parts with the widest token tile ((8, 4, 4) for the 4096 x 14336
    down shape at 1024 tokens, (7, 4, 4) for 4100 x 8192 at 512): integer
    inputs, 384 sampled rows against the oracle exactly (the fp32 partial
    sums of the parts and their total are exact integers)."""
    W = synth.integer_weights(rows, cols, seed=rows + 3, dtype="f16")
    keep = synth.random_mask(rows, cols, 2, 4, seed=batch + 1)
    xi = np.random.default_rng(rows).integers(-4, 5, size=(batch, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    Y = f64(native.nm_spmm_prefill(values, bits, t16(X, "f16")))
    idx = np.sort(np.random.default_rng(44).choice(rows, SAMPLE_ROWS, replace=False))
    idx[0], idx[-1] = 0, rows - 1
    want = oracle.masked_gemv(W, keep, X, False, rows_idx=idx, threads=8)
    assert np.array_equal(Y[:, idx], want)


def _split_case(rows, cols, batch, seed):
    """Integer inputs for a prefill shape that the launch splits in K, with
    the oracle's (exact) result."""
    W = synth.integer_weights(rows, cols, seed=seed, dtype="f16")
    keep = synth.random_mask(rows, cols, 2, 4, seed=seed + 1)
    xi = np.random.default_rng(seed + 2).integers(-4, 5, size=(batch, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    return values, bits, t16(X, "f16"), oracle.masked_gemv(W, keep, X, False, threads=8)


def test_prefill_split_workspace_kept_across_calls_and_streams():
    """Split-K calls keep one workspace per stream: a larger split grows it in
    stream order, a smaller one after it reuses it, and calls queued back to
    back on two streams each use their own; every result is exact.  (K in 4
    parts for all three shapes, 16.4, 16.8 and 32.8 MB of partial sums.)"""
    cases = [_split_case(1000, 2048, 1024, 51), _split_case(4100, 4096, 256, 52),
             _split_case(1000, 4096, 2048, 53)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    out = []
    for i1, i2 in ((0, 1), (2, 0), (1, 2), (0, 1)):
        with torch.cuda.stream(s1):
            v, b, X, _ = cases[i1]
            out.append((i1, native.nm_spmm_prefill(v, b, X)))
        with torch.cuda.stream(s2):
            v, b, X, _ = cases[i2]
            out.append((i2, native.nm_spmm_prefill(v, b, X)))
    torch.cuda.synchronize()
    for i, Y in out:
        assert np.array_equal(f64(Y), cases[i][3]), i


def test_prefill_split_in_graph_replays():
    """A split-K call captured in a HIP graph takes its own workspace (a
    memory node of the graph): replayed several times, with eager split-K
    calls and other eager work on the same stream between the replays, every
    replay and every eager call is exact."""
    values, bits, X, want = _split_case(4100, 4096, 256, 61)
    v2, b2, X2, want2 = _split_case(1000, 2048, 1024, 62)
    Y = torch.empty((256, 4100), device=DEV)
    native.nm_spmm_prefill(values, bits, X, out=Y)  # eager first: initialises everything
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        native.nm_spmm_prefill(values, bits, X, out=Y)
    for _ in range(3):
        Y.fill_(-1.0)
        Z = native.nm_spmm_prefill(v2, b2, X2)
        g.replay()
        Z2 = native.nm_spmm_prefill(v2, b2, X2)
        torch.cuda.synchronize()
        assert np.array_equal(f64(Y), want)
        assert np.array_equal(f64(Z), want2) and np.array_equal(f64(Z2), want2)
    del g


def test_prefill_zero_columns_and_empty_batch():
    values = torch.zeros((40, 0), dtype=torch.float16, device=DEV)
    bits = torch.zeros((40, 0), dtype=torch.int32, device=DEV)
    Y = torch.full((5, 40), 3.0, device=DEV)
    native.nm_spmm_prefill(values, bits, torch.zeros((5, 0), dtype=torch.float16, device=DEV), out=Y)
    assert torch.count_nonzero(Y).item() == 0
    W, keep, X = inputs(40, 64, 2, 4, "f16", 1, seed=5)
    v, b = gpu_pack(W, keep, 2, 4, "f16")
    Y0 = native.nm_spmm_prefill(v, b, torch.zeros((0, 64), dtype=torch.float16, device=DEV))
    assert Y0.shape == (0, 40)


def test_prefill_rejects_what_it_cannot_run():
    W, keep, X = inputs(32, 128, 4, 8, "f16", 4, seed=6)
    v, b = gpu_pack(W, keep, 4, 8, "f16")
    with pytest.raises(native.NMError):
        native.nm_spmm_prefill(v, b, t16(X, "f16"), 4, 8)
    W, keep, X = inputs(32, 96, 2, 4, "f16", 4, seed=7)
    v, b = gpu_pack(W, keep, 2, 4, "f16")
    with pytest.raises(native.NMError):
        native.nm_spmm_prefill(v, b, t16(X, "f16"))


# ---- the split reduction (k_split waves per row group) ----------------------

# K = 1024 c: a wave of a k_split group takes c / k_split chunks per lane per
# row, in load batches of 1 (2048, 14336), 2 (4096 at 4), 4 (8192 at 2) or
# 5 (10240 at 2) chunks per lane
SPLIT_SHAPES = [(96, 2048), (37, 4096), (130, 8192), (1, 4096), (64, 10240), (203, 14336),
                (50, 20480), (300, 4096)]


def _split_cfgs(cols):
    out = []
    for ks in (2, 4):
        if cols % (1024 * ks):
            continue
        for waves, rpw in ((ks, 1), (ks, 3), (2 * ks, 2), (4 * ks, 1), (16 // ks * ks, 4)):
            out.append(native.LaunchCfg(64 * waves, rpw, 0, VALU, ks))
    return out


@pytest.mark.parametrize("rows,cols", SPLIT_SHAPES)
def test_split_reduction_integer_exact(rows, cols):
    """2:4 at batch 1 with each row's load batches shared by 2 or 4 waves and
    their partial sums added through LDS: exact on integer inputs for every
    split, wave count and rows per wave, ragged row counts included."""
    W = synth.integer_weights(rows, cols, seed=81)
    keep = synth.random_mask(rows, cols, 2, 4, seed=82)
    xi = np.random.default_rng(83).integers(-4, 5, size=(1, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, "f16")
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    want = oracle.masked_gemv(W, keep, X, False)
    cfgs = _split_cfgs(cols)
    assert cfgs
    for cfg in cfgs:
        got = native.nm_resolve_launch(rows, cols, 1, 2, 4, cfg=cfg)
        assert got.k_split == cfg.k_split
        y = native.nm_spmv(values, bits, t16(X[0], "f16"), 2, 4, cfg=cfg)
        assert np.array_equal(f64(y), want[0]), cfg.as_tuple()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("rows,cols", [(203, 14336), (130, 8192), (300, 4096)])
def test_split_reduction_random(rows, cols, dtype):
    """Random weights and outlier activations: within rel-L2 1e-3 of the
    oracle, and the 16-bit output is the split launch's fp32 sum rounded."""
    W, keep, X = inputs(rows, cols, 2, 4, dtype, 1, seed=91)
    values, bits = gpu_pack(W, keep, 2, 4, dtype)
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16")
    for cfg in _split_cfgs(cols):
        y = native.nm_spmv(values, bits, t16(X[0], dtype), 2, 4, cfg=cfg)
        assert rel_l2(f64(y), want[0]) <= TOL, cfg.as_tuple()
        y16 = native.nm_spmv(values, bits, t16(X[0], dtype), 2, 4, out_dtype=TDT[dtype], cfg=cfg)
        assert np.array_equal(u16(y16), round16_f64(f64(y), dtype)), cfg.as_tuple()


def test_split_reduction_argument_rules():
    """k_split 2 or 4 only for 2:4 at batch 1 on the VALU row kernel with x
    whole in LDS, whole load batches per wave and a wave count it divides."""
    L = native.lib()
    c = native.LaunchCfg()

    def res(rows, cols, batch, n, m, cfg, dense=0):
        return L.nm_resolve_launch(rows, cols, batch, n, m, dense, ctypes.byref(cfg), ctypes.byref(c))

    ok = native.LaunchCfg(256, 2, 0, VALU, 2)
    assert res(512, 4096, 1, 2, 4, ok) == native.NM_OK and c.k_split == 2
    assert res(512, 4096, 1, 2, 4, native.LaunchCfg(256, 2, 0, VALU, 4)) == native.NM_OK
    assert res(512, 4096, 1, 2, 4, native.LaunchCfg(256, 2, 0, VALU, 3)) == native.NM_ERR_INVALID_ARG
    assert res(512, 4096, 1, 2, 4, native.LaunchCfg(256, 2, 0, VALU, -1)) == native.NM_ERR_INVALID_ARG
    assert res(512, 4096, 4, 2, 4, ok) == native.NM_ERR_UNSUPPORTED  # batch 4
    assert res(512, 4096, 1, 4, 8, ok) == native.NM_ERR_UNSUPPORTED  # 4:8
    assert res(512, 4096, 1, 1, 4, ok) == native.NM_ERR_UNSUPPORTED  # 1:4
    assert res(512, 3072, 1, 2, 4, native.LaunchCfg(256, 2, 0, VALU, 4)) == native.NM_ERR_UNSUPPORTED
    assert res(512, 4096, 1, 2, 4, native.LaunchCfg(192, 2, 0, VALU, 2)) == native.NM_ERR_UNSUPPORTED
    assert res(512, 4096, 1, 2, 4, native.LaunchCfg(256, 2, 1024, VALU, 2)) == native.NM_ERR_UNSUPPORTED
    assert res(512, 4096, 1, 2, 4, native.LaunchCfg(256, 2, 0, MFMA, 2)) == native.NM_ERR_UNSUPPORTED
    assert res(512, 4096, 1, 0, 0, ok, dense=1) == native.NM_ERR_UNSUPPORTED
    # the SwiGLU epilogue has no split form
    W = synth.weights(64, 2048, seed=3)
    keep = synth.topn_mask(W, 2, 4)
    values, bits = gpu_pack(W, keep, 2, 4, "f16")
    X = t16(synth.activations(1, 2048, seed=3), "f16")
    with pytest.raises(native.NMError) as e:
        native.nm_spmm_swiglu(values, bits, X, 2, 4, cfg=native.LaunchCfg(128, 2, 0, VALU, 2))
    assert e.value.status == native.NM_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("cols", [1024, 2080, 4096, 5120, 14336])
def test_4of8_plain_x_integer_exact_and_one_hot(cols, dtype):
    """4:8 at batch 1 takes x plainly in LDS with the per-byte pair selectors:
    exact on integer inputs (whole and ragged load batches), and a one-hot x
    picks out exactly the kept weight of that column in every row (the
    selector of each kept position, both 4-column windows of each byte)."""
    rows = 70
    W = synth.integer_weights(rows, cols, seed=111, dtype=dtype)
    keep = synth.random_mask(rows, cols, 4, 8, seed=112)
    xi = np.random.default_rng(113).integers(-4, 5, size=(1, cols)).astype(np.float32)
    X = synth.f32_to_16_bits(xi, dtype)
    values, bits = gpu_pack(W, keep, 4, 8, dtype)
    want = oracle.masked_gemv(W, keep, X, dtype == "bf16")
    for cfg in (None, (64, 1, 0, VALU), (256, 3, 0, VALU), (512, 2, 0, VALU)):
        y = native.nm_spmv(values, bits, t16(X[0], dtype), 4, 8, cfg=cfg)
        assert np.array_equal(f64(y), want[0]), cfg
    one = 0x3F80 if dtype == "bf16" else 0x3C00
    for j in (0, 3, 4, 7, 8, 13, cols - 1):
        xo = np.zeros((1, cols), dtype=np.uint16)
        xo[0, j] = one
        y = native.nm_spmv(values, bits, t16(xo[0], dtype), 4, 8)
        assert np.array_equal(f64(y), oracle.masked_gemv(W, keep, xo, dtype == "bf16")[0]), j
