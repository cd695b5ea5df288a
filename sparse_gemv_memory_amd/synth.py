"""Seeded synthetic inputs for N:M sparse GEMV workloads.

This module only draws inputs: weight matrices, N:M keep-masks and activation
vectors, as 16-bit bit patterns.  It holds none of the sparse product's
arithmetic (no packing, no products, no sums), so both the HIP path's tests
and the CPU oracle can take their inputs from it.

Recipe (numpy ``default_rng``, PCG64):

* weights: ``W = RNE16(0.02 * z)`` with ``z`` standard normal drawn in float32
  from ``default_rng(seed)``, shape (rows, cols);
* keep-mask: in each group of M consecutive columns of a row keep the N
  entries of largest magnitude, ties going to the lower column.  Magnitude is
  compared on the stored 16-bit pattern (sign bit cleared), which orders
  finite binary16 and bfloat16 values exactly like their absolute values;
* activations: ``x = RNE16(z)`` with ``z`` standard normal drawn in float32
  from ``default_rng(seed + 500)``, shape (batch, cols); with outliers,
  ``max(1, round(0.001 * cols))`` channels chosen without replacement (same
  channels for every batch row) are multiplied by 20 before rounding.

RNE16 is round-to-nearest-even from float32 to binary16 (numpy's cast) or to
bfloat16 (the integer rounding below).  The pruned weights the pages study
come from real checkpoints, which are not available here; these matrices have
the shapes of the Llama-3.1-8B, Llama-3.3-70B and Qwen3-32B linear layers the
pages evaluate and a top-N-of-M magnitude mask standing in for the solver's
mask.
"""

from __future__ import annotations

import numpy as np

F16 = "f16"
BF16 = "bf16"

W_STD = 0.02
X_SEED_OFFSET = 500
OUTLIER_FRACTION = 0.001
OUTLIER_SCALE = 20.0


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    out = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def f32_to_16_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def weights(rows: int, cols: int, seed: int, dtype: str = F16, std: float = W_STD) -> np.ndarray:
    """(rows, cols) uint16 bit patterns of N(0, std) weights."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    z *= np.float32(std)
    return f32_to_16_bits(z, dtype)


def topn_mask(w_bits: np.ndarray, n: int, m: int, chunk_rows: int = 4096) -> np.ndarray:
    """uint8 keep-mask: per group of m columns keep the n largest magnitudes.

    Ties go to the lower column: each entry gets the key
    ``magnitude * 32 + (31 - position_in_group)``, keys are distinct within a
    group, and the n largest keys are kept.
    """
    w = np.ascontiguousarray(w_bits).view(np.uint16)
    rows, cols = w.shape
    if m <= 0 or m > 32 or cols % m != 0 or not (0 <= n <= m):
        raise ValueError(f"bad pattern {n}:{m} for {cols} columns")
    keep = np.zeros((rows, cols), dtype=np.uint8)
    pos = (31 - np.arange(m, dtype=np.int32))
    for r0 in range(0, rows, chunk_rows):
        blk = w[r0:r0 + chunk_rows]
        mag = (blk & 0x7FFF).astype(np.int32).reshape(-1, m)
        key = (mag << 5) | pos
        if n == 0:
            k = np.zeros(key.shape, dtype=bool)
        else:
            thr = np.sort(key, axis=1)[:, m - n:m - n + 1]
            k = key >= thr
        keep[r0:r0 + chunk_rows] = k.reshape(blk.shape)
    return keep


def topk_row_mask(w_bits: np.ndarray, frac: float = 0.5) -> np.ndarray:
    """uint8 unstructured keep-mask: per row the round(frac * cols) largest
    magnitudes, ties to the lower column (key magnitude * 2**20 + (2**20 - 1
    - column), distinct within a row for cols <= 2**20)."""
    w = np.ascontiguousarray(w_bits).view(np.uint16)
    rows, cols = w.shape
    k = int(round(frac * cols))
    if cols > (1 << 20) or not (0 <= k <= cols):
        raise ValueError("bad shape or fraction")
    keep = np.zeros((rows, cols), dtype=np.uint8)
    if k == 0:
        return keep
    key = ((w & 0x7FFF).astype(np.int64) << 20) | ((1 << 20) - 1 - np.arange(cols, dtype=np.int64))
    idx = np.argpartition(-key, k - 1, axis=1)[:, :k]
    np.put_along_axis(keep, idx, 1, axis=1)
    return keep


def activations(batch: int, cols: int, seed: int, dtype: str = F16,
                outliers: bool = True) -> np.ndarray:
    """(batch, cols) uint16 bit patterns of N(0, 1) activations."""
    rng = np.random.default_rng(seed + X_SEED_OFFSET)
    z = rng.standard_normal((batch, cols), dtype=np.float32)
    if outliers and cols > 0:
        n_out = max(1, int(round(OUTLIER_FRACTION * cols)))
        ch = rng.choice(cols, size=n_out, replace=False)
        z[:, ch] *= np.float32(OUTLIER_SCALE)
    return f32_to_16_bits(z, dtype)


def integer_weights(rows: int, cols: int, seed: int, dtype: str = F16, lo: int = -4,
                    hi: int = 4) -> np.ndarray:
    """Small integers in [lo, hi], exact in binary16 and bfloat16."""
    rng = np.random.default_rng(seed)
    z = rng.integers(lo, hi + 1, size=(rows, cols)).astype(np.float32)
    return f32_to_16_bits(z, dtype)


def random_mask(rows: int, cols: int, n: int, m: int, seed: int) -> np.ndarray:
    """A uniformly random valid N:M keep-mask (n of every m, positions random)."""
    rng = np.random.default_rng(seed)
    g = rng.random((rows * cols // m, m))
    order = np.argsort(g, axis=1, kind="stable")
    keep = np.zeros((rows * cols // m, m), dtype=np.uint8)
    np.put_along_axis(keep, order[:, :n], 1, axis=1)
    return keep.reshape(rows, cols)


def layer_seed(config: int, layer: int, matrix: int) -> int:
    """Seed of matrix ``matrix`` of layer ``layer`` in workload ``config``.

    Workload 1 (the single 4096x4096 matrix) uses seed 0.
    """
    if config == 1:
        return 0
    return 1_000_000 * config + 1_000 * layer + matrix
