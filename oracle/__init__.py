"""CPU oracle for N:M bitmask sparse GEMV -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP product path never imports,
links or executes it, and it shares no code with that path: the arithmetic
lives in ``nm_oracle.c`` (plain C, fp64), built with gcc, and this module only
marshals numpy arrays into it.

Functions and the passages they follow (SparseDecoding, arXiv 2610.12327):

* :func:`pack` / :func:`unpack` -- bitmask indexing with values in increasing
  column order ("Method", kernel subsection, item (1) "Bitmask indexing"), one
  bit at a time.
* :func:`count_bad_groups` -- the N:M constraint (N kept in each group of M
  consecutive weights; "Related work", N:M paragraph).
* :func:`masked_gemv` -- the dense product of the masked weights with x in
  fp64, which is what the sparse kernel computes exactly up to rounding
  ("Method", "Decoding is dominated by SpMV operations").
* :func:`decode16` -- binary16 / bfloat16 bit patterns to float64 from the
  format definitions.
* :func:`hessian` -- H = scale * X X^T over the first ntok columns of a
  feature-major X (column t = the layer's input at decode step t): the
  Hessian H = 2 X X^T of the layer-wise objective ("Method", OBS paragraph
  and the decode-time calibration paragraph), a plain triple loop in fp64.
* :func:`select_nm` -- the N:M mask-selection step: in each group of M keep
  the N weights of largest w^2 * s[c], s = diag(H) for the |w| * ||x_c|| order
  of the Wanda backend or s = 1 / diag(H^-1) for the OBS saliency of one weight
  ("Method", OBS paragraph; "Experiments" setup naming SparseGPT and Wanda),
  chosen greedily one largest score at a time, scores in fp32.
* :func:`silu_mul` / :func:`swiglu_gemv` -- silu(gate) * up on the masked
  products of a row-interleaved gate/up matrix, the MLP step of the Llama and
  Qwen decoder layers whose end-to-end decoding the pages time ("Experiments",
  Table 3 paragraph; the layer itself is those models' published
  architecture, not spelled out on the pages).

Every function here is pinned in ``tests/test_oracle_pins.py`` against facts
that do not come from this code (library routines, closed forms, brute force,
exhaustive enumeration, the worked bit-count example printed on the pages).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nm_oracle.c")
_LIB = os.path.join(_HERE, "libnm_oracle.so")
# A build of nm_oracle.c to load instead (the sanitizer test runs the pins
# against an AddressSanitizer / UBSan build this way); unset: _LIB.
_LIB_OVERRIDE = os.environ.get("NM_ORACLE_LIB")

OK = 0
ERR_UNSUPPORTED = -2
ERR_SHAPE = -3
ERR_MASK = -5

_lib = None


def build() -> str:
    """Compile nm_oracle.c with gcc into libnm_oracle.so (always rebuilds)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.oracle_decode16.argtypes = [p, i64, ci, p]
    lib.oracle_decode16.restype = None
    lib.oracle_pattern_supported.argtypes = [ci, ci]
    lib.oracle_pattern_supported.restype = ci
    lib.oracle_count_bad_groups.argtypes = [p, i64, i64, ci, ci]
    lib.oracle_count_bad_groups.restype = i64
    lib.oracle_pack.argtypes = [p, p, i64, i64, ci, ci, p, p]
    lib.oracle_pack.restype = ci
    lib.oracle_unpack.argtypes = [p, p, i64, i64, ci, ci, p, p]
    lib.oracle_unpack.restype = ci
    lib.oracle_bitmask_row_ptr.argtypes = [p, i64, i64, p]
    lib.oracle_bitmask_row_ptr.restype = None
    lib.oracle_pack_bitmask.argtypes = [p, p, i64, i64, p, p, p]
    lib.oracle_pack_bitmask.restype = ci
    lib.oracle_unpack_bitmask.argtypes = [p, p, p, i64, i64, p, p]
    lib.oracle_unpack_bitmask.restype = ci
    lib.oracle_masked_gemv_f64.argtypes = [p, p, ci, p, ci, i64, i64, p, i64, ci, p]
    lib.oracle_masked_gemv_f64.restype = None
    lib.oracle_silu_mul_f64.argtypes = [p, p, i64, p]
    lib.oracle_silu_mul_f64.restype = None
    lib.oracle_hessian_f64.argtypes = [p, ci, i64, i64, i64, ctypes.c_double, ci, p]
    lib.oracle_hessian_f64.restype = None
    lib.oracle_select_nm.argtypes = [p, ci, p, i64, i64, i64, ci, ci, p]
    lib.oracle_select_nm.restype = ci
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _bits16(a) -> np.ndarray:
    """View a float16 / uint16 / int16 array as contiguous uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype.itemsize != 2:
        raise TypeError(f"expected a 16-bit array, got {a.dtype}")
    return a.view(np.uint16)


def _keep_u8(keep) -> np.ndarray:
    return np.ascontiguousarray(keep).astype(np.uint8, copy=False)


def decode16(bits, is_bf16: bool) -> np.ndarray:
    """float64 values of binary16 (is_bf16=False) or bfloat16 bit patterns."""
    b = _bits16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode16(_ptr(b), b.size, int(bool(is_bf16)), _ptr(out))
    return out


def pattern_supported(n: int, m: int) -> bool:
    return bool(_load().oracle_pattern_supported(n, m))


def count_bad_groups(keep, n: int, m: int) -> int:
    k = _keep_u8(keep)
    rows, cols = k.shape
    return int(_load().oracle_count_bad_groups(_ptr(k), rows, cols, n, m))


def pack(W, keep, n: int, m: int):
    """Return (status, values uint16[rows, cols*n/m], bits uint32[rows, cols/32])."""
    w = _bits16(W)
    k = _keep_u8(keep)
    rows, cols = w.shape
    if k.shape != w.shape:
        raise ValueError("W and keep must have the same shape")
    vcols = cols * n // m if m else 0
    values = np.zeros((rows, max(vcols, 0)), dtype=np.uint16)
    bits = np.zeros((rows, cols // 32), dtype=np.uint32)
    st = _load().oracle_pack(_ptr(w), _ptr(k), rows, cols, n, m, _ptr(values), _ptr(bits))
    return st, values, bits


def unpack(values, bits, cols: int, n: int, m: int):
    """Return (status, W uint16[rows, cols], keep uint8[rows, cols])."""
    v = _bits16(values)
    b = np.ascontiguousarray(bits, dtype=np.uint32)
    rows = b.shape[0]
    W = np.zeros((rows, cols), dtype=np.uint16)
    keep = np.zeros((rows, cols), dtype=np.uint8)
    st = _load().oracle_unpack(_ptr(v), _ptr(b), rows, cols, n, m, _ptr(W), _ptr(keep))
    return st, W, keep


def pack_bitmask(W, keep):
    """Unstructured bitmask pack of any keep-mask.  Returns (status, values
    uint16[row_ptr[-1]], bits uint32[rows, cols/32], row_ptr int64[rows+1])."""
    w = _bits16(W)
    k = _keep_u8(keep)
    rows, cols = w.shape
    if k.shape != w.shape:
        raise ValueError("W and keep must have the same shape")
    row_ptr = np.zeros(rows + 1, dtype=np.int64)
    _load().oracle_bitmask_row_ptr(_ptr(k), rows, cols, _ptr(row_ptr))
    values = np.zeros(int(row_ptr[-1]), dtype=np.uint16)
    bits = np.zeros((rows, cols // 32), dtype=np.uint32)
    st = _load().oracle_pack_bitmask(_ptr(w), _ptr(k), rows, cols, _ptr(row_ptr), _ptr(values),
                                     _ptr(bits))
    return st, values, bits, row_ptr


def unpack_bitmask(values, bits, row_ptr, cols: int):
    """Return (status, W uint16[rows, cols], keep uint8[rows, cols])."""
    v = _bits16(values)
    b = np.ascontiguousarray(bits, dtype=np.uint32)
    rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
    rows = b.shape[0]
    W = np.zeros((rows, cols), dtype=np.uint16)
    keep = np.zeros((rows, cols), dtype=np.uint8)
    st = _load().oracle_unpack_bitmask(_ptr(v), _ptr(b), _ptr(rp), rows, cols, _ptr(W), _ptr(keep))
    return st, W, keep


def masked_gemv(W, keep, x, is_bf16: bool, rows_idx=None, threads: int = 1) -> np.ndarray:
    """fp64 y[b, i] = sum_c keep[r, c] * W[r, c] * x[b, c] for r = rows_idx[i].

    ``keep=None`` gives the dense product.  x is (batch, cols) or (cols,);
    the result is (batch, nrows) float64 (or (nrows,) for 1-D x).
    """
    w = _bits16(W)
    rows, cols = w.shape
    xb = _bits16(x)
    squeeze = xb.ndim == 1
    if squeeze:
        xb = xb.reshape(1, -1)
    if xb.shape[1] != cols:
        raise ValueError("x length must equal the number of columns")
    batch = xb.shape[0]
    if rows_idx is None:
        idx = None
        nrows = rows
    else:
        idx = np.ascontiguousarray(rows_idx, dtype=np.int64)
        if idx.size and (idx.min() < 0 or idx.max() >= rows):
            raise IndexError("row index out of range")
        nrows = idx.size
    k = None if keep is None else _keep_u8(keep)
    if k is not None and k.shape != w.shape:
        raise ValueError("W and keep must have the same shape")
    y = np.zeros((batch, nrows), dtype=np.float64)
    _load().oracle_masked_gemv_f64(
        _ptr(w), None if k is None else _ptr(k), int(bool(is_bf16)), _ptr(xb), batch,
        rows, cols, None if idx is None else _ptr(idx), nrows, int(threads), _ptr(y))
    return y[0] if squeeze else y


def silu_mul(g, u) -> np.ndarray:
    """fp64 h = silu(g) * u elementwise, silu(z) = z / (1 + exp(-z))."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    if g.shape != u.shape:
        raise ValueError("g and u must have the same shape")
    h = np.empty_like(g)
    _load().oracle_silu_mul_f64(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def swiglu_gemv(W, keep, x, is_bf16: bool, threads: int = 1) -> np.ndarray:
    """fp64 h[b, r] = silu(g[b, r]) * u[b, r] where g and u are the masked
    products of rows 2r (gate) and 2r + 1 (up) of the row-interleaved W."""
    w = _bits16(W)
    if w.shape[0] % 2:
        raise ValueError("W must hold (gate, up) row pairs")
    y = masked_gemv(W, keep, x, is_bf16, threads=threads)
    return silu_mul(y[..., 0::2], y[..., 1::2])


def hessian(X, ntok=None, scale: float = 2.0, is_bf16: bool = False, threads: int = 1) -> np.ndarray:
    """fp64 H[i, j] = scale * sum_{t < ntok} X[i, t] X[j, t] for the d x ld
    16-bit pattern array X (feature-major)."""
    xb = _bits16(X)
    if xb.ndim != 2:
        raise ValueError("X must be 2-D (d, ld)")
    d, ld = xb.shape
    ntok = ld if ntok is None else int(ntok)
    if not 0 <= ntok <= ld:
        raise ValueError("ntok must be in [0, ld]")
    H = np.zeros((d, d), dtype=np.float64)
    _load().oracle_hessian_f64(_ptr(xb), int(bool(is_bf16)), d, ntok, ld, float(scale),
                               int(threads), _ptr(H))
    return H


def select_nm(W, colw, n: int, m: int, is_bf16: bool, cstride: int = 1) -> np.ndarray:
    """uint8 keep-mask of the rows x cols 16-bit W: in each group of m columns
    the n of largest fp32 score (w * w) * s[c], s[c] = colw.flat[c * cstride],
    ties to the lower column, NaN scores as -inf."""
    w = _bits16(W)
    if w.ndim != 2:
        raise ValueError("W must be 2-D")
    rows, cols = w.shape
    cw = np.ascontiguousarray(colw, dtype=np.float32).ravel()
    if cols and cw.size < (cols - 1) * cstride + 1:
        raise ValueError("colw too short for cols and cstride")
    keep = np.zeros((rows, cols), dtype=np.uint8)
    st = _load().oracle_select_nm(_ptr(w), int(bool(is_bf16)), _ptr(cw), int(cstride), rows, cols,
                                  int(n), int(m), _ptr(keep))
    if st == ERR_UNSUPPORTED:
        raise ValueError(f"pattern {n}:{m} not supported")
    if st == ERR_SHAPE:
        raise ValueError("cols must be a multiple of m")
    return keep
