"""ctypes binding of libnm_sparse.so (the C ABI in include/nm_sparse.h).

Argument marshalling only: every step of the product runs in the HIP kernels
of the library.  PyTorch supplies device memory and the current HIP stream.
There is no fallback: if the library is not built, or a tensor is not on the
GPU, the call raises.

The functions carry the C names:

* :func:`nm_packed_bytes` -- packed buffer sizes;
* :func:`nm_pack` -- dense W + keep-mask -> (values, bits);
* :func:`nm_spmv` -- batch-1 sparse product;
* :func:`nm_spmm_small` -- batch 1..8 sparse product;
* :func:`nm_dense_gemv` -- dense comparison product;
* :func:`nm_default_launch` -- the launch shape the library would choose.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

from .build import LIB

NM_OK = 0
NM_ERR_INVALID_ARG = -1
NM_ERR_UNSUPPORTED = -2
NM_ERR_SHAPE = -3
NM_ERR_ALIGN = -4
NM_ERR_MASK = -5
NM_ERR_HIP = -6

NM_F16 = 0
NM_BF16 = 1
NM_F32 = 2

_DT = {torch.float16: NM_F16, torch.bfloat16: NM_BF16, torch.float32: NM_F32}


class NMError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {status_string(status)}"
        if status == NM_ERR_HIP:
            msg += f" (hipError {lib().nm_last_hip_error()})"
        super().__init__(msg)


NM_KERNEL_AUTO, NM_KERNEL_VALU, NM_KERNEL_MFMA = 0, 1, 2


class LaunchCfg(ctypes.Structure):
    """nm_launch_cfg: (threads_per_wg, rows_per_wave, seg_cols, kernel, k_split); 0 = library's choice."""
    _fields_ = [("threads_per_wg", ctypes.c_int), ("rows_per_wave", ctypes.c_int),
                ("seg_cols", ctypes.c_int), ("kernel", ctypes.c_int), ("k_split", ctypes.c_int)]

    def as_tuple(self):
        return (self.threads_per_wg, self.rows_per_wave, self.seg_cols, self.kernel, self.k_split)


_lib = None


def lib():
    """Load libnm_sparse.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run `python -m sparse_gemv_memory_amd.build` "
                           "or __graft_entry__.build() first")
    _lib = declare(ctypes.CDLL(LIB))
    return _lib


def declare(L):
    """Set the argument and result types of every entry point of a loaded
    libnm_sparse.so; returns L."""
    p, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.nm_status_string.argtypes = [ci]
    L.nm_status_string.restype = ctypes.c_char_p
    L.nm_last_hip_error.argtypes = []
    L.nm_last_hip_error.restype = ci
    L.nm_packed_bytes.argtypes = [i64, i64, ci, ci, ci, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.nm_packed_bytes.restype = ci
    L.nm_pack.argtypes = [p, p, i64, i64, ci, ci, ci, p, p, p]
    L.nm_pack.restype = ci
    L.nm_pack_noalloc.argtypes = [p, p, i64, i64, ci, ci, ci, p, p, p]
    L.nm_pack_noalloc.restype = ci
    L.nm_spmv.argtypes = [p, p, p, p, i64, i64, ci, ci, ci, ci, p]
    L.nm_spmv.restype = ci
    L.nm_spmm_small.argtypes = [p, p, p, p, ci, i64, i64, ci, ci, ci, ci, p]
    L.nm_spmm_small.restype = ci
    L.nm_spmm_small_cfg.argtypes = [p, p, p, p, ci, i64, i64, ci, ci, ci, ci,
                                    ctypes.POINTER(LaunchCfg), p]
    L.nm_spmm_small_cfg.restype = ci
    L.nm_spmm_swiglu.argtypes = [p, p, p, p, ci, i64, i64, ci, ci, ci, ci, p]
    L.nm_spmm_swiglu.restype = ci
    L.nm_spmm_swiglu_cfg.argtypes = [p, p, p, p, ci, i64, i64, ci, ci, ci, ci,
                                     ctypes.POINTER(LaunchCfg), p]
    L.nm_spmm_swiglu_cfg.restype = ci
    L.nm_spmm_prefill.argtypes = [p, p, p, p, i64, i64, i64, ci, ci, ci, ci, p]
    L.nm_spmm_prefill.restype = ci
    L.nm_hessian_accumulate.argtypes = [p, p, i64, i64, i64, ci, ctypes.c_float, p]
    L.nm_hessian_accumulate.restype = ci
    L.nm_select_nm.argtypes = [p, p, i64, i64, i64, ci, ci, ci, p, p]
    L.nm_select_nm.restype = ci
    L.nm_dense_gemv.argtypes = [p, p, p, ci, i64, i64, ci, ci, p]
    L.nm_dense_gemv.restype = ci
    L.nm_dense_gemv_cfg.argtypes = [p, p, p, ci, i64, i64, ci, ci, ctypes.POINTER(LaunchCfg), p]
    L.nm_dense_gemv_cfg.restype = ci
    L.nm_default_launch.argtypes = [i64, i64, ci, ci, ci, ci, ctypes.POINTER(LaunchCfg)]
    L.nm_default_launch.restype = ci
    L.nm_resolve_launch.argtypes = [i64, i64, ci, ci, ci, ci, ctypes.POINTER(LaunchCfg),
                                    ctypes.POINTER(LaunchCfg)]
    L.nm_resolve_launch.restype = ci
    L.nm_bitmask_offsets.argtypes = [p, i64, i64, p, ctypes.POINTER(i64), p]
    L.nm_bitmask_offsets.restype = ci
    L.nm_pack_bitmask.argtypes = [p, p, i64, i64, ci, p, p, p, p]
    L.nm_pack_bitmask.restype = ci
    L.nm_spmm_bitmask.argtypes = [p, p, p, p, p, ci, i64, i64, ci, ci, p]
    L.nm_spmm_bitmask.restype = ci
    L.nm_stream_read.argtypes = [p, sz, p, ci, ci, p]
    L.nm_stream_read.restype = ci
    return L


def status_string(status: int) -> str:
    return lib().nm_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != NM_OK:
        raise NMError(status, what)


def _dev(t: torch.Tensor, name: str) -> Optional[int]:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() or None


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _in_dt(t: torch.Tensor) -> int:
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")
    return _DT[t.dtype]


def _cfg_ptr(cfg):
    if cfg is None:
        return None
    c = LaunchCfg(*cfg) if not isinstance(cfg, LaunchCfg) else cfg
    return ctypes.byref(c)


def nm_packed_bytes(rows: int, cols: int, n: int, m: int, dtype=torch.float16) -> Tuple[int, int]:
    vb, bb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().nm_packed_bytes(rows, cols, n, m, _DT[dtype], ctypes.byref(vb), ctypes.byref(bb)),
           "nm_packed_bytes")
    return vb.value, bb.value


def nm_pack(W: torch.Tensor, keep: torch.Tensor, n: int, m: int):
    """Pack a (rows, cols) fp16/bf16 W and a same-shape keep-mask.

    Returns (values, bits): values (rows, cols*n/m) of W's dtype and bits
    (rows, cols/32) int32 holding the uint32 mask words.  Raises NMError with
    status NM_ERR_MASK if a group does not keep exactly n of m.
    """
    if W.dim() != 2 or keep.shape != W.shape:
        raise ValueError("W must be 2-D and keep must have its shape")
    if keep.dtype not in (torch.uint8, torch.bool, torch.int8):
        raise TypeError("keep must be uint8, int8 or bool")
    rows, cols = W.shape
    dt = _in_dt(W)
    vcols = cols * n // m if m > 0 and n >= 0 else 0  # the library validates n, m
    values = _packed_values(rows, vcols, _padded_elems(rows, cols, n, m, W.dtype), W.dtype, W.device)
    bits = torch.empty((rows, cols // 32), dtype=torch.int32, device=W.device)
    with torch.cuda.device(W.device):
        st = lib().nm_pack(_dev(W, "W"), _dev(keep, "keep"), rows, cols, n, m, dt,
                           _dev(values, "values"), _dev(bits, "bits"), _stream(W.device))
    _check(st, "nm_pack")
    return values, bits


def nm_pack_noalloc(W: torch.Tensor, keep: torch.Tensor, n: int, m: int, values: torch.Tensor,
                    bits: torch.Tensor):
    """nm_pack into caller-provided values and bits (as nm_pack returns
    them), with the library's static device counter instead of a per-call
    allocation."""
    if W.dim() != 2 or keep.shape != W.shape:
        raise ValueError("W must be 2-D and keep must have its shape")
    if keep.dtype not in (torch.uint8, torch.bool, torch.int8):
        raise TypeError("keep must be uint8, int8 or bool")
    rows, cols = W.shape
    if values.dtype != W.dtype or bits.dtype != torch.int32 or \
            values.numel() * 2 < _padded_elems(rows, cols, n, m, W.dtype) * 2 or \
            bits.numel() * 32 < rows * cols:
        raise ValueError("values / bits too small or of the wrong dtype")
    with torch.cuda.device(W.device):
        st = lib().nm_pack_noalloc(_dev(W, "W"), _dev(keep, "keep"), rows, cols, n, m, _in_dt(W),
                                   _dev(values, "values"), _dev(bits, "bits"), _stream(W.device))
    _check(st, "nm_pack_noalloc")
    return values, bits


def _padded_elems(rows: int, cols: int, n: int, m: int, dtype) -> int:
    """16-bit elements of nm_packed_bytes' values size (the row-major values
    rounded up to 16 bytes); 0 for a pattern the library rejects."""
    vb = ctypes.c_size_t()
    bb = ctypes.c_size_t()
    st = lib().nm_packed_bytes(rows, cols, n, m, _DT[dtype], ctypes.byref(vb), ctypes.byref(bb))
    return vb.value // 2 if st == NM_OK else 0


def _packed_values(rows: int, vcols: int, elems: int, dtype, device) -> torch.Tensor:
    """A (rows, vcols) tensor whose storage holds max(elems, rows * vcols)
    elements (the packed-size padding stays allocated behind the view)."""
    flat = torch.empty((max(elems, rows * vcols),), dtype=dtype, device=device)
    return flat[:rows * vcols].view(rows, vcols)


def clone_packed(values: torch.Tensor) -> torch.Tensor:
    """A copy of packed values that keeps nm_packed_bytes' padding (a plain
    clone() allocates only rows * cols*n/m elements)."""
    out = torch.empty((values.untyped_storage().nbytes() // 2 - values.storage_offset(),),
                      dtype=values.dtype, device=values.device)
    out[:values.numel()].copy_(values.reshape(-1))
    return out[:values.numel()].view(values.shape)


def _sparse_args(values, bits, X, n, m):
    if values.dim() != 2 or bits.dim() != 2 or values.shape[0] != bits.shape[0]:
        raise ValueError("values and bits must be 2-D with the same number of rows")
    if bits.dtype not in (torch.int32, torch.uint32):
        raise TypeError("bits must be int32 (uint32 mask words)")
    if values.dtype != X.dtype:
        raise TypeError("values and x must have the same dtype")
    rows = values.shape[0]
    cols = bits.shape[1] * 32
    if m <= 0 or n < 0 or values.shape[1] != cols * n // m:
        raise ValueError("values must hold cols*n/m elements per row")
    need = _padded_elems(rows, cols, n, m, values.dtype)
    have = values.untyped_storage().nbytes() // 2 - values.storage_offset()
    if values.is_contiguous() and have < need:
        raise ValueError("values must be allocated with nm_packed_bytes' size (nm_pack's "
                         "output, or clone_packed of it)")
    return rows, cols


def nm_spmv(values, bits, x, n: int, m: int, out_dtype=torch.float32, out=None, cfg=None):
    """y = W_sparse . x for one token; x has shape (cols,) or (1, cols)."""
    rows, cols = _sparse_args(values, bits, x, n, m)
    if x.numel() != cols:
        raise ValueError("x must have cols elements")
    y = out if out is not None else torch.empty((rows,), dtype=out_dtype, device=values.device)
    if y.numel() != rows or y.dtype != out_dtype:
        raise ValueError("out has the wrong shape or dtype")
    with torch.cuda.device(values.device):
        if cfg is None:
            st = lib().nm_spmv(_dev(values, "values"), _dev(bits, "bits"), _dev(x, "x"),
                               _dev(y, "y"), rows, cols, n, m, _in_dt(x), _DT[out_dtype],
                               _stream(values.device))
        else:
            st = lib().nm_spmm_small_cfg(_dev(values, "values"), _dev(bits, "bits"), _dev(x, "x"),
                                         _dev(y, "y"), 1, rows, cols, n, m, _in_dt(x),
                                         _DT[out_dtype], _cfg_ptr(cfg), _stream(values.device))
    _check(st, "nm_spmv")
    return y


def nm_spmm_small(values, bits, X, n: int, m: int, out_dtype=torch.float32, out=None, cfg=None):
    """Y = X . W_sparse^T for X of shape (batch, cols), 1 <= batch <= 8."""
    rows, cols = _sparse_args(values, bits, X, n, m)
    if X.dim() != 2 or X.shape[1] != cols:
        raise ValueError("X must be (batch, cols)")
    batch = X.shape[0]
    Y = out if out is not None else torch.empty((batch, rows), dtype=out_dtype, device=values.device)
    if tuple(Y.shape) != (batch, rows) or Y.dtype != out_dtype:
        raise ValueError("out has the wrong shape or dtype")
    with torch.cuda.device(values.device):
        st = lib().nm_spmm_small_cfg(_dev(values, "values"), _dev(bits, "bits"), _dev(X, "X"),
                                     _dev(Y, "Y"), batch, rows, cols, n, m, _in_dt(X),
                                     _DT[out_dtype], _cfg_ptr(cfg), _stream(values.device))
    _check(st, "nm_spmm_small")
    return Y


def nm_spmm_prefill(values, bits, X, n: int = 2, m: int = 4, out_dtype=torch.float32, out=None):
    """Y = X . W_sparse^T for X of shape (batch, cols), any batch (2:4 only),
    on the sparse matrix cores with a GEMM tiling."""
    rows, cols = _sparse_args(values, bits, X, n, m)
    if X.dim() != 2 or X.shape[1] != cols:
        raise ValueError("X must be (batch, cols)")
    batch = X.shape[0]
    Y = out if out is not None else torch.empty((batch, rows), dtype=out_dtype, device=values.device)
    if tuple(Y.shape) != (batch, rows) or Y.dtype != out_dtype:
        raise ValueError("out has the wrong shape or dtype")
    with torch.cuda.device(values.device):
        st = lib().nm_spmm_prefill(_dev(values, "values"), _dev(bits, "bits"), _dev(X, "X"),
                                   _dev(Y, "Y"), batch, rows, cols, n, m, _in_dt(X),
                                   _DT[out_dtype], _stream(values.device))
    _check(st, "nm_spmm_prefill")
    return Y


def nm_spmm_swiglu(values, bits, X, n: int, m: int, out_dtype=torch.float32, out=None, cfg=None):
    """H = silu(G) * U for X of shape (batch, cols), 1 <= batch <= 8, where the
    packed matrix interleaves gate row r (packed row 2r) and up row r (2r + 1);
    H has shape (batch, rows // 2)."""
    rows, cols = _sparse_args(values, bits, X, n, m)
    if rows % 2:
        raise ValueError("the packed matrix must hold (gate, up) row pairs")
    if X.dim() != 2 or X.shape[1] != cols:
        raise ValueError("X must be (batch, cols)")
    batch, inter = X.shape[0], rows // 2
    H = out if out is not None else torch.empty((batch, inter), dtype=out_dtype, device=values.device)
    if tuple(H.shape) != (batch, inter) or H.dtype != out_dtype:
        raise ValueError("out has the wrong shape or dtype")
    with torch.cuda.device(values.device):
        st = lib().nm_spmm_swiglu_cfg(_dev(values, "values"), _dev(bits, "bits"), _dev(X, "X"),
                                      _dev(H, "H"), batch, inter, cols, n, m, _in_dt(X),
                                      _DT[out_dtype], _cfg_ptr(cfg), _stream(values.device))
    _check(st, "nm_spmm_swiglu")
    return H


def nm_hessian_accumulate(H: torch.Tensor, X: torch.Tensor, ntok: Optional[int] = None,
                          scale: float = 2.0) -> torch.Tensor:
    """H += scale * X[:, :ntok] @ X[:, :ntok]^T in place (H: (d, d) fp32; X:
    (d, ld) fp16/bf16, feature-major: column t is one decode-step activation)."""
    if H.dtype != torch.float32 or H.dim() != 2 or H.shape[0] != H.shape[1]:
        raise ValueError("H must be a square float32 matrix")
    if X.dim() != 2 or X.shape[0] != H.shape[0]:
        raise ValueError("X must be (d, ld) with d = H's size")
    d, ld = X.shape
    ntok = ld if ntok is None else ntok
    with torch.cuda.device(H.device):
        st = lib().nm_hessian_accumulate(_dev(H, "H"), _dev(X, "X"), d, ntok, ld, _in_dt(X),
                                         float(scale), _stream(H.device))
    _check(st, "nm_hessian_accumulate")
    return H


def nm_select_nm(W: torch.Tensor, colw: torch.Tensor, n: int, m: int,
                 cstride: int = 1, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Keep-mask (rows, cols) uint8: in each m-group of each row the n columns
    with the largest fp32 score (W * W) * s, s[c] = colw.flatten()[c * cstride],
    ties to the lower column.  For a Hessian H (d x d, fp32) pass H and
    cstride = d + 1 to use its diagonal."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    rows, cols = W.shape
    if colw.dtype != torch.float32:
        raise TypeError("colw must be float32")
    if not colw.is_contiguous():
        raise ValueError("colw must be contiguous")
    if cols and colw.numel() < (cols - 1) * cstride + 1:
        raise ValueError("colw too short for cols and cstride")
    keep = out if out is not None else torch.empty((rows, cols), dtype=torch.uint8, device=W.device)
    if keep.shape != (rows, cols) or keep.dtype != torch.uint8:
        raise ValueError("out must be a (rows, cols) uint8 tensor")
    with torch.cuda.device(W.device):
        st = lib().nm_select_nm(_dev(W, "W"), _dev(colw, "colw"), cstride, rows, cols, n, m,
                                _in_dt(W), _dev(keep, "keep"), _stream(W.device))
    _check(st, "nm_select_nm")
    return keep


def nm_dense_gemv(W, X, out_dtype=torch.float32, out=None, cfg=None):
    """Y = X . W^T, dense, for X of shape (batch, cols) or (cols,)."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    rows, cols = W.shape
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    if X2.shape[1] != cols or W.dtype != X.dtype:
        raise ValueError("X must be (batch, cols) with W's dtype")
    batch = X2.shape[0]
    Y = out if out is not None else torch.empty((batch, rows), dtype=out_dtype, device=W.device)
    with torch.cuda.device(W.device):
        st = lib().nm_dense_gemv_cfg(_dev(W, "W"), _dev(X2, "X"), _dev(Y, "Y"), batch, rows, cols,
                                     _in_dt(W), _DT[out_dtype], _cfg_ptr(cfg), _stream(W.device))
    _check(st, "nm_dense_gemv")
    return Y.reshape(-1) if squeeze else Y


def nm_default_launch(rows: int, cols: int, batch: int, n: int = 2, m: int = 4,
                      dense: bool = False) -> LaunchCfg:
    c = LaunchCfg()
    _check(lib().nm_default_launch(rows, cols, batch, n, m, int(bool(dense)), ctypes.byref(c)),
           "nm_default_launch")
    return c


def nm_resolve_launch(rows: int, cols: int, batch: int, n: int = 2, m: int = 4,
                      dense: bool = False, cfg: Optional[LaunchCfg] = None) -> LaunchCfg:
    """The launch shape a _cfg call with overrides cfg would use."""
    c = LaunchCfg()
    _check(lib().nm_resolve_launch(rows, cols, batch, n, m, int(bool(dense)), _cfg_ptr(cfg),
                                   ctypes.byref(c)), "nm_resolve_launch")
    return c


def nm_stream_read(buf: torch.Tensor, out: torch.Tensor, grid: int = 512, threads_per_wg: int = 256,
                   nbytes: Optional[int] = None):
    """Read nbytes (default: all) of buf once with the calibration read kernel;
    out (int32 or uint32, at least grid * threads_per_wg / 64 elements)
    receives one word per wave."""
    nbytes = buf.numel() * buf.element_size() if nbytes is None else nbytes
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    if out.numel() * out.element_size() < 4 * grid * (threads_per_wg // 64):
        raise ValueError("out needs one 4-byte word per wave of the grid")
    with torch.cuda.device(buf.device):
        st = lib().nm_stream_read(_dev(buf, "buf"), nbytes, _dev(out, "out"), grid,
                                  threads_per_wg, _stream(buf.device))
    _check(st, "nm_stream_read")


def _vptr(values: torch.Tensor) -> Optional[int]:
    """Device address of packed values; an empty view (no kept weight) still
    passes its padded storage, which the library never reads as data."""
    if values.numel() == 0 and values.untyped_storage().nbytes() > 0:
        return values.untyped_storage().data_ptr()
    return _dev(values, "values")


def nm_pack_bitmask(W: torch.Tensor, keep: torch.Tensor):
    """Unstructured bitmask pack of a (rows, cols) fp16/bf16 W under any keep
    mask.  Returns (values, bits, offs): values 1-D of W's dtype (the kept
    weights, rows one after another; storage padded to 16 bytes), bits
    (rows, cols/32) int32, offs int64 (rows * ceil(cols/2048) + 1 window
    offsets)."""
    if W.dim() != 2 or keep.shape != W.shape:
        raise ValueError("W must be 2-D and keep must have its shape")
    if keep.dtype not in (torch.uint8, torch.bool, torch.int8):
        raise TypeError("keep must be uint8, int8 or bool")
    rows, cols = W.shape
    dt = _in_dt(W)
    nwr = (cols // 32 + 63) // 64
    offs = torch.empty((rows * nwr + 1,), dtype=torch.int64, device=W.device)
    total = ctypes.c_int64()
    with torch.cuda.device(W.device):
        _check(lib().nm_bitmask_offsets(_dev(keep, "keep"), rows, cols, _dev(offs, "offs"),
                                        ctypes.byref(total), _stream(W.device)), "nm_bitmask_offsets")
        n = total.value
        values = _packed_values(1, n, max(8, (n + 7) // 8 * 8), W.dtype, W.device).view(n)
        bits = torch.empty((rows, cols // 32), dtype=torch.int32, device=W.device)
        _check(lib().nm_pack_bitmask(_dev(W, "W"), _dev(keep, "keep"), rows, cols, dt,
                                     _dev(offs, "offs"), _vptr(values), _dev(bits, "bits"),
                                     _stream(W.device)), "nm_pack_bitmask")
    return values, bits, offs


def nm_spmm_bitmask(values, bits, offs, X, out_dtype=torch.float32, out=None):
    """Y = X . W^T for an unstructured bitmask matrix (nm_pack_bitmask's
    output); X of shape (batch, cols) with 1 <= batch <= 8, or (cols,)."""
    if bits.dim() != 2 or bits.dtype not in (torch.int32, torch.uint32):
        raise ValueError("bits must be (rows, cols/32) int32")
    rows, cols = bits.shape[0], bits.shape[1] * 32
    nwr = (cols // 32 + 63) // 64
    if offs.dtype != torch.int64 or offs.numel() != rows * nwr + 1:
        raise ValueError("offs must hold rows * ceil(cols/2048) + 1 int64 offsets")
    if values.dtype != X.dtype:
        raise TypeError("values and X must have the same dtype")
    have = values.untyped_storage().nbytes() // 2 - values.storage_offset()
    if values.numel() and have < (values.numel() + 7) // 8 * 8:
        raise ValueError("values must keep nm_pack_bitmask's 16-byte padding")
    squeeze = X.dim() == 1
    X2 = X.reshape(1, -1) if squeeze else X
    if X2.shape[1] != cols:
        raise ValueError("X must have cols columns")
    batch = X2.shape[0]
    Y = out if out is not None else torch.empty((batch, rows), dtype=out_dtype, device=X.device)
    with torch.cuda.device(X.device):
        st = lib().nm_spmm_bitmask(_vptr(values), _dev(bits, "bits"), _dev(offs, "offs"),
                                   _dev(X2, "X"), _dev(Y, "Y"), batch, rows, cols, _in_dt(X2),
                                   _DT[out_dtype], _stream(X.device))
    _check(st, "nm_spmm_bitmask")
    return Y.reshape(-1) if squeeze else Y

