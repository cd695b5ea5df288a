"""The C ABI without a GPU: the library loads, exports every function declared
in include/*.h, and rejects bad arguments on the host before any HIP call.

Fake device addresses are passed where a pointer is needed: a rejected call
never dereferences or launches anything, and rows == 0 returns NM_OK without
touching the device.
"""

import ctypes
import glob
import os
import re

import pytest

from sparse_gemv_memory_amd import build as nbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INV, UNSUP, SHAPE, ALIGN = 0, -1, -2, -3, -4
F16, BF16, F32 = 0, 1, 2

P = 0x7F0000000000  # a 256-byte aligned fake address, never dereferenced


@pytest.fixture(scope="session")
def L():
    from sparse_gemv_memory_amd import native
    # NM_CAPI_LIB: another build of the same sources to check instead (the
    # sanitizer test points it at a host-side AddressSanitizer / UBSan build)
    other = os.environ.get("NM_CAPI_LIB")
    if other:
        return native.declare(ctypes.CDLL(other))
    if not os.path.exists(nbuild.LIB):
        nbuild.build()
    return native.lib()


def _declared():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(nm_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("nm_packed_bytes", "nm_pack", "nm_spmv", "nm_spmm_small", "nm_dense_gemv",
              "nm_status_string", "nm_spmm_swiglu", "nm_hessian_accumulate", "nm_select_nm",
              "nm_spmm_prefill"):
        assert n in names


def test_library_exports_every_declared_function(L):
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert missing == []


def test_binding_declares_every_argument_type(L):
    # an undeclared ctypes function masks Python ints to 32 bits, which would
    # turn a 64-bit device address into a wild pointer
    undeclared = [n for n in _declared() if getattr(L, n).argtypes is None]
    assert undeclared == []


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert L.nm_status_string(s).decode().startswith("NM_")
    assert L.nm_status_string(123).decode() == "unknown nm_status"
    assert L.nm_last_hip_error() == 0


def _pb(L, rows, cols, n, m, dt=F16):
    vb, bb = ctypes.c_size_t(), ctypes.c_size_t()
    st = L.nm_packed_bytes(rows, cols, n, m, dt, ctypes.byref(vb), ctypes.byref(bb))
    return st, vb.value, bb.value


def test_packed_bytes_closed_form(L):
    # K*N/M values and K/32 words per row; the same bytes for every 50% pattern
    for n, m in ((2, 4), (4, 8), (8, 16), (16, 32)):
        assert _pb(L, 14336, 4096, n, m) == (OK, 14336 * 4096, 14336 * 4096 // 8)
    assert _pb(L, 0, 4096, 2, 4) == (OK, 0, 0)
    assert _pb(L, 3, 0, 2, 4, BF16) == (OK, 0, 0)
    assert _pb(L, 4, 48, 2, 4)[0] == SHAPE
    # other densities: K*N/M values per row, the total rounded up to 16 bytes
    assert _pb(L, 14336, 4096, 1, 4) == (OK, 14336 * 4096 // 2, 14336 * 4096 // 8)
    assert _pb(L, 14336, 4096, 3, 4) == (OK, 14336 * 4096 * 3 // 2, 14336 * 4096 // 8)
    assert _pb(L, 1, 32, 1, 32) == (OK, 16, 4)  # 2 bytes of values, padded
    assert _pb(L, 3, 64, 5, 16) == (OK, 128, 24)  # 3 * 20 values = 120 bytes -> 128
    for n, m in ((0, 4), (4, 4), (3, 6), (2, 64), (-1, 4)):
        assert _pb(L, 4, 64, n, m)[0] == UNSUP
    assert _pb(L, 4, 64, 2, 4, F32)[0] == UNSUP
    assert _pb(L, -1, 64, 2, 4)[0] == INV
    assert L.nm_packed_bytes(1, 32, 2, 4, F16, None, None) == INV


def _spmv(L, values=P, bits=P, x=P, y=P, rows=8, cols=64, n=2, m=4, i=F16, o=F32):
    return L.nm_spmv(values, bits, x, y, rows, cols, n, m, i, o, None)


def test_spmv_rejects_bad_arguments(L):
    assert _spmv(L, rows=-1) == INV
    assert _spmv(L, cols=-32) == INV
    assert _spmv(L, cols=48) == SHAPE
    assert _spmv(L, cols=2 ** 31) == INV
    assert _spmv(L, n=3, m=6) == UNSUP
    assert _spmv(L, n=0, m=4) == UNSUP
    assert _spmv(L, n=32, m=64) == UNSUP
    assert _spmv(L, n=4, m=4) == UNSUP
    assert _spmv(L, i=F32) == UNSUP
    assert _spmv(L, i=F16, o=BF16) == UNSUP
    assert _spmv(L, values=None) == INV
    assert _spmv(L, bits=None) == INV
    assert _spmv(L, x=None) == INV
    assert _spmv(L, y=None) == INV
    assert _spmv(L, values=P + 8) == ALIGN
    assert _spmv(L, bits=P + 2) == ALIGN
    assert _spmv(L, x=P + 4) == ALIGN
    assert _spmv(L, y=P + 2, o=F32) == ALIGN
    assert _spmv(L, y=P + 1, o=F16) == ALIGN


def test_empty_calls_do_nothing(L):
    # rows == 0: nothing to compute, no device work, NULL pointers allowed
    assert _spmv(L, values=None, bits=None, x=P, y=None, rows=0) == OK
    assert _spmv(L, values=None, bits=None, x=None, y=None, rows=0, cols=0) == OK
    assert _spmv(L, values=None, bits=None, x=None, y=None, rows=0) == INV  # x has cols elements
    assert L.nm_spmm_small(None, None, P, None, 4, 0, 64, 2, 4, F16, F32, None) == OK
    assert L.nm_dense_gemv(None, P, None, 8, 0, 64, BF16, F32, None) == OK
    assert L.nm_pack(None, None, 0, 64, 2, 4, F16, None, None, None) == OK
    assert L.nm_pack(None, None, 5, 0, 2, 4, F16, None, None, None) == OK


def test_spmm_small_batch_range(L):
    for b in (0, 9, -1):
        assert L.nm_spmm_small(P, P, P, P, b, 8, 64, 2, 4, F16, F32, None) == INV
    assert L.nm_spmm_small(P, P, P, P, 2, 8, 96 + 8, 2, 4, F16, F32, None) == SHAPE


def _swiglu(L, values=P, bits=P, x=P, h=P, batch=1, inter=4, cols=64, n=2, m=4, i=F16, o=F32):
    return L.nm_spmm_swiglu(values, bits, x, h, batch, inter, cols, n, m, i, o, None)


def test_swiglu_rejects_bad_arguments(L):
    assert _swiglu(L, inter=-1) == INV
    assert _swiglu(L, inter=2 ** 30) == INV  # 2 * inter rows exceed INT32_MAX
    assert _swiglu(L, batch=0) == INV
    assert _swiglu(L, batch=9) == INV
    assert _swiglu(L, cols=48) == SHAPE
    assert _swiglu(L, n=1, m=4) == UNSUP
    assert _swiglu(L, i=F16, o=BF16) == UNSUP
    assert _swiglu(L, values=None) == INV
    assert _swiglu(L, h=None) == INV
    assert _swiglu(L, x=P + 4) == ALIGN
    assert _swiglu(L, h=P + 2) == ALIGN
    assert _swiglu(L, values=None, bits=None, h=None, inter=0) == OK  # nothing to compute


def test_hessian_rejects_bad_arguments(L):
    def h(H=P, X=P, d=64, ntok=16, ld=16, i=F16):
        return L.nm_hessian_accumulate(H, X, d, ntok, ld, i, 2.0, None)
    assert h(d=-1) == INV
    assert h(ntok=-1) == INV
    assert h(ntok=24, ld=16) == INV  # ld < ntok
    assert h(d=23171) == INV
    assert h(ld=12, ntok=12) == SHAPE
    assert h(i=F32) == UNSUP
    assert h(H=None) == INV
    assert h(X=None) == INV
    assert h(H=P + 2) == ALIGN
    assert h(X=P + 8) == ALIGN
    assert h(H=None, X=None, d=0) == OK  # nothing to do
    assert h(X=None, ntok=0) == OK


def test_prefill_rejects_bad_arguments(L):
    def pf(v=P, b=P, x=P, y=P, batch=16, rows=64, cols=128, n=2, m=4, i=F16, o=F32):
        return L.nm_spmm_prefill(v, b, x, y, batch, rows, cols, n, m, i, o, None)
    assert pf(batch=-1) == INV
    assert pf(rows=-1) == INV
    assert pf(n=4, m=8) == UNSUP  # the sparse instruction is 2:4
    assert pf(n=1) == UNSUP
    assert pf(i=F32) == UNSUP
    assert pf(o=BF16) == UNSUP  # f16 input, bf16 output
    assert pf(cols=96) == SHAPE
    assert pf(rows=1 << 20, cols=1 << 12) == INV  # rows * cols > INT32_MAX
    assert pf(batch=1 << 20, cols=1 << 11) == INV  # batch * cols * 2 > INT32_MAX
    # sizes whose products wrap int64 are rejected before any multiplication
    assert pf(rows=(1 << 35) + 3, cols=1 << 29) == INV
    assert pf(batch=(1 << 40) + 1, cols=1 << 24) == INV
    assert pf(batch=1, rows=1, cols=(1 << 40)) == INV
    assert pf(y=None) == INV
    assert pf(v=None) == INV
    assert pf(x=P + 8) == ALIGN
    assert pf(v=P + 8) == ALIGN
    assert pf(y=P + 2) == ALIGN
    assert pf(batch=0, v=None, b=None, x=None, y=None) == OK
    assert pf(rows=0, v=None, b=None, x=None, y=None) == OK


def test_select_rejects_bad_arguments(L):
    def sel(W=P, c=P, cs=1, rows=4, cols=64, n=2, m=4, dt=F16, k=P):
        return L.nm_select_nm(W, c, cs, rows, cols, n, m, dt, k, None)
    assert sel(rows=-1) == INV
    assert sel(cols=-32) == INV
    assert sel(cs=0) == INV
    assert sel(cols=48) == SHAPE
    assert sel(n=1) == UNSUP
    assert sel(m=64, n=32) == UNSUP
    assert sel(dt=F32) == UNSUP
    assert sel(W=None) == INV
    assert sel(c=None) == INV
    assert sel(k=None) == INV
    assert sel(W=P + 1) == ALIGN
    assert sel(c=P + 2) == ALIGN
    assert sel(W=None, c=None, k=None, rows=0) == OK  # nothing to do
    assert sel(W=None, c=None, k=None, cols=0) == OK


def test_dense_rejects_bad_arguments(L):
    assert L.nm_dense_gemv(P, P, P, 0, 8, 64, F16, F32, None) == INV
    assert L.nm_dense_gemv(P, P, P, 9, 8, 64, F16, F32, None) == INV
    assert L.nm_dense_gemv(P, P, P, 1, 8, 40, F16, F32, None) == SHAPE
    assert L.nm_dense_gemv(P, P, P, 1, 8, 64, F32, F32, None) == UNSUP
    assert L.nm_dense_gemv(None, P, P, 1, 8, 64, F16, F32, None) == INV
    assert L.nm_dense_gemv(P + 2, P, P, 1, 8, 64, F16, F32, None) == ALIGN


def test_pack_rejects_bad_arguments(L):
    def pack(W=P, keep=P, rows=4, cols=64, n=2, m=4, dt=F16, v=P, b=P):
        return L.nm_pack(W, keep, rows, cols, n, m, dt, v, b, None)
    assert pack(rows=-1) == INV
    assert pack(cols=96 + 16) == SHAPE
    assert pack(n=2, m=6) == UNSUP
    assert pack(n=8, m=8) == UNSUP
    assert pack(dt=F32) == UNSUP
    assert pack(W=None) == INV
    assert pack(keep=None) == INV
    assert pack(v=None) == INV
    assert pack(b=None) == INV
    assert pack(W=P + 1) == ALIGN
    assert pack(v=P + 2) == ALIGN
    assert pack(b=P + 2) == ALIGN


def test_launch_cfg_validation_is_host_only(L):
    from sparse_gemv_memory_amd.native import LaunchCfg
    c = LaunchCfg()
    assert L.nm_default_launch(8, 48, 1, 2, 4, 0, ctypes.byref(c)) == SHAPE
    assert L.nm_default_launch(8, 64, 9, 2, 4, 0, ctypes.byref(c)) == INV
    assert L.nm_default_launch(8, 64, 1, 2, 4, 0, None) == INV
    assert L.nm_default_launch(8, 64, 1, 3, 6, 0, ctypes.byref(c)) == UNSUP
    assert L.nm_default_launch(8, 64, 1, 4, 4, 0, ctypes.byref(c)) == UNSUP


def test_bitmask_entry_points_reject_bad_arguments(L):
    total = ctypes.c_int64()
    off = L.nm_bitmask_offsets
    assert off(P, 4, 48, P, ctypes.byref(total), None) == SHAPE
    assert off(P, -1, 64, P, ctypes.byref(total), None) == INV
    assert off(P, 4, 64, None, ctypes.byref(total), None) == INV
    assert off(P, 4, 64, P + 4, ctypes.byref(total), None) == ALIGN
    pack = L.nm_pack_bitmask
    assert pack(P, P, 4, 48, F16, P, P, P, None) == SHAPE
    assert pack(P, P, 4, 64, F32, P, P, P, None) == UNSUP
    assert pack(None, P, 4, 64, F16, P, P, P, None) == INV
    assert pack(P, P, 4, 64, F16, P, P + 8, P, None) == ALIGN
    assert pack(None, None, 0, 64, F16, None, None, None, None) == OK
    spmm = L.nm_spmm_bitmask
    assert spmm(P, P, P, P, P, 0, 4, 64, F16, F32, None) == INV
    assert spmm(P, P, P, P, P, 9, 4, 64, F16, F32, None) == INV
    assert spmm(P, P, P, P, P, 1, 4, 48, F16, F32, None) == SHAPE
    assert spmm(P, P, P, P, P, 1, 4, 64, F32, F32, None) == UNSUP
    assert spmm(P, P, P, P, P, 1, 4, 64, F16, BF16, None) == UNSUP
    assert spmm(P, P, None, P, P, 1, 4, 64, F16, F32, None) == INV
    assert spmm(P, P, P + 4, P, P, 1, 4, 64, F16, F32, None) == ALIGN
    assert spmm(P + 8, P, P, P, P, 1, 4, 64, F16, F32, None) == ALIGN
    assert spmm(None, None, None, P, None, 1, 0, 64, F16, F32, None) == OK

