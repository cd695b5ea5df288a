"""nm_pack_noalloc, the allocation-free pack, against nm_pack through the C
ABI: bit-identical values and bits on two calls in a row, the second with a
smaller matrix (the shared device counter must not carry over), the same
NM_ERR_MASK status for an invalid mask, and NM_OK again on the call after
one that failed.  Runs alone in a fresh process and after the other tests."""

import ctypes

import numpy as np
import pytest
import torch

from sparse_gemv_memory_amd import native, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def t16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).to(DEV)


def raw_pack(fn, W, keep, n, m, values, bits):
    L = native.lib()
    rows, cols = W.shape
    st = getattr(L, fn)(W.data_ptr(), keep.data_ptr(), rows, cols, n, m, native.NM_F16,
                        values.data_ptr(), bits.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st


def buffers(rows, cols, n, m):
    vb, bb = native.nm_packed_bytes(rows, cols, n, m)
    # filled with a pattern so that unwritten bytes would show
    return (torch.full((vb // 2,), 0x5A5A, dtype=torch.int16, device=DEV).view(torch.float16),
            torch.full((bb // 4,), 0x33, dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (16, 32), (3, 8)])
def test_noalloc_pack_matches_nm_pack_twice(n, m):
    for rows, cols, seed in ((300, 4160, 1), (37, 256, 2)):  # the second call smaller
        W = synth.weights(rows, cols, seed=seed)
        keep = torch.from_numpy(synth.topn_mask(W, n, m)).to(DEV)
        Wd = t16(W)
        va, ba = buffers(rows, cols, n, m)
        vb, bb = buffers(rows, cols, n, m)
        assert raw_pack("nm_pack", Wd, keep, n, m, va, ba) == native.NM_OK
        assert raw_pack("nm_pack_noalloc", Wd, keep, n, m, vb, bb) == native.NM_OK
        assert torch.equal(va.view(torch.int16), vb.view(torch.int16))
        assert torch.equal(ba, bb)


def test_noalloc_pack_reports_and_clears_invalid_groups():
    rows, cols, n, m = 64, 512, 2, 4
    W = synth.weights(rows, cols, seed=5)
    good = synth.topn_mask(W, n, m)
    bad = good.copy()
    bad[7, 8:12] = 1  # one group keeps 4 of 4
    Wd = t16(W)
    v, b = buffers(rows, cols, n, m)
    assert raw_pack("nm_pack", Wd, torch.from_numpy(bad).to(DEV), n, m, v, b) == native.NM_ERR_MASK
    assert raw_pack("nm_pack_noalloc", Wd, torch.from_numpy(bad).to(DEV), n, m, v, b) == native.NM_ERR_MASK
    # the next call starts from a cleared counter
    va, ba = buffers(rows, cols, n, m)
    assert raw_pack("nm_pack_noalloc", Wd, torch.from_numpy(good).to(DEV), n, m, v, b) == native.NM_OK
    assert raw_pack("nm_pack", Wd, torch.from_numpy(good).to(DEV), n, m, va, ba) == native.NM_OK
    assert torch.equal(va.view(torch.int16), v.view(torch.int16)) and torch.equal(ba, b)


def test_noalloc_pack_binding_and_host_checks():
    W = synth.weights(32, 128, seed=9)
    keep = torch.from_numpy(synth.topn_mask(W, 2, 4)).to(DEV)
    v, b = buffers(32, 128, 2, 4)
    native.nm_pack_noalloc(t16(W), keep, 2, 4, v, b)
    ref_v, ref_b = native.nm_pack(t16(W), keep, 2, 4)
    assert torch.equal(ref_v.view(torch.int16).reshape(-1), v.view(torch.int16)[:ref_v.numel()])
    assert torch.equal(ref_b.reshape(-1), b)
    L = native.lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.nm_pack_noalloc(None, None, 1 << 31, 32, 2, 4, native.NM_F16, None, None, s) == \
        native.NM_ERR_INVALID_ARG
    assert L.nm_pack_noalloc(None, None, 0, 32, 2, 4, native.NM_F16, None, None, s) == native.NM_OK
