"""N:M bitmask sparse GEMV for AMD Instinct MI355X (gfx950).

The product path is the HIP library ``libnm_sparse.so`` (C ABI in
``include/nm_sparse.h``); :mod:`.native` is its thin ctypes binding.
:mod:`.synth` draws seeded synthetic inputs and :mod:`.workloads` lists the
layer shapes.
"""

from .native import (  # noqa: F401
    NM_KERNEL_AUTO,
    NM_KERNEL_MFMA,
    NM_KERNEL_VALU,
    NMError,
    LaunchCfg,
    nm_default_launch,
    nm_dense_gemv,
    nm_hessian_accumulate,
    nm_pack,
    nm_select_nm,
    nm_packed_bytes,
    nm_spmm_small,
    nm_spmm_prefill,
    nm_spmm_swiglu,
    nm_spmv,
)
