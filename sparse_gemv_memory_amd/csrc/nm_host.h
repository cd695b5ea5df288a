// nm_host.h -- host-side helpers shared by the library's translation units:
// argument checks and the record of the last HIP error behind NM_ERR_HIP
// (read by nm_last_hip_error).  Defined in nm_sparse.hip; not exported from
// the shared library.

#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "nm_sparse.h"

#define NM_INTERNAL __attribute__((visibility("hidden")))

namespace nm_host {

// HIP error code of the last call that returned NM_ERR_HIP on this thread.
extern thread_local int g_last_hip NM_INTERNAL;

// Record e and return NM_ERR_HIP.
NM_INTERNAL nm_status hip_fail(hipError_t e);

// A 50% pattern the kernels are built for: N = M/2, M in {4, 8, 16, 32}.
NM_INTERNAL bool pattern_ok(int n, int m);

// Any N:M pattern the format holds: M in {4, 8, 16, 32}, 1 <= N < M (each
// aligned 32-bit mask word then holds exactly 32 N / M set bits).
NM_INTERNAL bool pattern_any_ok(int n, int m);

// The product for the patterns other than 50% (nm_generic.hip): launch
// shape (threads_per_wg, rows_per_wave, seg_cols; kernel NM_KERNEL_VALU), its
// check against the LDS budget, and the launch itself (arguments already
// checked by the caller).
NM_INTERNAL nm_status generic_default_cfg(int64_t rows, int64_t cols, int batch, int n, int m,
                                          int cus, size_t lds_budget, nm_launch_cfg *cfg);
NM_INTERNAL nm_status generic_check_cfg(const nm_launch_cfg &c, int batch, int n, int m,
                                        size_t lds_budget);
// Unstructured bitmasks (nm_generic.hip): window offsets, pack, product.
NM_INTERNAL nm_status bitmask_offsets(const uint8_t *keep, int64_t rows, int64_t cols,
                                      int64_t *offs, int64_t *total, void *stream);
NM_INTERNAL nm_status bitmask_pack(const uint16_t *W, const uint8_t *keep, int64_t rows,
                                   int64_t cols, const int64_t *offs, uint16_t *values,
                                   uint32_t *bits, void *stream);
NM_INTERNAL nm_status bitmask_launch(const void *values, const uint32_t *bits,
                                     const int64_t *offs, const void *X, void *Y, int batch,
                                     int64_t rows, int64_t cols, nm_dtype in_dt, nm_dtype out_dt,
                                     int cus, size_t lds_budget, void *stream);
NM_INTERNAL nm_status generic_launch(const void *values, const uint32_t *bits, const void *X,
                                     void *Y, int batch, int64_t rows, int64_t cols, int n, int m,
                                     nm_dtype in_dt, nm_dtype out_dt, const nm_launch_cfg &cfg,
                                     void *stream);

NM_INTERNAL bool is16(nm_dtype d);

// fp32 output, or the input's own 16-bit type.
NM_INTERNAL bool out_ok(nm_dtype in, nm_dtype out);

NM_INTERNAL bool aligned(const void *p, uintptr_t a);

}  // namespace nm_host
