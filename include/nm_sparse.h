/*
 * nm_sparse.h -- C ABI of the N:M bitmask sparse GEMV library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation: at decode time every pruned linear layer computes
 * y = W_sparse . x for one token (batch 1) or a few tokens (batch 2..8).
 * W keeps N of every M consecutive weights of a row (N:M semi-structured
 * sparsity) and is stored as
 *   - values: the kept weights of each row in increasing column order, and
 *   - bits:   one bit per column, 32 columns per 32-bit word, a set bit
 *             meaning "this column's weight is kept".
 * Passages that define it, in "SparseDecoding: Decoding-Aware Pruning for
 * Accurate and Efficient LLM Inference" (paper text):
 *   - Method, kernel subsection, opening paragraph: decoding is dominated by
 *     N:M SpMV at batch one and small batch;
 *   - same subsection, item (1) "Bitmask indexing": a row's mask has one
 *     bit per column and its kept weights are stored in column order, so the
 *     k-th set bit of the row names the column of its k-th stored value; at
 *     50% that costs 2 bits of metadata per kept weight;
 *   - same subsection, item (2) "Fixed-step bitmask traversal": under a 50%
 *     N:M pattern with M <= 32, a 32-bit mask word covers whole groups, so
 *     its count of set bits is always 16 and a per-word loop has a fixed
 *     trip count; each step takes the lowest set bit as the next kept column;
 *   - Appendix C (kernel implementation): one compiled kernel per N:M pattern,
 *     N and M fixed at compile time.
 *
 * Layout (shared by every entry point):
 *   - rows R = output features (d_out), cols K = input features (d_in);
 *     dense W is R x K row-major (leading dimension K);
 *   - N:M groups run along a row (along K); only the 50% patterns
 *     N = M/2, M in {4, 8, 16, 32} are supported;
 *   - K must be a multiple of 32 (hence of M);
 *   - values: R x (K/2) 16-bit elements, row-major, row stride K/2;
 *     the 16 kept values of word w of a row are values[r][16w .. 16w+15];
 *   - bits:   R x (K/32) uint32 words, row-major, row stride K/32;
 *     bit b (LSB = 0) of word w is column 32w + b;
 *   - x: batch x K row-major (one token per row); y: batch x R row-major,
 *     i.e. y = x . W_sparse^T, the convention of torch.nn.functional.linear.
 *
 * Ownership and streams: every pointer below is a device pointer the caller
 * allocated and owns; the library keeps no pointer after a call returns and
 * allocates no memory, except nm_pack (see there).  `stream` is a hipStream_t
 * passed as void* (NULL = the null stream); all device work of a call is
 * enqueued on it.  nm_spmv, nm_spmm_small and nm_dense_gemv return as soon as
 * the work is enqueued.
 *
 * Errors: every function returns an nm_status.  All argument checks run on
 * the host before any HIP call, so a call that returns NM_ERR_INVALID_ARG,
 * NM_ERR_UNSUPPORTED, NM_ERR_SHAPE or NM_ERR_ALIGN has done nothing on the
 * device.  NM_ERR_HIP means a HIP runtime call or a kernel launch failed
 * (nm_last_hip_error() gives the HIP error code).  A pointer may be NULL only
 * when the buffer it stands for holds zero bytes.
 */
#ifndef NM_SPARSE_H
#define NM_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NM_OK = 0,
  NM_ERR_INVALID_ARG = -1, /* NULL pointer, negative size, batch out of range */
  NM_ERR_UNSUPPORTED = -2, /* N:M pattern or dtype combination not supported */
  NM_ERR_SHAPE = -3,       /* K not a multiple of 32 */
  NM_ERR_ALIGN = -4,       /* a pointer is not aligned as required */
  NM_ERR_MASK = -5,        /* nm_pack: some M-group does not keep exactly N */
  NM_ERR_HIP = -6          /* HIP runtime or launch failure */
} nm_status;

typedef enum { NM_F16 = 0, NM_BF16 = 1, NM_F32 = 2 } nm_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *nm_status_string(int status);

/* HIP error code (hipError_t as int) of the last NM_ERR_HIP returned on the
 * calling thread, 0 if none. */
int nm_last_hip_error(void);

/* Patterns.  Every entry point taking n, m accepts the 50% patterns the
 * pages evaluate, N = M/2 with M in {4, 8, 16, 32} ("Experiments", Table 3
 * paragraph).  nm_packed_bytes, nm_pack, nm_spmv, nm_spmm_small(_cfg) and
 * nm_default_launch also accept any 0 < N < M with M in {4, 8, 16, 32}: every
 * aligned 32-bit mask word then holds exactly P = 32N/M set bits, so word w's
 * values start at w*P of the row and each word is walked in P fixed steps
 * (the fixed-count argument of Method item (2), which the pages make at 50%).
 * Those densities run on two generic kernels.  P = 4, 8, 12 and 24 (1:8, 1:4,
 * 3:8, 3:4, and 2:16, 6:16, 8:32, 24:32) take the direct kernel: each lane
 * loads whole mask words and their 2P value bytes straight into registers
 * with 8- or 16-byte loads.  Every other P takes the window kernel, which
 * copies the values of 64 mask words at a time into LDS with 16-byte loads.
 * Both read whole 16-byte chunks of values, so the last one may reach into
 * the padding that nm_packed_bytes adds (values_bytes rounded up to 16).
 * The other entry points reject these densities with NM_ERR_UNSUPPORTED. */

/* Sizes in bytes of the packed buffers of an R x K matrix under pattern N:M
 * with 16-bit elements of type dt (Method item (1): K*N/M values and K/32
 * words per row).  Pure host arithmetic.
 *   values_bytes = rows * cols * n / m * 2 rounded up to a multiple of 16
 *                  (the rounding adds bytes only at densities other than 50%),
 *   bits_bytes = rows * cols / 8.
 * Errors: NM_ERR_INVALID_ARG (negative sizes, NULL outputs),
 * NM_ERR_UNSUPPORTED (pattern, dt not 16-bit), NM_ERR_SHAPE (cols % 32). */
int nm_packed_bytes(int64_t rows, int64_t cols, int n, int m, nm_dtype dt,
                    size_t *values_bytes, size_t *bits_bytes);

/* Pack a dense matrix and its keep-mask into values + bits (Method item (1)).
 *   W:      device, rows x cols 16-bit elements (dt = NM_F16 or NM_BF16),
 *           row-major, 2-byte aligned; copied as raw bit patterns, so -0.0,
 *           subnormals, inf and NaN survive unchanged;
 *   keep:   device, rows x cols bytes, row-major; nonzero = kept;
 *   values: device, rows x cols*n/m 16-bit elements (output), 16-byte aligned,
 *           allocated with at least nm_packed_bytes' values_bytes;
 *   bits:   device, rows x cols/32 uint32 (output), 4-byte aligned.
 * The mask decides what is kept, never the value: a kept zero is stored.
 * Validates that every M-group of every row keeps exactly N entries.  The
 * call is synchronous: it waits for `stream` to read back the count of
 * invalid groups, and allocates (and frees) 4 bytes of device memory for it.
 * Returns NM_ERR_MASK when any group is invalid; values and bits then hold
 * unspecified contents, but nothing outside them was written. */
int nm_pack(const void *W, const uint8_t *keep, int64_t rows, int64_t cols,
            int n, int m, nm_dtype dt, void *values, uint32_t *bits,
            void *stream);

/* nm_pack for callers that cannot allocate device memory (code under HIP
 * graph capture elsewhere in the process, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, checks, output and status as
 * nm_pack, but the invalid-group counter lives in a 256-byte device array of
 * the library (one per GPU, looked up on the first call on that device and
 * held until the process ends) instead of a per-call hipMalloc / hipFree.
 * The counter does not grow with the matrix, so any size nm_pack accepts is
 * accepted (rows or cols above INT32_MAX give NM_ERR_INVALID_ARG, as there).
 * Calls on one GPU share that counter: the library serialises them within
 * the process (the call is synchronous, like nm_pack), and the counter is
 * cleared by a kernel on `stream` at the start of every call. */
int nm_pack_noalloc(const void *W, const uint8_t *keep, int64_t rows, int64_t cols,
                    int n, int m, nm_dtype dt, void *values, uint32_t *bits,
                    void *stream);

/* Batch-1 sparse matrix-vector product (Method, kernel subsection; the
 * decoding-specialised N:M SpMV):
 *   y[r] = sum over kept columns c of row r of W[r][c] * x[c],  r < rows.
 *   values, bits: as produced by nm_pack for pattern n:m (values 16-byte
 *           aligned and allocated with nm_packed_bytes' values_bytes, bits
 *           4-byte aligned); bits must hold exactly 32n/m set bits per word
 *           -- a word that does not yields an unspecified result for its row
 *           but no access outside the buffers;
 *   x:      device, cols elements of in_dt, 16-byte aligned;
 *   y:      device, rows elements of out_dt (overwritten), aligned to its
 *           element size.
 * in_dt is NM_F16 or NM_BF16 (values and x share it); out_dt is NM_F32 or
 * in_dt (then rounded to nearest, ties to even).  Products are exact in
 * fp32 and every sum is accumulated in fp32.  Asynchronous on `stream`. */
int nm_spmv(const void *values, const uint32_t *bits, const void *x, void *y,
            int64_t rows, int64_t cols, int n, int m, nm_dtype in_dt,
            nm_dtype out_dt, void *stream);

/* Small-batch product, the same operation for 1 <= batch <= 8 tokens (Method,
 * kernel subsection: batch-one and small-batch decoding):
 *   Y[b][r] = sum over kept c of W[r][c] * X[b][c].
 *   X: device, batch x cols row-major, 16-byte aligned;
 *   Y: device, batch x rows row-major (overwritten).
 * Other arguments, precision and errors as nm_spmv; batch outside 1..8 gives
 * NM_ERR_INVALID_ARG.  An x at a column that row r pruned never enters
 * Y[b][r], so Inf or NaN there leaves the sum finite, on every kernel.  (The
 * decompressed-tile matrix-core path, N:M other than 2:4 at batch >= 5 by
 * default, multiplies a zero-filled dense tile; where that gives NaN for a
 * 256-column block, the block is summed again over its kept columns only.) */
int nm_spmm_small(const void *values, const uint32_t *bits, const void *X,
                  void *Y, int batch, int64_t rows, int64_t cols, int n, int m,
                  nm_dtype in_dt, nm_dtype out_dt, void *stream);

/* Fused gate/up product with the SwiGLU epilogue: the MLP step around the
 * sparse product in the decoder layers of the Llama and Qwen models whose
 * end-to-end decoding the pages time (Experiments, Table 3 paragraph).  The
 * pages do not describe the layer; silu(gate) * up is those model families'
 * published MLP.
 *   H[b][r] = silu(G[b][r]) * U[b][r],  0 <= r < inter,  silu(z) = z / (1 + e^-z),
 * where G and U are the products (as nm_spmm_small) of the gate and up
 * projections.  The packed matrix holds 2 * inter rows with the two
 * projections interleaved: gate row r is packed row 2r and up row r is packed
 * row 2r + 1 (nm_pack of the row-interleaved dense matrix).  The sums are
 * fp32; silu is evaluated in fp32 (hardware exp) and H is fp32 or rounded to
 * in_dt.
 *   X: batch x cols; H: batch x inter row-major (overwritten).
 * Other arguments, precision and errors as nm_spmm_small; inter < 0 or
 * 2 * inter > INT32_MAX gives NM_ERR_INVALID_ARG.  With the VALU kernels the
 * epilogue needs all of x in LDS (cols * batch * 2 bytes within the LDS
 * budget; else NM_ERR_UNSUPPORTED) and an even rows_per_wave in an explicit
 * launch shape (else NM_ERR_INVALID_ARG). */
int nm_spmm_swiglu(const void *values, const uint32_t *bits, const void *X,
                   void *H, int batch, int64_t inter, int64_t cols, int n, int m,
                   nm_dtype in_dt, nm_dtype out_dt, void *stream);

/* Calibration side: accumulate the Hessian of the layer-wise reconstruction
 * objective (Method, OBS paragraph: H = 2 X X^T, shared by all rows; the
 * decode-time calibration paragraph: X's columns are the layer's input
 * activations at the decode steps of the dense model, prefill excluded):
 *   H[i][j] += scale * sum_{t < ntok} X[i][t] * X[j][t],  i, j < d.
 *   H: device, d x d fp32 row-major, updated in place (both triangles, so
 *      it stays symmetric); 4-byte aligned.
 *   X: device, d x ld 16-bit (in_dt = NM_F16 or NM_BF16) row-major, i.e.
 *      feature-major: column t is the activation of step t; only the first
 *      ntok columns are read.  ld % 8 == 0 (else NM_ERR_SHAPE), 16-byte
 *      aligned.
 *   scale: 2 gives the pages' H; calls with successive batches of columns
 *      accumulate H over the decode steps.
 * Products of 16-bit values are exact in fp32; sums are fp32 (matrix cores).
 * Errors: NM_ERR_INVALID_ARG (negative sizes, ld < ntok, d > 23170 or
 * d * ld > 2^31 - 1, NULL pointers), NM_ERR_UNSUPPORTED (in_dt),
 * NM_ERR_ALIGN.  d == 0 or ntok == 0 does nothing.  Asynchronous on stream.
 * Concurrent calls on the same H race. */
int nm_hessian_accumulate(float *H, const void *X, int64_t d, int64_t ntok,
                          int64_t ld, nm_dtype in_dt, float scale, void *stream);

/* Calibration side: N:M mask selection (the "N:M mask-selection step" of
 * the pruning solver).  In every group of m consecutive weights of a row,
 * keep[r][c] = 1 for the n columns with the largest score W[r][c]^2 * s[c],
 * ties to the lower column, else 0.  The score is computed in fp32 as
 * (w * w) * s[c]; a NaN score is taken as -inf.
 * Two per-column weights s give the criteria of the pages' backends ("Method",
 * OBS paragraph, and the "Experiments" setup naming SparseGPT and Wanda):
 *   s[c] = H[c][c] for H = 2 X X^T (nm_hessian_accumulate's output, read
 *          with cstride = cols + 1) ranks by |w| * ||x_c||, Wanda's criterion;
 *   s[c] = 1 / [H^-1]_cc ranks by the OBS saliency w^2 / [H^-1]_cc of removing
 *          the weight alone (the compensating update is the solver's, not this
 *          call's).
 *   W:    device, rows x cols 16-bit (dt), row-major, 2-byte aligned;
 *   colw: device fp32, s[c] = colw[c * cstride], 4-byte aligned;
 *   keep: device, rows x cols bytes (output), ready for nm_pack.
 * Errors: NM_ERR_INVALID_ARG, NM_ERR_UNSUPPORTED (pattern, dt), NM_ERR_SHAPE
 * (cols % 32), NM_ERR_ALIGN.  Asynchronous on stream. */
int nm_select_nm(const void *W, const float *colw, int64_t cstride,
                 int64_t rows, int64_t cols, int n, int m, nm_dtype dt,
                 uint8_t *keep, void *stream);

/* Dense comparison, the decode GEMV the sparse kernel replaces (Experiments,
 * Table 3 paragraph: speedups are against the dense model's decode):
 *   Y[b][r] = sum over all c of W[r][c] * X[b][c],  1 <= batch <= 8.
 *   W: device, rows x cols row-major 16-bit (in_dt), 16-byte aligned;
 *   X, Y, precision, errors: as nm_spmm_small (cols must be a multiple of
 *   32 here too). */
int nm_dense_gemv(const void *W, const void *X, void *Y, int batch,
                  int64_t rows, int64_t cols, nm_dtype in_dt, nm_dtype out_dt,
                  void *stream);

/* Kernel family of a launch.
 *   NM_KERNEL_VALU: vector-ALU kernels (every pattern, the dense product);
 *   NM_KERNEL_MFMA: the product on gfx950's matrix cores.  2:4 runs on the
 *                   sparse instruction (v_smfmac_f32_16x16x64), which takes
 *                   a 2:4 tile as its kept values plus a 2-bit in-group
 *                   position per value, derived on the fly from the bitmask
 *                   words.  4:8, 8:16 and 16:32 are expanded into a dense
 *                   tile in LDS and run on v_mfma_f32_16x16x32.  Only for
 *                   cols % 64 == 0, cols <= 2^25 and rows * cols <= 2^31 - 1.
 * The library's choice (NM_KERNEL_AUTO) takes the matrix cores for 2:4 at
 * batch >= 3 and for the other patterns at batch >= 5 where they can run,
 * the VALU kernels otherwise; except that 2:4 at batch 3 and 4 stays on the
 * VALU kernel (x stored plainly per token in LDS) with at most 1024 rows,
 * where that measured faster.  2:4 at batch 2 takes the VALU kernel
 * wherever all of x fits in LDS (cols <= 39680). */
typedef enum { NM_KERNEL_AUTO = 0, NM_KERNEL_VALU = 1, NM_KERNEL_MFMA = 2 } nm_kernel;

/* Launch shape of the sparse and dense kernels, for tuning sweeps.  Fields
 * set to 0 take the library's choice for the shape.
 * VALU kernels:
 *   threads_per_wg: a multiple of 64 in 64..1024;
 *   rows_per_wave:  rows processed by one wavefront (1..64 when x fits LDS
 *                   whole, else 1, 2 or 4 processed together);
 *   seg_cols:       columns of x staged in LDS at a time (multiple of 32);
 *                   seg_cols >= cols stages all of x once per workgroup.
 * MFMA kernel (one 16-row tile per workgroup):
 *   threads_per_wg: waves per workgroup x 64; the waves split K;
 *   rows_per_wave:  depth of each wave's LDS ring, 2..4 blocks of 256
 *                   columns (waves x (depth x block bytes + tile bytes)
 *                   must fit the LDS, else NM_ERR_INVALID_ARG);
 *   seg_cols:       ignored.
 * kernel: an nm_kernel (0 = the library's choice).
 * k_split: 0 = the library's choice, 1 = each row reduced by one wavefront,
 *   2 or 4 = the split reduction (Appendix C splits a row's reduction over
 *   several programs for shapes with few rows): k_split consecutive waves of
 *   a workgroup share each group of rows_per_wave rows, wave s taking the
 *   row's load batches s, s + k_split, ...; their partial row sums are added
 *   in a fixed order (wave 0, 1, ...) through LDS, so results are
 *   deterministic.  Only for the VALU kernel at batch 1 with 2:4, all of x in
 *   LDS (seg_cols >= cols), cols % (1024 * k_split) == 0, threads_per_wg / 64
 *   a multiple of k_split and no SwiGLU epilogue; elsewhere k_split > 1 gives
 *   NM_ERR_UNSUPPORTED, and values other than 0, 1, 2, 4 NM_ERR_INVALID_ARG. */
typedef struct {
  int threads_per_wg;
  int rows_per_wave;
  int seg_cols;
  int kernel;
  int k_split;
} nm_launch_cfg;

/* The launch shape nm_spmm_small (pattern n:m) or nm_dense_gemv (dense != 0;
 * n and m ignored) would use for a call.  Pure host arithmetic apart from one
 * query of the current device's properties on first use.  Errors as the
 * product's argument checks. */
int nm_default_launch(int64_t rows, int64_t cols, int batch, int n, int m,
                      int dense, nm_launch_cfg *cfg);

/* The launch shape nm_spmm_small_cfg (n:m) or nm_dense_gemv_cfg (dense != 0)
 * would use with the overrides in `user` (NULL or all fields 0 = the
 * default): the fields `user` leaves at 0 are the library's choice for the
 * kernel `user` names, with that kernel's launch rules for the pattern.
 * Host only apart from one query of the current device's properties on first
 * use.  Errors as the _cfg call's (an invalid or unsupported override gives
 * the same status that call would return). */
int nm_resolve_launch(int64_t rows, int64_t cols, int batch, int n, int m, int dense,
                      const nm_launch_cfg *user, nm_launch_cfg *cfg);

/* nm_spmm_small / nm_dense_gemv with an explicit launch shape (cfg may be
 * NULL for the default).  Invalid shapes give NM_ERR_INVALID_ARG; asking for
 * the MFMA kernel where it cannot run gives NM_ERR_UNSUPPORTED. */
int nm_spmm_small_cfg(const void *values, const uint32_t *bits, const void *X,
                      void *Y, int batch, int64_t rows, int64_t cols, int n,
                      int m, nm_dtype in_dt, nm_dtype out_dt,
                      const nm_launch_cfg *cfg, void *stream);
int nm_dense_gemv_cfg(const void *W, const void *X, void *Y, int batch,
                      int64_t rows, int64_t cols, nm_dtype in_dt,
                      nm_dtype out_dt, const nm_launch_cfg *cfg, void *stream);
/* nm_spmm_swiglu with an explicit launch shape of its 2 * inter packed rows
 * (cfg may be NULL). */
int nm_spmm_swiglu_cfg(const void *values, const uint32_t *bits, const void *X,
                       void *H, int batch, int64_t inter, int64_t cols, int n,
                       int m, nm_dtype in_dt, nm_dtype out_dt,
                       const nm_launch_cfg *cfg, void *stream);

/* Unstructured bitmasks: the bitmask format of Method item (1) for any keep
 * mask (the pages evaluate 50% unstructured pruning for quality,
 * "Experiments").  Values are the kept weights in column order, rows one
 * after another; bits as for N:M.  A word's count now varies, so an offset
 * index replaces the fixed row stride: offs[r * nwr + t] is the index in
 * values of the first kept weight of window t of row r, a window being 64
 * mask words (2048 columns) and nwr = ceil(cols / 2048); offs has rows * nwr
 * + 1 entries and the last one is the number of kept weights.  offs[r * nwr]
 * is the row's start (the CSR row pointer).
 *
 * nm_bitmask_offsets: fills offs (device, int64, rows * nwr + 1 entries,
 *   8-byte aligned) from keep (device, rows x cols bytes, nonzero = kept) and
 *   writes the number of kept weights to *total (host).  Synchronous on
 *   `stream`.
 * nm_pack_bitmask: with offs from nm_bitmask_offsets, writes values (device,
 *   16-byte aligned, at least total elements rounded up to a multiple of 8:
 *   the product reads whole 16-byte chunks) and bits (device, rows x cols/32
 *   uint32).  Raw 16-bit patterns are moved.  Synchronous; allocates and frees
 *   4 bytes of device memory for its check; NM_ERR_MASK when keep and offs
 *   disagree (values then unspecified, nothing outside a window's range
 *   written).
 * nm_spmm_bitmask: Y[b][r] = sum over kept c of W[r][c] * X[b][c] for
 *   1 <= batch <= 8, X batch x cols, Y batch x rows (as nm_spmm_small);
 *   fp32 accumulation; asynchronous on `stream`.  Words inconsistent with
 *   offs give unspecified results for their rows but no access outside the
 *   buffers.
 * Errors as nm_spmm_small (cols % 32 != 0 gives NM_ERR_SHAPE). */
int nm_bitmask_offsets(const uint8_t *keep, int64_t rows, int64_t cols, int64_t *offs,
                       int64_t *total, void *stream);
int nm_pack_bitmask(const void *W, const uint8_t *keep, int64_t rows, int64_t cols,
                    nm_dtype dt, const int64_t *offs, void *values, uint32_t *bits,
                    void *stream);
int nm_spmm_bitmask(const void *values, const uint32_t *bits, const int64_t *offs,
                    const void *X, void *Y, int batch, int64_t rows, int64_t cols,
                    nm_dtype in_dt, nm_dtype out_dt, void *stream);

/* Prefill-side product on the sparse matrix cores: Y = X . W^T for 2:4 W and
 * any number of tokens.  The pages contrast the structured-sparsity matrix
 * path with the dense GEMM: it gains in prefill and loses in decode
 * ("Introduction" and Figure 1(b)); this entry point is that path here, fed
 * from the same stored format.  A GEMM tiling (224 or 256 rows x 64, 128 or
 * 256 tokens per workgroup of 8 waves, v_smfmac_f32_16x16x64, chosen per
 * shape so that the workgroups fill the compute units) reuses each weight
 * byte for up to 256 tokens, where the decode entry points stream the
 * weights once per call for at most 8 tokens.  A workgroup takes up to
 * 160 KiB of LDS.  Where the tiles alone would leave compute units idle, K
 * is cut into 2, 4 or 8 parts: the fp32 partial products go to a workspace
 * of parts x batch x rows x 4 bytes and a second kernel adds them in part
 * order, so the result is deterministic.  The library keeps that workspace
 * between calls, one per (device, stream), grown with hipMallocAsync and
 * hipFreeAsync on `stream` when a call needs more (it holds the largest
 * split a stream has needed, e.g. 64 MiB for 4096 x 14336 at 512 tokens,
 * until the process ends); calls on one stream share it, which is safe
 * because they run in stream order.  A call made while `stream` is being
 * captured into a HIP graph takes its own workspace with hipMallocAsync and
 * frees it with hipFreeAsync after the sum (memory nodes of the graph), so a
 * graph shares no memory with other work.  The call stays asynchronous.
 *   values, bits: nm_pack output for 2:4 (rows x cols/2 and rows x cols/32),
 *                 device; values and X 16-byte aligned, bits 4-byte aligned;
 *   X:            device, batch x cols, in_dt, row-major (token-major);
 *   Y:            device, batch x rows, out_dt (NM_F32 or in_dt), row-major;
 *   cols % 64 == 0; rows * cols and batch * cols * 2 at most INT32_MAX.
 * batch == 0 or rows == 0 does nothing; cols == 0 writes zeros.
 * Errors: NM_ERR_INVALID_ARG, NM_ERR_UNSUPPORTED (not 2:4, dtypes, or a
 * device whose workgroups get less LDS than the smallest tile's 88 KiB),
 * NM_ERR_SHAPE (cols % 64), NM_ERR_ALIGN, NM_ERR_HIP.  Asynchronous on
 * stream. */
int nm_spmm_prefill(const void *values, const uint32_t *bits, const void *X, void *Y,
                    int64_t batch, int64_t rows, int64_t cols, int n, int m,
                    nm_dtype in_dt, nm_dtype out_dt, void *stream);

/* Calibration read (measurement only, not part of the product path): loads
 * every byte of buf once with 128-bit loads and writes one word per wavefront
 * of the grid to out (grid * threads_per_wg / 64 uint32, device), so the
 * loads cannot be elided.  Gives the device's achievable HBM read rate and
 * the per-launch fixed cost beside the sparse kernel, and is the read of
 * known size that scales the fetch-size counters.
 *   buf: device, bytes % 16 == 0, 16-byte aligned; grid >= 1 workgroups of
 *   threads_per_wg (64..1024, a power of two).  Asynchronous on `stream`. */
int nm_stream_read(const void *buf, size_t bytes, uint32_t *out, int grid,
                   int threads_per_wg, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NM_SPARSE_H */
