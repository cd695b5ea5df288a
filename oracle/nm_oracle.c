/*
 * nm_oracle.c -- plain, slow, obviously-correct CPU oracle for N:M bitmask
 * sparse GEMV.  TEST INFRASTRUCTURE ONLY: only the test-suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  The HIP
 * product path never includes, links or calls anything here, and this file
 * shares no code with it.
 *
 * What it computes, and where the pages define it (SparseDecoding, arXiv
 * 2610.12327):
 *   - N:M semi-structured sparsity: N kept weights in every group of M
 *     consecutive weights of a row ("Related work", N:M sparsity paragraph).
 *   - Bitmask indexing: a row's mask has one bit per column, set for a kept
 *     weight, and the kept weights are stored in column order, so the k-th
 *     set bit of a row gives the column of its k-th stored value ("Method",
 *     kernel subsection, item (1) "Bitmask indexing"; the learnaivisually
 *     explainer, "Why the pruned model was not faster").
 *   - Aligned 32-bit words: a 50% pattern with M <= 32 keeps half of every
 *     group and a word covers whole groups, so each word's set-bit count is
 *     16 ("Method", item (2) "Fixed-step bitmask traversal").
 *   - The product itself: the method reaches exactly the dense product of the
 *     masked weight matrix with x, so the oracle computes that definition in
 *     fp64 from the dense masked form, never from the packed form.
 *
 * Readings of points the pages leave open:
 *   - bit b (LSB = 0) of word w of a row <-> column 32*w + b, so an LSB-first
 *     scan visits kept columns in increasing order;
 *   - values are row-major, row stride cols*N/M elements; bits row-major, row
 *     stride cols/32 words; cols must be a multiple of 32 and of M;
 *   - groups run along a row (along the reduction dimension);
 *   - the mask decides what is kept, not the value: kept zeros are stored,
 *     values are moved as raw 16-bit patterns.
 *
 * Floating point: inputs are IEEE binary16 or bfloat16 bit patterns, decoded
 * here from their definitions; every product and sum is done in double, in
 * increasing column order.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC -o libnm_oracle.so nm_oracle.c
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define OR_OK 0
#define OR_ERR_SHAPE -3
#define OR_ERR_MASK -5
#define OR_ERR_UNSUPPORTED -2

/* ---- number decoding from the format definitions ---------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent 0 encodes zero/subnormals (value = frac * 2^-24), exponent 31
 * encodes infinities and NaNs. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * Exponent 0 encodes zero/subnormals (value = frac * 2^-133), 255 encodes
 * infinities and NaNs. */
double oracle_bf16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);
    return sign ? -v : v;
}

static double decode16(uint16_t h, int is_bf16) {
    return is_bf16 ? oracle_bf16_to_f64(h) : oracle_f16_to_f64(h);
}

/* Vectorised decoders so a caller can check them on every bit pattern. */
void oracle_decode16(const uint16_t *in, int64_t count, int is_bf16, double *out) {
    for (int64_t i = 0; i < count; ++i) out[i] = decode16(in[i], is_bf16);
}

/* ---- format checks ------------------------------------------------------ */

/* N:M patterns whose groups tile an aligned 32-bit word: M in {4, 8, 16, 32}
 * and 0 < N < M.  The pages evaluate the 50% ones (N = M/2); at any N the
 * same format holds, each aligned word then carrying exactly 32*N/M kept
 * columns (the fixed-count argument of "Method", item (2), which the pages
 * make at 50%). */
int oracle_pattern_supported(int n, int m) {
    return (m == 4 || m == 8 || m == 16 || m == 32) && n > 0 && n < m;
}

/* Number of M-groups of `keep` that do not hold exactly N kept entries.
 * keep is rows x cols, row-major, nonzero byte = kept. */
int64_t oracle_count_bad_groups(const uint8_t *keep, int64_t rows, int64_t cols,
                                int n, int m) {
    int64_t bad = 0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < cols / m; ++g) {
            int cnt = 0;
            for (int j = 0; j < m; ++j) cnt += keep[r * cols + g * m + j] != 0;
            if (cnt != n) ++bad;
        }
    return bad;
}

/* ---- pack / unpack, one bit at a time ------------------------------------ */

/* W: rows x cols 16-bit patterns; keep as above.
 * values: rows x (cols*n/m) 16-bit patterns, each row the kept W entries in
 * increasing column order.  bits: rows x (cols/32) words, bit b of word w set
 * iff column 32w+b is kept. */
int oracle_pack(const uint16_t *W, const uint8_t *keep, int64_t rows, int64_t cols,
                int n, int m, uint16_t *values, uint32_t *bits) {
    if (!oracle_pattern_supported(n, m)) return OR_ERR_UNSUPPORTED;
    if (cols % 32 != 0 || cols % m != 0) return OR_ERR_SHAPE;
    if (oracle_count_bad_groups(keep, rows, cols, n, m) != 0) return OR_ERR_MASK;
    const int64_t vrow = cols * n / m, wrow = cols / 32;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t j = 0;
        for (int64_t w = 0; w < wrow; ++w) {
            uint32_t word = 0;
            for (int b = 0; b < 32; ++b) {
                int64_t c = 32 * w + b;
                if (keep[r * cols + c]) {
                    word |= (uint32_t)1 << b;
                    values[r * vrow + j] = W[r * cols + c];
                    ++j;
                }
            }
            bits[r * wrow + w] = word;
        }
        if (j != vrow) return OR_ERR_MASK; /* cannot happen once groups are valid */
    }
    return OR_OK;
}

/* Inverse of oracle_pack: positions that are not kept become +0 (0x0000) and
 * keep = 0 there. */
int oracle_unpack(const uint16_t *values, const uint32_t *bits, int64_t rows, int64_t cols,
                  int n, int m, uint16_t *W, uint8_t *keep) {
    if (!oracle_pattern_supported(n, m)) return OR_ERR_UNSUPPORTED;
    if (cols % 32 != 0 || cols % m != 0) return OR_ERR_SHAPE;
    const int64_t vrow = cols * n / m, wrow = cols / 32;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t j = 0;
        for (int64_t c = 0; c < cols; ++c) {
            uint32_t word = bits[r * wrow + c / 32];
            int set = (word >> (c % 32)) & 1u;
            if (set) {
                if (j >= vrow) return OR_ERR_MASK;
                W[r * cols + c] = values[r * vrow + j];
                ++j;
            } else {
                W[r * cols + c] = 0;
            }
            keep[r * cols + c] = (uint8_t)set;
        }
        if (j != vrow) return OR_ERR_MASK;
    }
    return OR_OK;
}

/* ---- unstructured bitmasks (any keep mask) ------------------------------- */

/* The same bitmask format for an arbitrary keep mask (the pages evaluate 50%
 * unstructured pruning for quality, "Experiments"): each row's kept weights
 * in increasing column order, rows one after another, row r starting at
 * values[row_ptr[r]]; row_ptr has rows + 1 entries, row_ptr[0] = 0 and
 * row_ptr[rows] = the number of kept weights.  A word's count now varies, so
 * its values start at the row's start plus the set bits of the words before
 * it. */
void oracle_bitmask_row_ptr(const uint8_t *keep, int64_t rows, int64_t cols,
                            int64_t *row_ptr) {
    row_ptr[0] = 0;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t cnt = 0;
        for (int64_t c = 0; c < cols; ++c) cnt += keep[r * cols + c] != 0;
        row_ptr[r + 1] = row_ptr[r] + cnt;
    }
}

int oracle_pack_bitmask(const uint16_t *W, const uint8_t *keep, int64_t rows, int64_t cols,
                        const int64_t *row_ptr, uint16_t *values, uint32_t *bits) {
    if (cols % 32 != 0) return OR_ERR_SHAPE;
    const int64_t wrow = cols / 32;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t j = row_ptr[r];
        for (int64_t w = 0; w < wrow; ++w) {
            uint32_t word = 0;
            for (int b = 0; b < 32; ++b) {
                int64_t c = 32 * w + b;
                if (keep[r * cols + c]) {
                    word |= (uint32_t)1 << b;
                    values[j++] = W[r * cols + c];
                }
            }
            bits[r * wrow + w] = word;
        }
        if (j != row_ptr[r + 1]) return OR_ERR_MASK;
    }
    return OR_OK;
}

int oracle_unpack_bitmask(const uint16_t *values, const uint32_t *bits, const int64_t *row_ptr,
                          int64_t rows, int64_t cols, uint16_t *W, uint8_t *keep) {
    if (cols % 32 != 0) return OR_ERR_SHAPE;
    const int64_t wrow = cols / 32;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t j = row_ptr[r];
        for (int64_t c = 0; c < cols; ++c) {
            int set = (bits[r * wrow + c / 32] >> (c % 32)) & 1u;
            if (set) {
                if (j >= row_ptr[r + 1]) return OR_ERR_MASK;
                W[r * cols + c] = values[j++];
            } else {
                W[r * cols + c] = 0;
            }
            keep[r * cols + c] = (uint8_t)set;
        }
        if (j != row_ptr[r + 1]) return OR_ERR_MASK;
    }
    return OR_OK;
}

/* ---- the product ---------------------------------------------------------- */

/* y[b][i] = sum_{c=0}^{cols-1} [keep[r][c] != 0] * W[r][c] * x[b][c], r = row_idx[i]
 * (or r = i when row_idx is NULL), summed in double in increasing c.
 * W and x are 16-bit patterns of the same type (is_bf16 selects which).
 * x is batch x cols row-major; y is batch x nrows row-major. keep == NULL
 * means every entry is kept (the dense product). */
void oracle_masked_gemv_f64(const uint16_t *W, const uint8_t *keep, int is_bf16,
                            const uint16_t *x, int batch, int64_t rows, int64_t cols,
                            const int64_t *row_idx, int64_t nrows, int threads,
                            double *y) {
    (void)rows;
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = row_idx ? row_idx[i] : i;
        for (int b = 0; b < batch; ++b) {
            double s = 0.0;
            for (int64_t c = 0; c < cols; ++c) {
                if (keep && !keep[r * cols + c]) continue;
                s += decode16(W[r * cols + c], is_bf16) * decode16(x[(int64_t)b * cols + c], is_bf16);
            }
            y[(int64_t)b * nrows + i] = s;
        }
    }
}

/* ---- the SwiGLU step around the product ------------------------------------ */

/* h[i] = silu(g[i]) * u[i] with silu(z) = z * sigmoid(z) = z / (1 + exp(-z)),
 * in double.  The MLP of the Llama / Qwen decoder layers timed end to end on
 * the pages applies this to the gate and up projections (the pages do not
 * spell the layer out; it is those models' published architecture). */
void oracle_silu_mul_f64(const double *g, const double *u, int64_t n, double *h) {
    for (int64_t i = 0; i < n; ++i) h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* ---- the calibration side: the layer Hessian -------------------------------- */

/* H[i][j] = scale * sum_{t < ntok} x[i][t] * x[j][t] in double, i, j < d, where
 * X is d x ld 16-bit patterns (feature-major: column t is one decode-step
 * activation) and H is d x d row-major.  With scale = 2 this is H = 2 X X^T
 * of the layer-wise reconstruction objective, over the first ntok columns. */
void oracle_hessian_f64(const uint16_t *X, int is_bf16, int64_t d, int64_t ntok, int64_t ld,
                        double scale, int threads, double *H) {
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t i = 0; i < d; ++i) {
        for (int64_t j = 0; j < d; ++j) {
            double s = 0.0;
            for (int64_t t = 0; t < ntok; ++t)
                s += decode16(X[i * ld + t], is_bf16) * decode16(X[j * ld + t], is_bf16);
            H[i * d + j] = scale * s;
        }
    }
}

/* ---- the calibration side: N:M mask selection ------------------------------- */

/* keep[r][c] for the rows x cols 16-bit W: in each group of m consecutive
 * columns of a row, choose n columns one at a time, each time the unchosen
 * column of largest score (w * w) * s[c] (first in column order among equal
 * scores), s[c] = colw[c * cstride].  The score is a float (fp32) product,
 * the precision in which the decision is fixed; a NaN score counts as -inf.
 * With s = diag(H), H = 2 X X^T, this is the |w| * ||x_c|| order of the Wanda
 * backend; with s = 1 / diag(H^-1), the OBS saliency of removing one weight
 * ("Method", OBS paragraph). */
int oracle_select_nm(const uint16_t *W, int is_bf16, const float *colw, int64_t cstride,
                     int64_t rows, int64_t cols, int n, int m, uint8_t *keep) {
    /* the calibration side is built for the 50% patterns only */
    if (!oracle_pattern_supported(n, m) || 2 * n != m) return OR_ERR_UNSUPPORTED;
    if (cols % m != 0) return OR_ERR_SHAPE;
    float score[32];
    int chosen[32];
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < cols; g += m) {
            for (int e = 0; e < m; ++e) {
                const float w = (float)decode16(W[r * cols + g + e], is_bf16);
                const float ww = w * w;
                const float sc = ww * colw[(g + e) * cstride];
                score[e] = isnan(sc) ? -INFINITY : sc;
                chosen[e] = 0;
            }
            for (int k = 0; k < n; ++k) {
                int best = -1;
                for (int e = 0; e < m; ++e)
                    if (!chosen[e] && (best < 0 || score[e] > score[best])) best = e;
                chosen[best] = 1;
            }
            for (int e = 0; e < m; ++e) keep[r * cols + g + e] = (uint8_t)chosen[e];
        }
    }
    return OR_OK;
}
