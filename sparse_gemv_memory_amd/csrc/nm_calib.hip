// nm_calib.hip -- the calibration side of the method: the layer Hessian
// H = 2 X X^T accumulated from decode-step activations, and the N:M mask
// chosen from it ("Method": the OBS paragraph and the decode-time
// calibration paragraphs of SparseDecoding; the solver backends SparseGPT and
// Wanda named in "Experiments").  These kernels feed the pruning solver; the
// product path is in nm_sparse.hip.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "nm_device.h"
#include "nm_host.h"
#include "nm_sparse.h"

namespace {

using namespace nm_host;

// ---------------------------------------------------------------------------
// Calibration side: H += scale * X X^T (the Hessian of the layer-wise
// reconstruction objective, H = 2 X X^T, with X's columns the layer's input
// activations at the decode steps; Method, OBS paragraph and the
// decode-time calibration paragraph).  A GEMM-shaped contraction over
// tokens, so it runs on the dense matrix cores: X is feature-major (row i =
// feature i over the tokens), so a 16x16x32 operand lane reads 8 consecutive
// tokens of one feature, A and B alike.  Each workgroup owns a 128 x 128
// tile of H in the upper triangle and also writes its mirror; 32-token
// chunks of the two 128-feature row blocks are staged in LDS (rows padded to
// 80 bytes, so a 16-lane read hits distinct banks), double-buffered with one
// barrier per chunk; H is read, added to and written once per call (each
// element belongs to exactly one workgroup, so there are no atomics).

constexpr int kHTile = 128;     // H tile edge
constexpr int kHChunk = 32;     // tokens per staged chunk
constexpr int kHRow = 80;       // LDS bytes per staged feature row (64 + 16 pad)
constexpr int kHBuf = 2 * kHTile * kHRow;  // one buffer: the i and the j row blocks
constexpr int kHQRow = 64 * 4 + 16;         // epilogue: one wave's 64 x 64 fp32 quarter, padded rows
constexpr int kHQuarter = 64 * kHQRow;
constexpr int kHLds = 4 * kHQuarter > 2 * kHBuf ? 4 * kHQuarter : 2 * kHBuf;

template <bool BF>
__global__ __launch_bounds__(256) void nm_hessian_kernel(float *__restrict__ H,
                                                         const uint16_t *__restrict__ X, int d,
                                                         int ntok, int ldx, float scale, int T) {
  __shared__ __attribute__((aligned(16))) char lds[kHLds];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q = lane >> 4;
  // upper-triangle tile (ti <= tj) of this workgroup, row by row
  int p = blockIdx.x, ti = 0;
  while (p >= T - ti) { p -= T - ti; ++ti; }
  const int tj = ti + p;
  const int i0 = ti * kHTile, j0 = tj * kHTile;

  // staging: piece s of this thread = row (tid + 256 s) / 4 of the i block
  // (s = 0, 1) or of the j block (s = 2, 3), 16-byte chunk (tid & 3)
  u32x4_t stg[4];
  auto load_chunk = [&](int t0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int piece = tid + 256 * (s & 1);
      const int row = piece >> 2, c = piece & 3;
      const int f = ((s >> 1) ? j0 : i0) + row;
      const int t = t0 + 8 * c;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (f < d && t < ntok) {
        v = *reinterpret_cast<const u32x4_t *>(X + (int64_t)f * ldx + t);
        const int left = ntok - t;  // tokens beyond ntok contribute nothing
        if (left < 8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (2 * e >= left) v[e] = 0u;
            else if (2 * e + 1 >= left) v[e] &= 0xffffu;
          }
        }
      }
      stg[s] = v;
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int piece = tid + 256 * (s & 1);
      const int row = piece >> 2, c = piece & 3;
      *(__attribute__((address_space(3))) u32x4_t *)(size_t)(
          (uint32_t)(size_t)(lds_ptr)lds + buf * kHBuf + (s >> 1) * kHTile * kHRow + row * kHRow +
          16 * c) = stg[s];
    }
  };

  const int wi = w & 1, wj = w >> 1;  // this wave's 64 x 64 quarter of the tile
  f4v_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = (f4v_t){0.f, 0.f, 0.f, 0.f};

  const int nchunks = (ntok + kHChunk - 1) / kHChunk;
  if (nchunks > 0) load_chunk(0);
  for (int k = 0; k < nchunks; ++k) {
    const int buf = k & 1;
    store_chunk(buf);
    __syncthreads();  // chunk k is in LDS; every wave is done with chunk k - 1
    if (k + 1 < nchunks) load_chunk((k + 1) * kHChunk);
    const uint32_t base = (uint32_t)(size_t)(lds_ptr)lds + buf * kHBuf;
    u32x4_t av[4], bv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
      av[a] = ld<u32x4_t>((lds_ptr)(size_t)(base + (64 * wi + 16 * a + n) * kHRow + 16 * q));
#pragma unroll
    for (int b = 0; b < 4; ++b)
      bv[b] = ld<u32x4_t>((lds_ptr)(size_t)(base + kHTile * kHRow +
                                            (64 * wj + 16 * b + n) * kHRow + 16 * q));
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = dmfma<BF>(av[a], bv[b], acc[a][b]);
  }

  // Epilogue through LDS: each wave parks its 64 x 64 quarter (lane: rows
  // 4q..4q+3, column n of each 16 x 16) and then updates H with 16-byte
  // loads and stores, 16 lanes per 256-byte row segment: H[i][j] += scale *
  // Q[i][j], and for tiles off the diagonal the mirror H[j][i] += scale *
  // Q[i][j] from the quarter read column-wise.  Rows or columns past d and
  // segments that do not fill 4 columns take a scalar path.
  __syncthreads();  // every wave is done with the staging buffers
  const uint32_t qb = (uint32_t)(size_t)(lds_ptr)lds + (uint32_t)(w * kHQuarter);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lds_st<float>(qb + (16 * a + 4 * q + r) * kHQRow + 4 * (16 * b + n), scale * acc[a][b][r]);
  // (each wave reads back only its own quarter: LDS operations of one wave
  // complete in order, so no barrier is needed here)
  const int qi0 = i0 + 64 * wi, qj0 = j0 + 64 * wj;
  const int c4 = lane & 15, rsub = lane >> 4;  // 16 lanes x 16 bytes per row, 4 rows per pass
  const bool mirror = ti != tj;
  // whole 16-byte segments (inside the matrix and aligned) take the vector
  // path; the others (ragged d) are updated element by element
  auto vec_ok = [&](int64_t row, int col0) {
    return row < d && col0 + 3 < d && ((((uintptr_t)(H + row * d + col0)) & 15) == 0);
  };
  // 16 passes in groups of GP: the H segments of a group (and of its mirror)
  // are loaded together, so 2 GP loads per lane are in flight, then added to
  // and stored (GP = 4 keeps the register count, and the main loop's
  // occupancy, where it is without the epilogue)
  constexpr int GP = 4;
#pragma unroll
  for (int g0 = 0; g0 < 16; g0 += GP) {
  f4v_t hd[16], hm[16];
#pragma unroll
  for (int pass = g0; pass < g0 + GP; ++pass) {
    const int rr = 4 * pass + rsub;
    hd[pass] = (f4v_t){0.f, 0.f, 0.f, 0.f};
    hm[pass] = (f4v_t){0.f, 0.f, 0.f, 0.f};
    if (vec_ok(qi0 + rr, qj0 + 4 * c4))
      hd[pass] = *reinterpret_cast<const f4v_t *>(H + (int64_t)(qi0 + rr) * d + qj0 + 4 * c4);
    if (mirror && vec_ok(qj0 + rr, qi0 + 4 * c4))
      hm[pass] = *reinterpret_cast<const f4v_t *>(H + (int64_t)(qj0 + rr) * d + qi0 + 4 * c4);
  }
  // add the quarter (row-wise for H, column-wise for the mirror) and store
#pragma unroll
  for (int pass = g0; pass < g0 + GP; ++pass) {
    const int rr = 4 * pass + rsub;
    const f4v_t v = ld<f4v_t>((lds_ptr)(size_t)(qb + rr * kHQRow + 16 * c4));
    float mv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) mv[e] = ld<float>((lds_ptr)(size_t)(qb + (4 * c4 + e) * kHQRow + 4 * rr));
    {
      const int64_t row = qi0 + rr;
      const int col0 = qj0 + 4 * c4;
      if (vec_ok(row, col0)) {
        *reinterpret_cast<f4v_t *>(H + row * d + col0) = hd[pass] + v;
      } else if (row < d) {
        for (int e = 0; e < 4; ++e)
          if (col0 + e < d) H[row * d + col0 + e] += v[e];
      }
    }
    if (mirror) {
      const int64_t row = qj0 + rr;
      const int col0 = qi0 + 4 * c4;
      if (vec_ok(row, col0)) {
        f4v_t h = hm[pass];
        h[0] += mv[0]; h[1] += mv[1]; h[2] += mv[2]; h[3] += mv[3];
        *reinterpret_cast<f4v_t *>(H + row * d + col0) = h;
      } else if (row < d) {
        for (int e = 0; e < 4; ++e)
          if (col0 + e < d) H[row * d + col0 + e] += mv[e];
      }
    }
  }
  }
}

// ---------------------------------------------------------------------------
// Calibration side: N:M mask selection.  In every group of M consecutive
// weights of a row, keep the N with the largest score w^2 * s[c] for a
// per-column weight s: s = diag(H), H = 2 X X^T, orders the weights by
// |w| * ||x_c|| (the Wanda backend the pages name); s = 1 / diag(H^-1) gives
// the OBS saliency of one weight.  Ties go to the lower column.  The score is
// an fp32 product of exact fp32 values, (w * w) * s, so the decision is
// reproducible bit for bit; a NaN score is taken as -inf.
// A workgroup owns a block of 256 M columns: it stages the block's column
// weights in LDS once (s may be strided, e.g. the diagonal of H), then walks
// `rpb` rows, one lane per group of M; a column's rank is the number of
// columns of its group that beat it.

template <int M, bool VEC>
__device__ __forceinline__ void load_group(const uint16_t *__restrict__ p, uint16_t (&b)[M]) {
  if constexpr (VEC && M == 4) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    const uint32_t u[2] = {v.x, v.y};
#pragma unroll
    for (int c = 0; c < 4; ++c) b[c] = (uint16_t)(u[c >> 1] >> (16 * (c & 1)));
  } else if constexpr (VEC) {
#pragma unroll
    for (int q = 0; q < M / 8; ++q) {
      const uint4 v = reinterpret_cast<const uint4 *>(p)[q];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) b[8 * q + c] = (uint16_t)(u[c >> 1] >> (16 * (c & 1)));
    }
  } else {
#pragma unroll
    for (int c = 0; c < M; ++c) b[c] = p[c];
  }
}

template <int M, bool VEC>
__device__ __forceinline__ void store_group(uint8_t *__restrict__ p, const uint8_t (&k)[M]) {
  if constexpr (VEC) {
#pragma unroll
    for (int q = 0; q < M / 4; ++q)
      reinterpret_cast<uint32_t *>(p)[q] = (uint32_t)k[4 * q] | ((uint32_t)k[4 * q + 1] << 8) |
                                           ((uint32_t)k[4 * q + 2] << 16) |
                                           ((uint32_t)k[4 * q + 3] << 24);
  } else {
#pragma unroll
    for (int c = 0; c < M; ++c) p[c] = k[c];
  }
}

template <bool BF, int M, bool VEC>
__global__ __launch_bounds__(256) void nm_select_kernel(const uint16_t *__restrict__ W,
                                                        const float *__restrict__ colw,
                                                        int64_t cstride, int64_t R, int K, int N,
                                                        int rpb, uint8_t *__restrict__ keep) {
  __shared__ float cw[256 * M];
  const int cb = blockIdx.x * (256 * M);  // first column of the block
  const int ncols = min(256 * M, K - cb);   // a multiple of M (M divides 32 and K)
  for (int c = threadIdx.x; c < ncols; c += 256) cw[c] = colw[(int64_t)(cb + c) * cstride];
  __syncthreads();
  const int c0 = threadIdx.x * M;
  if (c0 >= ncols) return;
  const int64_t r0 = (int64_t)blockIdx.y * rpb;
  const int64_t r1 = min(R, r0 + rpb);
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t off = r * K + cb + c0;
    uint16_t b[M];
    load_group<M, VEC>(W + off, b);
    float sc[M];
#pragma unroll
    for (int c = 0; c < M; ++c) {
      const float w = BF ? __uint_as_float((uint32_t)b[c] << 16)
                         : (float)__builtin_bit_cast(_Float16, b[c]);
      const float s = (w * w) * cw[c0 + c];
      sc[c] = (s == s) ? s : -__builtin_inff();
    }
    uint8_t k[M];
#pragma unroll
    for (int c = 0; c < M; ++c) {
      int rank = 0;
#pragma unroll
      for (int e = 0; e < M; ++e) rank += (sc[e] > sc[c]) || (sc[e] == sc[c] && e < c);
      k[c] = rank < N ? 1 : 0;
    }
    store_group<M, VEC>(keep + off, k);
  }
}

}  // namespace

extern "C" {

int nm_hessian_accumulate(float *H, const void *X, int64_t d, int64_t ntok, int64_t ld,
                          nm_dtype in_dt, float scale, void *stream) {
  if (d < 0 || ntok < 0 || ld < ntok) return NM_ERR_INVALID_ARG;
  if (d > 23170 || d * ld > INT32_MAX) return NM_ERR_INVALID_ARG;  // 32-bit tile and row offsets
  if (!is16(in_dt)) return NM_ERR_UNSUPPORTED;
  if (ld % 8 != 0) return NM_ERR_SHAPE;
  if (d == 0) return NM_OK;
  if (!H || (!X && ntok > 0)) return NM_ERR_INVALID_ARG;
  if (!aligned(H, 4) || !aligned(X, 16)) return NM_ERR_ALIGN;
  if (ntok == 0) return NM_OK;
  const int T = (int)((d + kHTile - 1) / kHTile);
  const int64_t grid = (int64_t)T * (T + 1) / 2;
  auto fn = in_dt == NM_BF16 ? nm_hessian_kernel<true> : nm_hessian_kernel<false>;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, H,
                     (const uint16_t *)X, (int)d, (int)ntok, (int)ld, scale, T);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

int nm_select_nm(const void *W, const float *colw, int64_t cstride, int64_t rows, int64_t cols,
                 int n, int m, nm_dtype dt, uint8_t *keep, void *stream) {
  if (rows < 0 || cols < 0 || cstride < 1) return NM_ERR_INVALID_ARG;
  if (!pattern_ok(n, m) || !is16(dt)) return NM_ERR_UNSUPPORTED;
  if (cols % 32 != 0) return NM_ERR_SHAPE;
  if (rows == 0 || cols == 0) return NM_OK;
  if (!W || !colw || !keep) return NM_ERR_INVALID_ARG;
  if (!aligned(W, 2) || !aligned(colw, 4)) return NM_ERR_ALIGN;
  if (cols > INT32_MAX) return NM_ERR_INVALID_ARG;
  const int64_t gx = (cols + 256 * m - 1) / (256 * m);
  const int64_t rpb = rows <= 16 * 65535LL ? 16 : (rows + 65534) / 65535;
  const int64_t gy = (rows + rpb - 1) / rpb;
  if (gy > 65535 || rpb > INT32_MAX) return NM_ERR_INVALID_ARG;
  const bool bf = dt == NM_BF16;
  // vector loads of a lane's group and stores of its keep bytes when both
  // buffers are 16-byte aligned (row starts are then aligned too: K % 32 == 0)
  const bool vec = aligned(W, 16) && aligned(keep, 16);
  auto go = [&](auto fn) {
    hipLaunchKernelGGL(fn, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, (hipStream_t)stream,
                       (const uint16_t *)W, colw, cstride, rows, (int)cols, n, (int)rpb, keep);
  };
  auto by_m = [&](auto bft, auto vect) {
    constexpr bool B_ = decltype(bft)::value, V_ = decltype(vect)::value;
    switch (m) {
      case 4: go(nm_select_kernel<B_, 4, V_>); break;
      case 8: go(nm_select_kernel<B_, 8, V_>); break;
      case 16: go(nm_select_kernel<B_, 16, V_>); break;
      default: go(nm_select_kernel<B_, 32, V_>); break;
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  if (bf)
    vec ? by_m(T{}, T{}) : by_m(T{}, F{});
  else
    vec ? by_m(F{}, T{}) : by_m(F{}, F{});
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

}  // extern "C"
