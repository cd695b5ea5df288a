// nm_prefill.hip -- the prefill-side 2:4 product on the sparse matrix cores.
//
// Y = X . W^T for a 2:4 W in the stored format (kept values in increasing
// column order, one mask bit per column) and any number of tokens: the
// prefill regime, where the pages contrast the sparse matrix-core path with
// the dense GEMM ("Introduction" and Figure 1(b): the structured-sparsity
// path gains in prefill and loses in decode).  The decode kernels of
// nm_sparse.hip stream the weights once per call for at most 8 tokens; here
// the weights and the tokens are both tiled, so each weight byte read from
// memory serves up to 128 tokens and each token serves 256 rows.
//
// Tiling (gfx950, v_smfmac_f32_16x16x64_{f16,bf16}):
//   - a workgroup of 4 waves owns 256 rows x 128 tokens of Y; wave w owns rows
//     128 (w & 1) .. +128 and tokens 64 (w >> 1) .. +64, i.e. 8 x 4 output
//     tiles of 16 x 16 (32 accumulators of 4 floats per lane);
//   - K is walked in steps of 64 columns.  Each step's operands are staged in
//     LDS by direct-to-LDS buffer loads, double-buffered with one barrier per
//     step: the 256 rows' 32 kept values (64 bytes) and 2 mask words each,
//     and the 128 tokens' 64 x values (128 bytes) each;
//   - operand layouts are those of the instruction: lane l = 16 j + n holds
//     A row n, columns 16 j .. 16 j + 15 (its 8 kept values, and the 2-bit
//     in-group positions derived from the mask nibbles); B token n, columns
//     8 j .. 8 j + 7 and 32 + 8 j .. 32 + 8 j + 7; D rows 4 j .. 4 j + 3 of
//     token n;
//   - LDS rows are XOR-swizzled by 16-byte chunk (values: chunk c of row r
//     at c ^ ((r >> 2) & 3); x: chunk c of token t at c ^ ((t >> 1) & 7)),
//     so the 16 rows or tokens a quarter-wave reads fall on distinct banks.
// Ragged edges: rows past R load row R - 1 and are not stored; tokens past
// the batch read zeros (buffer range check); K must be a multiple of 64.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "nm_device.h"
#include "nm_host.h"
#include "nm_sparse.h"

namespace {

using namespace nm_host;

constexpr int kPRows = 256;                 // rows per workgroup
constexpr int kPToks = 128;                 // tokens per workgroup
constexpr int kPValRow = 64;                // LDS bytes of a row's values per step
constexpr int kPValBytes = kPRows * kPValRow;       // 16 KiB
constexpr int kPMaskBytes = kPRows * 8;             // 2 KiB: 2 words per row
constexpr int kPXRow = 128;                 // LDS bytes of a token's x per step
constexpr int kPXBytes = kPToks * kPXRow;           // 16 KiB
constexpr int kPStage = kPValBytes + kPMaskBytes + kPXBytes;
constexpr int kPDma = 4 + 2 + 4;  // direct-to-LDS loads per wave per step

__host__ __device__ constexpr int prefill_lds(int ns) { return ns * kPStage; }

#ifndef NM_PREFILL_STAGES
#define NM_PREFILL_STAGES 4
#endif
constexpr int kPrefillStages = NM_PREFILL_STAGES;  // ring depth (LDS: 34 KiB per step)

// An LDS read the compiler may not repeat or drop: the fragments of the next
// step are read once, into registers, while the current step's products run.
template <typename T>
__device__ __forceinline__ T vld(uint32_t addr) {
  return *(volatile __attribute__((address_space(3))) T *)(size_t)addr;
}

// Direct-to-LDS load of 4 bytes per lane with the default cache policy: the
// weights are reused by every token tile of their row tile, so they must stay
// in L2 (the streaming policy of the decode kernels measured 20% slower here).
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(size_t)lds, 4, voff, soff, 0, 0);
}

template <bool BF, int NS>
__global__ __launch_bounds__(256) void nm_spmm_prefill_kernel(
    const uint16_t *__restrict__ values, const uint32_t *__restrict__ bits,
    const uint16_t *__restrict__ x, void *__restrict__ y, int B, int R, int K, int nrt, int ntt,
    int out_kind) {
  static_assert(NS >= 3 && (NS - 2) * kPDma < 64, "ring depth");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, j = lane >> 4;
  // Tile of this workgroup.  Workgroups go to the 8 XCDs round-robin
  // (block b on XCD b % 8), and each XCD has its own L2: XCD x takes a
  // contiguous range of tiles, ordered by groups of 4 row tiles x all token
  // tiles, so the workgroups running together on one XCD share their
  // weights and activations through its L2.
  const int T = nrt * ntt;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int tile = xcd * (T / 8) + min(xcd, T % 8) + slot;
  const int group = tile / (4 * ntt);
  const int first_r = 4 * group, gr = min(nrt - first_r, 4);
  const int in = tile - group * 4 * ntt;
  const int rt = first_r + in % gr, tt = in / gr;
  const int row0 = rt * kPRows, tok0 = tt * kPToks;
  const int nk = K >> 6;
  const uint32_t base = (uint32_t)(size_t)(lds_ptr)lds;

  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void *)values, 0, (int)((int64_t)R * K), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void *)bits, 0, (int)((int64_t)R * K / 8), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, (int)((int64_t)B * K * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc((void *)values, 0, 0,
                                                                      kRsrcWord3);

  // Per-lane source offsets of step 0 (bytes); a step adds 64 (values),
  // 8 (masks) or 128 (x) through the scalar offset.
  // values: instruction q of wave w fills LDS bytes 1024 (4 q + w) .. + 1024,
  // i.e. rows 16 (4 q + w) .. + 16, lane i -> row (i >> 2), position i & 3
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 16 * (4 * q + w) + (lane >> 2);
    const int p = lane & 3;
    const int c = p ^ ((r >> 2) & 3);
    const int gr = min(row0 + r, R - 1);
    voff[q] = gr * K + 16 * c;
  }
  // masks: instruction q of wave w fills LDS bytes 256 (4 q + w) .. + 256,
  // i.e. rows 32 (4 q + w) .. + 32, lane i -> row (i >> 1), word i & 1
  int moff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 32 * (4 * q + w) + (lane >> 1);
    const int gr = min(row0 + r, R - 1);
    moff[q] = gr * (K / 8) + 4 * (lane & 1);
  }
  // x: instruction q of wave w fills LDS bytes 1024 (4 q + w) .. + 1024,
  // i.e. tokens 8 (4 q + w) .. + 8, lane i -> token (i >> 3), position i & 7
  int xoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = 8 * (4 * q + w) + (lane >> 3);
    const int p = lane & 7;
    const int c = p ^ ((t >> 1) & 7);
    // a token past the batch points at the end of x: the range check reads zeros
    xoff[q] = (int)min((int64_t)(tok0 + t) * K * 2, (int64_t)B * K * 2) + 16 * c;
  }

  // step s into ring slot s % NS; a step past the last loads from
  // zero-size resources (no memory traffic, same instruction count), so the
  // wait counts below are the same at every step
  auto issue = [&](int s) {
    const bool real = s < nk;
    const __amdgpu_buffer_rsrc_t V = real ? rv : r0, M = real ? rb : r0, X = real ? rx : r0;
    const uint32_t st = base + (uint32_t)((s % NS) * kPStage);
#pragma unroll
    for (int q = 0; q < 4; ++q) lds_load16(V, st + 1024 * (4 * q + w), voff[q], 64 * s);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      lds_load4(M, st + kPValBytes + 256 * (4 * q + w), moff[q], 8 * s);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      lds_load16(X, st + kPValBytes + kPMaskBytes + 1024 * (4 * q + w), xoff[q], 128 * s);
  };

  f4v_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = (f4v_t){0.f, 0.f, 0.f, 0.f};

  const int wr = w & 1, wc = w >> 1;
  // operands of one step: A fragments and raw mask words of the 8 row tiles,
  // B fragments of the 4 token tiles
  struct Frag {
    u32x4_t a[8];
    uint32_t mw[8];
    u32x4_t b[4][2];
  };
  auto read_frags = [&](Frag &f, int s) {
    const uint32_t st = base + (uint32_t)((s % NS) * kPStage);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 128 * wr + 16 * i + n;
      f.a[i] = vld<u32x4_t>(st + r * kPValRow + 16 * (j ^ ((r >> 2) & 3)));
      f.mw[i] = vld<uint32_t>(st + kPValBytes + r * 8 + 4 * (j >> 1));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tk = 64 * wc + 16 * t + n;
      const uint32_t xr = st + kPValBytes + kPMaskBytes + tk * kPXRow;
      const int sw = (tk >> 1) & 7;
      f.b[t][0] = vld<u32x4_t>(xr + 16 * (j ^ sw));
      f.b[t][1] = vld<u32x4_t>(xr + 16 * ((4 + j) ^ sw));
    }
  };
  // Software pipeline: the products of step s run while the fragments of
  // step s + 1 are read from LDS.  Steps s + 2 .. s + NS - 1 are in flight.
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);
  wait_vmcnt<(NS - 2) * kPDma>();  // step 0 has landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frag cur;
  read_frags(cur, 0);
  for (int s = 0; s < nk; ++s) {
    // step s + 1 has landed (NS - 3 younger steps stay in flight); the
    // fragments of step s are in registers, so after the barrier every
    // wave is done with slot (s - 1) % NS, which is refilled next
    wait_vmcnt<(NS - 3) * kPDma>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(s + NS - 1);
    Frag nxt;
    read_frags(nxt, s + 1);
    int idx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) idx[i] = nib_codes(cur.mw[i] >> ((j & 1) * 16));
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i][t] = smfmac<BF>(cur.a[i], cur.b[t][0], cur.b[t][1], idx[i], acc[i][t]);
    // issue order: one product, one LDS read of the next step, 24 times,
    // then the last 8 products
#pragma unroll
    for (int k = 0; k < 24; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    cur = nxt;
  }
  wait_vmcnt<0>();  // the trailing dummy loads still write LDS

  // lane (j, n) of tile (i, t): rows 4 j .. 4 j + 3 of row tile i, token n
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int tok = tok0 + 64 * wc + 16 * t + n;
    if (tok >= B) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = row0 + 128 * wr + 16 * i + 4 * j;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (r + e < R) store_out(y, (int64_t)tok * R + r + e, acc[i][t][e], out_kind);
    }
  }
}

}  // namespace

extern "C" {

int nm_spmm_prefill(const void *values, const uint32_t *bits, const void *X, void *Y,
                    int64_t batch, int64_t rows, int64_t cols, int n, int m, nm_dtype in_dt,
                    nm_dtype out_dt, void *stream) {
  if (batch < 0 || rows < 0 || cols < 0) return NM_ERR_INVALID_ARG;
  if (!pattern_ok(n, m) || !is16(in_dt) || !out_ok(in_dt, out_dt)) return NM_ERR_UNSUPPORTED;
  if (n != 2 || m != 4) return NM_ERR_UNSUPPORTED;  // the sparse instruction is 2:4
  if (cols % 64 != 0) return NM_ERR_SHAPE;
  if (batch == 0 || rows == 0) return NM_OK;
  // each size alone first, so the products below cannot overflow int64
  if (batch > INT32_MAX || rows > INT32_MAX || cols > INT32_MAX) return NM_ERR_INVALID_ARG;
  if (rows * cols > INT32_MAX || batch * cols * 2 > INT32_MAX) return NM_ERR_INVALID_ARG;
  if (!Y || (cols > 0 && (!values || !bits || !X))) return NM_ERR_INVALID_ARG;
  if (!aligned(values, 16) || !aligned(bits, 4) || !aligned(X, 16) ||
      !aligned(Y, out_dt == NM_F32 ? 4 : 2))
    return NM_ERR_ALIGN;
  const int64_t nrt = (rows + kPRows - 1) / kPRows, ntt = (batch + kPToks - 1) / kPToks;
  if (nrt * ntt > INT32_MAX) return NM_ERR_INVALID_ARG;
  constexpr int NS = kPrefillStages;
  auto go = [&](auto fn) {
    hipLaunchKernelGGL(fn, dim3((unsigned)(nrt * ntt)), dim3(256), prefill_lds(NS), (hipStream_t)stream,
                       (const uint16_t *)values, bits, (const uint16_t *)X, Y, (int)batch,
                       (int)rows, (int)cols, (int)nrt, (int)ntt, (int)out_dt);
  };
  if (in_dt == NM_BF16)
    go(nm_spmm_prefill_kernel<true, NS>);
  else
    go(nm_spmm_prefill_kernel<false, NS>);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

}  // extern "C"
