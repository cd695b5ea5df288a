// nm_prefill.hip -- the prefill-side 2:4 product on the sparse matrix cores.
//
// Y = X . W^T for a 2:4 W in the stored format (kept values in increasing
// column order, one mask bit per column) and any number of tokens: the
// prefill regime, where the pages contrast the sparse matrix-core path with
// the dense GEMM ("Introduction" and Figure 1(b): the structured-sparsity
// path gains in prefill and loses in decode).  The decode kernels of
// nm_sparse.hip stream the weights once per call for at most 8 tokens; here
// the weights and the tokens are both tiled, so each weight byte read from
// memory serves 256 tokens and each token serves up to 256 rows.
//
// Tiling (gfx950, v_smfmac_f32_16x16x64_{f16,bf16}):
//   - a workgroup of 8 waves (two per SIMD) owns 32 RT rows x 256 tokens of Y
//     (RT = 8 or 7 row tiles of 16 per wave, chosen per shape so that the
//     tiles fill the compute units in whole rounds); wave w owns rows
//     16 RT (w & 1) .. + 16 RT and tokens 64 (w >> 1) .. + 64, i.e. RT x 4
//     output tiles of 16 x 16;
//   - K is walked in steps of 64 columns.  A step's operands are staged in
//     LDS by direct-to-LDS buffer loads in a ring of 3 stages (48 KiB each:
//     the rows' 32 kept values (64 bytes) and the tokens' 64 x values (128
//     bytes)); the mask words come 4 steps at a time (32 bytes per row) into
//     a ring of 2 slots, since a load of 8 bytes per row costs as much
//     issue as one of 64.  The loads of step s + 2 are issued among the
//     products of step s, and one barrier per step both publishes step s + 1
//     and frees the slot of step s;
//   - operand layouts are those of the instruction: lane l = 16 j + n holds
//     A row n, columns 16 j .. 16 j + 15 (its 8 kept values, and the 2-bit
//     in-group positions derived from the mask nibbles); B token n, columns
//     8 j .. 8 j + 7 and 32 + 8 j .. 32 + 8 j + 7; D rows 4 j .. 4 j + 3 of
//     token n.  Two row tiles share one index register: the lane's 16 mask
//     bits of each are packed with v_perm, converted at once, and each
//     product takes its half (the instruction's ABID field);
//   - LDS rows are XOR-swizzled by 16-byte chunk (values: chunk c of row r
//     at c ^ ((r >> 2) & 3); x: chunk c of token t at c ^ ((t >> 1) & 7);
//     mask words: the two 16-byte halves of row r swapped when bit 3 of r is
//     set), so the reads in MFMA layout spread over the banks; every lane's
//     read address is a per-lane base plus per-tile immediates.
// Ragged edges: rows past R load row R - 1 and are not stored; tokens past
// the batch read zeros (buffer range check); K must be a multiple of 64.

#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>
#include <type_traits>
#include <vector>

#include "nm_device.h"
#include "nm_host.h"
#include "nm_sparse.h"

namespace {

using namespace nm_host;

constexpr int kPWaves = 8;                           // waves per workgroup
constexpr int kPValBytes = 256 * 64;                 // values of up to 256 rows per step
constexpr int kPNS = 3;                              // stages in the ring
constexpr int kPMaskSlot = 256 * 32;                 // mask words of 4 steps, 256 rows

// LDS of a workgroup with TT token tiles of 16 per wave (64 TT tokens): the
// ring of stages (values, then x of 64 TT tokens, 128 bytes each), then the
// two mask slots; 160 KiB at TT = 4.
__host__ __device__ constexpr int prefill_stage(int tt) { return kPValBytes + 8192 * tt; }
__host__ __device__ constexpr int prefill_mask_base(int tt) { return kPNS * prefill_stage(tt); }
__host__ __device__ constexpr int prefill_lds(int tt) {
  return prefill_mask_base(tt) + 2 * kPMaskSlot;
}

// An LDS read the compiler may not repeat or drop.
template <typename T>
__device__ __forceinline__ T vld(uint32_t addr) {
  return *(volatile __attribute__((address_space(3))) T *)(size_t)addr;
}

// In-group position codes of 8 nibbles at once (two 16-bit mask halves, each
// nibble holding exactly 2 set bits p0 < p1 -> p0 | p1 << 2), by the rule of
// nib_codes.
__device__ __forceinline__ int nib_codes2(uint32_t m) {
  const uint32_t s1 = m >> 1, s2 = m >> 2, s3 = m >> 3;
  const uint32_t c0 = ~m & s1 & 0x11111111u;
  const uint32_t c1 = ~m & ~s1 & 0x11111111u;
  const uint32_t c2 = (s3 | ~s2) & 0x11111111u;
  const uint32_t c3 = (s3 | s2) & 0x11111111u;
  return (int)(c0 | (c1 << 1) | (c2 << 2) | (c3 << 3));
}

// The 16x16x64 sparse product with its index set in half AB of idx.
template <bool BF, int AB>
__device__ __forceinline__ f4v_t smfmac_half(u32x4_t a, u32x4_t b0, u32x4_t b1, int idx, f4v_t c) {
  const u32x8_t b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
  if constexpr (BF)
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(b8v_t, a),
                                                    __builtin_bit_cast(b16v_t, b), c, idx, 0, AB);
  else
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(h8v_t, a),
                                                   __builtin_bit_cast(h16v_t, b), c, idx, 0, AB);
}

template <bool BF, int RT, int TT>
__global__ __launch_bounds__(512) void nm_spmm_prefill_kernel(
    const uint16_t *__restrict__ values, const uint32_t *__restrict__ bits,
    const uint16_t *__restrict__ x, void *__restrict__ y, int B, int R, int K, int nrt, int ntt,
    int out_kind, int vec, int ks, int kper, float *__restrict__ part) {
  static_assert(RT == 7 || RT == 8, "row tiles per wave");
  static_assert(TT == 1 || TT == 2 || TT == 4, "token tiles per wave");
  constexpr int kRows = 32 * RT;    // rows per workgroup
  constexpr int kToks = 64 * TT;    // tokens per workgroup
  constexpr int kStage = prefill_stage(TT);
  constexpr int kMaskBase = prefill_mask_base(TT);
  constexpr int kDma = 2 + TT;      // stage loads per wave per step
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, j = lane >> 4;
  // Tile and part of K of this workgroup.  Workgroups go to the 8 XCDs
  // round-robin (block b on XCD b % 8), and each XCD has its own L2: XCD x
  // takes a contiguous range of (tile, part) pairs, the tiles ordered by
  // groups of 4 row tiles x all token tiles, so the workgroups running
  // together on one XCD share their weights and activations through its L2.
  const int T = nrt * ntt, TV = T * ks;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int vt = xcd * (TV / 8) + min(xcd, TV % 8) + slot;
  const int tile = vt / ks, kpart = vt - tile * ks;
  const int group = tile / (4 * ntt);
  const int first_r = 4 * group, gr = min(nrt - first_r, 4);
  const int in = tile - group * 4 * ntt;
  const int rt = first_r + in % gr, tt = in / gr;
  const int row0 = rt * kRows, tok0 = tt * kToks;
  // steps of 64 columns of this part of K: sbeg .. sbeg + nk - 1 (kper is a
  // multiple of 4, so the parts start on a group of mask words)
  const int sbeg = min(K >> 6, kpart * kper);
  const int nk = min(K >> 6, sbeg + kper) - sbeg;
  const uint32_t base = (uint32_t)(size_t)(lds_ptr)lds;

  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void *)values, 0, (int)((int64_t)R * K), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void *)bits, 0, (int)((int64_t)R * K / 8), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, (int)((int64_t)B * K * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc((void *)values, 0, 0,
                                                                      kRsrcWord3);

  // Per-lane source offsets of step 0 (bytes); a step adds 64 (values) or
  // 128 (x) through the scalar offset, a group of 4 steps adds 32 (masks).
  // values: instruction q of wave w fills LDS bytes 1024 (8 q + w) .. + 1024,
  // i.e. rows 16 (8 q + w) .. + 16, lane i -> row (i >> 2), chunk slot i & 3;
  // the instructions past the workgroup's rows load from the empty resource
  const bool vreal[2] = {w < 2 * RT, 8 + w < 2 * RT};
  int voff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 16 * (8 * q + w) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    voff[q] = min(row0 + r, R - 1) * K + 16 * c + 64 * sbeg;
  }
  // masks: wave w fills LDS bytes 1024 w .. + 1024 of a mask slot, i.e. rows
  // 32 w .. + 32, lane i -> row (i >> 1), 16-byte half (i & 1) ^ (row >> 3 & 1)
  const bool mreal = w < RT;
  int moff;
  {
    const int r = 32 * w + (lane >> 1);
    moff = min(row0 + r, R - 1) * (K / 8) + 16 * ((lane & 1) ^ ((r >> 3) & 1)) + 8 * sbeg;
  }
  // x: instruction q of wave w fills LDS bytes 1024 (8 q + w) .. + 1024 of
  // the stage's x, i.e. tokens 8 (8 q + w) .. + 8, lane i -> token (i >> 3),
  // chunk slot i & 7; a token past the batch points at the end of x, where
  // the range check reads zeros
  int xoff[TT];
#pragma unroll
  for (int q = 0; q < TT; ++q) {
    const int t = 8 * (8 * q + w) + (lane >> 3);
    const int c = (lane & 7) ^ ((t >> 1) & 7);
    xoff[q] = (int)min((int64_t)(tok0 + t) * K * 2, (int64_t)B * K * 2) + 16 * c + 128 * sbeg;
  }
  // step s into stage slot s % 3; a step past the last loads from the empty
  // resource (no memory traffic, same instruction count), so the wait counts
  // below are the same at every step
  auto issue = [&](int s) {
    const bool real = s < nk;
    const uint32_t st = base + (uint32_t)((s % kPNS) * kStage);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      lds_load16(real && vreal[q] ? rv : r0, st + 1024 * (8 * q + w), voff[q], 64 * s);
#pragma unroll
    for (int q = 0; q < TT; ++q)
      lds_load16(real ? rx : r0, st + kPValBytes + 1024 * (8 * q + w), xoff[q], 128 * s);
  };
  // mask words of steps 4 S .. 4 S + 3 into mask slot S % 2; the group offset
  // goes into the vector offset, which the range check covers
  const int ngroups = (nk + 3) >> 2;
  auto issue_masks = [&](int S) {
    lds_load16(S < ngroups && mreal ? rb : r0, base + kMaskBase + (S & 1) * kPMaskSlot + 1024 * w,
               moff + 32 * S, 0);
  };

  const int wr = w & 1, wc = w >> 1;
  f4v_t acc[RT][TT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[i][t] = (f4v_t){0.f, 0.f, 0.f, 0.f};

  // per-lane LDS offsets: row tile i adds 1024 i (values) or 512 i (masks),
  // token tile t adds 2048 t
  const int r_lane = 16 * RT * wr + n;  // the lane's row within row tile 0
  const uint32_t a_off = (uint32_t)(r_lane * 64 + 16 * (j ^ ((n >> 2) & 3)));
  const uint32_t b_off0 =
      (uint32_t)(kPValBytes + (16 * TT * wc + n) * 128 + 16 * (j ^ ((n >> 1) & 7)));
  const uint32_t b_off1 =
      (uint32_t)(kPValBytes + (16 * TT * wc + n) * 128 + 16 * ((4 + j) ^ ((n >> 1) & 7)));
  // mask word 2 (s % 4) + (j >> 1) of the lane's row: its 16-byte half is
  // (s >> 1) & 1, swapped for rows with bit 3 set, and its word within the
  // half 2 (s & 1) + (j >> 1)
  const int hn = (n >> 3) & 1;
  const uint32_t m_lane = (uint32_t)(kMaskBase + r_lane * 32 + 4 * (j >> 1));
  const uint32_t m_off0 = m_lane + 16 * hn, m_off1 = m_lane + 16 * (hn ^ 1);
  // v_perm selector: the lane's 16-bit half of two mask words -> the low and
  // the high half of one register
  const uint32_t psel = (j & 1) ? 0x07060302u : 0x05040100u;

  issue_masks(0);
  issue(0);
  issue(1);
  wait_vmcnt<kDma>();  // the masks of steps 0..3 and step 0 have landed
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  int slot3 = 0;
  for (int s = 0; s < nk; ++s) {
    // the masks of the next 4 steps, before the stage 2 steps ahead: the
    // wait at the end of the iteration then leaves only that stage in flight
    if ((s & 3) == 0) issue_masks((s >> 2) + 1);
    const uint32_t st = base + (uint32_t)(slot3 * kStage);
    const uint32_t ms = base + ((s >> 2) & 1) * kPMaskSlot + 8 * (s & 1);
    const uint32_t mo = ((s >> 1) & 1) ? m_off1 : m_off0;
    u32x4_t a[RT];
    uint32_t mw[RT + 1];
    u32x4_t b[TT][2];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      a[i] = vld<u32x4_t>(st + a_off + 1024 * i);
      mw[i] = vld<uint32_t>(ms + mo + 512 * i);
    }
    mw[RT] = 0;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      b[t][0] = vld<u32x4_t>(st + b_off0 + 2048 * t);
      b[t][1] = vld<u32x4_t>(st + b_off1 + 2048 * t);
    }
    issue(s + 2);
#pragma unroll
    for (int i = 0; i < RT; i += 2) {
      const int idx = nib_codes2(__builtin_amdgcn_perm(mw[i + 1], mw[i], psel));
#pragma unroll
      for (int t = 0; t < TT; ++t)
        acc[i][t] = smfmac_half<BF, 0>(a[i], b[t][0], b[t][1], idx, acc[i][t]);
      if (i + 1 < RT) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
          acc[i + 1][t] = smfmac_half<BF, 1>(a[i + 1], b[t][0], b[t][1], idx, acc[i + 1][t]);
      }
    }
    // issue order: the LDS reads, then the products with the loads of step
    // s + 2 spread among them
    constexpr int kPer = RT * TT / kDma;  // products before each load
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * RT + 2 * TT, 0);
#pragma unroll
    for (int k = 0; k < kDma; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, RT * TT - kPer * kDma, 0);
    // every LDS read of this step has returned and step s + 1 has landed
    // (step s + 2 may be in flight): after the barrier, step s + 1 is
    // visible to all waves and slot s % 3 is free for step s + 3
    wait_lgkmcnt0();
    wait_vmcnt<kDma>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    slot3 = slot3 == kPNS - 1 ? 0 : slot3 + 1;
  }
  wait_vmcnt<0>();  // the trailing loads from the empty resource still write LDS

  // lane (j, n) of tile (i, t): rows 4 j .. 4 j + 3 of row tile i, token n;
  // one 16-byte (fp32) or 8-byte store per tile where vec (R % 4 == 0 and y
  // aligned to that size) and the 4 rows exist.  With K in several parts the
  // fp32 sums go to this part's slice of part (B x R each) instead.
  const int kind = part ? NM_F32 : out_kind & 0xff;
  if (part) {
    y = part + (int64_t)kpart * B * R;
    vec = (R & 3) == 0;
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int tok = tok0 + 16 * TT * wc + 16 * t + n;
    if (tok >= B) continue;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int r = row0 + 16 * RT * wr + 16 * i + 4 * j;
      const int64_t o = (int64_t)tok * R + r;
      if (vec && r + 3 < R) {
        if (kind == NM_F32) {
          *reinterpret_cast<f4v_t *>(static_cast<float *>(y) + o) = acc[i][t];
        } else {
          uint16_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = kind == NM_F16 ? __builtin_bit_cast(uint16_t, (_Float16)acc[i][t][e])
                                  : f32_to_bf16_rne(acc[i][t][e]);
          const uint2 v = {h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16};
          *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + o) = v;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (r + e < R) store_out(y, o + e, acc[i][t][e], kind);
      }
    }
  }
}

// Sum of the ks fp32 partial products of a split K (each n = B x R values,
// laid out as Y), in part order, into Y in out_kind; 4 values per thread
// where vec (n % 4 == 0 and Y aligned to 4 values).
__global__ __launch_bounds__(256) void nm_prefill_reduce_kernel(const float *__restrict__ part,
                                                               int ks, int64_t n, void *y,
                                                               int out_kind, int vec) {
  const int64_t i0 = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (i0 >= n) return;
  if (vec) {
    f4v_t s = *reinterpret_cast<const f4v_t *>(part + i0);
    for (int k = 1; k < ks; ++k) s += *reinterpret_cast<const f4v_t *>(part + k * n + i0);
    const int kind = out_kind & 0xff;
    if (kind == NM_F32) {
      *reinterpret_cast<f4v_t *>(static_cast<float *>(y) + i0) = s;
    } else {
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        h[e] = kind == NM_F16 ? __builtin_bit_cast(uint16_t, (_Float16)s[e]) : f32_to_bf16_rne(s[e]);
      const uint2 v = {h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16};
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + i0) = v;
    }
  } else {
    for (int64_t i = i0; i < i0 + 4 && i < n; ++i) {
      float s = part[i];
      for (int k = 1; k < ks; ++k) s += part[k * n + i];
      store_out(y, i, s, out_kind);
    }
  }
}

// Compute units and the LDS one workgroup may use, per device (queried once).
struct PrefillDev {
  int cus = 0;
  size_t lds = 0;
};
PrefillDev g_prefill_dev[64];
std::mutex g_prefill_mu;

nm_status prefill_device(PrefillDev *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return NM_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_prefill_mu);
  PrefillDev &d = g_prefill_dev[dev];
  if (d.cus == 0) {
    int cus = 0, lds = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return hip_fail(e);
    d.lds = (size_t)lds;
    d.cus = cus;
  }
  *out = d;
  return NM_OK;
}

// Split-K workspace of uncaptured calls: one per (device, stream), kept
// between calls and grown in stream order (the old one freed after the work
// already queued on the stream).  Calls on one stream run in order, so they
// can share it; the lock is held from the workspace lookup until both of a
// call's kernels are queued, so that calls made on one stream from several
// host threads cannot interleave their products and sums.  A call made
// while its stream is being captured takes a fresh stream-ordered
// allocation instead (a memory node of the graph), so that no graph shares
// memory with other work.  Measured on the 8B shapes (us per call, eager):
// 14336x4096 at 64 / 256 tokens 29.1 / 46.8 with an allocation per call,
// 24.8 / 42.8 with the kept workspace; 4096x14336 35.0 / 49.8 against
// 30.9 / 44.9.
struct PrefillWs {
  int dev;
  hipStream_t stream;
  float *ptr;
  size_t bytes;
};
std::vector<PrefillWs> g_prefill_ws;
std::mutex g_prefill_ws_mu;

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
  const int vec = rows % 4 == 0 && aligned(Y, out_dt == NM_F32 ? 16 : 8);
  PrefillDev dev;
  const nm_status ds = prefill_device(&dev);
  if (ds != NM_OK) return ds;
  // Tile shape: 7 or 8 row tiles and 1, 2 or 4 token tiles per wave, and K in
  // 1, 2, 4 or 8 parts (each at least 8 steps).  The time of a shape is taken as the rounds of
  // workgroups over the compute units times the bytes a workgroup stages
  // (values and mask words of 32 RT rows, x of 64 TT tokens, per step, over
  // its part of K), plus, for a split K, 2.5 times the bytes of the fp32
  // partial products written and summed (HBM traffic, at a lower rate than
  // the staging; the weight was fitted to a sweep of every tile shape and
  // split on the 8B gate and down shapes at 64..2048 tokens, where this
  // choice came within 2% of the fastest).  Small batches take narrow token
  // tiles, and a split K where the tiles alone leave compute units idle; ties
  // go to the earlier choice.
  const int64_t nk = cols / 64;
  int best_rt = 0, best_tt = 0, best_ks = 1;
  int64_t best = INT64_MAX, best_kper = nk;
  for (int ks : {1, 2, 4, 8}) {
    const int64_t kper = ((nk + ks - 1) / ks + 3) / 4 * 4;
    if (ks > 1 && (nk < 8 * ks || kper * (ks - 1) >= nk)) continue;
    for (int tt : {4, 2, 1}) {
      if ((size_t)prefill_lds(tt) > dev.lds) continue;
      for (int rt : {8, 7}) {
        const int64_t tiles =
            (rows + 32 * rt - 1) / (32 * rt) * ((batch + 64 * tt - 1) / (64 * tt)) * ks;
        int64_t c = (tiles + dev.cus - 1) / dev.cus * kper * (2304 * rt + 8192 * tt);
        if (ks > 1) c += 5 * (ks + 1) * batch * rows * 4 / (2 * dev.cus);
        if (c < best) best = c, best_rt = rt, best_tt = tt, best_ks = ks, best_kper = kper;
      }
    }
  }
  if (best_rt == 0) return NM_ERR_UNSUPPORTED;
  const int64_t nrt = (rows + 32 * best_rt - 1) / (32 * best_rt);
  const int64_t ntt = (batch + 64 * best_tt - 1) / (64 * best_tt);
  if (nrt * ntt * best_ks > INT32_MAX) return NM_ERR_INVALID_ARG;
  float *part = nullptr;
  bool part_owned = false;  // a per-call allocation, freed after the sum
  const hipStream_t hs = (hipStream_t)stream;
  std::unique_lock<std::mutex> ws_lock(g_prefill_ws_mu, std::defer_lock);
  if (best_ks > 1) {
    // the partial products (a split K is chosen only where the tiles leave
    // compute units idle, so they are small beside the weights)
    if ((batch * rows + 1023) / 1024 > INT32_MAX) return NM_ERR_INVALID_ARG;
    const size_t need = (size_t)best_ks * batch * rows * 4;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(hs, &cs);
    if (e != hipSuccess) return hip_fail(e);
    if (cs != hipStreamCaptureStatusNone) {
      e = hipMallocAsync((void **)&part, need, hs);
      if (e != hipSuccess) return hip_fail(e);
      part_owned = true;
    } else {
      int dv = 0;
      e = hipGetDevice(&dv);
      if (e != hipSuccess) return hip_fail(e);
      ws_lock.lock();
      PrefillWs *w = nullptr;
      for (PrefillWs &c : g_prefill_ws)
        if (c.dev == dv && c.stream == hs) w = &c;
      if (!w) {
        g_prefill_ws.push_back(PrefillWs{dv, hs, nullptr, 0});
        w = &g_prefill_ws.back();
      }
      if (w->bytes < need) {
        if (w->ptr) {
          e = hipFreeAsync(w->ptr, hs);
          w->ptr = nullptr;
          w->bytes = 0;
          if (e != hipSuccess) return hip_fail(e);
        }
        e = hipMallocAsync((void **)&w->ptr, need, hs);
        if (e != hipSuccess) {
          w->ptr = nullptr;
          return hip_fail(e);
        }
        w->bytes = need;
      }
      part = w->ptr;
    }
  }
  auto go = [&](auto fn, int tt) {
    hipLaunchKernelGGL(fn, dim3((unsigned)(nrt * ntt * best_ks)), dim3(kPWaves * kWave),
                       prefill_lds(tt), hs, (const uint16_t *)values, bits, (const uint16_t *)X, Y,
                       (int)batch, (int)rows, (int)cols, (int)nrt, (int)ntt, (int)out_dt, vec,
                       best_ks, (int)best_kper, part);
  };
  auto pick = [&](auto bf) {
    constexpr bool BF = decltype(bf)::value;
    const int key = best_rt * 10 + best_tt;
    switch (key) {
      case 84: go(nm_spmm_prefill_kernel<BF, 8, 4>, 4); break;
      case 82: go(nm_spmm_prefill_kernel<BF, 8, 2>, 2); break;
      case 81: go(nm_spmm_prefill_kernel<BF, 8, 1>, 1); break;
      case 74: go(nm_spmm_prefill_kernel<BF, 7, 4>, 4); break;
      case 72: go(nm_spmm_prefill_kernel<BF, 7, 2>, 2); break;
      default: go(nm_spmm_prefill_kernel<BF, 7, 1>, 1); break;
    }
  };
  if (in_dt == NM_BF16)
    pick(std::true_type{});
  else
    pick(std::false_type{});
  if (best_ks > 1) {
    const int64_t n = batch * rows;
    const int rvec = n % 4 == 0 && aligned(Y, out_dt == NM_F32 ? 16 : 8);
    const int64_t groups = (n + 3) / 4;
    hipLaunchKernelGGL(nm_prefill_reduce_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                       hs, part, best_ks, n, Y, (int)out_dt, rvec);
    hipError_t e = hipGetLastError();
    if (part_owned) {
      const hipError_t f = hipFreeAsync(part, hs);
      if (e == hipSuccess) e = f;
    }
    return e == hipSuccess ? NM_OK : hip_fail(e);
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

}  // extern "C"
