// nm_sparse.hip -- N:M bitmask sparse GEMV for AMD Instinct MI355X (gfx950).
//
// Kernels and the C ABI declared in include/nm_sparse.h.  What is computed
// follows "SparseDecoding: Decoding-Aware Pruning for Accurate and Efficient
// LLM Inference" (paper text):
//   - Method, kernel subsection, item (1) "Bitmask indexing": per row one bit
//     per column, kept weights stored in increasing column order;
//   - item (2) "Fixed-step bitmask traversal": a 50% N:M pattern with M
//     dividing 32 keeps half of the 32 columns of every word, so the loop
//     over a word runs a known number of steps; each step takes the least
//     significant set bit as the next kept column and clears it;
//   - Appendix C: one kernel per pattern with N and M fixed at compile time.
// The Triton/A100 kernel described there is prior art only; the design here
// is for CDNA4.  Batch 1 (and every pattern at batch <= 4) runs on the
// vector ALUs, where the HBM-bound matrix-vector product belongs:
//   - x is staged once per workgroup in LDS (the paper's kernel read x
//     through L1 instead) in a padded layout, so the per-nonzero gathers of
//     a wavefront spread over the LDS banks;
//   - each lane owns one 16-byte chunk of a row's values (8 kept weights, one
//     half of a mask word), so a wavefront reads 1 KiB of contiguous values
//     per load instruction with 128-bit loads;
//   - each lane walks its half-word in a fixed 8-step LSB scan (v_ffbl_b32),
//     pairs two gathered x values into one register and accumulates with
//     v_dot2_f32_{f16,bf16} (fp16/bf16 products are exact in fp32);
//   - one wavefront per row (or a few rows), reduced across lanes at the end.
// At batch 2..8 the per-token multiply-adds make that kernel ALU-bound, and
// the small-batch product moves to the matrix cores (2:4 on the sparse
// instruction, the other patterns through a decompressed tile), fed from the
// same stored format through LDS; see nm_spmm_mfma_kernel.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "nm_sparse.h"
#include "nm_device.h"
#include "nm_host.h"

// Scratch of the allocation-free pack (nm_pack_noalloc): element 0 counts
// the invalid groups of the running call.  256 bytes per device, held until
// the process ends.  Host code must use the per-device address from
// hipGetSymbolAddress, never this name.
constexpr int kPackScratchInts = 64;
static __device__ __align__(256) int scratch[kPackScratchInts];

namespace nm_host {

thread_local int g_last_hip = 0;

nm_status hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return NM_ERR_HIP;
}

bool pattern_ok(int n, int m) {
  return (m == 4 || m == 8 || m == 16 || m == 32) && 2 * n == m;
}

bool is16(nm_dtype d) { return d == NM_F16 || d == NM_BF16; }

bool out_ok(nm_dtype in, nm_dtype out) { return out == NM_F32 || out == in; }

bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

}  // namespace nm_host

namespace {

using namespace nm_host;

// LDS layout of a segment of x for the sparse kernel.  Column c of the
// segment holds the BP batch values of that column in one slot of SB bytes;
// the 32 slots of a mask word are followed by PB pad bytes, and PB bytes sit
// in front of word 0.  The pad shifts consecutive words across LDS banks.  A
// tail of 16 slots keeps the reads of a malformed mask word (fewer set bits
// than its pattern requires: the scan walks into the sentinel bits, an empty
// 2:4 nibble decodes to column 32) inside the allocation.
template <int BP>
struct XLay {
  static constexpr int SB = 2 * BP;
  static constexpr int PB = SB < 4 ? 4 : SB;
  static constexpr int WS = 32 * SB + PB;
  static constexpr int FP = PB;
  static constexpr size_t bytes(int seg_cols) {
    return FP + (size_t)(seg_cols / 32) * WS + 16 * SB;
  }
};

// Byte offset of the split reduction's partial sums in the batch-1 row
// kernel's LDS: after the x image, 16-byte aligned.
__host__ __device__ constexpr size_t split_lds_offset(int K) {
  return (XLay<1>::bytes(K) + 15) / 16 * 16;
}

// Staging of x into the XLay<BP> layout, one 8-column group at a time: the
// group's 16-byte chunk of each batch row is loaded, and for BP > 1 the
// chunks are transposed in registers into 8 column slots of BP values.
template <int BP>
struct XGroup {
  uint4 r[BP];
};

// Load group g (columns s0 + 8g .. +7) of every batch row; rows b >= B read
// row B-1 and are zeroed, so the number of loads issued never depends on B.
template <int BP>
__device__ __forceinline__ void xgroup_load(XGroup<BP> &xg, const uint16_t *__restrict__ x,
                                            int B, int K, int s0, int g) {
#pragma unroll
  for (int b = 0; b < BP; ++b) {
    const int bb = b < B ? b : B - 1;
    xg.r[b] = reinterpret_cast<const uint4 *>(x + (int64_t)bb * K + s0)[g];
  }
#pragma unroll
  for (int b = 1; b < BP; ++b)
    if (b >= B) xg.r[b] = make_uint4(0, 0, 0, 0);
}

template <int BP>
__device__ __forceinline__ void xgroup_store(char *lds, const XGroup<BP> &xg, int g) {
  using L = XLay<BP>;
  const int c0 = 8 * g;  // segment column of the group's first column
  char *wbase = lds + L::FP + (c0 >> 5) * L::WS + (c0 & 31) * L::SB;
  if constexpr (BP == 1) {
    uint32_t *d = reinterpret_cast<uint32_t *>(wbase);
    d[0] = xg.r[0].x;
    d[1] = xg.r[0].y;
    d[2] = xg.r[0].z;
    d[3] = xg.r[0].w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t d[BP / 2];
#pragma unroll
      for (int p = 0; p < BP / 2; ++p) {
        const uint4 &a = xg.r[2 * p], &b = xg.r[2 * p + 1];
        const uint32_t da = (e >> 1) == 0 ? a.x : (e >> 1) == 1 ? a.y : (e >> 1) == 2 ? a.z : a.w;
        const uint32_t db = (e >> 1) == 0 ? b.x : (e >> 1) == 1 ? b.y : (e >> 1) == 2 ? b.z : b.w;
        d[p] = (e & 1) ? ((da >> 16) | (db & 0xffff0000u)) : ((da & 0xffffu) | (db << 16));
      }
      char *dst = wbase + e * L::SB;
      if constexpr (BP == 2) {
        *reinterpret_cast<uint32_t *>(dst) = d[0];
      } else if constexpr (BP == 4) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(d[0], d[1]);
      } else {
        *reinterpret_cast<uint4 *>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
      }
    }
  }
}

// Stage groups first, first + step, ... of the segment [s0, s0 + S).
template <int BP>
__device__ __forceinline__ void stage_x_sparse(char *lds, const uint16_t *__restrict__ x,
                                               int B, int K, int s0, int S, int first,
                                               int step) {
  for (int g = first; g < S / 8; g += step) {
    XGroup<BP> xg;
    xgroup_load<BP>(xg, x, B, K, s0, g);
    xgroup_store<BP>(lds, xg, g);
  }
}

// x values of a kept pair of a lane's chunk (LDS slots p0, p1), multiplied
// with the packed weight pair w and accumulated for every batch row.
template <bool BF, int BP, typename P>
__device__ __forceinline__ void accum_pair(P p0, P p1, uint32_t w, float (&acc)[BP]) {
  if constexpr (BP == 1) {
    // two 16-bit LDS reads into the low and high halves of one register
    u16x2_t pr;
    pr[0] = ld<uint16_t>(p0);
    pr[1] = ld<uint16_t>(p1);
    acc[0] = dot2<BF>(w, __builtin_bit_cast(uint32_t, pr), acc[0]);
  } else {
    uint32_t X0[BP / 2], X1[BP / 2];
    if constexpr (BP == 2) {
      X0[0] = ld<uint32_t>(p0);
      X1[0] = ld<uint32_t>(p1);
    } else if constexpr (BP == 4) {
      const u32x2_t a = ld<u32x2_t>(p0);
      const u32x2_t b = ld<u32x2_t>(p1);
      X0[0] = a[0]; X0[1] = a[1];
      X1[0] = b[0]; X1[1] = b[1];
    } else {
      const u32x4_t a = ld<u32x4_t>(p0);
      const u32x4_t b = ld<u32x4_t>(p1);
      X0[0] = a[0]; X0[1] = a[1]; X0[2] = a[2]; X0[3] = a[3];
      X1[0] = b[0]; X1[1] = b[1]; X1[2] = b[2]; X1[3] = b[3];
    }
#pragma unroll
    for (int d = 0; d < BP / 2; ++d) {
      // (x0[b], x1[b]) pairs for batch rows b = 2d and 2d+1
      const uint32_t lo = (X0[d] & 0xffffu) | (X1[d] << 16);
      const uint32_t hi = (X0[d] >> 16) | (X1[d] & 0xffff0000u);
      acc[2 * d] = dot2<BF>(w, lo, acc[2 * d]);
      acc[2 * d + 1] = dot2<BF>(w, hi, acc[2 * d + 1]);
    }
  }
}

// The BP batch values of one x slot, as loaded from LDS.
template <int BP> struct SlotT { using T = u32x4_t; };
template <> struct SlotT<1> { using T = uint16_t; };
template <> struct SlotT<2> { using T = uint32_t; };
template <> struct SlotT<4> { using T = u32x2_t; };

// accum_pair on x slots already in registers.
template <bool BF, int BP>
__device__ __forceinline__ void accum_slots(typename SlotT<BP>::T a, typename SlotT<BP>::T b,
                                            uint32_t w, float (&acc)[BP]) {
  if constexpr (BP == 1) {
    acc[0] = dot2<BF>(w, (uint32_t)a | ((uint32_t)b << 16), acc[0]);
  } else if constexpr (BP == 2) {
    acc[0] = dot2<BF>(w, (a & 0xffffu) | (b << 16), acc[0]);
    acc[1] = dot2<BF>(w, (a >> 16) | (b & 0xffff0000u), acc[1]);
  } else {
#pragma unroll
    for (int d = 0; d < BP / 2; ++d) {
      acc[2 * d] = dot2<BF>(w, (a[d] & 0xffffu) | (b[d] << 16), acc[2 * d]);
      acc[2 * d + 1] = dot2<BF>(w, (a[d] >> 16) | (b[d] & 0xffff0000u), acc[2 * d + 1]);
    }
  }
}

// Generic fixed-step traversal (item (2)): the chunk's 8 kept weights are
// the 8 lowest set bits of m; each step takes the lowest set bit as the next
// kept column and clears it, and two steps feed one pair.  TOGETHER: the 8
// columns are found first and their x slots read together, one LDS round trip
// per chunk (8:16: gate 14336x4096 13.64 -> 13.26 us, k 1024x4096 3.70 ->
// 3.40 at batch 1); else each pair's reads follow its two steps, which
// overlaps the reads with the longer chain of 16:32 (whose odd lanes first
// clear 8 bits; 1-3% faster that way).
template <bool BF, int BP, bool TOGETHER = true>
__device__ __forceinline__ void chunk8_scan(const char *wb, uint32_t m, const uint4 v,
                                            float (&acc)[BP]) {
  using T = typename SlotT<BP>::T;
  const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
  if constexpr (!TOGETHER) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // m is never zero here (see the callers), so v_ffbl_b32 is well defined
      const int c0 = __builtin_ctz(m);
      m &= m - 1;
      const int c1 = __builtin_ctz(m);
      m &= m - 1;
      accum_pair<BF, BP>(wb + c0 * XLay<BP>::SB, wb + c1 * XLay<BP>::SB, vv[j], acc);
    }
    return;
  }
  int c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // m is never zero here (see the callers), so v_ffbl_b32 is well defined
    c[e] = __builtin_ctz(m) * XLay<BP>::SB;
    m &= m - 1;
  }
  T xs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) xs[e] = ld<T>(wb + c[e]);
#pragma unroll
  for (int j = 0; j < 4; ++j) accum_slots<BF, BP>(xs[2 * j], xs[2 * j + 1], vv[j], acc);
}

// 16:32: a word keeps 16 columns, lane h of the pair takes kept values
// 8h .. 8h + 7.  Lane 0 takes the word's 8 lowest set bits.  Lane 1 takes
// its 8 highest: it scans the bit-reversed word from the bottom, so both
// lanes walk 8 steps (rather than lane 1 first clearing 8 bits), finds the
// columns in descending order (column 31 - f), and so meets its values in
// reverse: the pair of steps 2j, 2j + 1 holds values 15 - 2j and 14 - 2j,
// which are the halves of the lane's value word 3 - j swapped.
template <bool BF, int BP>
__device__ __forceinline__ void chunk16_scan(const char *wb, uint32_t m, uint32_t h,
                                             const uint4 v, float (&acc)[BP]) {
  using T = typename SlotT<BP>::T;
  const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
  const uint32_t flip = h ? 31u : 0u;
  m = h ? __builtin_bitreverse32(m) : m;
  int c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // 16 set bits, so m is never zero here
    c[e] = (int)(((uint32_t)__builtin_ctz(m) ^ flip) * XLay<BP>::SB);
    m &= m - 1;
  }
  T xs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) xs[e] = ld<T>(wb + c[e]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = h ? __builtin_amdgcn_alignbit(vv[3 - j], vv[3 - j], 16) : vv[j];
    accum_slots<BF, BP>(xs[2 * j], xs[2 * j + 1], w, acc);
  }
}

// 2:4: nibble j of the lane's 16 columns holds exactly the pair j of kept
// weights, so its lowest and highest set bits are their columns: one ffbl and
// one ffbh per pair replace the serial scan.  A malformed nibble (no set bit)
// gives columns -1 and 32, inside the LDS pads.
// base - hz * SB in one v_mad_i32_i24 (the slot of column 31 - hz relative to
// column 31's slot); hz <= 32 and SB <= 16 fit the 24-bit operands.
template <int SB>
__device__ __forceinline__ uint32_t slot_from_top(int hz, uint32_t base31) {
  uint32_t r;
  if constexpr (SB == 2)
    asm("v_mad_i32_i24 %0, %1, -2, %2" : "=v"(r) : "v"(hz), "v"(base31));
  else if constexpr (SB == 4)
    asm("v_mad_i32_i24 %0, %1, -4, %2" : "=v"(r) : "v"(hz), "v"(base31));
  else if constexpr (SB == 8)
    asm("v_mad_i32_i24 %0, %1, -8, %2" : "=v"(r) : "v"(hz), "v"(base31));
  else
    asm("v_mad_i32_i24 %0, %1, -16, %2" : "=v"(r) : "v"(hz), "v"(base31));
  return r;
}

template <bool BF, int BP>
__device__ __forceinline__ void chunk8_nibbles(const char *lds, uint32_t base, uint32_t m,
                                               const uint4 v, float (&acc)[BP]) {
  constexpr int SB = XLay<BP>::SB;
  const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
  // LDS addresses as 32-bit integers, so that the slot arithmetic (one
  // lshl_add and one mad_i24 per pair) yields the final address
  const uint32_t b0 = (uint32_t)(size_t)(lds_ptr)lds + base;
  const uint32_t b31 = b0 + 31 * SB;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t n = m & (0xfu << (4 * j));
    const uint32_t o0 = b0 + (uint32_t)ffbl_hw(n) * SB;
    const uint32_t o1 = slot_from_top<SB>(ffbh_hw(n), b31);
    accum_pair<BF, BP>((lds_ptr)(size_t)o0, (lds_ptr)(size_t)o1, vv[j], acc);
  }
}

// Pattern kinds: the traversal a kernel is compiled for (Appendix C: one
// kernel per pattern, with N and M fixed at compile time).  kPat24x is 2:4 at
// batch 1 in the row kernel, with x stored plainly (see chunk24x); kPat24xE
// is the same where the load batches divide the row exactly (no chunk of a
// batch lies past the row end, so the guards of run_batch are left out).
enum { kPat24 = 0, kPatHalf = 1, kPat1632 = 2, kPat24x = 3, kPat24xE = 4, kPat48x = 5, kPat48xE = 6 };

// x stored plainly in LDS (column c at byte 2c): 2:4 at any batch, 4:8 at batch 1
__host__ __device__ constexpr bool plain_x(int pk) {
  return pk == kPat24x || pk == kPat24xE || pk == kPat48x || pk == kPat48xE;
}
__host__ __device__ constexpr bool is48(int pk) { return pk == kPat48x || pk == kPat48xE; }
__host__ __device__ constexpr bool exact_kind(int pk) { return pk == kPat24xE || pk == kPat48xE; }

__host__ __device__ constexpr int pattern_kind(int m) {
  return m == 4 ? kPat24 : m == 32 ? kPat1632 : kPatHalf;
}

// Process value chunk q (< nch) of a row with the lane's registers: select
// the lane's 16 columns of mask word q >> 1 and decode its 8 kept columns.
//   kPat24, kPatHalf (M <= 16): a half-word's 16 columns hold exactly 8 kept
//         weights, so the odd lane takes the upper 16 bits of the word;
//   kPat1632 (16:32): the 8 kept weights of the odd lane are set bits 8..15
//         of the word, so it first clears the 8 lowest set bits.
// 2:4 at batch 1 with x stored plainly in LDS (column c at byte 2c): the
// chunk's 16 columns are 32 contiguous bytes, read with two 16-byte LDS loads
// instead of one 2-byte gather per kept weight.  Pair j of the chunk is the
// two kept weights of nibble j, at in-group positions p0 < p1; its x operand
// {x[4j+p0], x[4j+p1]} is cut out of the group's two words by one v_perm
// with byte selector [2p0, 2p0+1, 2p1, 2p1+1].  The positions come from two
// 8-entry byte tables (themselves read with v_perm) indexed by n >> 1, which
// is unique for the six nibbles with two set bits (3, 5, 6, 9, 10, 12 ->
// 1..6).  No LDS address depends on the mask, so a malformed mask word only
// makes its row's sum undefined.
constexpr uint32_t kPos0Lo = 0x02000000u, kPos0Hi = 0x00040200u;  // n >> 1 -> 2 p0
constexpr uint32_t kPos1Lo = 0x04040200u, kPos1Hi = 0x00060606u;  // n >> 1 -> 2 p1

// chunk24x_ops takes the chunk's 32 bytes of x (xa: columns 0..7, xc:
// columns 8..15) already read from LDS.
template <bool BF>
__device__ __forceinline__ void chunk24x_ops(int q, uint32_t mw, const uint4 v, const u32x4_t xa,
                                             const u32x4_t xc, float &acc) {
  const uint32_t m = (mw >> ((q & 1) << 4)) & 0xffffu;
  const uint32_t X[8] = {xa[0], xa[1], xa[2], xa[3], xc[0], xc[1], xc[2], xc[3]};
  // table indices n >> 1 of nibbles 0, 2, 1, 3 in bytes 0..3
  const uint32_t t = m >> 1;
  const uint32_t S = (t & 0x0707u) | (((t >> 4) & 0x0707u) << 16);
  const uint32_t P0 = __builtin_amdgcn_perm(kPos0Hi, kPos0Lo, S);
  const uint32_t P1 = __builtin_amdgcn_perm(kPos1Hi, kPos1Lo, S);
  const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
  // selector bytes [b, b, 4 + b, 4 + b] with b the byte of nibble j in P0 / P1
  constexpr uint32_t kPick[4] = {0x04040000u, 0x06060202u, 0x05050101u, 0x07070303u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel = __builtin_amdgcn_perm(P1, P0, kPick[j]) | 0x01000100u;
    const uint32_t xs = __builtin_amdgcn_perm(X[2 * j + 1], X[2 * j], sel);
    acc = dot2<BF>(vv[j], xs, acc);
  }
}

// chunk24x_ops for BP tokens whose x rows are stored plainly one after
// another in LDS (token b's columns at b * xrow): the nibble selectors are
// computed once and cut every token's pair operand out of its own 32 bytes.
template <bool BF, int BP>
__device__ __forceinline__ void chunk24x_multi(const char *lds, int xrow, int q, uint32_t mw,
                                               const uint4 v, float (&acc)[BP]) {
  const uint32_t m = (mw >> ((q & 1) << 4)) & 0xffffu;
  const uint32_t t = m >> 1;
  const uint32_t S = (t & 0x0707u) | (((t >> 4) & 0x0707u) << 16);
  const uint32_t P0 = __builtin_amdgcn_perm(kPos0Hi, kPos0Lo, S);
  const uint32_t P1 = __builtin_amdgcn_perm(kPos1Hi, kPos1Lo, S);
  const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
  constexpr uint32_t kPick[4] = {0x04040000u, 0x06060202u, 0x05050101u, 0x07070303u};
  uint32_t sel[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sel[j] = __builtin_amdgcn_perm(P1, P0, kPick[j]) | 0x01000100u;
#pragma unroll
  for (int b = 0; b < BP; ++b) {
    const lds_ptr xb = (lds_ptr)lds + b * xrow + 32 * q;
    const u32x4_t xa = ld<u32x4_t>(xb), xc = ld<u32x4_t>(xb + 16);
    const uint32_t X[8] = {xa[0], xa[1], xa[2], xa[3], xc[0], xc[1], xc[2], xc[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[b] = dot2<BF>(vv[j], __builtin_amdgcn_perm(X[2 * j + 1], X[2 * j], sel[j]), acc[b]);
  }
}

// chunk24x_multi with every token's 32 bytes of x already read from LDS
// (xa[b]: columns 0..7 of token b, xc[b]: columns 8..15).
template <bool BF, int BP>
__device__ __forceinline__ void chunk24x_multi_ops(int q, uint32_t mw, const uint4 v,
                                                   const u32x4_t (&xa)[BP],
                                                   const u32x4_t (&xc)[BP], float (&acc)[BP]) {
  const uint32_t m = (mw >> ((q & 1) << 4)) & 0xffffu;
  const uint32_t t = m >> 1;
  const uint32_t S = (t & 0x0707u) | (((t >> 4) & 0x0707u) << 16);
  const uint32_t P0 = __builtin_amdgcn_perm(kPos0Hi, kPos0Lo, S);
  const uint32_t P1 = __builtin_amdgcn_perm(kPos1Hi, kPos1Lo, S);
  const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
  constexpr uint32_t kPick[4] = {0x04040000u, 0x06060202u, 0x05050101u, 0x07070303u};
  uint32_t sel[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sel[j] = __builtin_amdgcn_perm(P1, P0, kPick[j]) | 0x01000100u;
#pragma unroll
  for (int b = 0; b < BP; ++b) {
    const uint32_t X[8] = {xa[b][0], xa[b][1], xa[b][2], xa[b][3],
                           xc[b][0], xc[b][1], xc[b][2], xc[b][3]};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[b] = dot2<BF>(vv[j], __builtin_amdgcn_perm(X[2 * j + 1], X[2 * j], sel[j]), acc[b]);
  }
}

// Read chunk q's 32 bytes of x of every token (token b's row at b * xrow).
template <int BP>
__device__ __forceinline__ void x_multi(const char *lds, int xrow, int q, u32x4_t (&xa)[BP],
                                        u32x4_t (&xc)[BP]) {
#pragma unroll
  for (int b = 0; b < BP; ++b) {
    const lds_ptr xb = (lds_ptr)lds + b * xrow + 32 * q;
    xa[b] = ld<u32x4_t>(xb);
    xc[b] = ld<u32x4_t>(xb + 16);
  }
}

template <bool BF>
__device__ __forceinline__ void chunk24x(const char *lds, int q, uint32_t mw, const uint4 v,
                                         float &acc) {
  const lds_ptr xb = (lds_ptr)lds + 32 * q;
  chunk24x_ops<BF>(q, mw, v, ld<u32x4_t>(xb), ld<u32x4_t>(xb + 16), acc);
}

// 4:8 at batch 1 with x stored plainly.  Every byte of a valid 4:8 mask word
// keeps exactly 4 of its 8 columns, i.e. the chunk's two bytes hold the kept
// pairs (p0, p1), (p2, p3) of their own 8 columns (four x registers).  The
// pair's x operand is cut out of the two 4-column windows with two v_perm and
// joined with an or: a selector byte of 12 yields zero, so each window
// contributes only the columns that lie in it.  The four selectors of a mask
// byte (pair 0: window 0, window 1; pair 1: window 0, window 1) come from a
// 256-entry table in LDS (pair48_table); a malformed byte selects some
// columns of its own 8, so only its row's sum is undefined.
constexpr int kPair48TableBytes = 256 * 16;

__device__ __forceinline__ uint32_t pair48_sel(int a, int c, int w) {
  const uint32_t sa = (a >> 2) == w ? (uint32_t)(2 * (a & 3)) : 12u;
  const uint32_t sc = (c >> 2) == w ? (uint32_t)(2 * (c & 3)) : 12u;
  const uint32_t sa1 = sa == 12u ? 12u : sa + 1, sc1 = sc == 12u ? 12u : sc + 1;
  return sa | (sa1 << 8) | (sc << 16) | (sc1 << 24);
}

// Table entry of mask byte b: the selectors of its two kept pairs.
__device__ __forceinline__ u32x4_t pair48_entry(uint32_t b) {
  int p[4];
  uint32_t t = b;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    p[k] = ffbl_hw(t) & 7;  // an exhausted (malformed) byte repeats a column
    t &= t - 1;
  }
  return (u32x4_t){pair48_sel(p[0], p[1], 0), pair48_sel(p[0], p[1], 1), pair48_sel(p[2], p[3], 0),
                   pair48_sel(p[2], p[3], 1)};
}

template <bool BF>
__device__ __forceinline__ void chunk48x_ops(const char *table, int q, uint32_t mw, const uint4 v,
                                             const u32x4_t xa, const u32x4_t xc, float &acc) {
  const uint32_t m = (mw >> ((q & 1) << 4)) & 0xffffu;
  const u32x4_t e0 = ld<u32x4_t>((lds_ptr)table + 16 * (m & 0xffu));
  const u32x4_t e1 = ld<u32x4_t>((lds_ptr)table + 16 * (m >> 8));
  const uint32_t x0 = __builtin_amdgcn_perm(xa[1], xa[0], e0[0]) | __builtin_amdgcn_perm(xa[3], xa[2], e0[1]);
  const uint32_t x1 = __builtin_amdgcn_perm(xa[1], xa[0], e0[2]) | __builtin_amdgcn_perm(xa[3], xa[2], e0[3]);
  const uint32_t x2 = __builtin_amdgcn_perm(xc[1], xc[0], e1[0]) | __builtin_amdgcn_perm(xc[3], xc[2], e1[1]);
  const uint32_t x3 = __builtin_amdgcn_perm(xc[1], xc[0], e1[2]) | __builtin_amdgcn_perm(xc[3], xc[2], e1[3]);
  acc = dot2<BF>(v.x, x0, acc);
  acc = dot2<BF>(v.y, x1, acc);
  acc = dot2<BF>(v.z, x2, acc);
  acc = dot2<BF>(v.w, x3, acc);
}

// The plain-x chunk of a batch-1 kind: x operands already read from LDS.
template <bool BF, int PK>
__device__ __forceinline__ void chunk_plain_ops(const char *lds, int nch, int q, uint32_t mw,
                                                const uint4 v, const u32x4_t xa, const u32x4_t xc,
                                                float &acc) {
  if constexpr (is48(PK))
    chunk48x_ops<BF>(lds + 32 * nch, q, mw, v, xa, xc, acc);  // the table follows x
  else
    chunk24x_ops<BF>(q, mw, v, xa, xc, acc);
}

template <bool BF, int BP, int PK>
__device__ __forceinline__ void chunk(const char *lds, int q, uint32_t mw, const uint4 v,
                                      float (&acc)[BP]) {
  using L = XLay<BP>;
  if constexpr (plain_x(PK)) {  // (run_batch handles the plain kinds itself)
    if constexpr (BP == 1) chunk24x<BF>(lds, q, mw, v, acc[0]);
    return;
  }
  const uint32_t h = q & 1;
  uint32_t base = L::FP + (uint32_t)(q >> 1) * L::WS;
  uint32_t m = mw;
  if constexpr (PK == kPat24) {
    m >>= (h << 4);
    base += h * (16 * L::SB);
    chunk8_nibbles<BF, BP>(lds, base, m, v, acc);
  } else if constexpr (PK == kPatHalf) {
    // the lane's 16 columns in the low half; the sentinel bits above them
    // keep every scan step on a nonzero word
    m = (m >> (h << 4)) | 0xffff0000u;
    base += h * (16 * L::SB);
    chunk8_scan<BF, BP>(lds + base, m, v, acc);
  } else {
    // a word without exactly 16 set bits is replaced by one that keeps the
    // scan in range (its row's result is then undefined)
    if (__popc(m) != 16) m = 0xffffu;
    if constexpr (BP == 1) {
      // (one token: lane 1 clears its 8 lower set bits first; the reversed
      // scan measured 1-8% slower here, 15% faster on 6144x4096 at batch 2-4)
      if (h) {
#pragma unroll
        for (int k = 0; k < 8; ++k) m &= m - 1;
      }
      chunk8_scan<BF, BP, false>(lds + base, m, v, acc);
    } else {
      chunk16_scan<BF, BP>(lds + base, m, h, v, acc);
    }
  }
}

// Registers of one load batch: U value chunks and their mask words.
template <int U>
struct Batch {
  uint4 v[U];
  uint32_t m[U];
};

// Load batch t of a row segment: lane l gets value chunks t*64U + l + 64u
// (u < U) and their mask words.  Raw buffer loads: the resource holds the
// batch's base and the bytes left in the segment, so the per-lane offsets are
// loop-invariant and a chunk past the end reads zeros (the hardware range
// check) without touching memory.  nch = 0 makes a dummy
// batch that keeps the wait counts uniform and costs no memory traffic.
// MF: the mask words are issued before the values, so the first chunk of a
// batch waits for one value load less.
template <int U, bool MF = false>
__device__ __forceinline__ void load_batch(Batch<U> &bt, const uint4 *vrow,
                                           const uint32_t *brow, int nch, int t, int lane) {
  // the resources start at the batch (scalar arithmetic) and end at the row
  // end, so the range check, which covers the vector offsets, zeroes every
  // chunk past the row
  const int c0 = t * (kWave * U), left = nch - c0 > 0 ? nch - c0 : 0;
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void *)(vrow + c0), 0, left * 16, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void *)(brow + c0 / 2), 0, left * 2, kRsrcWord3);
  if constexpr (MF) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      bt.m[u] = __builtin_amdgcn_raw_buffer_load_b32(rb, (lane >> 1) * 4 + u * kWave * 2, 0,
                                                     kStreamAux);
#pragma unroll
    for (int u = 0; u < U; ++u)
      bt.v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rv, lane * 16 + u * kWave * 16, 0, kStreamAux));
    return;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    bt.v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rv, lane * 16 + u * kWave * 16, 0, kStreamAux));
    bt.m[u] = __builtin_amdgcn_raw_buffer_load_b32(rb, (lane >> 1) * 4 + u * kWave * 2, 0,
                                                   kStreamAux);
  }
}

// Consume a load batch.  A chunk past the row end (zeros, see load_batch) is
// computed like any other at the row's last column range, without a branch,
// and its sum is dropped by a select.  Straight-line code keeps the wait
// counts of the pipeline exact.
// qb (plain-x kinds): the batch's first chunk, t * 64 * U, a wave-uniform
// value.  A batch that ends inside the row takes the guard-free code; in the
// row's last batch, groups of 64 chunks wholly past the row end are skipped by
// a uniform branch.
template <bool BF, int BP, int PK, int U>
__device__ __forceinline__ void run_batch(const char *lds, const Batch<U> &bt, int q0, int nch,
                                          float (&acc)[BP], int qb = 0) {
  if constexpr (plain_x(PK) && BP > 1) {
    // 2:4 at batch 2..8 with x stored plainly (token b's row at b * 32 nch)
    static_assert(!is48(PK), "the plain 4:8 kind is for batch 1");
    if (exact_kind(PK) || qb + kWave * U <= nch) {
      // the x operands of a chunk are read for up to 4 tokens at once, ahead
      // of their use (their LDS addresses do not depend on the loaded data,
      // so the first reads overlap the wait for the batch), within 32..64
      // registers of x (the row kernel's launch bound leaves 128 VGPRs): every
      // chunk's at batch 2 in the exact kind (the other kind also holds the
      // ragged batch's code), else a chunk's at a time, at batch 8 in two
      // halves of 4 tokens
      if constexpr (U * BP <= 8 && exact_kind(PK)) {
        u32x4_t xa[U][BP], xc[U][BP];
#pragma unroll
        for (int u = 0; u < U; ++u) x_multi<BP>(lds, 32 * nch, q0 + kWave * u, xa[u], xc[u]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
          chunk24x_multi_ops<BF, BP>(q0 + kWave * u, bt.m[u], bt.v[u], xa[u], xc[u], acc);
      } else {
        constexpr int G = BP < 4 ? BP : 4;  // tokens per group of reads
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int g = 0; g < BP; g += G) {
            u32x4_t xa[G], xc[G];
            x_multi<G>(lds + g * 32 * nch, 32 * nch, q0 + kWave * u, xa, xc);
            __builtin_amdgcn_sched_barrier(0);
            float part[G];
#pragma unroll
            for (int b = 0; b < G; ++b) part[b] = acc[g + b];
            chunk24x_multi_ops<BF, G>(q0 + kWave * u, bt.m[u], bt.v[u], xa, xc, part);
#pragma unroll
            for (int b = 0; b < G; ++b) acc[g + b] = part[b];
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (qb + kWave * u >= nch) break;  // uniform: the rest of the batch is past the row end
      const int q = q0 + kWave * u;
      float part[BP];
#pragma unroll
      for (int b = 0; b < BP; ++b) part[b] = 0.f;
      chunk24x_multi<BF, BP>(lds, 32 * nch, min(q, nch - 1), bt.m[u], bt.v[u], part);
#pragma unroll
      for (int b = 0; b < BP; ++b) acc[b] += q < nch ? part[b] : 0.f;
    }
    return;
  } else if constexpr (plain_x(PK)) {
    if (exact_kind(PK) || qb + kWave * U <= nch) {
      // the x operands of every chunk first: their LDS addresses do not
      // depend on the loaded data, so the reads overlap the wait for the batch
      u32x4_t xa[U], xc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const lds_ptr xb = (lds_ptr)lds + 32 * (q0 + kWave * u);
        xa[u] = ld<u32x4_t>(xb);
        xc[u] = ld<u32x4_t>(xb + 16);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
        chunk_plain_ops<BF, PK>(lds, nch, q0 + kWave * u, bt.m[u], bt.v[u], xa[u], xc[u], acc[0]);
      return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (qb + kWave * u >= nch) break;
      const int q = q0 + kWave * u;
      const int qc = min(q, nch - 1);
      float part = 0.f;
      const lds_ptr xb = (lds_ptr)lds + 32 * qc;
      chunk_plain_ops<BF, PK>(lds, nch, qc, bt.m[u], bt.v[u], ld<u32x4_t>(xb), ld<u32x4_t>(xb + 16),
                              part);
      acc[0] += q < nch ? part : 0.f;
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int q = q0 + kWave * u;
    const int qc = min(q, nch - 1);
    float part[BP];
#pragma unroll
    for (int b = 0; b < BP; ++b) part[b] = 0.f;
    chunk<BF, BP, PK>(lds, qc, bt.m[u], bt.v[u], part);
#pragma unroll
    for (int b = 0; b < BP; ++b) acc[b] += q < nch ? part[b] : 0.f;
  }
}

template <int BP>
__device__ __forceinline__ void finish_row(float (&acc)[BP], void *y, int B, int64_t R,
                                           int64_t r, int lane, int out_kind) {
#pragma unroll
  for (int b = 0; b < BP; ++b) {
    const float s = wave_sum_to_63(acc[b]);
    if (lane == kWave - 1 && b < B) store_out(y, (int64_t)b * R + r, s, out_kind);
    acc[b] = 0.f;
  }
}

// Reduce the row sums of the wave's row i and park them in lane i of res
// (no store inside the item loop; the wave stores its rows once at the end).
template <int BP>
__device__ __forceinline__ void collect_row(float (&acc)[BP], float (&res)[BP], int i, int lane) {
#pragma unroll
  for (int b = 0; b < BP; ++b) {
    const float s = wave_sum_to_63(acc[b]);
    const float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), kWave - 1));
    res[b] = lane == i ? sv : res[b];
    acc[b] = 0.f;
  }
}

// Sparse product when all of x fits the LDS budget (the common case).  x is
// staged once per workgroup; wave w of the grid owns the rpw consecutive rows
// from w * rpw.  Its work is a sequence of items (row, load batch of U chunks
// per lane) run as a two-stage software pipeline: the loads of item k+1 are
// in flight while item k is consumed.  U is chosen per shape so that it
// divides the row's chunks per lane (no idle load slots in the last batch).  The first item's loads are issued
// before x is committed to LDS, so the x and weight latencies overlap.
// xdma (the plain-x kinds only): x's LDS image is x itself, BP rows of K
// values, and is copied by direct-to-LDS loads issued before the weights',
// instead of passing through registers; the host takes it where the image is
// large beside the workgroup's weights (batch >= 2, or at most 4 rows per
// workgroup).
template <bool BF, int BP, int PK, int U, int XS, int KS = 1>
__global__ __launch_bounds__(1024) void nm_spmv_rows_kernel(
    const uint4 *__restrict__ values, const uint32_t *__restrict__ bits,
    const uint16_t *__restrict__ x, void *__restrict__ y, int B, int64_t R, int K, int rpw,
    int out_kind, int xdma) {
  // XS: x groups per thread held in registers before the weight loads (the
  // host picks enough for all of x where it can: a group left to the staging
  // loop below waits for every outstanding load, the weights' included)
  // KS: waves per row group (the split reduction; 1 = one wave per row)
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wpg = blockDim.x / kWave;
  const int nch = K >> 4;                                // value chunks per row
  const int nb = (nch + kWave * U - 1) / (kWave * U);    // load batches per row
  // wave index as a wave-uniform (scalar) value: the item loop below is then
  // scalar control flow and the wait counts of the pipeline stay exact
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // row group of the wave and its place in the group: with KS > 1 the KS
  // waves of a group share its rows, wave `sub` taking the load batches
  // sub, sub + KS, ... of each row (KS divides nb; exact kinds only)
  const int grp = wid / KS, sub = wid - grp * KS;
  const int nbs = nb / KS;                               // this wave's batches per row
  const int64_t r0 = ((int64_t)blockIdx.x * (wpg / KS) + grp) * rpw;
  const int64_t left = R - r0;
  const int nrows = left <= 0 ? 0 : (left < rpw ? (int)left : rpw);
  const int nitems = nrows * nbs;
  const int64_t cpr = nch, wpr = K >> 5;
  static_assert(KS == 1 || PK == kPat24xE, "the split reduction is built for the exact 2:4 kind");

  float acc[BP];
#pragma unroll
  for (int b = 0; b < BP; ++b) acc[b] = 0.f;
  const bool swiglu = (out_kind >> kEpiShift) == kEpiSwiglu;
  if (K == 0) {  // every sum is empty
    if (swiglu) {  // silu(0) * 0 for every pair of the wave (r0 and nrows are even)
      if (lane == 0)
        for (int r = 0; r < nrows; r += 2)
          for (int b = 0; b < B; ++b) store_out(y, (int64_t)b * (R / 2) + (r0 + r) / 2, 0.f, out_kind);
      return;
    }
    for (int r = 0; r < nrows; ++r) finish_row<BP>(acc, y, B, R, r0 + r, lane, out_kind);
    return;
  }

  // x: the first XS groups per thread are loaded, then the weights of the
  // wave's first two items, then the groups are written to LDS.  Every load
  // here is issued unconditionally (indices clamped, dummy batches) so that
  // the waits before the LDS writes count exactly and leave the weight loads
  // in flight.  With xdma the waves instead copy x's image in 1 KiB pieces
  // (lane i's 16 bytes of piece p land at byte 1024 p + 16 i; rows of the
  // image past B read as zeros through the range check), then issue the
  // weights, and wait for the copies only.
  const int ngx = K >> 3;
  // (the host takes xdma at every batch >= 2: those kinds have no other path)
  constexpr bool kDmaOnly = plain_x(PK) && BP >= 2;
  const bool xd = kDmaOnly || (plain_x(PK) && xdma != 0);
  if (xd) {
    const __amdgpu_buffer_rsrc_t rxs =
        __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, B * K * 2, kRsrcWord3);
    const int nq = BP * ngx;  // 16-byte pieces of the image
    const uint32_t lbase = (uint32_t)(size_t)(lds_ptr)lds;
    for (int q0 = wid * kWave; q0 < nq; q0 += wpg * kWave)
      if (q0 + lane < nq) lds_load16(rxs, lbase + 16 * q0, 16 * (q0 + lane), 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  XGroup<BP> xg[XS];
  if constexpr (kDmaOnly) {
    (void)xg;
  } else if constexpr (plain_x(PK)) {
    // buffer loads (rows past B read as zeros); under xdma the resource is
    // empty, so the same loads are issued without a branch and move no data
    const __amdgpu_buffer_rsrc_t rxg =
        __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, xd ? 0 : B * K * 2, kRsrcWord3);
#pragma unroll
    for (int s = 0; s < XS; ++s)
#pragma unroll
      for (int b = 0; b < BP; ++b)
        xg[s].r[b] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       rxg, b * K * 2 + 16 * min((int)threadIdx.x + s * (int)blockDim.x, ngx - 1), 0, 0));
  } else {
#pragma unroll
    for (int s = 0; s < XS; ++s)
      xgroup_load<BP>(xg[s], x, B, K, 0, min((int)threadIdx.x + s * (int)blockDim.x, ngx - 1));
  }
  // the wave's items k = 0, 1 are in flight before x is committed to LDS;
  // an item past the wave's last is a dummy load (no memory traffic)
  auto item_load = [&](Batch<U> &bt, int k) {
    const bool real = k < nitems;
    const int ii = real ? k / nbs : 0, tt = real ? sub + KS * (k - ii * nbs) : 0;
    const int64_t r = real ? r0 + ii : 0;
    load_batch<U, plain_x(PK)>(bt, values + r * cpr, bits + r * wpr, real ? nch : 0, tt, lane);
  };
  Batch<U> A, Bt;
  item_load(A, 0);
  item_load(Bt, 1);
  // clamped groups rewrite group ngx-1 with the same data it already holds
  if constexpr (is48(PK)) {  // the 4:8 pair selectors, after x
    u32x4_t *table = reinterpret_cast<u32x4_t *>(lds + 2 * (size_t)K);
    for (int b = threadIdx.x; b < 256; b += blockDim.x) table[b] = pair48_entry((uint32_t)b);
  }
  if (xd) {
    // the copies were issued before the two items' 4U loads, and loads
    // complete in issue order
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<4 * U>();
    // the empty register loads are consumed here too, so that the compiler
    // keeps them ahead of the branch (used on one side only, it would sink
    // them below the weight loads of the other)
    if constexpr (!kDmaOnly) {
#pragma unroll
      for (int s = 0; s < XS; ++s)
#pragma unroll
        for (int b = 0; b < BP; ++b)
          asm volatile("" ::"v"(xg[s].r[b].x), "v"(xg[s].r[b].y), "v"(xg[s].r[b].z),
                       "v"(xg[s].r[b].w));
    }
  } else if constexpr (plain_x(PK) && !kDmaOnly) {  // token b's group g at byte b * 2K + 16 g
#pragma unroll
    for (int s = 0; s < XS; ++s)
#pragma unroll
      for (int b = 0; b < BP; ++b)
        reinterpret_cast<uint4 *>(lds)[b * ngx + min((int)threadIdx.x + s * (int)blockDim.x, ngx - 1)] =
            xg[s].r[b];
    for (int g = threadIdx.x + XS * blockDim.x; g < ngx; g += blockDim.x)
#pragma unroll
      for (int b = 0; b < BP; ++b)
        reinterpret_cast<uint4 *>(lds)[b * ngx + g] =
            b < B ? reinterpret_cast<const uint4 *>(x + (int64_t)b * K)[g] : make_uint4(0, 0, 0, 0);
  } else if constexpr (!plain_x(PK)) {
#pragma unroll
    for (int s = 0; s < XS; ++s)
      xgroup_store<BP>(lds, xg[s], min((int)threadIdx.x + s * (int)blockDim.x, ngx - 1));
    stage_x_sparse<BP>(lds, x, B, K, 0, K, threadIdx.x + XS * blockDim.x, blockDim.x);
  }
  __syncthreads();

  float res[BP];  // lane i holds the sums of the wave's row i
#pragma unroll
  for (int b = 0; b < BP; ++b) res[b] = 0.f;
  // two-buffer pipeline: while one batch is consumed the other is in flight
  for (int k = 0; k < nitems; k += 2) {
    const int i = k / nbs, j = k - i * nbs, t = sub + KS * j;
    run_batch<BF, BP, PK, U>(lds, A, t * kWave * U + lane, nch, acc, t * kWave * U);
    if (j == nbs - 1) collect_row<BP>(acc, res, i, lane);
    item_load(A, k + 2);
    if (k + 1 >= nitems) break;
    const int i1 = (k + 1) / nbs, j1 = (k + 1) - i1 * nbs, t1 = sub + KS * j1;
    run_batch<BF, BP, PK, U>(lds, Bt, t1 * kWave * U + lane, nch, acc, t1 * kWave * U);
    if (j1 == nbs - 1) collect_row<BP>(acc, res, i1, lane);
    item_load(Bt, k + 3);
  }
  if constexpr (KS > 1) {
    // the split reduction: each wave's partial row sums (lane i: row i of the
    // group) meet in LDS after the x image; the group's first wave adds them
    // in wave order and stores the rows
    float *part = reinterpret_cast<float *>(lds + split_lds_offset(K));
    if (lane < rpw) part[wid * rpw + lane] = res[0];
    __syncthreads();
    if (sub == 0 && lane < nrows) {
      float sum = part[grp * KS * rpw + lane];
#pragma unroll
      for (int w = 1; w < KS; ++w) sum += part[(grp * KS + w) * rpw + lane];
      store_out(y, r0 + lane, sum, out_kind);
    }
    return;
  }
  if (swiglu) {
    // the wave's rows come in (gate, up) pairs at even offsets: lane 2p
    // takes its up sum from lane 2p + 1 and stores pair p
#pragma unroll
    for (int b = 0; b < BP; ++b) {
      const float u = __shfl_down(res[b], 1);
      if ((lane & 1) == 0 && lane < nrows && b < B)
        store_out(y, (int64_t)b * (R / 2) + (r0 + lane) / 2, silu(res[b]) * u, out_kind);
    }
    return;
  }
  if (lane < nrows) {
#pragma unroll
    for (int b = 0; b < BP; ++b)
      if (b < B) store_out(y, (int64_t)b * R + r0 + lane, res[b], out_kind);
  }
}

// Sparse product when x does not fit the LDS budget in one piece.
// Workgroup g owns rows g*WPG*RPW + i*WPG + wave (i < RPW), processed
// together; K is walked in segments of `seg` columns, each staged in LDS once
// per workgroup, and the RPW x BP accumulators live in registers throughout.
// Lane l of a wave handles value chunks l, l+64, ... of the segment; chunk q
// is half (q & 1) of mask word q >> 1 (see chunk()).
template <bool BF, int BP, int PK, int RPW>
__global__ __launch_bounds__(1024) void nm_spmv_seg_kernel(
    const uint4 *__restrict__ values, const uint32_t *__restrict__ bits,
    const uint16_t *__restrict__ x, void *__restrict__ y, int B, int64_t R,
    int K, int seg, int out_kind) {
  constexpr int U = RPW >= 4 ? 2 : 4;  // chunks per lane per load batch
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wpg = blockDim.x / kWave;
  const int64_t row0 =
      (int64_t)blockIdx.x * wpg * RPW + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t cpr = K >> 4;  // 16-byte value chunks per row
  const int64_t wpr = K >> 5;  // mask words per row

  float acc[RPW][BP];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int b = 0; b < BP; ++b) acc[i][b] = 0.f;

  for (int s0 = 0; s0 < K; s0 += seg) {
    const int S = min(seg, K - s0);
    if (s0) __syncthreads();  // all waves are done with the previous segment
    stage_x_sparse<BP>(lds, x, B, K, s0, S, threadIdx.x, blockDim.x);
    __syncthreads();
    const int nch = S >> 4;
    const int64_t cbeg = s0 >> 4;
    for (int t0 = 0; t0 < nch; t0 += kWave * U) {
      Batch<U> bt[RPW];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        // rows past R reload row R-1 (wave-uniform) and are never stored
        const int64_t r = min(row0 + (int64_t)i * wpg, R - 1);
        load_batch<U>(bt[i], values + r * cpr + cbeg, bits + r * wpr + (cbeg >> 1), nch,
                      t0 / (kWave * U), lane);
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i)
        run_batch<BF, BP, PK, U>(lds, bt[i], t0 + lane, nch, acc[i]);
    }
  }

#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int64_t r = row0 + (int64_t)i * wpg;
    if (r < R) finish_row<BP>(acc[i], y, B, R, r, lane, out_kind);  // uniform per wave
  }
}

// ---------------------------------------------------------------------------
// 2:4 small batch on the sparse matrix cores.
//
// At batch 2..8 the VALU kernel's work per kept weight grows with the batch
// (one dot2 per token per pair plus the gathers), so for 2:4 the product runs
// on gfx950's v_smfmac_f32_16x16x64_{f16,bf16}: A is a 16 x 64 2:4-sparse
// tile given as its kept values plus a 2-bit in-group position per kept
// value, B a dense 64 x 16 tile, D += A.B in fp32.  The bitmask format maps
// onto it directly (Method item (1)): a lane's 16 columns of a row hold
// exactly 8 kept values, 16 contiguous bytes of `values`, and their position
// codes come from the lane's 16 mask bits.  Operand layout (established on
// the device against a CPU product): lane l = 16 j + n holds
//   A: row n of the tile, dense columns 16 j .. 16 j + 15 of the step;
//   B: column n (the token), dense columns 8 j .. 8 j + 7 and
//      32 + 8 j .. 32 + 8 j + 7 of the step;
//   D: rows 4 j .. 4 j + 3 of the tile, column n.
// N = 16 columns hold the batch; columns beyond it are computed from
// whatever the lanes hold and never stored.
//
// Loads.  A's layout asks one load instruction for 16 rows x 64 bytes,
// which streams HBM at about half the rate of row-contiguous requests, so
// every operand goes through LDS: a block (256 columns of the 16-row tile:
// 4 KiB of values, 512 B of mask words, and 512 B of x per token) is copied
// by direct-to-LDS buffer loads (buffer_load ... lds, 16 or 4 bytes per
// lane, lane i's data landing at base + i * size), each instruction reading
// whole 256-byte row segments.  The 16-byte chunks are XOR-swizzled within a
// row (values: chunk c of row r at position c ^ r; x: chunk c of token t at
// c ^ t; mask word w of row r at w ^ (r >> 2 & 7)), so the reads in MFMA
// layout hit distinct LDS banks.  Each wave streams its own K range through a
// private ring of NB such blocks with explicit vmcnt waits; the waves of a
// workgroup split K and add their tiles through LDS at the end.

constexpr int kMfmaSparse24 = 0;   // 2:4 on v_smfmac
constexpr int kMfmaDenseHalf = 1;  // 4:8, 8:16: decompressed tile, v_mfma
constexpr int kMfmaDense1632 = 2;  // 16:32: decompressed tile, v_mfma

constexpr int kMBlkCols = 256;                  // columns per block
constexpr int kMValBytes = 16 * kMBlkCols;      // 16 rows x 128 values x 2 B
constexpr int kMMaskBytes = 16 * kMBlkCols / 8;  // 16 rows x 8 words x 4 B
constexpr int kMXTok = 2 * kMBlkCols;           // x bytes per token per block

// LDS bytes of one ring slot for a padded batch BP (x for BP tokens); the
// 2:4 kind keeps its mask words in a ring of its own (two blocks per slot).
__host__ __device__ constexpr int mfma_slot_bytes(int bp, int kind) {
  return kMValBytes + (kind == 0 ? 0 : kMMaskBytes) + kMXTok * bp;
}
// Mask ring of the 2:4 kind: slots of two blocks' mask words (16 rows x 64
// bytes), enough that a slot is refilled only after both blocks are done.
__host__ __device__ constexpr int mfma_mask_slots(int nb) { return (nb + 2) / 2; }

// Dense 16 x 64 tile of the decompressing kinds: rows padded to 144 bytes
// (64 x 2 + 16), so the 16 rows of a 16-lane read start on distinct banks.
constexpr int kMTileRow = 144;
constexpr int kMTileBytes = 16 * kMTileRow;

// LDS of one wave: its ring, and the dense tile of the decompressing kinds.
__host__ __device__ constexpr int mfma_wave_bytes(int bp, int nb, int kind) {
  return nb * mfma_slot_bytes(bp, kind) +
         (kind == kMfmaSparse24 ? 1024 * mfma_mask_slots(nb) : kMTileBytes);
}

// Operands of one 64-column step of the matrix-core kernel.
struct MfmaOps {
  u32x4_t a, x0, x1;
  uint32_t w;
};

template <bool BF, int BP, int NB, int KIND>
__global__ __launch_bounds__(1024) void nm_spmm_mfma_kernel(
    const uint16_t *__restrict__ values, const uint32_t *__restrict__ bits,
    const uint16_t *__restrict__ x, void *__restrict__ y, int B, int64_t R, int K,
    int out_kind) {
  constexpr int XQ = BP / 2;          // x instructions per block (2 tokens each)
  constexpr int ND = 4 + 2 + XQ;      // direct-to-LDS instructions per block (not 2:4)
  constexpr int SLOT = mfma_slot_bytes(BP, KIND);
  constexpr bool M2 = KIND == kMfmaSparse24;     // masks by pairs of blocks
  constexpr int MS = mfma_mask_slots(NB);
  constexpr int XB = M2 ? kMValBytes : kMValBytes + kMMaskBytes;  // x within a slot
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int W = blockDim.x / kWave;
  const int n = lane & 15, j = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int nsteps = K >> 6;                              // 64-column steps
  const int per = (((nsteps + W - 1) / W) + 3) & ~3;      // whole blocks per wave
  const int sbeg = min(nsteps, wid * per), send = min(nsteps, sbeg + per);
  const int mysteps = send - sbeg;
  const int nblk = (mysteps + 3) >> 2;
  constexpr int WBYTES = mfma_wave_bytes(BP, NB, KIND);
  const uint32_t ring = (uint32_t)(size_t)(lds_ptr)lds + (uint32_t)(wid * WBYTES);

  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void *)values, 0, (int)(R * (int64_t)K), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)bits, 0, (int)(R * (int64_t)K / 8), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void *)x, 0, B * K * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc((void *)values, 0, 0,
                                                                      kRsrcWord3);
  // Per-lane source offsets of the wave's first block (bytes).  Rows past R
  // load row R - 1 (never stored); tokens past B read zeros (range check).
  int voff[4], boff[2], xoff[XQ];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rr = 4 * q + (lane >> 4);
    const int64_t r = min(row0 + rr, R - 1);
    voff[q] = (int)(r * K) + 64 * sbeg + 16 * ((lane & 15) ^ rr);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int rr = 8 * q + (lane >> 3);
    const int64_t r = min(row0 + rr, R - 1);
    boff[q] = (int)(r * (K / 8)) + 8 * sbeg + 4 * ((lane & 7) ^ ((rr >> 2) & 7));
  }
  // 2:4: the mask words of blocks 2p, 2p + 1 (64 bytes per row) in one load,
  // lane i -> row i >> 2, 16-byte piece (i & 3) ^ (row >> 2 & 3)
  const int mrow = lane >> 2;
  const int moff2 = (int)(min(row0 + mrow, R - 1) * (K / 8)) + 8 * sbeg +
                    16 * ((lane & 3) ^ ((mrow >> 2) & 3));
  const int npairs = (nblk + 1) >> 1;
  const uint32_t mring = ring + (uint32_t)(NB * SLOT);
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int t = 2 * q + (lane >> 5);
    xoff[q] = t * K * 2 + 128 * sbeg + 16 * ((lane & 31) ^ (t & 7));
  }

  // block b of the wave into ring slot b % NB; b >= nblk loads from
  // zero-size resources (no memory traffic, same instruction count)
  auto issue = [&](int b) {
    const bool real = b < nblk;
    const __amdgpu_buffer_rsrc_t V = real ? rv : r0, M = real ? rb : r0, X = real ? rx : r0;
    const uint32_t sl = ring + (uint32_t)((b % NB) * SLOT);
    // the block offset goes into the vector offset, which the range check
    // covers (the scalar offset is not checked): a wave's last block may
    // reach past its K range, and on the last rows past the arrays
    if constexpr (M2) {
      if ((b & 1) == 0)
        lds_load16_nt((b >> 1) < npairs ? rb : r0, mring + (uint32_t)(((b >> 1) % MS) * 1024),
                      moff2 + 64 * (b >> 1), 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      lds_load16_nt(V, sl + 1024 * q, voff[q] + kMValBytes / 16 * b, 0);
    if constexpr (!M2) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        lds_load4_nt(M, sl + kMValBytes + 256 * q, boff[q] + kMMaskBytes / 16 * b, 0);
    }
#pragma unroll
    for (int q = 0; q < XQ; ++q)
      lds_load16(X, sl + XB + 1024 * q, xoff[q] + kMXTok * b, 0);
  };

  // reader addresses within a slot, step 0 (steps add constant offsets only
  // after the swizzle, so they are recomputed per step)
  const int tn = min(n, B - 1);
  f4v_t acc = {0.f, 0.f, 0.f, 0.f};
  // operands of step s of the block in slot sl
  auto fetch = [&](uint32_t sl, int s, int b) {
    MfmaOps o;
    o.a = ld<u32x4_t>((lds_ptr)(size_t)(sl + n * 256 + 16 * ((4 * s + j) ^ n)));
    if constexpr (M2)
      o.w = ld<uint32_t>((lds_ptr)(size_t)(mring + ((b >> 1) % MS) * 1024 + n * 64 +
                                           16 * ((2 * (b & 1) + (s >> 1)) ^ ((n >> 2) & 3)) +
                                           4 * (2 * (s & 1) + (j >> 1))));
    else
      o.w = ld<uint32_t>((lds_ptr)(size_t)(sl + kMValBytes + n * 32 +
                                           4 * ((2 * s + (j >> 1)) ^ ((n >> 2) & 7))));
    const uint32_t xb = sl + XB + tn * kMXTok;
    o.x0 = ld<u32x4_t>((lds_ptr)(size_t)(xb + 16 * ((8 * s + j) ^ (tn & 7))));
    o.x1 = ld<u32x4_t>((lds_ptr)(size_t)(xb + 16 * ((8 * s + 4 + j) ^ (tn & 7))));
    return o;
  };
  auto mac = [&](const MfmaOps &o) {
    acc = smfmac<BF>(o.a, o.x0, o.x1, nib_codes(o.w >> ((j & 1) * 16)), acc);
  };
  // Decompressing kinds, step s: lane (j, n) takes chunk 4 s + j of row n
  // (8 kept values) and the columns of its 8 kept values within its 32-column
  // mask word: the word's 8 lowest set bits for an even chunk, the next 8 for
  // an odd one (for M <= 16 simply the word's low or high half).  It zeroes
  // its 16 columns of the step's dense tile row, writes its 8 values at their
  // columns (the zeroing of every lane precedes every value write: one
  // wave's LDS operations complete in order), and the two 16x16x32 products
  // read the tile in MFMA layout.  (Running a block's four steps phase by
  // phase on four tiles measured slower: the larger LDS footprint costs more
  // waves per CU than the overlap gains.)
  const uint32_t tile = ring + (uint32_t)(NB * SLOT);
  auto chunk_of = [&](uint32_t sl, int s) {
    return ld<u32x4_t>((lds_ptr)(size_t)(sl + n * 256 + 16 * ((4 * s + j) ^ n)));
  };
  auto word_of = [&](uint32_t sl, int s) {
    return ld<uint32_t>((lds_ptr)(size_t)(sl + kMValBytes + n * 32 +
                                          4 * ((2 * s + (j >> 1)) ^ ((n >> 2) & 7))));
  };
  // the set bits of mask word w that belong to the lane's chunk: its lowest
  // 8 kept columns for an even chunk, the next 8 for an odd one
  auto chunk_bits = [&](uint32_t w) -> uint32_t {
    if constexpr (KIND == kMfmaDenseHalf) {
      return w & ((j & 1) ? 0xffff0000u : 0x0000ffffu);
    } else {
      uint32_t hi = w;
#pragma unroll
      for (int k = 0; k < 8; ++k) hi &= hi - 1;
      return (j & 1) ? hi : w;
    }
  };
  auto scatter = [&](uint32_t tile, u32x4_t v, uint32_t w) {
    uint32_t m = chunk_bits(w);
    const uint32_t row = tile + (uint32_t)(n * kMTileRow);
    lds_st<u32x4_t>(row + 32 * j, (u32x4_t){0u, 0u, 0u, 0u});
    lds_st<u32x4_t>(row + 32 * j + 16, (u32x4_t){0u, 0u, 0u, 0u});
    const uint32_t wb = row + 64 * (j >> 1);  // column 0 of the lane's word
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = ffbl_hw(m) & 31;  // an exhausted (malformed) word writes column 31
      m &= m - 1;
      lds_st<uint16_t>(wb + 2 * c, (uint16_t)(v[k >> 1] >> (16 * (k & 1))));
    }
  };
  auto tile_a = [&](uint32_t tile, int t) {
    return ld<u32x4_t>((lds_ptr)(size_t)(tile + n * kMTileRow + 64 * t + 16 * j));
  };
  auto x_of = [&](uint32_t sl, int s, int t) {
    const uint32_t xb = sl + XB + tn * kMXTok;
    return ld<u32x4_t>((lds_ptr)(size_t)(xb + 16 * ((8 * s + 4 * t + j) ^ (tn & 7))));
  };
  auto dense_step = [&](uint32_t sl, int s) {
    scatter(tile, chunk_of(sl, s), word_of(sl, s));
#pragma unroll
    for (int t = 0; t < 2; ++t) acc = dmfma<BF>(tile_a(tile, t), x_of(sl, s, t), acc);
  };
  // Kept-column product of the block in slot sl, the decompressing kinds'
  // fallback.  The tile product multiplies the zeros stored at pruned
  // entries with x, so Inf or NaN in x at a column that some row of the tile
  // pruned makes the block's sums NaN, while the product sums kept weights
  // only (Method, item (1)).  Here lane (j, n) walks the 8 kept values of
  // chunk 4 s + j of row n (the columns scatter would write) against every
  // token's x in the block, in fp32 (16-bit products are exact); the four
  // lanes of a row are added, and the row sums reach the output layout
  // (rows 4 j .. 4 j + 3, token n) through the wave's tile.
  auto exact_block = [&](uint32_t sl, int ns) -> f4v_t {
    float p[BP];
#pragma unroll
    for (int t = 0; t < BP; ++t) p[t] = 0.f;
    for (int s = 0; s < ns; ++s) {
      const u32x4_t v = chunk_of(sl, s);
      uint32_t m = chunk_bits(word_of(sl, s));
      const int cb = 64 * s + 32 * (j >> 1);  // block column of the word's bit 0
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = cb + (ffbl_hw(m) & 31);  // an exhausted (malformed) word repeats column 31
        m &= m - 1;
        const float w = half_to_f32<BF>((uint16_t)(v[k >> 1] >> (16 * (k & 1))));
#pragma unroll
        for (int t = 0; t < BP; ++t) {
          const uint32_t xa = sl + XB + t * kMXTok +
                              16 * ((c >> 3) ^ (t & 7)) + 2 * (c & 7);
          p[t] = fmaf(w, half_to_f32<BF>(ld<uint16_t>((lds_ptr)(size_t)xa)), p[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < BP; ++t) {
      p[t] += __shfl_xor(p[t], 16);
      p[t] += __shfl_xor(p[t], 32);
    }
    // the tile's last reads (the block's products) precede these writes:
    // one wave's LDS operations complete in order
    if (j == 0) {
#pragma unroll
      for (int t = 0; t < BP; ++t) lds_st<float>(tile + 4 * (n * BP + t), p[t]);
    }
    f4v_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = ld<float>((lds_ptr)(size_t)(tile + 4 * ((4 * j + i) * BP + tn)));
    return r;
  };
  auto compute = [&](int b) {
    const uint32_t sl = ring + (uint32_t)((b % NB) * SLOT);
    const int ns = min(4, mysteps - 4 * b);
    if constexpr (KIND != kMfmaSparse24) {
      // the block's tile product from zero; a NaN in it means Inf or NaN in
      // the block's x, and the block is summed again over kept columns only
      const f4v_t prev = acc;
      acc = (f4v_t){0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < ns; ++s) dense_step(sl, s);
      const bool nan = acc[0] != acc[0] || acc[1] != acc[1] || acc[2] != acc[2] || acc[3] != acc[3];
      if (__builtin_amdgcn_ballot_w64(nan) != 0) acc = exact_block(sl, ns);
      acc += prev;
    } else if (ns == 4) {  // whole block: every LDS read is issued before the first product
      MfmaOps o[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) o[s] = fetch(sl, s, b);
#pragma unroll
      for (int s = 0; s < 4; ++s) mac(o[s]);
    } else {  // the wave's ragged last block
      for (int s = 0; s < ns; ++s) mac(fetch(sl, s, b));
    }
  };

#pragma unroll
  for (int b = 0; b < NB - 1; ++b) issue(b);
  for (int b = 0; b < nblk; ++b) {
    // the slot about to be refilled was read by the previous block's
    // compute: its LDS reads have returned before the refill is issued
    wait_lgkmcnt0();
    __builtin_amdgcn_sched_barrier(0);
    issue(b + NB - 1);
    // block b has landed; NB - 1 blocks stay in flight (with the 2:4 kind,
    // each even block among them also carries a mask load)
    if constexpr (M2) {
      constexpr int D = 4 + XQ;
      if (b & 1)
        wait_vmcnt<(NB - 1) * D + NB / 2>();  // evens among b+1..b+NB-1, b odd
      else
        wait_vmcnt<(NB - 1) * D + (NB - 1) / 2>();
    } else {
      wait_vmcnt<(NB - 1) * ND>();
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(b);
  }
  wait_vmcnt<0>();  // the trailing dummy loads still write LDS
  __builtin_amdgcn_sched_barrier(0);

  // partial tiles of the W waves -> LDS (each wave's own ring) -> wave 0
  if (W > 1) {
    wait_lgkmcnt0();
    float *mine = reinterpret_cast<float *>(lds + wid * WBYTES);
#pragma unroll
    for (int i = 0; i < 4; ++i) mine[i * kWave + lane] = acc[i];
    __syncthreads();
    if (wid != 0) return;
    for (int w = 1; w < W; ++w) {
      const float *other = reinterpret_cast<const float *>(lds + w * WBYTES);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += other[i * kWave + lane];
    }
  }
  if (n < B) {
    if ((out_kind >> kEpiShift) == kEpiSwiglu) {
      // rows 4j, 4j+1 and 4j+2, 4j+3 of the tile are (gate, up) pairs
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int64_t r = row0 + 4 * j + i;
        if (r < R) store_out(y, (int64_t)n * (R / 2) + r / 2, silu(acc[i]) * acc[i + 1], out_kind);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + 4 * j + i;
        if (r < R) store_out(y, (int64_t)n * R + r, acc[i], out_kind);
      }
    }
  }
}

// Dense comparison when x fits the LDS budget, built like the sparse row
// kernel so that the speedup is measured against an equally tuned dense
// GEMV: x staged once per workgroup as BP contiguous rows; each wave walks
// its rows as a two-stage pipeline of load batches (lane l takes 16-byte
// chunks, 8 columns each, t*64U + l + 64u), with the same raw buffer loads
// and nt policy as the sparse weights.
template <int U>
struct DBatch {
  uint4 v[U];
};

template <int U>
__device__ __forceinline__ void dload_batch(DBatch<U> &bt, const uint4 *wrow, int nch, int t,
                                            int lane) {
  // the resource starts at the batch and ends at the row end (the range check
  // covers the vector offsets only)
  const int c0 = t * (kWave * U), left = nch - c0 > 0 ? nch - c0 : 0;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void *)(wrow + c0), 0, left * 16, kRsrcWord3);
#pragma unroll
  for (int u = 0; u < U; ++u)
    bt.v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            r, lane * 16 + u * kWave * 16, 0, kStreamAux));
}

template <bool BF, int BP, int U>
__device__ __forceinline__ void drun_batch(const char *lds, int K, const DBatch<U> &bt, int q0,
                                           int nch, float (&acc)[BP]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int q = q0 + kWave * u;
    const int qc = min(q, nch - 1);
#pragma unroll
    for (int b = 0; b < BP; ++b) {
      const uint4 xq = *reinterpret_cast<const uint4 *>(lds + (size_t)b * K * 2 + (size_t)qc * 16);
      float a = 0.f;
      a = dot2<BF>(bt.v[u].x, xq.x, a);
      a = dot2<BF>(bt.v[u].y, xq.y, a);
      a = dot2<BF>(bt.v[u].z, xq.z, a);
      a = dot2<BF>(bt.v[u].w, xq.w, a);
      acc[b] += q < nch ? a : 0.f;
    }
  }
}

template <bool BF, int BP>
__global__ __launch_bounds__(1024) void nm_dense_rows_kernel(
    const uint4 *__restrict__ W, const uint16_t *__restrict__ x, void *__restrict__ y, int B,
    int64_t R, int K, int rpw, int out_kind) {
  constexpr int U = 4;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wpg = blockDim.x / kWave;
  const int nch = K >> 3;  // 16-byte chunks per row
  const int nb = (nch + kWave * U - 1) / (kWave * U);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t r0 = ((int64_t)blockIdx.x * wpg + wid) * rpw;
  const int64_t left = R - r0;
  const int nrows = left <= 0 ? 0 : (left < rpw ? (int)left : rpw);
  const int nitems = nrows * nb;

  float acc[BP];
#pragma unroll
  for (int b = 0; b < BP; ++b) acc[b] = 0.f;
  if (K == 0) {
    for (int r = 0; r < nrows; ++r) finish_row<BP>(acc, y, B, R, r0 + r, lane, out_kind);
    return;
  }
  auto item_load = [&](DBatch<U> &bt, int k) {
    const bool real = k < nitems;
    const int ii = real ? k / nb : 0, tt = real ? k - ii * nb : 0;
    const int64_t r = real ? r0 + ii : 0;
    dload_batch<U>(bt, W + r * nch, real ? nch : 0, tt, lane);
  };
  DBatch<U> A, Bt;
  item_load(A, 0);
  item_load(Bt, 1);
  for (int b = 0; b < BP; ++b) {
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)(b < B ? b : 0) * K);
    uint4 *dst = reinterpret_cast<uint4 *>(lds + (size_t)b * K * 2);
    for (int j = threadIdx.x; j < nch; j += blockDim.x)
      dst[j] = b < B ? src[j] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  float res[BP];
#pragma unroll
  for (int b = 0; b < BP; ++b) res[b] = 0.f;
  for (int k = 0; k < nitems; k += 2) {
    const int i = k / nb, t = k - i * nb;
    drun_batch<BF, BP, U>(lds, K, A, t * kWave * U + lane, nch, acc);
    if (t == nb - 1) collect_row<BP>(acc, res, i, lane);
    item_load(A, k + 2);
    if (k + 1 >= nitems) break;
    const int i1 = (k + 1) / nb, t1 = (k + 1) - i1 * nb;
    drun_batch<BF, BP, U>(lds, K, Bt, t1 * kWave * U + lane, nch, acc);
    if (t1 == nb - 1) collect_row<BP>(acc, res, i1, lane);
    item_load(Bt, k + 3);
  }
  if (lane < nrows) {
#pragma unroll
    for (int b = 0; b < BP; ++b)
      if (b < B) store_out(y, (int64_t)b * R + r0 + lane, res[b], out_kind);
  }
}

// Dense comparison when x does not fit the LDS budget in one piece.
// Dense comparison: lane l handles 16-byte chunks (8 columns) l, l+64, ...
// of a row; x is staged in LDS as BP contiguous rows of `seg` columns.
template <bool BF, int BP, int RPW>
__global__ __launch_bounds__(1024) void nm_dense_kernel(
    const uint4 *__restrict__ W, const uint16_t *__restrict__ x,
    void *__restrict__ y, int B, int64_t R, int K, int seg, int out_kind) {
  constexpr int U = RPW >= 4 ? 2 : 4;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int wpg = blockDim.x / kWave;
  const int64_t row0 = (int64_t)blockIdx.x * wpg * RPW + wid;
  const int64_t cpr = K >> 3;  // 16-byte chunks per row

  float acc[RPW][BP];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int b = 0; b < BP; ++b) acc[i][b] = 0.f;

  for (int s0 = 0; s0 < K; s0 += seg) {
    const int S = min(seg, K - s0);
    if (s0) __syncthreads();
    for (int b = 0; b < BP; ++b) {
      const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)b * K + s0);
      uint4 *dst = reinterpret_cast<uint4 *>(lds + (size_t)b * seg * 2);
      for (int j = threadIdx.x; j < S / 8; j += blockDim.x)
        dst[j] = (b < B) ? src[j] : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    const int nch = S >> 3;
    const int64_t cbeg = s0 >> 3;
    for (int t0 = 0; t0 < nch; t0 += kWave * U) {
      uint4 v[RPW][U];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int64_t r = row0 + (int64_t)i * wpg;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = t0 + kWave * u + lane;
          v[i][u] = (r < R && q < nch) ? W[r * cpr + cbeg + q] : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = t0 + kWave * u + lane;
        if (q < nch) {
#pragma unroll
          for (int b = 0; b < BP; ++b) {
            const uint4 xq =
                *reinterpret_cast<const uint4 *>(lds + (size_t)b * seg * 2 + (size_t)q * 16);
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
              float a = acc[i][b];
              a = dot2<BF>(v[i][u].x, xq.x, a);
              a = dot2<BF>(v[i][u].y, xq.y, a);
              a = dot2<BF>(v[i][u].z, xq.z, a);
              a = dot2<BF>(v[i][u].w, xq.w, a);
              acc[i][b] = a;
            }
          }
        }
      }
    }
  }

#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int64_t r = row0 + (int64_t)i * wpg;
    if (r < R) {
#pragma unroll
      for (int b = 0; b < BP; ++b) {
        const float s = wave_sum_to_63(acc[i][b]);
        if (lane == kWave - 1 && b < B) store_out(y, (int64_t)b * R + r, s, out_kind);
      }
    }
  }
}

// Pack (Method item (1)).  One wavefront per row, 64 columns per step: lane l
// tests column c0 + l, a ballot forms the two 32-bit words, and the count of
// set bits below the lane (an mbcnt-style prefix) is the kept weight's slot
// among its word's 16 values.  Lanes at the start of each M-group check that
// the group keeps exactly M/2; the number of bad groups is added to *bad.
template <int M>
__global__ __launch_bounds__(256) void nm_pack_kernel(
    const uint16_t *__restrict__ W, const uint8_t *__restrict__ keep,
    int64_t R, int K, int N, uint16_t *__restrict__ values,
    uint32_t *__restrict__ bits, int *__restrict__ bad) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wpg = blockDim.x / kWave;
  const uint32_t lb = lane & 31;
  const uint32_t below = (1u << lb) - 1u;
  const uint32_t gmask = (M == 32) ? 0xffffffffu : ((1u << (M & 31)) - 1u);
  const uint32_t P = 32 / M * N;  // values per 32-bit mask word
  int nbad = 0;
  for (int64_t r = (int64_t)blockIdx.x * wpg + threadIdx.x / kWave; r < R;
       r += (int64_t)gridDim.x * wpg) {
    const uint16_t *wr = W + r * K;
    const uint8_t *kr = keep + r * K;
    uint16_t *vr = values + r * (K / 32) * P;
    uint32_t *br = bits + r * (K / 32);
    for (int c0 = 0; c0 < K; c0 += kWave) {
      const int c = c0 + lane;
      const bool in = c < K;
      const bool kept = in && kr[c] != 0;
      const uint16_t wv = in ? wr[c] : (uint16_t)0;
      const uint64_t bal = __ballot(kept);
      const uint32_t word = (lane < 32) ? (uint32_t)bal : (uint32_t)(bal >> 32);
      const uint32_t slot = __popc(word & below);
      const int64_t wg = (c0 >> 5) + (lane >> 5);
      if (kept && slot < P) vr[wg * P + slot] = wv;
      if (in && lb == 0) br[wg] = word;
      bool badg = false;
      if (in && (lb % M) == 0) badg = __popc((word >> lb) & gmask) != N;
      nbad += badg ? 1 : 0;
    }
  }
  // sum over the wave, one atomic per wave
  for (int o = kWave / 2; o > 0; o >>= 1) nbad += __shfl_xor(nbad, o, kWave);
  if (lane == 0 && nbad) atomicAdd(bad, nbad);
}

// Calibration read: every 16-byte chunk of buf is loaded once with the same
// 128-bit non-temporal buffer loads as the sparse kernel's weights (wave w
// reads chunks w*64*U + l + 64u, grid-strided), and each wave writes one
// word so the loads cannot be dropped.  It gives the achievable HBM read rate
// and the per-launch fixed cost, and is the plain read of known size that
// scales the fetch-size counters.
__global__ __launch_bounds__(1024) void nm_stream_read_kernel(const char *__restrict__ buf,
                                                               int64_t nchunks,
                                                               uint32_t *__restrict__ out) {
  constexpr int U = 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / kWave) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
  uint32_t acc = 0;
  for (int64_t c0 = wave * kWave * U; c0 < nchunks; c0 += nwaves * kWave * U) {
    const int64_t left = nchunks - c0;
    const int nbytes = (int)((left < kWave * U ? left : kWave * U) * 16);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void *)(buf + c0 * 16), 0, nbytes, kRsrcWord3);
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, lane * 16 + u * kWave * 16, 0, kStreamAux));
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  const int sv = __reduce_or_sync(~0ull, (int)acc);
  if (lane == 0) out[wave] = (uint32_t)sv;
}

// Zero n ints of p (one workgroup): the scratch counter is cleared by a
// kernel on the call's stream rather than a memset node.
__global__ __launch_bounds__(64) void nm_zero_ints_kernel(int *__restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// ---------------------------------------------------------------------------
// host side

struct DevInfo {
  bool init = false;
  int cus = 0;
  size_t lds_per_wg = 0;
};
constexpr int kMaxDev = 64;
DevInfo g_dev[kMaxDev];
std::mutex g_dev_mu;

nm_status device_info(DevInfo *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDev) return NM_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_dev_mu);
  DevInfo &d = g_dev[dev];
  if (!d.init) {
    int cus = 0, lds = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e);
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return hip_fail(e);
    d.cus = cus;
    d.lds_per_wg = (size_t)lds;
    d.init = true;
  }
  *out = d;
  return NM_OK;
}

// Argument checks common to the products; nothing here touches HIP.
nm_status check_dims(int64_t rows, int64_t cols, int batch) {
  if (rows < 0 || cols < 0 || batch < 1 || batch > 8) return NM_ERR_INVALID_ARG;
  if (rows > INT32_MAX || cols > INT32_MAX) return NM_ERR_INVALID_ARG;
  if (cols % 32 != 0) return NM_ERR_SHAPE;
  return NM_OK;
}

int pad_batch(int b) { return b <= 1 ? 1 : b <= 2 ? 2 : b <= 4 ? 4 : 8; }

size_t sparse_lds_bytes(int bp, int seg) {
  switch (bp) {
    case 1: return XLay<1>::bytes(seg);
    case 2: return XLay<2>::bytes(seg);
    case 4: return XLay<4>::bytes(seg);
    default: return XLay<8>::bytes(seg);
  }
}

size_t dense_lds_bytes(int bp, int seg) { return (size_t)bp * seg * 2; }

size_t lds_bytes(bool dense, int bp, int seg) {
  return dense ? dense_lds_bytes(bp, seg) : sparse_lds_bytes(bp, seg);
}

// Widest segment (multiple of 32 columns) whose LDS image fits `budget`.
int max_seg(bool dense, int bp, size_t budget) {
  int lo = 32, hi = 1 << 20;
  if (lds_bytes(dense, bp, lo) > budget) return 0;
  while (lo < hi) {
    int mid = ((lo + hi) / 2 + 31) / 32 * 32;
    if (mid >= hi) mid = hi;
    if (lds_bytes(dense, bp, mid) <= budget) lo = mid; else hi = mid - 32;
  }
  return lo;
}

size_t lds_budget(const DevInfo &di) {
  return di.lds_per_wg < kLdsCap ? di.lds_per_wg : kLdsCap;
}

// Chunks per lane per load batch of a split launch: the largest of 4, 5, 2, 1
// that divides a wave's share of the row's chunks per lane (K / 1024 / ks).
int split_batch_chunks(int64_t cols, int ks) {
  const int64_t c = cols / 1024 / ks;
  return c % 4 == 0 ? 4 : c % 5 == 0 ? 5 : c % 2 == 0 ? 2 : 1;
}

// Does 4:8 at this batch take the plain-x kind with the pair table?  Batch 1,
// K > 0, and x plus the table within the LDS a workgroup may use.
bool plain48_ok(int64_t cols, int bp, int n, int m) {
  return bp == 1 && n == 4 && m == 8 && cols > 0 &&
         (size_t)cols * 2 + 256 * 16 <= kLdsCap;
}

// LDS of a split launch: the x image and one partial sum per row per wave.
size_t split_lds_bytes(int64_t cols, int waves, int rpw) {
  return split_lds_offset((int)cols) + (size_t)waves * rpw * 4;
}

// Is this a launch of the single-segment row kernel (all of x in LDS)?
bool rows_kernel(bool dense, int64_t cols, int seg) {
  (void)dense;
  return seg >= cols;
}

int threads_for_lds(size_t lds) {
  return lds <= 40 * 1024 ? 256 : lds <= 80 * 1024 ? 512 : 1024;
}

// Can the matrix-core kernel run this shape?  Its buffer resources address
// the whole values array and the batch's x with 32-bit offsets.
bool mfma_ok(int64_t rows, int64_t cols, int n, int m) {
  return pattern_ok(n, m) && cols % 64 == 0 && cols <= (1 << 25) && rows * cols <= INT32_MAX;
}

// Matrix-core kind of a pattern: 2:4 on the sparse instruction, the others
// through a decompressed tile.
int mfma_kind(int n, int m) {
  return (n == 2 && m == 4) ? kMfmaSparse24 : m == 32 ? kMfmaDense1632 : kMfmaDenseHalf;
}

// LDS of the matrix-core kernel: every wave's ring of `nb` blocks (and tile).
size_t mfma_lds_bytes(int waves, int nb, int bp, int kind) {
  return (size_t)waves * mfma_wave_bytes(bp < 2 ? 2 : bp, nb, kind);
}

// Launch shape of the matrix-core kernel: threads_per_wg / 64 waves split K
// for one 16-row tile; rows_per_wave is each wave's ring depth (blocks).
// Measured on the 8B, 70B and Qwen3-32B shapes at batch 2..8 (2:4): four
// waves per workgroup, halved while a wave would walk fewer than 32 steps of
// 64 columns and the grid keeps at least 1024 waves (14336x4096 at batch 8:
// 14.9 us with two waves against 16.2 with four; 8192x5120 11.5 against
// 12.5; 4096x4096, 256 tiles, keeps four: 6.4 against 7.4); a ring of three
// blocks while at least 8 waves of such workgroups fit a CU's LDS, else two
// (two waves of three blocks at batch 8 leave 6 waves per CU: 17.5 us on
// 14336x4096).  For the decompressing kinds (measured on the 8B shapes at
// batch 2..8) the ring of two blocks is best, with about 8 waves per CU in
// total, at most 8 per workgroup.
void mfma_default(int64_t rows, int64_t cols, int batch, int kind, const DevInfo &di,
                  nm_launch_cfg *cfg) {
  const int bp = pad_batch(batch) < 2 ? 2 : pad_batch(batch);
  const int64_t nsteps = cols / 64;
  const int64_t tiles = (rows + 15) / 16;
  const size_t budget = lds_budget(di);
  int w = 4;
  if (kind != kMfmaSparse24) {
    const int64_t t = 8LL * di.cus / (tiles > 0 ? tiles : 1);
    w = t < 1 ? 1 : t > 8 ? 8 : (int)t;
  }
  while (w > 1 && nsteps / w < 8) --w;  // at least two blocks of K per wave
  if (kind == kMfmaSparse24) {
    while (w > 1 && nsteps / w < 32 && tiles * (w / 2) >= 1024) w /= 2;
    // one wave per workgroup where two would walk fewer than 64 steps and the
    // grid still holds 1024 tiles (25600x5120: 27.3 us at batch 2 against
    // 30.3 with two waves; 14336x4096, 896 tiles, keeps two)
    if (w == 2 && nsteps / 2 < 64 && tiles >= 1024) w = 1;
  }
  const int nb =
      (kind == kMfmaSparse24 && (int64_t)(kLdsCap / mfma_lds_bytes(w, 3, bp, kind)) * w >= 8) ? 3 : 2;
  while (w > 1 && mfma_lds_bytes(w, nb, bp, kind) > budget) --w;
  cfg->kernel = NM_KERNEL_MFMA;
  cfg->k_split = 1;
  cfg->threads_per_wg = w * kWave;
  cfg->rows_per_wave = nb;
  cfg->seg_cols = cols > 0 ? (int)cols : 64;
}

// Batch from which the auto choice takes the matrix-core kernel: 2:4 on the
// sparse instruction, the other patterns through the decompressed tile.
constexpr int kMfmaMinBatch = 2;
constexpr int kDenseMfmaMinBatch = 5;  // measured: the VALU kernel wins at batch <= 4

// 2:4 shapes where the VALU row kernel with x stored plainly per token beats
// the sparse matrix cores although batch >= kMfmaMinBatch.  Measured on the
// 13 shapes of the 8B, 70B and Qwen3-32B layers (us, cache-cold, one box,
// each kernel at its default launch, VALU / matrix cores):
//  - batch 2: every shape (1024x4096 3.29 / 4.84, 6144x4096 6.79 / 8.22,
//    14336x4096 12.47 / 13.88, 4096x14336 12.93 / 13.10, 8192x8192 13.96 /
//    14.30, 28672x8192 41.63 / 42.24, 8192x28672 41.00 / 43.60, 5120x8192
//    9.86 / 12.45, 5120x25600 24.90 / 35.13);
//  - batch 3 and 4: at most 1024 rows (1024x4096 3.86 / 5.02, 1024x8192
//    5.26 / 6.88); above that the matrix cores win on every shape but
//    5120x8192 (11.3 / 12.8), e.g. 14336x4096 14.61 / 14.10, 8192x8192
//    15.83 / 14.58, 5120x25600 50.98 / 36.28.
bool valu_beats_mfma_24(int64_t rows, int64_t cols, int batch) {
  (void)cols;
  if (batch > 4) return false;
  return batch == 2 || rows <= 1024;
}

int rows_batch_chunks(int64_t cols, int bp);

// pair: the rows come in (gate, up) pairs for the SwiGLU epilogue, so a
// wave of the row kernel must own an even number of rows.  allow_mfma =
// false gives the VALU kernels' shape for the pattern (a caller that forces
// NM_KERNEL_VALU), with the same pattern-specific launch rules as the
// automatic choice.
nm_status default_cfg(int64_t rows, int64_t cols, int batch, int n, int m, bool dense,
                      nm_launch_cfg *cfg, bool pair = false, bool allow_mfma = true) {
  DevInfo di;
  nm_status st = device_info(&di);
  if (st != NM_OK) return st;
  const bool sp24 = mfma_kind(n, m) == kMfmaSparse24;
  if (allow_mfma && !dense && mfma_ok(rows, cols, n, m) &&
      batch >= (sp24 ? kMfmaMinBatch : kDenseMfmaMinBatch) &&
      !(sp24 && valu_beats_mfma_24(rows, cols, batch) &&
        sparse_lds_bytes(pad_batch(batch), (int)cols) <= lds_budget(di))) {
    mfma_default(rows, cols, batch, mfma_kind(n, m), di, cfg);
    return NM_OK;
  }
  cfg->kernel = NM_KERNEL_VALU;
  cfg->k_split = 1;
  const int bp = pad_batch(batch);
  const size_t budget = lds_budget(di);
  const int smax = max_seg(dense, bp, budget);
  const size_t full = lds_bytes(dense, bp, cols > 0 ? (int)cols : 32);
  if (!dense && sp24 && bp >= 2 && full <= budget && cols > 0 && rows > 0) {
    // 2:4 at batch 2..8 (x staged by direct-to-LDS copies): the CU's rows
    // (rows / CUs) split evenly over one workgroup of 4 waves where K <= 4096
    // or where K >= 8192 with 32 or more rows per CU, else of 8 (no more
    // waves than rows), and over two workgroups where a wave would hold more
    // than 8 rows; at batch 2 with K >= 8192, 32 or more rows per CU and room
    // for two workgroups per CU, 4 rows per wave.  Measured on the 13 shapes
    // of the 8B, 70B and Qwen3-32B layers at batch 2 (us; a sweep of 256/512
    // threads x 1..16 rows per wave): within 4% of the best launch on each,
    // and up to 23% faster than the row-kernel rules below (5120x25600 24.90
    // against 32.23, 6144x4096 6.79 against 8.62, 8192x8192 13.96 against
    // 17.82, 5120x8192 9.86 against 13.23).
    const int64_t per_cu = (rows + di.cus - 1) / di.cus;
    int64_t w = cols <= 4096 || (cols >= 8192 && per_cu >= 32) ? 4 : 8;
    if (per_cu < w) w = per_cu;
    int64_t rpw = (per_cu + w - 1) / w;
    if (rpw > 8) rpw = (rpw + 1) / 2;
    if (bp == 2 && cols >= 8192 && per_cu >= 32 && 2 * full <= kLdsCap) rpw = 4;
    if (pair) rpw += rpw & 1;  // (gate, up) pairs stay within a wave
    cfg->seg_cols = (int)cols;
    cfg->threads_per_wg = (int)w * kWave;
    cfg->rows_per_wave = (int)(rpw < 64 ? rpw : 64);
    return NM_OK;
  }
  if (full <= budget) {
    // row kernel: x staged once per workgroup.  Measured on the 8B, 70B and
    // Qwen3-32B shapes:
    //  - very few rows (<= 8 per CU) split evenly over the CUs: one row per
    //    wave and one workgroup per CU, so x is staged once per CU;
    //  - few rows (<= 32 per CU) split evenly over the CUs: exactly two
    //    workgroups per CU; for the sparse product at batch 1 with
    //    K <= 16384, 4 or else 2 rows per wave while a workgroup keeps at
    //    least 4 waves (a longer pipeline per wave: 70B q 8192x8192 -20%,
    //    Qwen3 q and 8B down 4-5%, 8B q/o 3%); for 2:4, 4 rows already while
    //    it keeps 2 waves (the fused 8B q|k|v 6144x4096 -13% with 3 waves of
    //    4 rows instead of 6 of 2; the scan of the other 50% patterns ran
    //    20-48% slower so on 4096-row shapes), otherwise one row per wave
    //    (better or equal at K >= 25600);
    //  - otherwise, rows split evenly: 256 threads and the same number of
    //    rows rpw (<= 8) for every wave, at least two workgroups per CU, so
    //    x is staged rarely and no CU finishes early;
    //  - otherwise one row per wave, and the hardware balances the groups.
    cfg->seg_cols = cols > 0 ? (int)cols : 32;
    const int64_t two_per_cu = 2LL * di.cus;
    const int rmin = pair ? 2 : 1;  // rows per wave in the one-row shapes
    if (rows > 0 && rows % (rmin * di.cus) == 0 && rows / di.cus <= 8) {
      cfg->threads_per_wg = (int)(rows / (rmin * di.cus)) * kWave;
      cfg->rows_per_wave = rmin;
      return NM_OK;
    }
    // 2:4, and 4:8 in its plain-x kind, at batch 1 with 12..24 rows per CU
    // (a multiple of 4) and K <= 8192: one workgroup of 4 waves per CU, so x
    // is staged once per CU (4096x4096 5.11 us against 5.57 with two 2-wave
    // workgroups, 4:8 bf16 5.18 against 5.77; 6144x4096 6.36 against 6.63,
    // 4:8 6.38 against 6.77; 5120x8192 9.05 against 9.34); at 32 rows per CU
    // (8192x8192) and at K = 14336 two workgroups stay ahead
    if (!dense && (sp24 || plain48_ok(cols, bp, n, m)) && bp == 1 && !pair && cols <= 8192 &&
        rows % di.cus == 0 && rows / di.cus > 8 && rows / di.cus <= 24 && (rows / di.cus) % 4 == 0) {
      cfg->threads_per_wg = 4 * kWave;
      cfg->rows_per_wave = (int)(rows / di.cus / 4);
      return NM_OK;
    }
    // 8:16 and 16:32 (the scan) at batch 1 with 24 rows per CU: two workgroups
    // of 4 waves per CU, 3 rows a wave (6144x4096 bf16: 7.84 / 7.99 us
    // against 8.59 / 9.03 with 6 waves of 2 rows)
    if (!dense && (m == 16 || m == 32) && 2 * n == m && bp == 1 && !pair && cols <= 8192 &&
        rows == 24LL * di.cus) {
      cfg->threads_per_wg = 4 * kWave;
      cfg->rows_per_wave = 3;
      return NM_OK;
    }
    if (full <= budget / 2 && rows % (rmin * two_per_cu) == 0 && rows / two_per_cu <= 16) {
      int rpw = rmin;
      // (2:4 rows whose load batches hold 2 chunks per lane keep one row per
      // wave: 8 waves per workgroup measured 3% faster for K = 14336; 4:8 in
      // its plain-x kind follows the 2:4 rules, measured equal or better)
      const bool plain_rules = m == 4 || plain48_ok(cols, bp, n, m);
      if (!dense && bp == 1 && cols <= 16384 && !(plain_rules && rows_batch_chunks(cols, bp) == 2))
        for (int r = 4; r >= 2; r -= 2)
          if (rows % (r * two_per_cu) == 0 &&
              rows / (r * two_per_cu) >= (r == 4 && plain_rules ? 2 : 4)) {
            rpw = r;
            break;
          }
      cfg->threads_per_wg = (int)(rows / (rpw * two_per_cu)) * kWave;
      cfg->rows_per_wave = rpw;
      return NM_OK;
    }
    cfg->threads_per_wg = threads_for_lds(full);
    const int64_t per_cu_rows = (int64_t)di.cus * (cfg->threads_per_wg / kWave);
    int rpw = rmin;
    if (rows % per_cu_rows == 0) {
      const int64_t q = rows / per_cu_rows;  // rows per wave if one workgroup per CU
      for (int d = 8; d >= 2; d -= pair ? 2 : 1)
        if (q % d == 0 && q / d >= 2) { rpw = d; break; }
    }
    cfg->rows_per_wave = rpw;
    return NM_OK;
  }
  int seg;
  if (cols <= smax) {
    seg = cols > 0 ? (int)cols : 32;
  } else {
    seg = smax >= 1024 ? smax / 1024 * 1024 : smax;
  }
  cfg->seg_cols = seg;
  cfg->threads_per_wg = threads_for_lds(lds_bytes(dense, bp, seg));
  cfg->rows_per_wave = bp == 1 ? 1 : 2;
  return NM_OK;
}

nm_status check_cfg(const nm_launch_cfg &c, int64_t rows, int64_t cols, int n, int m,
                    bool dense, int bp, const DevInfo &di, bool pair = false) {
  const int t = c.threads_per_wg;
  if (t < kWave || t > 1024 || t % kWave != 0) return NM_ERR_INVALID_ARG;
  if (!(c.k_split == 0 || c.k_split == 1 || c.k_split == 2 || c.k_split == 4))
    return NM_ERR_INVALID_ARG;
  if (c.k_split > 1) {
    // the split reduction: 2:4 at batch 1 on the VALU row kernel, x whole in
    // LDS, whole load batches per wave, no epilogue
    if (dense || c.kernel != NM_KERNEL_VALU || bp != 1 || !(n == 2 && m == 4) || pair ||
        !rows_kernel(false, cols, c.seg_cols) || cols % (1024LL * c.k_split) != 0 ||
        (t / kWave) % c.k_split != 0)
      return NM_ERR_UNSUPPORTED;
    if (c.rows_per_wave < 1 || c.rows_per_wave > 64) return NM_ERR_INVALID_ARG;
    if (split_lds_bytes(cols, t / kWave, c.rows_per_wave) > lds_budget(di)) return NM_ERR_INVALID_ARG;
    return NM_OK;
  }
  if (c.kernel == NM_KERNEL_MFMA) {
    if (dense || !mfma_ok(rows, cols, n, m)) return NM_ERR_UNSUPPORTED;
    if (c.rows_per_wave < 2 || c.rows_per_wave > 4) return NM_ERR_INVALID_ARG;
    if (mfma_lds_bytes(t / kWave, c.rows_per_wave, bp, mfma_kind(n, m)) > lds_budget(di))
      return NM_ERR_INVALID_ARG;
    return NM_OK;
  }
  if (c.kernel != NM_KERNEL_VALU) return NM_ERR_INVALID_ARG;
  if (c.seg_cols <= 0 || c.seg_cols % 32 != 0) return NM_ERR_INVALID_ARG;
  if (rows_kernel(dense, cols, c.seg_cols)) {
    if (c.rows_per_wave < 1 || c.rows_per_wave > 64) return NM_ERR_INVALID_ARG;
    if (lds_bytes(dense, bp, cols > 0 ? (int)cols : 32) > lds_budget(di)) return NM_ERR_INVALID_ARG;
    if (!dense && plain48_ok(cols, bp, n, m) && (size_t)cols * 2 + 256 * 16 > lds_budget(di))
      return NM_ERR_INVALID_ARG;
    return NM_OK;
  }
  if (!(c.rows_per_wave == 1 || c.rows_per_wave == 2 || c.rows_per_wave == 4))
    return NM_ERR_INVALID_ARG;
  if (lds_bytes(dense, bp, c.seg_cols) > lds_budget(di)) return NM_ERR_INVALID_ARG;
  return NM_OK;
}

nm_status resolve_cfg(int64_t rows, int64_t cols, int batch, int n, int m, bool dense,
                      const nm_launch_cfg *user, nm_launch_cfg *out, bool pair = false) {
  DevInfo di;
  nm_status st = device_info(&di);
  if (st != NM_OK) return st;
  if (user && user->kernel == NM_KERNEL_MFMA && !dense && mfma_ok(rows, cols, n, m))
    mfma_default(rows, cols, batch, mfma_kind(n, m), di, out);
  else if (user && user->kernel == NM_KERNEL_VALU)
    st = default_cfg(rows, cols, batch, n, m, dense, out, pair, false);
  else
    st = default_cfg(rows, cols, batch, n, m, dense, out, pair);
  if (st != NM_OK) return st;
  if (user) {
    if (user->kernel) out->kernel = user->kernel;
    if (user->threads_per_wg) out->threads_per_wg = user->threads_per_wg;
    if (user->rows_per_wave) out->rows_per_wave = user->rows_per_wave;
    if (user->seg_cols) out->seg_cols = user->seg_cols;
    if (user->k_split) out->k_split = user->k_split;
  }
  return check_cfg(*out, rows, cols, n, m, dense, pad_batch(batch), di, pair);
}

typedef void (*seg_fn)(const uint4 *, const uint32_t *, const uint16_t *, void *, int,
                       int64_t, int, int, int);
// Does the row kernel copy x to LDS by direct-to-LDS loads (its plain-x
// kinds)?  Where x's image is large beside the workgroup's weights: batch >= 2,
// or at most 4 rows per workgroup.  Measured (us, cache-cold, 2:4 fp16): k
// 1024x4096 batch 1 / 2 / 4: 3.36 / 3.77 / 4.51 -> 2.99 / 3.26 / 3.94; 70B k
// 1024x8192 batch 1 / 4: 4.41 / 6.75 -> 3.92 / 5.33; 14336x4096 batch 2:
// 13.24 -> 12.38; but at batch 1 with 12 or more rows per workgroup the
// register path stays ahead (14336x4096 11.57 against 11.80, 6144x4096 6.50
// against 6.85).
int x_by_dma(int bp, int64_t rows_per_wg) { return bp >= 2 || rows_per_wg <= 4 ? 1 : 0; }

typedef void (*rows_fn)(const uint4 *, const uint32_t *, const uint16_t *, void *, int,
                        int64_t, int, int, int, int);
typedef void (*dense_fn)(const uint4 *, const uint16_t *, void *, int, int64_t,
                         int, int, int);

template <bool BF, int BP, int PK>
seg_fn pick_seg_rpw(int rpw) {
  switch (rpw) {
    case 1: return nm_spmv_seg_kernel<BF, BP, PK, 1>;
    case 2: return nm_spmv_seg_kernel<BF, BP, PK, 2>;
    default: return nm_spmv_seg_kernel<BF, BP, PK, 4>;
  }
}

template <bool BF, int PK>
seg_fn pick_seg_bp(int bp, int rpw) {
  switch (bp) {
    case 1: return pick_seg_rpw<BF, 1, PK>(rpw);
    case 2: return pick_seg_rpw<BF, 2, PK>(rpw);
    case 4: return pick_seg_rpw<BF, 4, PK>(rpw);
    default: return pick_seg_rpw<BF, 8, PK>(rpw);
  }
}

template <bool BF>
seg_fn pick_seg_pk(int pk, int bp, int rpw) {
  switch (pk) {
    case kPat24: return pick_seg_bp<BF, kPat24>(bp, rpw);
    case kPatHalf: return pick_seg_bp<BF, kPatHalf>(bp, rpw);
    default: return pick_seg_bp<BF, kPat1632>(bp, rpw);
  }
}

seg_fn pick_seg(bool bf, int pk, int bp, int rpw) {
  return bf ? pick_seg_pk<true>(pk, bp, rpw) : pick_seg_pk<false>(pk, bp, rpw);
}

template <bool BF, int PK>
rows_fn pick_rows_bp(int bp, int u, int xs) {
  switch (bp) {
    case 1:
      if (xs > 4)
        return u == 5 ? nm_spmv_rows_kernel<BF, 1, PK, 5, 8> : nm_spmv_rows_kernel<BF, 1, PK, 4, 8>;
      return u == 5 ? nm_spmv_rows_kernel<BF, 1, PK, 5, 4> : nm_spmv_rows_kernel<BF, 1, PK, 4, 4>;
    case 2: return nm_spmv_rows_kernel<BF, 2, PK, 4, 1>;
    case 4: return nm_spmv_rows_kernel<BF, 4, PK, 4, 1>;
    default: return nm_spmv_rows_kernel<BF, 8, PK, 4, 1>;
  }
}

template <bool BF, int PK, int XS>
rows_fn pick_rows_24x_u(int u) {
  switch (u) {
    case 2: return nm_spmv_rows_kernel<BF, 1, PK, 2, XS>;
    case 5: return nm_spmv_rows_kernel<BF, 1, PK, 5, XS>;
    default: return nm_spmv_rows_kernel<BF, 1, PK, 4, XS>;
  }
}

template <bool BF, int PK>
rows_fn pick_rows_24x_xs(int u, int xs) {
  return xs > 4 ? pick_rows_24x_u<BF, PK, 8>(u) : pick_rows_24x_u<BF, PK, 4>(u);
}

template <bool BF>
rows_fn pick_rows_24x(int u, int xs, bool exact) {
  return exact ? pick_rows_24x_xs<BF, kPat24xE>(u, xs) : pick_rows_24x_xs<BF, kPat24x>(u, xs);
}

// 2:4 at batch 2..8 (padded to 2, 4, 8): x stored plainly per token.
template <bool BF, int PK>
rows_fn pick_rows_24xm_bp(int bp) {
  switch (bp) {
    case 2: return nm_spmv_rows_kernel<BF, 2, PK, 4, 1>;
    case 4: return nm_spmv_rows_kernel<BF, 4, PK, 4, 1>;
    default: return nm_spmv_rows_kernel<BF, 8, PK, 4, 1>;
  }
}

template <bool BF>
rows_fn pick_rows_pk(int pk, int bp, int u, int xs, bool exact) {
  switch (pk) {
    case kPat24:
      if (bp == 1) return pick_rows_24x<BF>(u, xs, exact);
      return exact ? pick_rows_24xm_bp<BF, kPat24xE>(bp) : pick_rows_24xm_bp<BF, kPat24x>(bp);
    case kPatHalf: return pick_rows_bp<BF, kPatHalf>(bp, u, xs);
    default: return pick_rows_bp<BF, kPat1632>(bp, u, xs);
  }
}

// xs: x groups (8 columns each at batch 1) a thread needs to stage all of x;
// exact: the row's value chunks are a whole number of load batches (only the
// 2:4 batch-1 kernel has a separate kind for it)
rows_fn pick_rows(bool bf, int pk, int bp, int u, int xs, bool exact) {
  return bf ? pick_rows_pk<true>(pk, bp, u, xs, exact) : pick_rows_pk<false>(pk, bp, u, xs, exact);
}

// 4:8 at batch 1 with x stored plainly and the pair-selector table.
template <bool BF, int PK>
rows_fn pick_rows_48x_xs(int u, int xs) {
  return xs > 4 ? pick_rows_24x_u<BF, PK, 8>(u) : pick_rows_24x_u<BF, PK, 4>(u);
}

rows_fn pick_rows48(bool bf, int u, int xs, bool exact) {
  if (bf) return exact ? pick_rows_48x_xs<true, kPat48xE>(u, xs) : pick_rows_48x_xs<true, kPat48x>(u, xs);
  return exact ? pick_rows_48x_xs<false, kPat48xE>(u, xs) : pick_rows_48x_xs<false, kPat48x>(u, xs);
}

// LDS of the 4:8 plain kind: x (2 bytes per column) and the 4 KiB table.
size_t plain48_lds_bytes(int64_t cols) {
  return (size_t)cols * 2 + kPair48TableBytes;
}

// The split-reduction kernels (2:4, batch 1, exact kind): KS waves per row
// group, U chunks per lane per load batch.
template <bool BF, int KS, int XS>
rows_fn pick_split_u(int u) {
  switch (u) {
    case 1: return nm_spmv_rows_kernel<BF, 1, kPat24xE, 1, XS, KS>;
    case 2: return nm_spmv_rows_kernel<BF, 1, kPat24xE, 2, XS, KS>;
    case 5: return nm_spmv_rows_kernel<BF, 1, kPat24xE, 5, XS, KS>;
    default: return nm_spmv_rows_kernel<BF, 1, kPat24xE, 4, XS, KS>;
  }
}

template <bool BF>
rows_fn pick_split_bf(int ks, int u, int xs) {
  if (ks == 2) return xs > 4 ? pick_split_u<BF, 2, 8>(u) : pick_split_u<BF, 2, 4>(u);
  return xs > 4 ? pick_split_u<BF, 4, 8>(u) : pick_split_u<BF, 4, 4>(u);
}

rows_fn pick_split(bool bf, int ks, int u, int xs) {
  return bf ? pick_split_bf<true>(ks, u, xs) : pick_split_bf<false>(ks, u, xs);
}


// Chunks per lane per load batch of the batch-1 row kernel: 4, or 5 when
// that divides the row's chunks per lane (K / 1024) and 4 does not, or 2 when
// neither does but 2 does, so the row's last batch has no idle slots
// (K = 5120, 25600: 5; K = 14336: 2, with one row per wave, see default_cfg).
// Measured on the 8B/70B/Qwen shapes: 5 helps the K = 5120k shapes; for
// K = 14336, 2 (12.0 us) beats a ragged last batch of 4 (12.4 us), and 7 costs
// occupancy and is slower than both.
int rows_batch_chunks(int64_t cols, int bp) {
  if (bp != 1 || cols % 1024 != 0) return 4;
  const int64_t c = cols / 1024;
  if (c % 4 == 0) return 4;
  if (c % 5 == 0) return 5;
  return c % 2 == 0 ? 2 : 4;
}

template <bool BF, int BP>
dense_fn pick_dense_rpw(int rpw) {
  switch (rpw) {
    case 1: return nm_dense_kernel<BF, BP, 1>;
    case 2: return nm_dense_kernel<BF, BP, 2>;
    default: return nm_dense_kernel<BF, BP, 4>;
  }
}

template <bool BF>
dense_fn pick_dense_bp(int bp, int rpw) {
  switch (bp) {
    case 1: return pick_dense_rpw<BF, 1>(rpw);
    case 2: return pick_dense_rpw<BF, 2>(rpw);
    case 4: return pick_dense_rpw<BF, 4>(rpw);
    default: return pick_dense_rpw<BF, 8>(rpw);
  }
}

dense_fn pick_dense(bool bf, int bp, int rpw) {
  return bf ? pick_dense_bp<true>(bp, rpw) : pick_dense_bp<false>(bp, rpw);
}

typedef void (*dense_rows_fn)(const uint4 *, const uint16_t *, void *, int, int64_t, int, int,
                              int);

template <bool BF>
dense_rows_fn pick_dense_rows_bp(int bp) {
  switch (bp) {
    case 1: return nm_dense_rows_kernel<BF, 1>;
    case 2: return nm_dense_rows_kernel<BF, 2>;
    case 4: return nm_dense_rows_kernel<BF, 4>;
    default: return nm_dense_rows_kernel<BF, 8>;
  }
}

dense_rows_fn pick_dense_rows(bool bf, int bp) {
  return bf ? pick_dense_rows_bp<true>(bp) : pick_dense_rows_bp<false>(bp);
}

typedef void (*mfma_fn)(const uint16_t *, const uint32_t *, const uint16_t *, void *, int,
                        int64_t, int, int);

template <bool BF, int BP, int KIND>
mfma_fn pick_mfma_nb(int nb) {
  switch (nb) {
    case 2: return nm_spmm_mfma_kernel<BF, BP, 2, KIND>;
    case 3: return nm_spmm_mfma_kernel<BF, BP, 3, KIND>;
    default: return nm_spmm_mfma_kernel<BF, BP, 4, KIND>;
  }
}

template <bool BF, int KIND>
mfma_fn pick_mfma_bp(int bp, int nb) {
  switch (bp) {
    case 2: return pick_mfma_nb<BF, 2, KIND>(nb);
    case 4: return pick_mfma_nb<BF, 4, KIND>(nb);
    default: return pick_mfma_nb<BF, 8, KIND>(nb);
  }
}

template <bool BF>
mfma_fn pick_mfma_kind(int kind, int bp, int nb) {
  switch (kind) {
    case kMfmaSparse24: return pick_mfma_bp<BF, kMfmaSparse24>(bp, nb);
    case kMfmaDenseHalf: return pick_mfma_bp<BF, kMfmaDenseHalf>(bp, nb);
    default: return pick_mfma_bp<BF, kMfmaDense1632>(bp, nb);
  }
}

mfma_fn pick_mfma(bool bf, int kind, int bp, int nb) {
  return bf ? pick_mfma_kind<true>(kind, bp, nb) : pick_mfma_kind<false>(kind, bp, nb);
}

// The launch shape of a sparse product with the caller's overrides (user may
// be NULL), checked: the 50% patterns through resolve_cfg, the other
// densities through the generic kernels' rules.
nm_status resolve_sparse(int64_t rows, int64_t cols, int batch, int n, int m,
                         const nm_launch_cfg *user, nm_launch_cfg *cfg, bool pair) {
  if (pattern_ok(n, m)) return resolve_cfg(rows, cols, batch, n, m, false, user, cfg, pair);
  DevInfo di;
  nm_status st = device_info(&di);
  if (st != NM_OK) return st;
  st = generic_default_cfg(rows, cols, batch, n, m, di.cus, lds_budget(di), cfg);
  if (st != NM_OK) return st;
  if (user) {
    if (!(user->k_split == 0 || user->k_split == 1 || user->k_split == 2 || user->k_split == 4))
      return NM_ERR_INVALID_ARG;
    if (user->k_split > 1) return NM_ERR_UNSUPPORTED;  // the split reduction is 2:4 only
    if (user->kernel) cfg->kernel = user->kernel;
    if (user->threads_per_wg) cfg->threads_per_wg = user->threads_per_wg;
    if (user->rows_per_wave) cfg->rows_per_wave = user->rows_per_wave;
    if (user->seg_cols) cfg->seg_cols = user->seg_cols;
  }
  return generic_check_cfg(*cfg, batch, n, m, lds_budget(di));
}

// epi: kEpiNone, or kEpiSwiglu (rows are (gate, up) pairs, Y has rows / 2
// columns per token).
int sparse_product(const void *values, const uint32_t *bits, const void *X,
                   void *Y, int batch, int64_t rows, int64_t cols, int n,
                   int m, nm_dtype in_dt, nm_dtype out_dt,
                   const nm_launch_cfg *user, void *stream, int epi = kEpiNone) {
  nm_status st = check_dims(rows, cols, batch);
  if (st != NM_OK) return st;
  if (!pattern_any_ok(n, m) || !is16(in_dt) || !out_ok(in_dt, out_dt)) return NM_ERR_UNSUPPORTED;
  if (!pattern_ok(n, m) && epi != kEpiNone) return NM_ERR_UNSUPPORTED;
  const bool empty_w = rows == 0 || cols == 0;
  if ((!values && !empty_w) || (!bits && !empty_w) || (!X && cols != 0) ||
      (!Y && rows != 0))
    return NM_ERR_INVALID_ARG;
  const uintptr_t ysz = out_dt == NM_F32 ? 4 : 2;
  if (!aligned(values, 16) || !aligned(bits, 4) || !aligned(X, 16) || !aligned(Y, ysz))
    return NM_ERR_ALIGN;
  if (rows == 0) return NM_OK;
  nm_launch_cfg cfg = {};
  const bool pair = epi == kEpiSwiglu;
  st = resolve_sparse(rows, cols, batch, n, m, user, &cfg, pair);
  if (st != NM_OK) return st;
  if (!pattern_ok(n, m))  // densities other than 50%: the generic kernels
    return generic_launch(values, bits, X, Y, batch, rows, cols, n, m, in_dt, out_dt, cfg, stream);
  if (pair && cfg.kernel != NM_KERNEL_MFMA) {
    // the epilogue lives in the row kernel: each wave an even number of rows
    if (!rows_kernel(false, cols, cfg.seg_cols)) return NM_ERR_UNSUPPORTED;
    if (cfg.rows_per_wave % 2 != 0) return NM_ERR_INVALID_ARG;
  }
  const int out_kind = (int)out_dt | (epi << kEpiShift);
  const int bp = pad_batch(batch);
  const bool bf = in_dt == NM_BF16;
  if (cfg.kernel == NM_KERNEL_MFMA) {
    const int waves = cfg.threads_per_wg / kWave, nb = cfg.rows_per_wave;
    const int mbp = bp < 2 ? 2 : bp;
    const int64_t grid = (rows + 15) / 16;
    const int kind = mfma_kind(n, m);
    hipLaunchKernelGGL(pick_mfma(bf, kind, mbp, nb), dim3((unsigned)grid),
                       dim3(cfg.threads_per_wg), mfma_lds_bytes(waves, nb, mbp, kind),
                       (hipStream_t)stream,
                       (const uint16_t *)values, bits, (const uint16_t *)X, Y, batch, rows,
                       (int)cols, out_kind);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? NM_OK : hip_fail(e);
  }
  const int pk = pattern_kind(m);
  const int wpg = cfg.threads_per_wg / kWave;
  if (cfg.k_split > 1) {  // the split reduction (checked by resolve_cfg)
    const int ks = cfg.k_split;
    const int64_t rows_per_wg = (int64_t)(wpg / ks) * cfg.rows_per_wave;
    const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
    if (grid > INT32_MAX) return NM_ERR_INVALID_ARG;
    const int xs = (int)((cols / 8 + cfg.threads_per_wg - 1) / cfg.threads_per_wg);
    hipLaunchKernelGGL(pick_split(bf, ks, split_batch_chunks(cols, ks), xs), dim3((unsigned)grid),
                       dim3(cfg.threads_per_wg), split_lds_bytes(cols, wpg, cfg.rows_per_wave),
                       (hipStream_t)stream, (const uint4 *)values, bits, (const uint16_t *)X, Y,
                       batch, rows, (int)cols, cfg.rows_per_wave, out_kind,
                       x_by_dma(bp, rows_per_wg));
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? NM_OK : hip_fail(e);
  }
  if (rows_kernel(false, cols, cfg.seg_cols)) {
    const int64_t rows_per_wg = (int64_t)wpg * cfg.rows_per_wave;
    const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
    if (grid > INT32_MAX) return NM_ERR_INVALID_ARG;
    const int xs = (int)((cols / 8 + cfg.threads_per_wg - 1) / cfg.threads_per_wg);
    const int ub = rows_batch_chunks(cols, bp);
    const bool exact = cols % (1024LL * ub) == 0;  // 16 columns per chunk, 64 lanes
    const int xdma = x_by_dma(bp, rows_per_wg);
    if (plain48_ok(cols, bp, n, m)) {
      hipLaunchKernelGGL(pick_rows48(bf, ub, xs, exact), dim3((unsigned)grid),
                         dim3(cfg.threads_per_wg), plain48_lds_bytes(cols), (hipStream_t)stream,
                         (const uint4 *)values, bits, (const uint16_t *)X, Y, batch, rows,
                         (int)cols, cfg.rows_per_wave, out_kind, xdma);
    } else {
      hipLaunchKernelGGL(pick_rows(bf, pk, bp, ub, xs, exact), dim3((unsigned)grid),
                         dim3(cfg.threads_per_wg),
                         sparse_lds_bytes(bp, cols > 0 ? (int)cols : 32), (hipStream_t)stream,
                         (const uint4 *)values, bits, (const uint16_t *)X, Y, batch, rows,
                         (int)cols, cfg.rows_per_wave, out_kind, xdma);
    }
  } else {
    const int64_t rows_per_wg = (int64_t)wpg * cfg.rows_per_wave;
    const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
    if (grid > INT32_MAX) return NM_ERR_INVALID_ARG;
    hipLaunchKernelGGL(pick_seg(bf, pk, bp, cfg.rows_per_wave), dim3((unsigned)grid),
                       dim3(cfg.threads_per_wg), sparse_lds_bytes(bp, cfg.seg_cols),
                       (hipStream_t)stream, (const uint4 *)values, bits, (const uint16_t *)X, Y,
                       batch, rows, (int)cols, cfg.seg_cols, (int)out_dt);
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

// Argument checks of the pack entry points (nothing here touches HIP);
// *empty: there is nothing to pack.
nm_status pack_check(const void *W, const uint8_t *keep, int64_t rows, int64_t cols, int n, int m,
                     nm_dtype dt, const void *values, const uint32_t *bits, bool *empty) {
  if (rows < 0 || cols < 0) return NM_ERR_INVALID_ARG;
  if (rows > INT32_MAX || cols > INT32_MAX) return NM_ERR_INVALID_ARG;
  if (!pattern_any_ok(n, m) || !is16(dt)) return NM_ERR_UNSUPPORTED;
  if (cols % 32 != 0) return NM_ERR_SHAPE;
  *empty = rows == 0 || cols == 0;
  if (!*empty && (!W || !keep || !values || !bits)) return NM_ERR_INVALID_ARG;
  if (!aligned(W, 2) || !aligned(values, 16) || !aligned(bits, 4)) return NM_ERR_ALIGN;
  return NM_OK;
}

// The pack kernel for pattern n:m on stream s; invalid groups are counted
// into *dbad (device), which the caller has cleared.
hipError_t pack_launch(const void *W, const uint8_t *keep, int64_t rows, int64_t cols, int n, int m,
                       void *values, uint32_t *bits, int *dbad, hipStream_t s) {
  const int threads = 256, wpg = threads / kWave;
  int64_t grid = (rows + wpg - 1) / wpg;
  if (grid > (1 << 20)) grid = 1 << 20;
  const int K = (int)cols;
  const uint16_t *w16 = (const uint16_t *)W;
  uint16_t *v16 = (uint16_t *)values;
  switch (m) {
    case 4: hipLaunchKernelGGL(nm_pack_kernel<4>, dim3((unsigned)grid), dim3(threads), 0, s, w16, keep, rows, K, n, v16, bits, dbad); break;
    case 8: hipLaunchKernelGGL(nm_pack_kernel<8>, dim3((unsigned)grid), dim3(threads), 0, s, w16, keep, rows, K, n, v16, bits, dbad); break;
    case 16: hipLaunchKernelGGL(nm_pack_kernel<16>, dim3((unsigned)grid), dim3(threads), 0, s, w16, keep, rows, K, n, v16, bits, dbad); break;
    default: hipLaunchKernelGGL(nm_pack_kernel<32>, dim3((unsigned)grid), dim3(threads), 0, s, w16, keep, rows, K, n, v16, bits, dbad); break;
  }
  return hipGetLastError();
}

// The device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU holds its own copy of the array
// at its own address; the array's name in host code is only a stand-in), and
// the lock that serialises the allocation-free calls on that device.
struct ScratchDev {
  bool init = false;
  int *ptr = nullptr;
  std::mutex mu;
};
ScratchDev g_scratch[kMaxDev];
std::mutex g_scratch_mu;

nm_status scratch_of_device(int **ptr, std::mutex **mu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDev) return NM_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  ScratchDev &d = g_scratch[dev];
  if (!d.init) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    d.ptr = static_cast<int *>(p);
    d.init = true;
  }
  *ptr = d.ptr;
  *mu = &d.mu;
  return NM_OK;
}

}  // namespace

extern "C" {

const char *nm_status_string(int status) {
  switch (status) {
    case NM_OK: return "NM_OK";
    case NM_ERR_INVALID_ARG: return "NM_ERR_INVALID_ARG: invalid argument";
    case NM_ERR_UNSUPPORTED: return "NM_ERR_UNSUPPORTED: unsupported pattern or dtype";
    case NM_ERR_SHAPE: return "NM_ERR_SHAPE: cols must be a multiple of 32";
    case NM_ERR_ALIGN: return "NM_ERR_ALIGN: misaligned pointer";
    case NM_ERR_MASK: return "NM_ERR_MASK: an M-group does not keep exactly N";
    case NM_ERR_HIP: return "NM_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown nm_status";
  }
}

int nm_last_hip_error(void) { return nm_host::g_last_hip; }

int nm_packed_bytes(int64_t rows, int64_t cols, int n, int m, nm_dtype dt,
                    size_t *values_bytes, size_t *bits_bytes) {
  if (rows < 0 || cols < 0 || !values_bytes || !bits_bytes) return NM_ERR_INVALID_ARG;
  if (!pattern_any_ok(n, m) || !is16(dt)) return NM_ERR_UNSUPPORTED;
  if (cols % 32 != 0) return NM_ERR_SHAPE;
  if (rows > INT32_MAX || cols > INT32_MAX) return NM_ERR_INVALID_ARG;
  const uint64_t rc = (uint64_t)rows * (uint64_t)cols;
  // rows x cols*n/m values, rounded up to 16 bytes (a whole last chunk for
  // the 16-byte loads; already whole at 50%)
  *values_bytes = (size_t)((rc / (uint64_t)m * (uint64_t)n * 2u + 15u) & ~(uint64_t)15);
  *bits_bytes = (size_t)(rc / 8u);
  return NM_OK;
}

int nm_pack(const void *W, const uint8_t *keep, int64_t rows, int64_t cols,
            int n, int m, nm_dtype dt, void *values, uint32_t *bits,
            void *stream) {
  bool empty = false;
  nm_status st = pack_check(W, keep, rows, cols, n, m, dt, values, bits, &empty);
  if (st != NM_OK || empty) return st;
  hipStream_t s = (hipStream_t)stream;
  int *dbad = nullptr;
  hipError_t e = hipMalloc((void **)&dbad, sizeof(int));
  if (e != hipSuccess) return hip_fail(e);
  int hbad = 0;
  e = hipMemsetAsync(dbad, 0, sizeof(int), s);
  if (e == hipSuccess) e = pack_launch(W, keep, rows, cols, n, m, values, bits, dbad, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&hbad, dbad, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  hipError_t ef = hipFree(dbad);
  if (e != hipSuccess) return hip_fail(e);
  if (ef != hipSuccess) return hip_fail(ef);
  return hbad ? NM_ERR_MASK : NM_OK;
}

int nm_pack_noalloc(const void *W, const uint8_t *keep, int64_t rows, int64_t cols,
                    int n, int m, nm_dtype dt, void *values, uint32_t *bits,
                    void *stream) {
  bool empty = false;
  nm_status st = pack_check(W, keep, rows, cols, n, m, dt, values, bits, &empty);
  if (st != NM_OK || empty) return st;
  int *dbad = nullptr;
  std::mutex *mu = nullptr;
  st = scratch_of_device(&dbad, &mu);
  if (st != NM_OK) return st;
  // one call at a time per device in this process: the calls share the
  // device's counter, and the call is synchronous
  std::lock_guard<std::mutex> g(*mu);
  hipStream_t s = (hipStream_t)stream;
  int hbad = 0;
  // the counter keeps the previous call's count: cleared by a one-thread
  // kernel on the call's stream, ordered before the pack
  hipLaunchKernelGGL(nm_zero_ints_kernel, dim3(1), dim3(kWave), 0, s, dbad, kPackScratchInts);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = pack_launch(W, keep, rows, cols, n, m, values, bits, dbad, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&hbad, dbad, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  return hbad ? NM_ERR_MASK : NM_OK;
}

int nm_spmv(const void *values, const uint32_t *bits, const void *x, void *y,
            int64_t rows, int64_t cols, int n, int m, nm_dtype in_dt,
            nm_dtype out_dt, void *stream) {
  return sparse_product(values, bits, x, y, 1, rows, cols, n, m, in_dt, out_dt,
                        nullptr, stream);
}

int nm_spmm_small(const void *values, const uint32_t *bits, const void *X,
                  void *Y, int batch, int64_t rows, int64_t cols, int n, int m,
                  nm_dtype in_dt, nm_dtype out_dt, void *stream) {
  return sparse_product(values, bits, X, Y, batch, rows, cols, n, m, in_dt,
                        out_dt, nullptr, stream);
}

int nm_spmm_small_cfg(const void *values, const uint32_t *bits, const void *X,
                      void *Y, int batch, int64_t rows, int64_t cols, int n,
                      int m, nm_dtype in_dt, nm_dtype out_dt,
                      const nm_launch_cfg *cfg, void *stream) {
  return sparse_product(values, bits, X, Y, batch, rows, cols, n, m, in_dt,
                        out_dt, cfg, stream);
}

int nm_spmm_swiglu(const void *values, const uint32_t *bits, const void *X, void *H,
                   int batch, int64_t inter, int64_t cols, int n, int m, nm_dtype in_dt,
                   nm_dtype out_dt, void *stream) {
  return nm_spmm_swiglu_cfg(values, bits, X, H, batch, inter, cols, n, m, in_dt, out_dt,
                            nullptr, stream);
}

int nm_spmm_swiglu_cfg(const void *values, const uint32_t *bits, const void *X, void *H,
                       int batch, int64_t inter, int64_t cols, int n, int m, nm_dtype in_dt,
                       nm_dtype out_dt, const nm_launch_cfg *cfg, void *stream) {
  if (inter < 0 || inter > INT32_MAX / 2) return NM_ERR_INVALID_ARG;
  return sparse_product(values, bits, X, H, batch, 2 * inter, cols, n, m, in_dt, out_dt, cfg,
                        stream, kEpiSwiglu);
}

int nm_default_launch(int64_t rows, int64_t cols, int batch, int n, int m, int dense,
                      nm_launch_cfg *cfg) {
  if (!cfg) return NM_ERR_INVALID_ARG;
  nm_status st = check_dims(rows, cols, batch);
  if (st != NM_OK) return st;
  if (!dense && !pattern_any_ok(n, m)) return NM_ERR_UNSUPPORTED;
  if (!dense && !pattern_ok(n, m)) {
    DevInfo di;
    st = device_info(&di);
    if (st != NM_OK) return st;
    return generic_default_cfg(rows, cols, batch, n, m, di.cus, lds_budget(di), cfg);
  }
  return default_cfg(rows, cols, batch, n, m, dense != 0, cfg);
}

int nm_resolve_launch(int64_t rows, int64_t cols, int batch, int n, int m, int dense,
                      const nm_launch_cfg *user, nm_launch_cfg *cfg) {
  if (!cfg) return NM_ERR_INVALID_ARG;
  nm_status st = check_dims(rows, cols, batch);
  if (st != NM_OK) return st;
  if (dense) return resolve_cfg(rows, cols, batch, 0, 0, true, user, cfg);
  if (!pattern_any_ok(n, m)) return NM_ERR_UNSUPPORTED;
  return resolve_sparse(rows, cols, batch, n, m, user, cfg, false);
}

int nm_dense_gemv_cfg(const void *W, const void *X, void *Y, int batch,
                      int64_t rows, int64_t cols, nm_dtype in_dt,
                      nm_dtype out_dt, const nm_launch_cfg *user,
                      void *stream) {
  nm_status st = check_dims(rows, cols, batch);
  if (st != NM_OK) return st;
  if (!is16(in_dt) || !out_ok(in_dt, out_dt)) return NM_ERR_UNSUPPORTED;
  const bool empty_w = rows == 0 || cols == 0;
  if ((!W && !empty_w) || (!X && cols != 0) || (!Y && rows != 0)) return NM_ERR_INVALID_ARG;
  const uintptr_t ysz = out_dt == NM_F32 ? 4 : 2;
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, ysz)) return NM_ERR_ALIGN;
  if (rows == 0) return NM_OK;
  nm_launch_cfg cfg = {};
  st = resolve_cfg(rows, cols, batch, 0, 0, true, user, &cfg);
  if (st != NM_OK) return st;
  const int bp = pad_batch(batch);
  const bool bf = in_dt == NM_BF16;
  const int64_t rows_per_wg = (int64_t)(cfg.threads_per_wg / kWave) * cfg.rows_per_wave;
  const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
  if (grid > INT32_MAX) return NM_ERR_INVALID_ARG;
  if (rows_kernel(true, cols, cfg.seg_cols)) {
    hipLaunchKernelGGL(pick_dense_rows(bf, bp), dim3((unsigned)grid), dim3(cfg.threads_per_wg),
                       dense_lds_bytes(bp, cols > 0 ? (int)cols : 32), (hipStream_t)stream,
                       (const uint4 *)W, (const uint16_t *)X, Y, batch, rows, (int)cols,
                       cfg.rows_per_wave, (int)out_dt);
  } else {
    hipLaunchKernelGGL(pick_dense(bf, bp, cfg.rows_per_wave), dim3((unsigned)grid),
                       dim3(cfg.threads_per_wg), dense_lds_bytes(bp, cfg.seg_cols),
                       (hipStream_t)stream, (const uint4 *)W, (const uint16_t *)X, Y, batch, rows,
                       (int)cols, cfg.seg_cols, (int)out_dt);
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

int nm_dense_gemv(const void *W, const void *X, void *Y, int batch,
                  int64_t rows, int64_t cols, nm_dtype in_dt, nm_dtype out_dt,
                  void *stream) {
  return nm_dense_gemv_cfg(W, X, Y, batch, rows, cols, in_dt, out_dt, nullptr,
                           stream);
}

int nm_stream_read(const void *buf, size_t bytes, uint32_t *out, int grid, int threads_per_wg,
                   void *stream) {
  if (!buf || !out || bytes == 0 || grid < 1) return NM_ERR_INVALID_ARG;
  if (bytes % 16 != 0) return NM_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(out, 4)) return NM_ERR_ALIGN;
  const int t = threads_per_wg;
  if (!(t == 64 || t == 128 || t == 256 || t == 512 || t == 1024)) return NM_ERR_INVALID_ARG;
  hipLaunchKernelGGL(nm_stream_read_kernel, dim3((unsigned)grid), dim3(t), 0, (hipStream_t)stream,
                     (const char *)buf, (int64_t)(bytes / 16), out);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

}  // extern "C"

