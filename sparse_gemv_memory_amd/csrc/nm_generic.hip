// nm_generic.hip -- N:M bitmask product at densities other than 50%.
//
// "SparseDecoding: Decoding-Aware Pruning for Accurate and Efficient LLM
// Inference", Method, kernel subsection: item (1) "Bitmask indexing" stores
// one bit per column and the kept weights in increasing column order; item
// (2) "Fixed-step bitmask traversal" rests on every aligned 32-bit word of a
// 50% N:M row holding the same number of set bits.  The same holds for any
// N:M pattern with M dividing 32: each word holds exactly P = 32 N / M set
// bits, so word w's values start at w * P within the row (no prefix sums) and
// each word is walked in P fixed steps, each taking the lowest set bit as the
// next kept column and clearing it.  The stored format is the one of the 50%
// kinds, with row stride K * N / M values.
//
// Kernel design (gfx950).  One wavefront walks a window of 64 mask words of a
// row, one word per lane.  The window's values are one contiguous run of 64 P
// values; the wave copies it from HBM straight into its LDS buffer with
// 16-byte direct-to-LDS buffer loads (range-checked, so nothing outside the
// window's 16-byte-aligned span is read), double-buffered so the next
// window's copy is in flight while this one is consumed.  Lane l then reads
// its P values at l * P from LDS and the x values of its kept columns from
// the LDS copy of x (column-major slots of all batch rows), and accumulates
// pairs with v_dot2_f32_{f16,bf16} (the products are exact in fp32).  x is
// staged per workgroup in segments when all of it does not fit the LDS
// budget.

#include <mutex>

#include "nm_device.h"
#include "nm_host.h"

namespace {

constexpr int kWinWords = 64;  // mask words per window (one per lane)

// Chunks of 16 bytes (8 values) one window can span: 64 P values plus up to
// 7 values of alignment slack in front.
__host__ __device__ constexpr int win_chunks(int p) { return 8 * p + 1; }
// Direct-to-LDS load instructions per window (64 chunks each).  A buffer of
// win_loads * 1 KiB >= 16 (8p + 1) bytes is a multiple of 128 bytes, so it
// also holds the up to 7 slots past lane 63's last value that the 8-step
// groups of the traversal read (and drop).
__host__ __device__ constexpr int win_loads(int p) { return (win_chunks(p) + 63) / 64; }

// LDS image of a segment of x: bit b of the segment's word w (column
// 32 w + b) holds the BP batch values of that column in one slot of SB bytes
// at w * WS + b * SB; each word's 32 slots are followed by PB pad bytes, so
// the words that the 64 lanes of a wave gather from at once (one word per
// lane) start in different LDS banks.
template <int BP>
struct XCols {
  static constexpr int SB = 2 * BP;
  static constexpr int PB = SB < 4 ? 4 : SB;
  static constexpr int WS = 32 * SB + PB;
  static constexpr size_t bytes(int seg_cols) { return (size_t)(seg_cols / 32) * WS; }
};

// x segment [s0, s0 + S) of every batch row into the XCols<BP> image (rows
// >= B hold zeros), one 8-column group at a time.
template <int BP>
__device__ __forceinline__ void stage_x_cols(char *lds, const uint16_t *__restrict__ x, int B,
                                             int K, int s0, int S) {
  using L = XCols<BP>;
  for (int g = threadIdx.x; g < S / 8; g += blockDim.x) {
    uint4 r[BP];
#pragma unroll
    for (int b = 0; b < BP; ++b) {
      const int bb = b < B ? b : B - 1;
      r[b] = reinterpret_cast<const uint4 *>(x + (int64_t)bb * K + s0)[g];
      if (b >= B) r[b] = make_uint4(0, 0, 0, 0);
    }
    char *dst = lds + (g >> 2) * L::WS + (8 * g & 31) * L::SB;
    if constexpr (BP == 1) {  // 4-byte aligned: four dword stores
      uint32_t *d = reinterpret_cast<uint32_t *>(dst);
      d[0] = r[0].x;
      d[1] = r[0].y;
      d[2] = r[0].z;
      d[3] = r[0].w;
    } else {
      uint16_t *d = reinterpret_cast<uint16_t *>(dst);
#pragma unroll
      for (int b = 0; b < BP; ++b) {
        uint16_t h[8];
        __builtin_memcpy(h, &r[b], 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e * BP + b] = h[e];
      }
    }
  }
}

// Sum of v over the wave, the same value in every lane (the DPP reduction
// into lane 63, then a read of lane 63 executed by the whole wave).
__device__ __forceinline__ float wave_total(float v) {
  const float s = wave_sum_to_63(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), kWave - 1));
}

// Kept pair (x slots at byte offsets a0, a1 of the XCols image; packed
// weights w) for every batch row.
template <bool BF, int BP>
__device__ __forceinline__ void pair_acc(const char *lds, int a0, int a1, uint32_t w,
                                         float (&acc)[BP]) {
  const lds_ptr x0 = (lds_ptr)lds + a0, x1 = (lds_ptr)lds + a1;
  if constexpr (BP == 1) {
    u16x2_t pr;
    pr[0] = ld<uint16_t>(x0);
    pr[1] = ld<uint16_t>(x1);
    acc[0] = dot2<BF>(w, __builtin_bit_cast(uint32_t, pr), acc[0]);
  } else {
    uint32_t a[BP / 2], b[BP / 2];
    if constexpr (BP == 2) {
      a[0] = ld<uint32_t>(x0);
      b[0] = ld<uint32_t>(x1);
    } else if constexpr (BP == 4) {
      const u32x2_t p = ld<u32x2_t>(x0), q = ld<u32x2_t>(x1);
      a[0] = p[0]; a[1] = p[1];
      b[0] = q[0]; b[1] = q[1];
    } else {
      const u32x4_t p = ld<u32x4_t>(x0), q = ld<u32x4_t>(x1);
#pragma unroll
      for (int d = 0; d < 4; ++d) { a[d] = p[d]; b[d] = q[d]; }
    }
#pragma unroll
    for (int d = 0; d < BP / 2; ++d) {
      acc[2 * d] = dot2<BF>(w, (a[d] & 0xffffu) | (b[d] << 16), acc[2 * d]);
      acc[2 * d + 1] = dot2<BF>(w, (a[d] >> 16) | (b[d] & 0xffff0000u), acc[2 * d + 1]);
    }
  }
}

// One kept weight v (low half; the high half is 0 and meets an x of 0, so the
// pair product adds exactly v * x).
template <bool BF, int BP>
__device__ __forceinline__ void single_acc(const char *lds, int a0, uint32_t v,
                                           float (&acc)[BP]) {
  const lds_ptr x0 = (lds_ptr)lds + a0;
#pragma unroll
  for (int b = 0; b < BP; ++b)
    acc[b] = dot2<BF>(v, (uint32_t)ld<uint16_t>(x0 + 2 * b), acc[b]);
}

// The BP batch values of one x slot, as loaded from LDS.
template <int BP> struct XSlot { using T = u32x4_t; };
template <> struct XSlot<1> { using T = uint16_t; };
template <> struct XSlot<2> { using T = uint32_t; };
template <> struct XSlot<4> { using T = u32x2_t; };

// Kept pair w (packed 16-bit values) against the x slots p, q of its two
// columns, already in registers.
template <bool BF, int BP>
__device__ __forceinline__ void pair_fma(typename XSlot<BP>::T p, typename XSlot<BP>::T q,
                                         uint32_t w, float (&acc)[BP]) {
  if constexpr (BP == 1) {
    acc[0] = dot2<BF>(w, (uint32_t)p | ((uint32_t)q << 16), acc[0]);
  } else if constexpr (BP == 2) {
    acc[0] = dot2<BF>(w, (p & 0xffffu) | (q << 16), acc[0]);
    acc[1] = dot2<BF>(w, (p >> 16) | (q & 0xffff0000u), acc[1]);
  } else {
#pragma unroll
    for (int d = 0; d < BP / 2; ++d) {
      acc[2 * d] = dot2<BF>(w, (p[d] & 0xffffu) | (q[d] << 16), acc[2 * d]);
      acc[2 * d + 1] = dot2<BF>(w, (p[d] >> 16) | (q[d] & 0xffff0000u), acc[2 * d + 1]);
    }
  }
}

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round
// trips): row shifts by 1, 2, 4, 8 within each row of 16 lanes, then lane 15
// of each row into the next and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Wave w of the grid owns rows w * rpw .. + rpw - 1.  Its work per segment of
// x is a sequence of items (row i, window t), copied into a ring of NB
// buffers per wave: the copies of items k + 1 .. k + NB - 1 are in flight
// while item k is consumed (with NB > 2 the item's mask words are copied into
// its buffer too, else they are loaded into registers).  Lane i accumulates
// the sums of the wave's row i across segments (rpw <= 64).
// UN: unstructured bitmask (any keep mask).  A word's count varies, so offs
// holds the value index of every 64-word window of every row (row r, window
// t at offs[r * nwr + t], nwr = windows per row, offs[R * nwr] = all kept
// values); lane l of a window finds its values at the window's start plus
// the set bits of the window's words before it (a wave prefix sum), and
// walks popc(word) steps.  seg is then a multiple of 64 words.  A window
// whose values do not fit a buffer (more than NI KiB with the copy's 16-byte
// alignment) has its values read by the lanes from global memory.
template <bool BF, int BP, int NI, bool UN = false, int NB = 2>
__global__ __launch_bounds__(1024) void nm_spmv_fixed_kernel(
    const uint16_t *__restrict__ values, const uint32_t *__restrict__ bits,
    const uint16_t *__restrict__ x, void *__restrict__ y, int B, int64_t R, int K, int P,
    int seg, int rpw, int out_kind, const int64_t *__restrict__ offs = nullptr) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wpg = blockDim.x / kWave;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t r0 = ((int64_t)blockIdx.x * wpg + wid) * rpw;
  const int64_t left = R - r0;
  const int nrows = left <= 0 ? 0 : (left < rpw ? (int)left : rpw);
  const int W = K >> 5;                   // mask words per row
  const int64_t vstride = (int64_t)W * P;  // values per row (N:M)
  const int nwr = (W + kWinWords - 1) / kWinWords;  // windows per row (UN)
  const uint32_t xbytes = ((uint32_t)XCols<BP>::bytes(seg) + 15u) & ~15u;
  // LDS address of the wave's NB window buffers (NI KiB each, and past
  // two buffers 256 bytes for the item's mask words)
  constexpr uint32_t kSlot = NI * 1024 + (NB > 2 ? 256 : 0);
  const uint32_t wbuf = (uint32_t)(size_t)(lds_ptr)lds + xbytes + (uint32_t)wid * (NB * kSlot);

  float res[BP];
#pragma unroll
  for (int b = 0; b < BP; ++b) res[b] = 0.f;

  for (int s0 = 0; s0 < K; s0 += seg) {
    const int S = K - s0 < seg ? K - s0 : seg;
    __syncthreads();  // every wave is done with the previous segment's x
    stage_x_cols<BP>(lds, x, B, K, s0, S);
    if constexpr (UN) {  // the pad after each word's slots reads as x = 0
      for (int w = threadIdx.x; w < (S >> 5); w += blockDim.x) {
        uint32_t *pad = reinterpret_cast<uint32_t *>(lds + w * XCols<BP>::WS + 32 * XCols<BP>::SB);
#pragma unroll
        for (int q = 0; q < XCols<BP>::PB / 4; ++q) pad[q] = 0u;
      }
    }
    __syncthreads();
    const int sw0 = s0 >> 5, sw = S >> 5;
    const int nwin = (sw + kWinWords - 1) / kWinWords;
    const int nitems = nrows * nwin;

    // Issue item k (a dummy past the last item: empty ranges, no memory
    // traffic, so the wait counts below stay the same for every item).
    auto issue = [&](int k, uint32_t &mword) {
      const bool real = k < nitems;
      const int i = real ? k / nwin : 0, t = real ? k - i * nwin : 0;
      const int64_t r = r0 + i;
      const int w0 = sw0 + t * kWinWords;
      const int nw = real ? min(kWinWords, sw - t * kWinWords) : 0;
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(bits + r * W + w0), 0, nw * 4, kRsrcWord3);
      const uint32_t dst = wbuf + (uint32_t)(k % NB) * kSlot;
      if constexpr (NB > 2)
        lds_load4_nt(rb, dst + NI * 1024, lane * 4, 0);
      else
        mword = __builtin_amdgcn_raw_buffer_load_b32(rb, lane * 4, 0, kStreamAux);
      int64_t vs, cnt;
      if constexpr (UN) {
        // a dummy item reads entry 0 (always present) and uses none of it
        const int64_t wi = real ? r * nwr + (w0 / kWinWords) : 0;
        const int64_t a = offs[wi], b = offs[wi + (real ? 1 : 0)];
        vs = real ? a : 0;
        cnt = real ? b - a : 0;
      } else {
        vs = r * vstride + (int64_t)w0 * P;
        cnt = (int64_t)nw * P;
      }
      const int64_t a0 = vs & ~(int64_t)7;
      const int nch = real ? (int)((vs + cnt - a0 + 7) >> 3) : 0;
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(values + a0), 0, nch * 16, kRsrcWord3);
#pragma unroll
      for (int j = 0; j < NI; ++j) lds_load16_nt(rv, dst + j * 1024, lane * 16 + j * 1024, 0);
    };

    float acc[BP];
#pragma unroll
    for (int b = 0; b < BP; ++b) acc[b] = 0.f;
    uint32_t mA = 0, mB = 0;
    issue(0, mA);
    issue(1, mB);
#pragma unroll
    for (int j = 2; j < NB; ++j) issue(j, mA);
    for (int k = 0; k < nitems; ++k) {
      // item k's mask words and window copy have landed (the 1 + NI loads
      // of each of the next NB - 1 items may still be in flight)
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<(NB - 1) * (1 + NI)>();
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t slot = wbuf + (uint32_t)(k % NB) * kSlot;
      uint32_t mw;
      if constexpr (NB > 2)
        mw = ld<uint32_t>((lds_ptr)(size_t)(slot + NI * 1024 + 4 * lane));
      else
        mw = (k & 1) ? mB : mA;
      const int i = k / nwin, t = k - i * nwin;
      const int64_t r = r0 + i;
      const int w0 = sw0 + t * kWinWords;
      const int nw = min(kWinWords, sw - t * kWinWords);
      // the lane's count and the offset of its values in the window
      int pl = P, ol = lane * P;
      int64_t vs, vcnt = 0;
      if constexpr (UN) {
        pl = __popc(mw);  // words past the row read 0
        ol = wave_incl_scan(pl) - pl;
        vs = offs[r * nwr + (w0 / kWinWords)];
        vcnt = offs[r * nwr + (w0 / kWinWords) + 1] - vs;
      } else {
        vs = r * vstride + (int64_t)w0 * P;
      }
      if (lane < nw) {
        // (UN: a lane's offset is clamped so that its reads stay inside the
        // buffer also where the words disagree with offs; a consistent
        // window copied whole never reaches the clamp)
        const int olb = UN ? min(ol, (int)(kSlot / 2) - 7 - 32) : ol;
        const uint32_t vb = slot + 2u * (uint32_t)((vs & 7) + (int64_t)olb);
        // byte offset of the word's x slots in the segment's image
        const int cb = (t * kWinWords + lane) * XCols<BP>::WS;
        uint32_t m = mw;
        if constexpr (UN) {
          // The counts differ between lanes, so the step loop runs a
          // wave-uniform number of 8-step groups (from ballots) with no
          // branch per step: a step past the lane's count finds no set bit
          // and takes the word's zeroed pad slot as its x (column 32), and
          // its value is zeroed, so it adds an exact 0.  Per-lane loop bounds
          // and a branch per pair left the kernel bound by instruction issue.
          const int ng = (__ballot(pl > 0) != 0) + (__ballot(pl > 8) != 0) +
                         (__ballot(pl > 16) != 0) + (__ballot(pl > 24) != 0);
          auto groups = [&](auto value) {
            for (int g = 0; g < ng; ++g) {
              const int j0 = 8 * g;
              int c[8];
              uint32_t v[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t f = (uint32_t)ffbl_hw(m);  // 0xffffffff once m == 0
                c[e] = cb + (int)(f < 32u ? f : 32u) * XCols<BP>::SB;
                m &= m - 1;
              }
              // the group's x slots and values are all requested before any
              // is used (the empty asm keeps every value load unconditional)
              typename XSlot<BP>::T xs[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) xs[e] = ld<typename XSlot<BP>::T>((lds_ptr)lds + c[e]);
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] = value(j0 + e);
#pragma unroll
              for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(v[e]));
#pragma unroll
              for (int e = 0; e < 8; e += 2) {
                const int left = pl - j0 - e;
                const uint32_t w = (left >= 1 ? v[e] : 0u) | (left >= 2 ? v[e + 1] << 16 : 0u);
                pair_fma<BF, BP>(xs[e], xs[e + 1], w, acc);
              }
            }
          };
          if ((vs & 7) + vcnt <= NI * 512) {  // the whole window is in the buffer
            groups([&](int j) -> uint32_t { return ld<uint16_t>((lds_ptr)(size_t)(vb + 2 * j)); });
          } else {
            // a window denser than the buffer holds (the copy stopped at its
            // end): the lane reads its values from global memory instead
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(values + vs), 0, (int)(2 * vcnt), kRsrcWord3);
            groups([&](int j) -> uint32_t {
              return __builtin_amdgcn_raw_buffer_load_b16(rw, 2 * (ol + j), 0, 0);
            });
          }
        } else
        // eight scan steps at a time: the columns first (a short VALU chain),
        // then every LDS read of the group, then the products.  Steps past P
        // read slots inside the buffer (see win_loads) and are dropped.
        for (int j0 = 0; j0 < pl; j0 += 8) {
          int c[8];
          uint32_t v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            c[e] = cb + (ffbl_hw(m) & 31) * XCols<BP>::SB;
            m &= m - 1;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = ld<uint16_t>((lds_ptr)(size_t)(vb + 2 * (j0 + e)));
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int left = pl - j0 - e;  // steps of this pair still inside the count
            if (left >= 2)
              pair_acc<BF, BP>(lds, c[e], c[e + 1], v[e] | (v[e + 1] << 16), acc);
            else if (left == 1)
              single_acc<BF, BP>(lds, c[e], v[e], acc);
          }
        }
      }
      if (t == nwin - 1) {  // the row's part of this segment is complete
#pragma unroll
        for (int b = 0; b < BP; ++b) {
          const float sv = wave_total(acc[b]);
          res[b] += lane == i ? sv : 0.f;
          acc[b] = 0.f;
        }
      }
      // the buffer of item k is read out before item k + 2 overwrites it
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkmcnt0();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NB > 2)
        issue(k + NB, mA);
      else if (k & 1)
        issue(k + 2, mB);
      else
        issue(k + 2, mA);
    }
    // the dummy items' copies land before the buffers are reused
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (lane < nrows) {
#pragma unroll
    for (int b = 0; b < BP; ++b)
      if (b < B) store_out(y, (int64_t)b * R + r0 + lane, res[b], out_kind);
  }
}

// Direct kernel for the common densities (P = 4, 8, 12, 24 kept columns per
// word: 1:8, 1:4, 3:8, 3:4).  Lane l of a wave owns mask words
// t * 64 U + 64 u + l of its row's part of the x segment (u < U): the word
// and its 2P value bytes (one contiguous run per word, 8- or 16-byte aligned)
// are loaded straight into registers with raw buffer loads (range-checked at
// the segment end), two load batches in flight per wave, and the word is
// walked in P unrolled steps, each kept pair meeting its x values from LDS in
// one dot2.  When all of x does not fit the LDS budget, K is walked in
// segments of seg columns; lane i carries the sums of the wave's row i across
// segments.
template <int P>
struct WordVals {
  static constexpr int kBytes = 2 * P;                  // value bytes per word
  static constexpr int kWidth = kBytes % 16 == 0 ? 16 : 8;  // bytes per load
  static constexpr int kLoads = kBytes / kWidth;
  static constexpr int kRegs = kBytes / 4;
};

template <int P, int U>
struct WordBatch {
  uint32_t m[U];
  uint32_t v[U][WordVals<P>::kRegs];
};

template <int P, int U>
__device__ __forceinline__ void word_batch_load(WordBatch<P, U> &bt, const uint16_t *vrow,
                                                const uint32_t *brow, int nw, int t, int lane) {
  using V = WordVals<P>;
  // resources from the batch's first word to the row end: the range check
  // (vector offsets) zeroes the words past the row
  const int w0 = t * kWave * U, left = nw - w0 > 0 ? nw - w0 : 0;
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void *)(brow + w0), 0, left * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(vrow + (int64_t)w0 * P), 0, left * V::kBytes, kRsrcWord3);
#pragma unroll
  for (int u = 0; u < U; ++u)
    bt.m[u] = __builtin_amdgcn_raw_buffer_load_b32(rb, (lane + kWave * u) * 4, 0, kStreamAux);
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int l = 0; l < V::kLoads; ++l) {
      const int off = (lane + kWave * u) * V::kBytes + l * V::kWidth;
      if constexpr (V::kWidth == 16) {
        const u32x4_t q = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kStreamAux));
#pragma unroll
        for (int e = 0; e < 4; ++e) bt.v[u][4 * l + e] = q[e];
      } else {
        const u32x2_t q = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, kStreamAux));
        bt.v[u][2 * l] = q[0];
        bt.v[u][2 * l + 1] = q[1];
      }
    }
  }
}

// The P kept weights of one word (mask m, values v) against the word's x
// slots at byte offset xw of the XCols image.  CH independent scans: with
// M <= 8 every byte of a valid word holds P / 4 kept columns (CH = 4), with
// M = 16 every half-word P / 2 (CH = 2); value j of chain h is value
// h * P / CH + j of the word (column order).  The chains are independent, so
// their steps overlap instead of forming one P-step dependence chain.  A
// malformed word only makes its row's sum undefined: every column stays in
// its chain's span.
template <bool BF, int BP, int P, int CH>
__device__ __forceinline__ void word_acc(const char *lds, int xw, uint32_t m,
                                         const uint32_t (&v)[WordVals<P>::kRegs],
                                         float (&acc)[BP]) {
  constexpr int Q = P / CH, SPAN = 32 / CH;
  static_assert(Q * CH == P, "chains split the word's kept columns evenly");
  int c[P];
#pragma unroll
  for (int h = 0; h < CH; ++h) {
    uint32_t mh = CH == 1 ? m : (m >> (SPAN * h)) & ((1u << (SPAN & 31)) - 1u);
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      c[h * Q + j] = xw + (SPAN * h + (ffbl_hw(mh) & (SPAN - 1))) * XCols<BP>::SB;
      mh &= mh - 1;
    }
  }
#pragma unroll
  for (int j = 0; j < P; j += 2) pair_acc<BF, BP>(lds, c[j], c[j + 1], v[j / 2], acc);
}

// SEGS: x in several segments (a build of its own, so that the one-segment
// case keeps the straight-line code of a single pass).
template <bool BF, int BP, int P, int U, int CH, bool SEGS>
__global__ __launch_bounds__(1024) void nm_spmv_fixedp_kernel(
    const uint16_t *__restrict__ values, const uint32_t *__restrict__ bits,
    const uint16_t *__restrict__ x, void *__restrict__ y, int B, int64_t R, int K, int rpw,
    int out_kind, int seg) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wpg = blockDim.x / kWave;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t r0 = ((int64_t)blockIdx.x * wpg + wid) * rpw;
  const int64_t left = R - r0;
  const int nrows = left <= 0 ? 0 : (left < rpw ? (int)left : rpw);
  const int W = K >> 5;

  float res[BP];
#pragma unroll
  for (int b = 0; b < BP; ++b) res[b] = 0.f;

  auto segment = [&](const int s0, const int S) {
    if (s0 > 0) __syncthreads();  // every wave is done with the previous segment's x
    stage_x_cols<BP>(lds, x, B, K, s0, S);
    __syncthreads();
    const int sw0 = s0 >> 5, sw = S >> 5;  // the segment's first word and its words
    const int nb = (sw + kWave * U - 1) / (kWave * U);  // load batches per row and segment
    const int nitems = nrows * nb;

    auto item_load = [&](WordBatch<P, U> &bt, int k) {
      const bool real = k < nitems;
      const int i = real ? k / nb : 0, t = real ? k - i * nb : 0;
      const int64_t r = real ? r0 + i : 0;
      word_batch_load<P, U>(bt, values + (r * W + sw0) * P, bits + r * W + sw0, real ? sw : 0, t,
                            lane);
    };
    auto consume = [&](const WordBatch<P, U> &bt, int t, float (&acc)[BP]) {
      const int wb = t * kWave * U;  // the batch's first word in the segment (wave-uniform)
      if (wb + kWave * U <= sw) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          word_acc<BF, BP, P, CH>(lds, (wb + kWave * u + lane) * XCols<BP>::WS, bt.m[u], bt.v[u], acc);
        return;
      }
      // the segment's last batch: words past its end read zeros and are dropped
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (wb + kWave * u >= sw) break;
        const int w = wb + kWave * u + lane;
        float part[BP];
#pragma unroll
        for (int b = 0; b < BP; ++b) part[b] = 0.f;
        word_acc<BF, BP, P, CH>(lds, min(w, sw - 1) * XCols<BP>::WS, bt.m[u], bt.v[u], part);
#pragma unroll
        for (int b = 0; b < BP; ++b) acc[b] += w < sw ? part[b] : 0.f;
      }
    };

    float acc[BP];
#pragma unroll
    for (int b = 0; b < BP; ++b) acc[b] = 0.f;
    WordBatch<P, U> A, Bt;
    item_load(A, 0);
    item_load(Bt, 1);
    for (int k = 0; k < nitems; k += 2) {
      {
        const int i = k / nb, t = k - i * nb;
        consume(A, t, acc);
        if (t == nb - 1) {
#pragma unroll
          for (int b = 0; b < BP; ++b) {
            // the lane-63 read is taken by every lane: inside a select on the
            // lane it would let the reduction's last step run for lane i only
            const float sv = wave_total(acc[b]);
            res[b] += lane == i ? sv : 0.f;
            acc[b] = 0.f;
          }
        }
      }
      item_load(A, k + 2);
      if (k + 1 >= nitems) break;
      {
        const int i = (k + 1) / nb, t = (k + 1) - i * nb;
        consume(Bt, t, acc);
        if (t == nb - 1) {
#pragma unroll
          for (int b = 0; b < BP; ++b) {
            // the lane-63 read is taken by every lane: inside a select on the
            // lane it would let the reduction's last step run for lane i only
            const float sv = wave_total(acc[b]);
            res[b] += lane == i ? sv : 0.f;
            acc[b] = 0.f;
          }
        }
      }
      item_load(Bt, k + 3);
    }
  };
  if constexpr (SEGS) {
    for (int s0 = 0; s0 < K; s0 += seg) segment(s0, K - s0 < seg ? K - s0 : seg);
  } else {
    segment(0, K);
  }
  if (lane < nrows) {
#pragma unroll
    for (int b = 0; b < BP; ++b)
      if (b < B) store_out(y, (int64_t)b * R + r0 + lane, res[b], out_kind);
  }
}

using fixedp_fn = void (*)(const uint16_t *, const uint32_t *, const uint16_t *, void *, int,
                           int64_t, int, int, int, int);

// The densities with a direct kernel, and its words per lane per load batch:
// two for P = 4, 8, 12 (a batch of 128 words is one row of K = 4096; four
// words per lane left half of each batch idle there and measured 2-8% slower
// for P = 4 and 8 on the 8B gate and down shapes, eight 6-19% slower, one
// 3-36% slower), one for P = 24, whose word already carries 48 value bytes
// (up to 8% faster than two, equal on gate at batch 1).
__host__ __device__ constexpr bool direct_p(int p) { return p == 4 || p == 8 || p == 12 || p == 24; }

template <bool BF, int BP, int CH, bool SEGS>
fixedp_fn pick_fixedp_p(int p) {
  switch (p) {
    case 4: return nm_spmv_fixedp_kernel<BF, BP, 4, 2, CH, SEGS>;
    case 8: return nm_spmv_fixedp_kernel<BF, BP, 8, 2, CH, SEGS>;
    case 12: return nm_spmv_fixedp_kernel<BF, BP, 12, 2, CH, SEGS>;
    default: return nm_spmv_fixedp_kernel<BF, BP, 24, 1, CH, SEGS>;
  }
}

// ch: independent scan chains per word (4 for M <= 8, 2 for M = 16, 1 for
// M = 32)
template <bool BF, int BP, bool SEGS>
fixedp_fn pick_fixedp_ch(int p, int ch) {
  return ch == 4 ? pick_fixedp_p<BF, BP, 4, SEGS>(p)
                 : ch == 2 ? pick_fixedp_p<BF, BP, 2, SEGS>(p) : pick_fixedp_p<BF, BP, 1, SEGS>(p);
}

template <bool BF, bool SEGS>
fixedp_fn pick_fixedp_bp(int bp, int p, int ch) {
  switch (bp) {
    case 1: return pick_fixedp_ch<BF, 1, SEGS>(p, ch);
    case 2: return pick_fixedp_ch<BF, 2, SEGS>(p, ch);
    case 4: return pick_fixedp_ch<BF, 4, SEGS>(p, ch);
    default: return pick_fixedp_ch<BF, 8, SEGS>(p, ch);
  }
}

template <bool BF>
fixedp_fn pick_fixedp(int bp, int p, int ch, bool segs) {
  return segs ? pick_fixedp_bp<BF, true>(bp, p, ch) : pick_fixedp_bp<BF, false>(bp, p, ch);
}

size_t xcols_bytes(int bp, int64_t cols) {
  switch (bp) {
    case 1: return XCols<1>::bytes((int)cols);
    case 2: return XCols<2>::bytes((int)cols);
    case 4: return XCols<4>::bytes((int)cols);
    default: return XCols<8>::bytes((int)cols);
  }
}

size_t fixedp_lds_bytes(int bp, int64_t cols) { return xcols_bytes(bp, cols); }

// ---- unstructured bitmasks: window offsets and pack ------------------------

// Kept entries of window t of row r (64 words = 2048 columns), one wave per
// window: cnt[r * nwr + t].
__global__ __launch_bounds__(256) void nm_bitmask_count_kernel(const uint8_t *__restrict__ keep,
                                                               int64_t R, int K,
                                                               int64_t *__restrict__ cnt) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nwr = (K / 32 + kWinWords - 1) / kWinWords;
  const int64_t nwave = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t q = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; q < R * nwr;
       q += nwave) {
    const int64_t r = q / nwr;
    const int c0 = (int)(q - r * nwr) * kWinWords * 32;
    const int c1 = min(c0 + kWinWords * 32, K);
    int n = 0;
    for (int c = c0 + lane; c < c1; c += kWave) n += keep[r * K + c] != 0;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) n += __shfl_xor(n, o, kWave);
    if (lane == 0) cnt[q] = n;
  }
}

// offs[0] = 0, offs[i + 1] = offs[i] + cnt[i] for i < n: one workgroup of
// 1024 threads, each scanning a contiguous block; cnt may alias offs + 1.
__global__ __launch_bounds__(1024) void nm_bitmask_scan_kernel(int64_t *__restrict__ offs,
                                                               int64_t n) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t b0 = t * per < n ? t * per : n, b1 = b0 + per < n ? b0 + per : n;
  int64_t sum = 0;
  for (int64_t i = b0; i < b1; ++i) sum += offs[i + 1];
  part[t] = sum;
  __syncthreads();
  if (t == 0) {
    int64_t run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int64_t v = part[i];
      part[i] = run;
      run += v;
    }
    offs[0] = 0;
  }
  __syncthreads();
  int64_t run = part[t];
  for (int64_t i = b0; i < b1; ++i) {
    run += offs[i + 1];
    offs[i + 1] = run;
  }
}

// Pack one window per wave: bit b of word w <-> column 32 w + b, kept values
// in column order from offs[window].  A window whose kept count does not
// match its offsets bumps *bad (the write stays inside the window's range).
__global__ __launch_bounds__(256) void nm_pack_bitmask_kernel(
    const uint16_t *__restrict__ W, const uint8_t *__restrict__ keep, int64_t R, int K,
    const int64_t *__restrict__ offs, uint16_t *__restrict__ values, uint32_t *__restrict__ bits,
    int *__restrict__ bad) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nwr = (K / 32 + kWinWords - 1) / kWinWords;
  const int64_t nwave = (int64_t)gridDim.x * (blockDim.x / kWave);
  const uint64_t below = lane ? (~0ull >> (kWave - lane)) : 0ull;
  int nbad = 0;
  for (int64_t q = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; q < R * nwr;
       q += nwave) {
    const int64_t r = q / nwr;
    const int c0 = (int)(q - r * nwr) * kWinWords * 32;
    const int c1 = min(c0 + kWinWords * 32, K);
    const int64_t vs = offs[q], cnt = offs[q + 1] - vs;
    int64_t run = 0;
    for (int c = c0; c < c1; c += kWave) {  // K % 32 == 0: whole words
      const int col = c + lane;
      const bool in = col < c1;
      const bool kept = in && keep[r * K + col] != 0;
      const uint64_t bal = __ballot(kept);
      const int64_t j = run + __popcll(bal & below);
      if (kept && j < cnt) values[vs + j] = W[r * K + col];
      if (in && (lane & 31) == 0)
        bits[r * (K / 32) + col / 32] = (uint32_t)(bal >> (lane & 32));
      run += __popcll(bal);
    }
    nbad += run != cnt ? 1 : 0;
  }
  if (lane == 0 && nbad) atomicAdd(bad, nbad);
}

using fixed_fn = void (*)(const uint16_t *, const uint32_t *, const uint16_t *, void *, int,
                          int64_t, int, int, int, int, int, const int64_t *);

template <bool BF, int BP>
fixed_fn pick_fixed_ni(int ni) {
  switch (ni) {
    case 1: return nm_spmv_fixed_kernel<BF, BP, 1>;
    case 2: return nm_spmv_fixed_kernel<BF, BP, 2>;
    case 3: return nm_spmv_fixed_kernel<BF, BP, 3>;
    default: return nm_spmv_fixed_kernel<BF, BP, 4>;
  }
}

template <bool BF>
fixed_fn pick_fixed_bp(int bp, int ni) {
  switch (bp) {
    case 1: return pick_fixed_ni<BF, 1>(ni);
    case 2: return pick_fixed_ni<BF, 2>(ni);
    case 4: return pick_fixed_ni<BF, 4>(ni);
    default: return pick_fixed_ni<BF, 8>(ni);
  }
}

int pad_b(int b) { return b <= 1 ? 1 : b <= 2 ? 2 : b <= 4 ? 4 : 8; }

size_t xcols_bytes(int bp, int64_t cols);

size_t fixed_lds_bytes(int bp, int seg, int waves, int ni, int nb = 2) {
  const size_t slot = (size_t)ni * 1024 + (nb > 2 ? 256 : 0);
  return ((xcols_bytes(bp, seg) + 15) & ~(size_t)15) + (size_t)waves * nb * slot;
}


}  // namespace

namespace nm_host {

bool pattern_any_ok(int n, int m) {
  return (m == 4 || m == 8 || m == 16 || m == 32) && n >= 1 && n < m;
}

nm_status generic_default_cfg(int64_t rows, int64_t cols, int batch, int n, int m, int cus,
                              size_t lds_budget, nm_launch_cfg *cfg) {
  const int p = 32 * n / m, ni = win_loads(p), bp = pad_b(batch);
  cfg->kernel = NM_KERNEL_VALU;
  cfg->k_split = 1;
  if (direct_p(p)) {
    // x in as few equal segments as fit the budget.  Workgroups of 4 waves,
    // about two per CU, unless only one x image fits a CU's LDS or there are
    // at most 16 rows per CU: then 16 waves, one row each, so that a CU still
    // holds 16 waves (measured: 2.0-2.4x faster at K = 14336, batch 4-8).
    const int64_t w = cols / 32;
    const int64_t maxw = (int64_t)((lds_budget - 16) / xcols_bytes(bp, 32));
    const int64_t nseg = w <= maxw ? 1 : (w + maxw - 1) / maxw;
    const int64_t segw = (w + nseg - 1) / nseg;
    cfg->seg_cols = segw > 0 ? (int)(segw * 32) : 32;
    const size_t xb = fixedp_lds_bytes(bp, cfg->seg_cols);
    const size_t per_cu = xb > 0 ? kLdsCap / xb : 16;
    const int waves = (per_cu < 2 || rows <= (int64_t)16 * cus) ? 16 : 4;
    cfg->threads_per_wg = waves * kWave;
    int64_t rpw = rows / ((int64_t)2 * cus * waves);
    cfg->rows_per_wave = (int)(rpw < 1 ? 1 : rpw > 8 ? 8 : rpw);
    return NM_OK;
  }
  const int waves = 4;
  cfg->threads_per_wg = waves * kWave;
  // about two workgroups per CU, at most 8 rows per wave
  int64_t rpw = rows / ((int64_t)2 * cus * waves);
  cfg->rows_per_wave = (int)(rpw < 1 ? 1 : rpw > 8 ? 8 : rpw);
  const size_t wave_area = fixed_lds_bytes(bp, 0, waves, ni);
  if (fixed_lds_bytes(bp, (int)cols, waves, ni) <= lds_budget) {
    cfg->seg_cols = cols > 0 ? (int)cols : 32;
  } else {
    // widest multiple of 2048 columns (whole windows) that fits
    const size_t ws = xcols_bytes(bp, 32);  // bytes per 32-column word
    const int64_t s = (int64_t)((lds_budget - wave_area - 16) / ws) * 32 / 2048 * 2048;
    cfg->seg_cols = (int)(s < 2048 ? 2048 : s);
  }
  return NM_OK;
}

nm_status generic_check_cfg(const nm_launch_cfg &c, int batch, int n, int m,
                            size_t lds_budget) {
  const int t = c.threads_per_wg;
  if (c.kernel != NM_KERNEL_VALU) return NM_ERR_UNSUPPORTED;
  if (t < kWave || t > 1024 || t % kWave != 0) return NM_ERR_INVALID_ARG;
  if (c.rows_per_wave < 1 || c.rows_per_wave > kWave) return NM_ERR_INVALID_ARG;
  if (c.seg_cols <= 0 || c.seg_cols % 32 != 0) return NM_ERR_INVALID_ARG;
  const int p = 32 * n / m;
  const size_t need = direct_p(p) ? fixedp_lds_bytes(pad_b(batch), c.seg_cols)
                                  : fixed_lds_bytes(pad_b(batch), c.seg_cols, t / kWave, win_loads(p));
  if (need > lds_budget) return NM_ERR_INVALID_ARG;
  return NM_OK;
}

nm_status bitmask_offsets(const uint8_t *keep, int64_t rows, int64_t cols, int64_t *offs,
                          int64_t *total, void *stream) {
  const int nwr = (int)((cols / 32 + kWinWords - 1) / kWinWords);
  const int64_t n = rows * nwr;
  hipStream_t s = (hipStream_t)stream;
  if (n > 0) {
    int64_t grid = (n + 3) / 4;
    if (grid > (1 << 20)) grid = 1 << 20;
    hipLaunchKernelGGL(nm_bitmask_count_kernel, dim3((unsigned)grid), dim3(256), 0, s, keep, rows,
                       (int)cols, offs + 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  hipLaunchKernelGGL(nm_bitmask_scan_kernel, dim3(1), dim3(1024), 0, s, offs, n);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(total, offs + n, sizeof(int64_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

nm_status bitmask_pack(const uint16_t *W, const uint8_t *keep, int64_t rows, int64_t cols,
                       const int64_t *offs, uint16_t *values, uint32_t *bits, void *stream) {
  const int nwr = (int)((cols / 32 + kWinWords - 1) / kWinWords);
  const int64_t n = rows * nwr;
  hipStream_t s = (hipStream_t)stream;
  int *dbad = nullptr;
  hipError_t e = hipMalloc((void **)&dbad, sizeof(int));
  if (e != hipSuccess) return hip_fail(e);
  int hbad = 0;
  e = hipMemsetAsync(dbad, 0, sizeof(int), s);
  if (e == hipSuccess) {
    int64_t grid = (n + 3) / 4;
    if (grid > (1 << 20)) grid = 1 << 20;
    hipLaunchKernelGGL(nm_pack_bitmask_kernel, dim3((unsigned)grid), dim3(256), 0, s, W, keep,
                       rows, (int)cols, offs, values, bits, dbad);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipMemcpyAsync(&hbad, dbad, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  const hipError_t ef = hipFree(dbad);
  if (e != hipSuccess) return hip_fail(e);
  if (ef != hipSuccess) return hip_fail(ef);
  return hbad ? NM_ERR_MASK : NM_OK;
}

nm_status bitmask_launch(const void *values, const uint32_t *bits, const int64_t *offs,
                         const void *X, void *Y, int batch, int64_t rows, int64_t cols,
                         nm_dtype in_dt, nm_dtype out_dt, int cus, size_t lds_budget,
                         void *stream) {
  // Three window buffers per wave of 3 KiB each: a window of up to 1528
  // values (75% of its 2048 columns) is copied whole, a denser one is read
  // from global memory by the lanes (the buffers sized for a full window,
  // 5 KiB, leave room for two per wave and fewer workgroups per CU: gate
  // 14336x4096 at batch 1 29.0 -> 26.8 us, down 4096x14336 31.7 -> 28.3)
  constexpr int kNI = 3;
  constexpr int kNB = 3;
  const int bp = pad_b(batch);
  // x whole, or in segments of whole windows, next to the waves' buffers
  auto seg_for = [&](int waves) -> int64_t {
    if (fixed_lds_bytes(bp, (int)cols, waves, kNI, kNB) <= lds_budget) return cols;
    const size_t wave_area = fixed_lds_bytes(bp, 0, waves, kNI, kNB);
    if (wave_area + 16 + xcols_bytes(bp, 2048) > lds_budget) return 0;
    return (int64_t)((lds_budget - wave_area - 16) / xcols_bytes(bp, 32)) * 32 / 2048 * 2048;
  };
  // 4-wave workgroups: about three per CU where three fit its LDS (batch 1:
  // gate 14336x4096 31.4 -> 29.1 us), else about two (a three-per-CU grid
  // then runs in one and a half rounds: 1.2x slower at batch 2-4); where only
  // one of them fits (batch 4-8 here), 8-wave workgroups, one per CU, every
  // row in one round (measured 1.2-1.4x faster there, slower at batch 1)
  int waves = 4;
  int64_t seg = seg_for(4), rpw;
  const size_t wg4 = seg > 0 ? fixed_lds_bytes(bp, (int)seg, 4, kNI, kNB) : 0;
  if (seg > 0 && 2 * wg4 > kLdsCap && seg_for(8) > 0) {
    waves = 8;
    seg = seg_for(8);
    rpw = (rows + (int64_t)cus * waves - 1) / ((int64_t)cus * waves);
  } else if (seg > 0 && 3 * wg4 <= kLdsCap) {
    rpw = (rows + (int64_t)3 * cus * waves - 1) / ((int64_t)3 * cus * waves);
  } else {
    rpw = rows / ((int64_t)2 * cus * waves);
  }
  if (seg <= 0) return NM_ERR_UNSUPPORTED;
  rpw = rpw < 1 ? 1 : rpw > 8 ? 8 : rpw;
  const int64_t grid = (rows + waves * rpw - 1) / (waves * rpw);
  if (grid > INT32_MAX) return NM_ERR_INVALID_ARG;
  using un_fn = void (*)(const uint16_t *, const uint32_t *, const uint16_t *, void *, int, int64_t,
                         int, int, int, int, int, const int64_t *);
  un_fn fn;
  const bool bf = in_dt == NM_BF16;
  switch (bp) {
    case 1: fn = bf ? nm_spmv_fixed_kernel<true, 1, kNI, true, kNB> : nm_spmv_fixed_kernel<false, 1, kNI, true, kNB>; break;
    case 2: fn = bf ? nm_spmv_fixed_kernel<true, 2, kNI, true, kNB> : nm_spmv_fixed_kernel<false, 2, kNI, true, kNB>; break;
    case 4: fn = bf ? nm_spmv_fixed_kernel<true, 4, kNI, true, kNB> : nm_spmv_fixed_kernel<false, 4, kNI, true, kNB>; break;
    default: fn = bf ? nm_spmv_fixed_kernel<true, 8, kNI, true, kNB> : nm_spmv_fixed_kernel<false, 8, kNI, true, kNB>; break;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(waves * kWave),
                     fixed_lds_bytes(bp, (int)seg, waves, kNI, kNB), (hipStream_t)stream,
                     (const uint16_t *)values, bits, (const uint16_t *)X, Y, batch, rows, (int)cols,
                     0, (int)seg, (int)rpw, (int)out_dt, offs);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

nm_status generic_launch(const void *values, const uint32_t *bits, const void *X, void *Y,
                         int batch, int64_t rows, int64_t cols, int n, int m, nm_dtype in_dt,
                         nm_dtype out_dt, const nm_launch_cfg &cfg, void *stream) {
  const int p = 32 * n / m, ni = win_loads(p), bp = pad_b(batch);
  const int waves = cfg.threads_per_wg / kWave;
  const int64_t rows_per_wg = (int64_t)waves * cfg.rows_per_wave;
  const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
  if (grid > INT32_MAX) return NM_ERR_INVALID_ARG;
  const int seg = cfg.seg_cols < cols ? cfg.seg_cols : (int)cols;
  if (direct_p(p) && cols > 0) {
    // x in segments of seg columns (checked against the budget)
    const int ch = m <= 8 ? 4 : m == 16 ? 2 : 1;
    const bool segs = seg < cols;
    const fixedp_fn fn = in_dt == NM_BF16 ? pick_fixedp<true>(bp, p, ch, segs)
                                          : pick_fixedp<false>(bp, p, ch, segs);
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(cfg.threads_per_wg),
                       fixedp_lds_bytes(bp, seg), (hipStream_t)stream, (const uint16_t *)values,
                       bits, (const uint16_t *)X, Y, batch, rows, (int)cols, cfg.rows_per_wave,
                       (int)out_dt, seg);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? NM_OK : hip_fail(e);
  }
  const fixed_fn fn = in_dt == NM_BF16 ? pick_fixed_bp<true>(bp, ni) : pick_fixed_bp<false>(bp, ni);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(cfg.threads_per_wg),
                     fixed_lds_bytes(bp, seg, waves, ni), (hipStream_t)stream,
                     (const uint16_t *)values, bits, (const uint16_t *)X, Y, batch, rows,
                     (int)cols, p, seg, cfg.rows_per_wave, (int)out_dt, (const int64_t *)nullptr);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? NM_OK : hip_fail(e);
}

}  // namespace nm_host

namespace {

// Compute units and the LDS one workgroup may use, per device (queried once).
struct GenDev {
  int cus = 0;
  size_t lds = 0;
};
GenDev g_gen_dev[64];
std::mutex g_gen_mu;

nm_status gen_device(GenDev *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return nm_host::hip_fail(e);
  if (dev < 0 || dev >= 64) return NM_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_gen_mu);
  GenDev &d = g_gen_dev[dev];
  if (d.cus == 0) {
    int cus = 0, lds = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return nm_host::hip_fail(e);
    d.lds = (size_t)lds < kLdsCap ? (size_t)lds : kLdsCap;
    d.cus = cus;
  }
  *out = d;
  return NM_OK;
}

nm_status bitmask_dims(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0 || rows > INT32_MAX || cols > INT32_MAX) return NM_ERR_INVALID_ARG;
  if (cols % 32 != 0) return NM_ERR_SHAPE;
  const int64_t nwr = (cols / 32 + kWinWords - 1) / kWinWords;
  if (rows * nwr > ((int64_t)1 << 40)) return NM_ERR_INVALID_ARG;
  return NM_OK;
}

}  // namespace

extern "C" {

int nm_bitmask_offsets(const uint8_t *keep, int64_t rows, int64_t cols, int64_t *offs,
                       int64_t *total, void *stream) {
  nm_status st = bitmask_dims(rows, cols);
  if (st != NM_OK) return st;
  if (!offs || !total || (!keep && rows > 0 && cols > 0)) return NM_ERR_INVALID_ARG;
  if (!nm_host::aligned(offs, 8)) return NM_ERR_ALIGN;
  return nm_host::bitmask_offsets(keep, rows, cols, offs, total, stream);
}

int nm_pack_bitmask(const void *W, const uint8_t *keep, int64_t rows, int64_t cols, nm_dtype dt,
                    const int64_t *offs, void *values, uint32_t *bits, void *stream) {
  nm_status st = bitmask_dims(rows, cols);
  if (st != NM_OK) return st;
  if (!nm_host::is16(dt)) return NM_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return NM_OK;
  if (!W || !keep || !offs || !values || !bits) return NM_ERR_INVALID_ARG;
  if (!nm_host::aligned(W, 2) || !nm_host::aligned(offs, 8) || !nm_host::aligned(values, 16) ||
      !nm_host::aligned(bits, 4))
    return NM_ERR_ALIGN;
  return nm_host::bitmask_pack((const uint16_t *)W, keep, rows, cols, offs, (uint16_t *)values,
                               bits, stream);
}

int nm_spmm_bitmask(const void *values, const uint32_t *bits, const int64_t *offs, const void *X,
                    void *Y, int batch, int64_t rows, int64_t cols, nm_dtype in_dt,
                    nm_dtype out_dt, void *stream) {
  nm_status st = bitmask_dims(rows, cols);
  if (st != NM_OK) return st;
  if (batch < 1 || batch > 8) return NM_ERR_INVALID_ARG;
  if (!nm_host::is16(in_dt) || !nm_host::out_ok(in_dt, out_dt)) return NM_ERR_UNSUPPORTED;
  const bool empty_w = rows == 0 || cols == 0;
  if ((!values && !empty_w) || (!bits && !empty_w) || (!offs && !empty_w) || (!X && cols != 0) ||
      (!Y && rows != 0))
    return NM_ERR_INVALID_ARG;
  const uintptr_t ysz = out_dt == NM_F32 ? 4 : 2;
  if (!nm_host::aligned(values, 16) || !nm_host::aligned(bits, 4) || !nm_host::aligned(offs, 8) ||
      !nm_host::aligned(X, 16) || !nm_host::aligned(Y, ysz))
    return NM_ERR_ALIGN;
  if (rows == 0) return NM_OK;
  GenDev d;
  st = gen_device(&d);
  if (st != NM_OK) return st;
  return nm_host::bitmask_launch(values, bits, offs, X, Y, batch, rows, cols, in_dt, out_dt, d.cus,
                                 d.lds, stream);
}

}  // extern "C"

