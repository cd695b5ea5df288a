// nm_device.h -- device helpers shared by the library's HIP kernels
// (gfx950): vector types, the 16-bit pair dot product and the wavefront sum,
// output conversion and epilogue codes, LDS access and direct-to-LDS buffer
// loads, the matrix-core wrappers, and explicit wait counts.  Included once
// per translation unit; everything here has internal linkage.

#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "nm_sparse.h"

namespace {

constexpr int kWave = 64;
constexpr size_t kLdsCap = 160 * 1024;  // LDS one workgroup may use (CU total on gfx950)

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// acc + w.lo * x.lo + w.hi * x.hi with 16-bit pairs and an fp32 accumulator.
template <bool BF>
__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  if constexpr (BF)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, w),
                                           __builtin_bit_cast(b2_t, x), acc,
                                           false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w),
                                  __builtin_bit_cast(h2_t, x), acc, false);
}

// v + (v of the DPP-selected lane); rows outside ROW_MASK add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false);
  return v + __int_as_float(t);
}

// Sum over the 64 lanes with DPP moves only (no LDS traffic); the result is
// valid in lane 63.
__device__ __forceinline__ float wave_sum_to_63(float v) {
  v = dpp_add<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]: pairs
  v = dpp_add<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]: quads
  v = dpp_add<0x141, 0xf>(v);  // row_half_mirror: 8 lanes
  v = dpp_add<0x140, 0xf>(v);  // row_mirror: 16 lanes (a row)
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// fp32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// A 16-bit pattern (bfloat16 if BF, else binary16) widened exactly to fp32.
template <bool BF>
__device__ __forceinline__ float half_to_f32(uint16_t h) {
  if constexpr (BF)
    return __uint_as_float((uint32_t)h << 16);
  else
    return (float)__builtin_bit_cast(_Float16, h);
}

// out_kind: the output nm_dtype in bits 0..7 and the epilogue above them.
constexpr int kEpiShift = 8;
constexpr int kEpiNone = 0;
constexpr int kEpiSwiglu = 1;  // rows 2r, 2r+1 -> silu(row 2r) * row 2r+1

__device__ __forceinline__ void store_out(void *y, int64_t idx, float v,
                                          int kind) {
  kind &= 0xff;
  if (kind == NM_F32)
    static_cast<float *>(y)[idx] = v;
  else if (kind == NM_F16)
    static_cast<_Float16 *>(y)[idx] = (_Float16)v;  // v_cvt_f16_f32, RNE
  else
    static_cast<uint16_t *>(y)[idx] = f32_to_bf16_rne(v);
}

typedef __attribute__((address_space(3))) const char *lds_ptr;

// Load a T from an LDS slot given either as a generic pointer into the
// dynamic LDS array or as an explicit LDS-address-space pointer.
template <typename T, typename P>
__device__ __forceinline__ T ld(P p) {
  if constexpr (__is_same(P, lds_ptr))
    return *(__attribute__((address_space(3))) const T *)p;
  else
    return *reinterpret_cast<const T *>(p);
}

// v_ffbl_b32 / v_ffbh_u32 with their hardware meaning for 0 (-1), which the
// C builtins leave undefined: index of the lowest set bit, and the number of
// zero bits above the highest set bit.
__device__ __forceinline__ int ffbl_hw(uint32_t x) {
  int r;
  asm("v_ffbl_b32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ int ffbh_hw(uint32_t x) {
  int r;
  asm("v_ffbh_u32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Word 3 of a raw buffer resource for the gfx9 family (gfx950): untyped
// 32-bit data, no swizzle; with stride 0 the range check is per byte offset.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the weight loads: nt (non-temporal).  Every weight byte is
// read exactly once per call, and streaming it with nt measured 7-9% more
// HBM read bandwidth on gfx950 than the default policy.
constexpr int kStreamAux = 2;

// SiLU in fp32: z * sigmoid(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

typedef _Float16 h8v_t __attribute__((ext_vector_type(8)));
typedef _Float16 h16v_t __attribute__((ext_vector_type(16)));
typedef __bf16 b8v_t __attribute__((ext_vector_type(8)));
typedef __bf16 b16v_t __attribute__((ext_vector_type(16)));
typedef float f4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void *lds_vptr;

// 2-bit in-group positions of the 8 kept values of a lane's 16 columns:
// nibble g (exactly 2 set bits at p0 < p1) -> p0 | p1 << 2 at bits 4g..4g+3.
// Branch-free: with bits b0..b3 of a nibble, p0 & 1 = ~b0 & b1,
// p0 >> 1 = ~b0 & ~b1, p1 & 1 = b3 | ~b2, p1 >> 1 = b3 | b2.
__device__ __forceinline__ int nib_codes(uint32_t m) {
  const uint32_t s1 = m >> 1, s2 = m >> 2, s3 = m >> 3;
  const uint32_t c0 = ~m & s1 & 0x1111u;
  const uint32_t c1 = ~m & ~s1 & 0x1111u;
  const uint32_t c2 = (s3 | ~s2) & 0x1111u;
  const uint32_t c3 = (s3 | s2) & 0x1111u;
  return (int)(c0 | (c1 << 1) | (c2 << 2) | (c3 << 3));
}

template <bool BF>
__device__ __forceinline__ f4v_t smfmac(u32x4_t a, u32x4_t b0, u32x4_t b1, int idx, f4v_t c) {
  const u32x8_t b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
  if constexpr (BF)
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(b8v_t, a),
                                                    __builtin_bit_cast(b16v_t, b), c, idx, 0, 0);
  else
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(h8v_t, a),
                                                   __builtin_bit_cast(h16v_t, b), c, idx, 0, 0);
}

template <bool BF>
__device__ __forceinline__ f4v_t dmfma(u32x4_t a, u32x4_t b, f4v_t c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8v_t, a),
                                                  __builtin_bit_cast(b8v_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v_t, a),
                                                 __builtin_bit_cast(h8v_t, b), c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ void lds_st(uint32_t addr, T v) {
  *(__attribute__((address_space(3))) T *)(size_t)addr = v;
}

// Kernel kinds of the matrix-core product.

// Direct-to-LDS buffer loads: lane i's 16 (or 4) bytes at voff + soff land
// at LDS address lds + 16 i (4 i); lds is wave-uniform.  The weights stream
// with the nt policy, x (read by every workgroup) with the default one.
__device__ __forceinline__ void lds_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff,
                                              int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(size_t)lds, 16, voff, soff, 0, 2);
}
__device__ __forceinline__ void lds_load4_nt(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff,
                                             int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(size_t)lds, 4, voff, soff, 0, 2);
}
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff,
                                           int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(size_t)lds, 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(n) alone (expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

}  // namespace
