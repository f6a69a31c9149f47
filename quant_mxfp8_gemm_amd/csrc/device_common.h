// device_common.h - gfx950 helpers shared by the MXFP8 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp8 {

// UE8M0 code of a 32-block from the bits of its (non-negative, finite) amax held as
// an IEEE binary32: the smallest e with amax <= 448 * 2^e = 1.75 * 2^(e+8). For a
// normal amax = (1 + f) * 2^(E-127) that is e = E - 135 when f <= 0.75 and E - 134
// otherwise; the code is e + 127, clamped to [0, 254] (zero and tiny blocks -> 0).
__device__ __forceinline__ uint32_t ue8m0_from_amax_f32_bits(uint32_t amax_bits) {
  int32_t e = (int32_t)(amax_bits >> 23) - 8 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  e = e < 0 ? 0 : e;
  e = e > 254 ? 254 : e;
  return (uint32_t)e;
}

// Same rule from the bits of a BF16 amax (7 stored mantissa bits: f <= 0.75 <=> m <= 96).
__device__ __forceinline__ uint32_t ue8m0_from_amax_bf16_bits(uint32_t amax_bits) {
  int32_t e = (int32_t)(amax_bits >> 7) - 8 + ((amax_bits & 0x7Fu) > 96u ? 1 : 0);
  e = e < 0 ? 0 : e;
  e = e > 254 ? 254 : e;
  return (uint32_t)e;
}

// 2^(127 - code) as fp32: the factor that maps a block onto the E4M3 range.
// Exact for code in [0, 253], which covers every finite input.
__device__ __forceinline__ float inv_scale_from_ue8m0(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

// Two fp32 -> two E4M3 (OCP, round to nearest even) packed in the low 16 bits.
// The inputs are already within +-448, so saturation never matters.
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four fp32 -> four E4M3 bytes in one dword (byte i = value i).
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Two fp32 values -> packed BF16 bits (lo in bits 0-15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950. On finite inputs (denormals included) it equals the bit-level
// rounding (u + 0x7FFF + ((u >> 16) & 1)) >> 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A lane's value from another lane of its row of 16, by DPP control code (gfx9 encoding).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(lo | (hi << 32)));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i of 8 <- lane 7 - i
constexpr int DPP_MIRROR = 0x140;       // lane i of 16 <- lane 15 - i

// 16-byte streaming load (data read once: do not keep it in the caches).
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Byte offset of (row r, K-block c) in the 128x4 swizzled scale layout; col_tiles = ceil(nblk/4).
__device__ __forceinline__ int64_t swizzled_offset(int64_t r, int64_t c, int64_t col_tiles) {
  return ((r >> 7) * col_tiles + (c >> 2)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (c & 3);
}

}  // namespace mxfp8
