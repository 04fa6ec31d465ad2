// Device helpers shared by the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

// Packed dot products with fp32 accumulation (v_dot2_f32_bf16 / v_dot2_f32_f16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// The 8 nibbles of a packed word as 4 pairs of 16-bit floats whose values
// are OFFSET + q: pair m holds nibbles m and m+4 (low, high half).  The high
// byte of each half is the exponent byte E (0x43: bf16 128 + q; 0x64: fp16
// 1024 + q), the nibble lands in the low mantissa bits, whose weight is
// exactly 1.  One shift and one and-or per pair (the first needs no shift).
template <uint32_t E>
__device__ __forceinline__ void nib_pairs(uint32_t w, uint32_t (&p)[4]) {
  constexpr uint32_t M = (E << 8) * 0x00010001u;
  p[0] = (w & 0x000F000Fu) | M;
  p[1] = ((w >> 4) & 0x000F000Fu) | M;
  p[2] = ((w >> 8) & 0x000F000Fu) | M;
  p[3] = ((w >> 12) & 0x000F000Fu) | M;
}
constexpr uint32_t kExpBf16 = 0x43u;  // bf16 128 + q
constexpr uint32_t kExpF16 = 0x64u;   // fp16 1024 + q

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f32_to_f16(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Whole-wavefront maximum / sum through DPP row shifts and row broadcasts
// (no LDS): within each row of 16 lanes a doubling scan leaves the row's
// result in its lane 15, then rows 1 and 3 take row 0's and row 2's, and
// rows 2-3 take lane 31's; lane 63 ends with the total, which is returned to
// every lane.  The order of the additions is fixed, so every call gives the
// same bits for the same inputs.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_zero(uint32_t v) {  // lanes without a source (or outside ROWS) read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}
// Unsigned maximum (0 is neutral); the result is returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_zero<0x111, 0xF>(v));  // row_shr:1
  v = max(v, dpp_zero<0x112, 0xF>(v));  // row_shr:2
  v = max(v, dpp_zero<0x114, 0xF>(v));  // row_shr:4
  v = max(v, dpp_zero<0x118, 0xF>(v));  // row_shr:8
  v = max(v, dpp_zero<0x142, 0xA>(v));  // row_bcast:15 into rows 1, 3
  v = max(v, dpp_zero<0x143, 0xC>(v));  // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ float dpp_add(float v, uint32_t s) { return v + __uint_as_float(s); }
// Sum of the 64 lanes (LAST = 63) or of lanes 0..31 (LAST = 31), returned to
// every lane; all 64 lanes must be active.
template <int LAST = 63>
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = dpp_add(v, dpp_zero<0x111, 0xF>(__float_as_uint(v)));
  v = dpp_add(v, dpp_zero<0x112, 0xF>(__float_as_uint(v)));
  v = dpp_add(v, dpp_zero<0x114, 0xF>(__float_as_uint(v)));
  v = dpp_add(v, dpp_zero<0x118, 0xF>(__float_as_uint(v)));
  v = dpp_add(v, dpp_zero<0x142, 0xA>(__float_as_uint(v)));
  if (LAST == 63) v = dpp_add(v, dpp_zero<0x143, 0xC>(__float_as_uint(v)));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), LAST));
}

// Sum over lanes that differ in the given xor bits (fixed butterfly order).
__device__ __forceinline__ float xor_sum(float v, int mask_lo, int mask_hi) {
  for (int m = mask_lo; m <= mask_hi; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace moe
