// Device-side helpers shared by the CSA2 kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

namespace csa2 {

constexpr int D = 512;
constexpr int DI = 64;
constexpr int BLOCK = 8;
constexpr int RECORD = 2176;
constexpr int SCALE_OFF = 2048;
constexpr int GROUP_ENTRIES = 512;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Lane shuffles within a wave64 (compile to ds_bpermute / DPP as the compiler sees fit).
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ float warp_max_xor(float v, int lo_mask_bits) {
  // butterfly max over lanes whose ids differ in the low `lo_mask_bits` bits
  for (int m = 1; m < (1 << lo_mask_bits); m <<= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

// Order-preserving map float -> uint32 (larger float -> larger key).  NaN and
// -inf both map to 0, which marks "not a candidate".
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (s != s || s == -__builtin_inff()) return 0u;
  if (s == 0.0f) return 0x80000000u;          // -0 and +0 are one score (a tie)
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Dequantise 8 MXFP4 codes (one dword; byte k holds element 2k in its low
// nibble and 2k+1 in its high nibble) with E8M0 scale byte sb into 8 bf16
// (4 dwords, element order kept).  gfx950's scaled FP4 -> bf16 conversion takes
// the scale as the float 2^(sb-127), passed by its bit pattern sb << 23; it is
// exact for every code and every sb in [0, 254].  Results are moved as whole
// 32-bit words: single-element access to __bf16 vectors is avoided on purpose.
__device__ __forceinline__ uint4 dequant8(uint32_t codes, uint32_t sb) {
  float sc = __uint_as_float(sb << 23);
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ uint4 as_uint4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace csa2
