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

// Lane exchanges within a wave64 without LDS round trips: DPP swaps inside a
// 16-lane row (quad xor 1 and xor 2, the 8-lane half-row mirror, the 16-lane
// row mirror) and gfx950's row swaps (v_permlane16_swap: lane l meets l ^ 16;
// v_permlane32_swap: l meets l ^ 32).  For a symmetric op, applying it to a
// value and its partner at every step leaves the group's result in every lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_QUAD_XOR1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_XOR2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7 - i within 8 lanes
constexpr int DPP_ROW_MIRROR = 0x140;  // lane i <-> 15 - i within 16 lanes

// op over the 8 lanes of an aligned group (3 DPP steps)
template <typename F>
__device__ __forceinline__ uint32_t group8_reduce(uint32_t x, F op) {
  x = op(x, dpp_mov<DPP_QUAD_XOR1>(x));
  x = op(x, dpp_mov<DPP_QUAD_XOR2>(x));
  return op(x, dpp_mov<DPP_HALF_MIRROR>(x));
}
// op of lane l and lane l ^ 16, then of l and l ^ 32 (the row swaps)
template <typename F>
__device__ __forceinline__ uint32_t cross_rows_reduce(uint32_t x, F op) {
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op((uint32_t)a[0], (uint32_t)a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op((uint32_t)c[0], (uint32_t)c[1]);
}
// op over the whole wave, result in every lane
template <typename F>
__device__ __forceinline__ uint32_t wave_allreduce(uint32_t x, F op) {
  x = group8_reduce(x, op);
  x = op(x, dpp_mov<DPP_ROW_MIRROR>(x));
  return cross_rows_reduce(x, op);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return wave_allreduce(x, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return wave_allreduce(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return wave_allreduce(x, [](uint32_t a, uint32_t b) { return a + b; });
}
// max over an aligned group of 4 lanes (2 DPP steps), and over each 32-lane
// half of the wave (lane l meets l ^ 16 last)
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t x) {
  x = max(x, dpp_mov<DPP_QUAD_XOR1>(x));
  return max(x, dpp_mov<DPP_QUAD_XOR2>(x));
}
__device__ __forceinline__ uint32_t half_wave_max_u32(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  x = group8_reduce(x, op);
  x = op(x, dpp_mov<DPP_ROW_MIRROR>(x));
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return op((uint32_t)a[0], (uint32_t)a[1]);
}
// float max over an aligned group of 8 lanes
__device__ __forceinline__ float group8_max(float v) {
  return __uint_as_float(group8_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
// float sum of lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float cross_rows_sum(float v) {
  return __uint_as_float(cross_rows_reduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

// Order-preserving map float -> uint32 (larger float -> larger key).  NaN and
// -inf both map to 0, which marks "not a candidate".
// (selects only: the top-K kernels convert 16-64 scores per thread, and
// early returns there became a branch per score)
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  k = s == 0.0f ? 0x80000000u : k;             // -0 and +0 are one score (a tie)
  return (s != s || s == -__builtin_inff()) ? 0u : k;
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

// Store one head's slice of an O^T accumulator as fp16 of acc * f * 2^shift
// (v_ldexp per value: no intermediate overflow).  Lane (head,
// hh) holds acc[mt][i] = dim 32mt + 8(i/4) + 4hh + i%4 (relative to dst); the
// lanes hh = 0 and hh = 1 of a head swap halves (v_permlane32_swap) so that each
// writes 16 contiguous dims [32mt + 16hh, +16) per mt: 32-byte stores.
__device__ __forceinline__ void store_o16_slice(const floatx16 (&acc)[4], float f, int shift, int hh,
                                                uint16_t* dst) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                 f2{ldexpf(acc[mt][2 * k] * f, shift), ldexpf(acc[mt][2 * k + 1] * f, shift)}, h2));
    // hh = 1 sends its dims 4-7, 12-15 (w[0..3]); hh = 0 sends 16-19, 24-27 (w[4..7])
    uint32_t x[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t snd = hh ? w[d] : w[4 + d];
      const auto r = __builtin_amdgcn_permlane32_swap(snd, snd, false, false);
      x[d] = hh ? r[0] : r[1];
    }
    const uint4 a = hh ? make_uint4(x[0], x[1], w[4], w[5]) : make_uint4(w[0], w[1], x[0], x[1]);
    const uint4 c = hh ? make_uint4(x[2], x[3], w[6], w[7]) : make_uint4(w[2], w[3], x[2], x[3]);
    uint4* o = reinterpret_cast<uint4*>(dst + 32 * mt + 16 * hh);
    o[0] = a;
    o[1] = c;
  }
}

// Workgroup L of an attention grid -> (unit, head group), unit = row * splits
// + split.  With several splits XCD x (= L % 8) runs the x-th contiguous
// eighth of the (unit, head group) order, so a row's splits and head groups
// share one XCD's L2 (the row's query comes from HBM once, and the two head
// groups of a split, dispatched together, share their reads).  With one split
// (many rows per sequence, as in prefill) unit u goes to XCD u % 8 and its
// head groups to ids 8 apart: measured to fetch a quarter of the L2 misses of
// the contiguous order there.  The split combine places its workgroups on the
// XCD of their row under the contiguous order (launch_combine).
__device__ __forceinline__ void map_unit(int L, int n_units, int hgroups, bool several_splits, int& unit,
                                         int& hgi) {
  if (several_splits) {
    const int per_xcd = ((n_units + 7) / 8) * hgroups;
    const int u = (L & 7) * per_xcd + (L >> 3);
    unit = u / hgroups;
    hgi = u - unit * hgroups;
  } else {
    unit = (L / (8 * hgroups)) * 8 + (L & 7);
    hgi = (L >> 3) % hgroups;
  }
}

}  // namespace csa2
