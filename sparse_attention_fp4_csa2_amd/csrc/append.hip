// Cache append: MXFP4 quantise + pack of new latent entries, indexer-key copy
// (bf16, or MXFP8 in the lower-precision key cache), group-sum recompute.
//
// Storage of the global latent cache in FP4 follows the news.promptgoblins.ai
// summary (Details, "FP4 KVCache precision") and the thelatestinai.com
// abstract; the format is MXFP4 as in the OCP Microscaling Formats v1.0
// specification (E2M1 elements, one E8M0 scale per 32 values).  Each entry is a
// merged pair of raw positions (paper-digest.app page, Core Mechanics).
//
// One wave quantises one 512-value entry: lane l owns values [8l, 8l+8), four
// lanes form a 32-value scale group.  All decisions are exact integer
// arithmetic on the bf16 bit patterns, so the packed bytes are reproducible
// bit for bit.
#include "device.h"
#include "launch.h"

namespace csa2 {

// floor(log2 |x|) for a nonzero finite bf16 magnitude pattern (sign cleared).
__device__ __forceinline__ int floor_log2_bf16(uint32_t mag) {
  uint32_t ef = mag >> 7;
  if (ef) return (int)ef - 127;
  // subnormal: mag = m * 2^-133 with 1 <= m < 128
  return (31 - __builtin_clz(mag)) - 133;
}

// E2M1 magnitude code (0..7) of |x| / 2^(sb-127), round to nearest, halfway to
// the even code, saturating at 6.  mag = bf16 magnitude bits of x.
__device__ __forceinline__ uint32_t e2m1_code(uint32_t mag, int sb) {
  uint32_t ef = mag >> 7;
  uint32_t sig = ef ? (0x80u | (mag & 0x7Fu)) : (mag & 0x7Fu);
  int ex = ef ? (int)ef : 1;
  // |x|/X * 4 = sig * 2^-u with u = sb + 5 - ex; halfway points *4 are the
  // integers 1 3 5 7 10 14 20
  int u = sb + 5 - ex;
  if (u < 0) return 7;           // far above 6: saturate
  if (u >= 9) return 0;          // below 0.125: rounds to 0
  const uint32_t T[7] = {1u, 3u, 5u, 7u, 10u, 14u, 20u};
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) c += (sig > (T[i] << u)) ? 1u : 0u;
  if (c < 7 && sig == (T[c] << u) && (c & 1u)) c += 1;   // exact tie -> even code
  return c;
}

// ---- MXFP8 indexer keys -------------------------------------------------
// E4M3 magnitude code (0..126) of |x| / 2^(sb-127), round to nearest, halfway
// to the even code, saturating at 448 (code 126).  mag = bf16 magnitude bits.
// |x| / X = sig * 2^p exactly; its E4M3 binade is e = floor(log2) + 7 (codes
// 8(e-1) .. 8(e-1)+15 step 2^(e-10) for e >= 1; below 2^-6 the step is 2^-9),
// so n = round(|x| / X / step) and code = 8 (max(e, 1) - 1) + n (n = 16 carries
// into the next binade).
__device__ __forceinline__ uint32_t e4m3_code(uint32_t mag, int sb) {
  const uint32_t ef = mag >> 7;
  const uint32_t sig = ef ? (0x80u | (mag & 0x7Fu)) : (mag & 0x7Fu);
  if (sig == 0) return 0;
  const int p = (ef ? (int)ef : 1) - 7 - sb;           // |x| / X = sig * 2^p
  const int lg = 31 - __builtin_clz(sig);               // floor(log2 sig)
  const int e = lg + p + 7;
  const int qe = (e > 1 ? e : 1) - 10;                  // log2 of the grid step
  const int s = qe - p;                                 // n = sig / 2^s
  uint32_t n;
  if (s <= 0) {
    n = sig << (-s);
  } else if (s >= 10) {
    n = 0;                                              // below half the smallest step
  } else {
    const uint32_t n0 = sig >> s, rem = sig & ((1u << s) - 1u), half = 1u << (s - 1);
    n = n0 + ((rem > half || (rem == half && (n0 & 1u))) ? 1u : 0u);
  }
  const uint32_t code = 8u * (uint32_t)((e > 1 ? e : 1) - 1) + n;
  return code > 126u ? 126u : code;
}

// MXFP8 key of new entry i at cache entry j, by one wave: lane d holds dim d;
// the 32 lanes of a scale group agree on the group's largest magnitude.
__device__ __forceinline__ void write_key8(const uint16_t* __restrict__ idx_key, int b, int i, int n_new,
                                           long long j, int cap, int lane, uint8_t* __restrict__ key8,
                                           uint8_t* __restrict__ key8_scale) {
  const uint32_t v = idx_key[((size_t)b * n_new + i) * DI + lane];
  uint32_t amax = v & 0x7FFFu;
  amax = half_wave_max_u32(amax);
  const int sb = amax ? min(max(floor_log2_bf16(amax) - 8 + 127, 0), 254) : 0;
  const uint32_t code = ((v >> 15) << 7) | e4m3_code(v & 0x7FFFu, sb);
  key8[((size_t)b * cap + (size_t)j) * DI + lane] = (uint8_t)code;
  if ((lane & 31) == 0) key8_scale[((size_t)b * cap + (size_t)j) * 2 + (lane >> 5)] = (uint8_t)sb;
}

// One wave per new entry: the latent's MXFP4 record bytes (latent may be
// null: keys only), and its indexer key as bf16 (key_cache) or MXFP8 (key8).
// Workgroup x of sequence b takes new entries 4x .. 4x + 3.
__device__ __forceinline__ void append_entries(
    const uint16_t* __restrict__ latent, const uint16_t* __restrict__ idx_key,
    const int32_t* __restrict__ start_entry, int n_new, int cap,
    uint8_t* __restrict__ cache, uint16_t* __restrict__ key_cache,
    uint8_t* __restrict__ key8, uint8_t* __restrict__ key8_scale, int x, int b) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = x * 4 + wave;                   // new entry index
  if (i >= n_new) return;
  const long long j = (long long)start_entry[b] + i;   // cache entry position
  if (j < 0 || j >= cap) return;
  if (key8 != nullptr) write_key8(idx_key, b, i, n_new, j, cap, lane, key8, key8_scale);
  if (latent == nullptr) return;

  const uint16_t* src = latent + ((size_t)b * n_new + i) * D + lane * 8;
  uint4 raw = *reinterpret_cast<const uint4*>(src);
  uint32_t v[8] = {raw.x & 0xFFFFu, raw.x >> 16, raw.y & 0xFFFFu, raw.y >> 16,
                   raw.z & 0xFFFFu, raw.z >> 16, raw.w & 0xFFFFu, raw.w >> 16};
  // group amax as an integer on the magnitude bits (monotonic for finite bf16)
  uint32_t amax = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = max(amax, v[k] & 0x7FFFu);
  amax = quad_max_u32(amax);
  const bool nonfinite = amax >= 0x7F80u;
  int sb = 0;
  if (!nonfinite && amax) sb = min(max(floor_log2_bf16(amax) - 2 + 127, 0), 254);

  uint32_t packed = 0;
  if (!nonfinite) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t code = ((v[k] >> 15) << 3) | e2m1_code(v[k] & 0x7FFFu, sb);
      packed |= code << (4 * k);
    }
  }
  uint8_t* rec = cache + ((size_t)b * (cap / BLOCK) + (size_t)(j / BLOCK)) * RECORD;
  const int slot = (int)(j % BLOCK);
  *reinterpret_cast<uint32_t*>(rec + slot * 256 + lane * 4) = packed;
  if ((lane & 3) == 0) rec[SCALE_OFF + slot * 16 + (lane >> 2)] = (uint8_t)(nonfinite ? 255 : sb);

  if (idx_key != nullptr && key_cache != nullptr && lane < 8) {
    const uint4* ks = reinterpret_cast<const uint4*>(idx_key + ((size_t)b * n_new + i) * DI) + lane;
    uint4* kd = reinterpret_cast<uint4*>(key_cache + ((size_t)b * cap + (size_t)j) * DI) + lane;
    *kd = *ks;
  }
}

// E4M3 code -> value (finite codes; exact in fp32 with the power-of-two scale)
__device__ __forceinline__ float e4m3_value(uint32_t c, int sb) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? ldexpf((float)(8u + m), (int)e - 10) : ldexpf((float)m, -9);
  return ldexpf((c & 0x80u) ? -mag : mag, sb - 127);
}

// Group sums, recomputed for every 512-entry group the append touches: the sum
// of the keys all 512 slots of the group hold once the append is done (slots
// that hold no entry are zero in a zero-initialised cache), so an overwritten
// entry counts once, with its new key.  A slot the append writes is read from
// the new keys themselves (MXFP8: quantised here exactly as the entry waves
// quantise it), every other slot from the key cache, so these workgroups share
// the append's launch without reading what its other workgroups write.  One
// 256-thread workgroup per (sequence, touched group gi): thread t sums dims
// [8(t%8), +8) over the slots t/8, t/8 + 32, ... in fp64, and the 32 partials
// meet in LDS in a fixed order.  fp64 holds the sum of 512 bf16 (or E4M3 x 2^k)
// values exactly unless they span more than ~40 binades, so the stored fp32 is
// the exact sum rounded once, whatever the order.
template <bool K8>
__device__ __forceinline__ void group_sum_unit(
    const uint16_t* __restrict__ idx_key, const uint16_t* __restrict__ key_cache,
    const uint8_t* __restrict__ key8, const uint8_t* __restrict__ key8_scale,
    const int32_t* __restrict__ start_entry, int n_new, int cap, float* __restrict__ group_sum, int gi, int b) {
  __shared__ double part[32][DI + 1];
  const int t = threadIdx.x, c = t & 7, r = t >> 3;
  const long long s0 = start_entry[b];
  const long long first = max(s0, 0LL), last = min(s0 + n_new, (long long)cap);   // written [first, last)
  if (first >= last) return;
  const long long g = first / GROUP_ENTRIES + gi;
  if (g * GROUP_ENTRIES >= last) return;
  double acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.0;
  constexpr int PER = GROUP_ENTRIES / 32;      // slots per thread, all requested before any is summed
  uint4 kw[PER];      // bf16 key words (new slot, or bf16 cache); MXFP8 cache: codes in .x .y, scale in .z
  bool fresh[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const long long j = g * GROUP_ENTRIES + r + 32 * i;
    fresh[i] = j >= first && j < last;
    const size_t e = (size_t)b * cap + (size_t)j;
    if (fresh[i]) {
      kw[i] = *reinterpret_cast<const uint4*>(idx_key + ((size_t)b * n_new + (size_t)(j - s0)) * DI + 8 * c);
    } else if constexpr (K8) {
      const uint2 cw = *reinterpret_cast<const uint2*>(key8 + e * DI + 8 * c);
      kw[i] = make_uint4(cw.x, cw.y, key8_scale[e * 2 + (c >> 2)], 0u);
    } else {
      kw[i] = *reinterpret_cast<const uint4*>(key_cache + e * DI + 8 * c);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t w4[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
    if constexpr (K8) {
      // a new key's 32-dim scale group spans the 4 threads c = 4(c/4) .. +3 of this slot
      uint32_t amax = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = max(amax, ((k & 1) ? (w4[k >> 1] >> 16) : w4[k >> 1]) & 0x7FFFu);
      amax = fresh[i] ? amax : 0u;
      amax = quad_max_u32(amax);
      const int sb_new = amax ? min(max(floor_log2_bf16(amax) - 8 + 127, 0), 254) : 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float v;
        if (fresh[i]) {
          const uint32_t h = ((k & 1) ? (w4[k >> 1] >> 16) : w4[k >> 1]) & 0xFFFFu;
          v = e4m3_value(((h >> 15) << 7) | e4m3_code(h & 0x7FFFu, sb_new), sb_new);
        } else {
          v = e4m3_value((w4[k >> 2] >> (8 * (k & 3))) & 0xFFu, (int)w4[2]);
        }
        acc[k] += (double)v;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc[k] += (double)__uint_as_float((k & 1) ? (w4[k >> 1] & 0xFFFF0000u) : (w4[k >> 1] << 16));
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) part[r][8 * c + k] = acc[k];
  __syncthreads();
  if (t < DI) {
    double sum = 0.0;
    for (int i = 0; i < 32; ++i) sum += part[i][t];
    group_sum[((size_t)b * (cap / GROUP_ENTRIES) + (size_t)g) * DI + t] = (float)sum;
  }
}

// One launch per append: workgroups [0, n_entry_wg) of each sequence write the
// new entries, the rest recompute the touched groups' sums (when group_sum is
// given).
template <bool K8>
__global__ __launch_bounds__(256) void append_kernel(
    const uint16_t* __restrict__ latent, const uint16_t* __restrict__ idx_key,
    const int32_t* __restrict__ start_entry, int n_new, int cap, uint8_t* __restrict__ cache,
    uint16_t* __restrict__ key_cache, uint8_t* __restrict__ key8, uint8_t* __restrict__ key8_scale,
    float* __restrict__ group_sum, int n_entry_wg) {
  const int b = blockIdx.y;
  if ((int)blockIdx.x < n_entry_wg)
    append_entries(latent, idx_key, start_entry, n_new, cap, cache, key_cache, key8, key8_scale, blockIdx.x, b);
  else
    group_sum_unit<K8>(idx_key, key_cache, key8, key8_scale, start_entry, n_new, cap, group_sum,
                       (int)blockIdx.x - n_entry_wg, b);
}

static int launch_append_t(bool k8, const uint16_t* latent, const uint16_t* idx_key, const int32_t* start_entry,
                           int B, int n_new, int cap, uint8_t* cache, uint16_t* key_cache, uint8_t* key8,
                           uint8_t* key8_scale, float* group_sum, hipStream_t stream) {
  const int n_entry_wg = (n_new + 3) / 4;
  const int n_group_wg = group_sum ? (n_new + GROUP_ENTRIES - 1) / GROUP_ENTRIES + 1 : 0;
  dim3 grid(n_entry_wg + n_group_wg, B);
  if (k8)
    append_kernel<true><<<grid, 256, 0, stream>>>(latent, idx_key, start_entry, n_new, cap, cache, nullptr, key8,
                                                  key8_scale, group_sum, n_entry_wg);
  else
    append_kernel<false><<<grid, 256, 0, stream>>>(latent, idx_key, start_entry, n_new, cap, cache, key_cache,
                                                   nullptr, nullptr, group_sum, n_entry_wg);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_append_key8(const uint16_t* latent, const uint16_t* idx_key, const int32_t* start_entry, int B,
                       int n_new, int cap, uint8_t* cache, uint8_t* key8, uint8_t* key8_scale, float* group_sum,
                       hipStream_t stream) {
  return launch_append_t(true, latent, idx_key, start_entry, B, n_new, cap, cache, nullptr, key8, key8_scale,
                         group_sum, stream);
}

int launch_append(const uint16_t* latent, const uint16_t* idx_key, const int32_t* start_entry,
                  int B, int n_new, int cap, uint8_t* cache, uint16_t* key_cache,
                  float* group_sum, hipStream_t stream) {
  return launch_append_t(false, latent, idx_key, start_entry, B, n_new, cap, cache, key_cache, nullptr, nullptr,
                         group_sum, stream);
}

}  // namespace csa2
