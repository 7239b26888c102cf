// Sparse indexer: entry scores, fused block max, and the coarse group stage.
//
// The pages name the indexer and its output -- up to 2048 blocks of 8 per
// query, rescored per layer in Reindex mode, two-level ("hierarchical") to trim
// decoder indexing (observer.broadside.tech card, Key ideas, "CSA2 with three
// static layer modes") -- but print no formula.  The score used here:
//   e_j = sum_h w_h * max(0, q_h . k_j),  block score = max over its visible,
//   present entries; coarse group score = the same formula on the group's mean key.
//
// The entry scores are a genuine [Hi x 64] x [64 x N] contraction per query
// row, done on v_mfma_f32_16x16x32_bf16: A = the row's indexer query (heads
// padded to 16), B = 16 keys per MFMA.  Keys are bf16, or MXFP8 (E4M3 codes
// with one E8M0 scale per 32 dims) converted to bf16 in registers on load
// (v_cvt_scalef32_pk_bf16_fp8: exact), which halves the bytes read.  The ReLU, weights, head sum and the
// 8-entry block max run in the epilogue, so entry scores never reach memory.
// Keys stream once from HBM with 32-byte loads per lane.
#include "device.h"
#include "launch.h"
#include "select.h"

namespace csa2 {

namespace {

constexpr int CH_FLAT = 512;    // entries per workgroup (flat)
constexpr int CH_GROUP = 512;   // entries per workgroup (one coarse group)
constexpr int UNROLL = 4;       // 16-entry tiles in flight per wave
constexpr int MAX_HI = 16;      // indexer heads (rows of the A operand)

__device__ __forceinline__ floatx4 mfma16(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// MXFP8 keys: E8M0 scale byte -> the float 2^(sb - 127) (sb = 0: the fp32
// subnormal 2^-127)
__device__ __forceinline__ float e8m0_float(uint32_t sb) {
  return __uint_as_float(sb ? sb << 23 : 1u << 22);
}
// 4 E4M3 codes (bytes of c, byte 0 first) times the scale -> 4 bf16 (the
// products are exact: 4 significant bits times a power of two)
__device__ __forceinline__ uint2 fp8x4_bf16(uint32_t c, float scale) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, scale, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, scale, true)));
}
__device__ __forceinline__ uint4 fp8x8_bf16(uint32_t lo, uint32_t hi, float scale) {
  const uint2 a = fp8x4_bf16(lo, scale), b = fp8x4_bf16(hi, scale);
  return make_uint4(a.x, a.y, b.x, b.y);
}

}  // namespace

// grid: (chunks, rows).  Flat: chunk x covers entries [x*CH, x*CH + CH) and
// writes block scores at [row][x*CH/8 ...] of a row of length n_out = cap/8.
// Group-restricted: chunk x covers group gsel[row][x] and writes at
// [row][x*64 ...] of a row of length n_out = 64 * n_groups_sel.
template <int CH, bool K8>
__global__ __launch_bounds__(256) void index_scores_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ key_cache, const uint8_t* __restrict__ key8,
    const uint8_t* __restrict__ key8_scale, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ q_pos, int Q, int Hi, int cap,
    const int32_t* __restrict__ gsel, int n_groups_sel, int n_out, float* __restrict__ scores) {
  const int x = blockIdx.x, row = blockIdx.y;
  const int b = row / Q;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15;            // entry within a 16-entry tile / head row of A
  const int kg = lane >> 4;           // k-group: dims [16kg, 16kg+16)

  int e0;
  if (gsel) {
    const int g = gsel[(size_t)row * n_groups_sel + x];
    e0 = g < 0 ? -1 : g * GROUP_ENTRIES;
  } else {
    e0 = x * CH;
  }
  float* out = scores + (size_t)row * n_out + (size_t)x * (CH / BLOCK);
  const int ne = n_entries[b];
  const int limit_vis = q_pos ? ((q_pos[row] - 1) >> 1) + 1 : 0x7FFFFFFF;   // visible iff j < limit
  const int jmax = min(min(ne, cap), limit_vis);          // entries [0, jmax) count

  if (e0 < 0) {
    // unused group slot: no candidates
    for (int i = threadIdx.x; i < CH / BLOCK; i += 256) out[i] = -__builtin_inff();
    return;
  }

  // A fragments: head n (< Hi), dims [16kg + 8ks, +8)
  uint4 qa[2];
  const size_t qoff = ((size_t)row * Hi + n) * DI + 16 * kg;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    qa[ks] = n < Hi ? *reinterpret_cast<const uint4*>(q_idx + qoff + 8 * ks) : make_uint4(0, 0, 0, 0);
  // weights of the 4 heads this lane's accumulator rows hold: 4kg + i
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * kg + i;
    wv[i] = h < Hi ? w[(size_t)row * Hi + h] : 0.f;
  }

  constexpr int PER_WAVE = CH / 4;              // entries per wave
  constexpr int TILES = PER_WAVE / 16;
  const int wbase = e0 + wave * PER_WAVE;
  const uint16_t* kbase = K8 ? nullptr : key_cache + (size_t)b * cap * DI;

  for (int t0 = 0; t0 < TILES; t0 += UNROLL) {
    uint4 kb[UNROLL][2];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int j = wbase + 16 * (t0 + u) + n;
      if (j < jmax) {
        if constexpr (K8) {
          const size_t ke = (size_t)b * cap + (size_t)j;
          const uint4 c = *reinterpret_cast<const uint4*>(key8 + ke * DI + 16 * kg);
          const float sc = e8m0_float(key8_scale[ke * 2 + (kg >> 1)]);
          kb[u][0] = fp8x8_bf16(c.x, c.y, sc);
          kb[u][1] = fp8x8_bf16(c.z, c.w, sc);
        } else {
          const uint4* kp = reinterpret_cast<const uint4*>(kbase + (size_t)j * DI + 16 * kg);
          kb[u][0] = kp[0];
          kb[u][1] = kp[1];
        }
      } else {
        kb[u][0] = make_uint4(0, 0, 0, 0);
        kb[u][1] = kb[u][0];
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      floatx4 acc = floatx4{};
      acc = mfma16(qa[0], kb[u][0], acc);
      acc = mfma16(qa[1], kb[u][1], acc);
      // acc[i]: head 4kg + i, entry n
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) part += wv[i] * fmaxf(acc[i], 0.f);
      part = cross_rows_sum(part);
      const int j = wbase + 16 * (t0 + u) + n;
      float s = j < jmax ? part : -__builtin_inff();
      s = group8_max(s);
      const int local_blk = (wave * PER_WAVE + 16 * (t0 + u) + n) / BLOCK;
      if ((lane == 0 || lane == 8) && x * (CH / BLOCK) + local_blk < n_out) out[local_blk] = s;
    }
  }
}

// Many query rows of one sequence (chunked prefill): the entry scores are a
// [rows*Hi x 64] x [64 x N] contraction on v_mfma_f32_32x32x16_bf16.  A wave
// holds 16 rows as four A sets of 32 (row, head) pairs (4 rows x 8 heads) and
// streams 32 keys at a time as B, so each key it loads serves 16 rows, and
// the 4 waves of a workgroup (64 rows) read the same keys through L1.
// Epilogue per A set: ReLU and weights over the lane's 4 heads of each row,
// then one lane swap per row pair (l, l^32) completes the head sums of rows
// {0, 1} in the low half and {2, 3} in the high one; causal mask per row;
// 8-entry block max in three DPP steps.  grid: (row tiles of 64, entry chunks
// of CH_ROWS): the workgroups resident at a time share a few key chunks in
// L2.  Hi <= 8.
constexpr int ROWS_W = 16;              // rows per wave
constexpr int ROWS_T = 4 * ROWS_W;      // rows per workgroup
constexpr int CH_ROWS = 1024;     // 64 row tiles x 66 chunks at prefill: 8+ rounds of 512 slots

__device__ __forceinline__ floatx16 mfma32_bf16(uint4 a, uint4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <bool K8>
__global__ __launch_bounds__(256) void index_rows_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const uint16_t* __restrict__ key_cache, const uint8_t* __restrict__ key8,
    const uint8_t* __restrict__ key8_scale, const int32_t* __restrict__ n_entries,
    const int32_t* __restrict__ q_pos, int Q, int Hi, int cap, int n_out, float* __restrict__ scores) {
  const int rt = blockIdx.x, chunk = blockIdx.y;
  const int tiles_per_seq = (Q + ROWS_T - 1) / ROWS_T;
  const int b = rt / tiles_per_seq;
  const int q0 = (rt - b * tiles_per_seq) * ROWS_T + ROWS_W * (threadIdx.x >> 6);   // this wave's first row
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int ne = min(n_entries[b], cap);

  // A set a: pair col = (row q0 + 4a + col/8, head col%8), dims 16ks + 8hh + [0, 8)
  uint4 qa[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int r = q0 + 4 * a + (col >> 3), h = col & 7;
    const bool ok = r < Q && h < Hi;
    const uint16_t* src = q_idx + (((size_t)b * Q + (ok ? r : 0)) * Hi + (ok ? h : 0)) * DI + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[a][ks] = ok ? *reinterpret_cast<const uint4*>(src + 16 * ks) : make_uint4(0, 0, 0, 0);
  }
  // accumulator value i of set a: row q0 + 4a + i/4, head 4hh + i%4
  float wv[4][16];
  int lim[16];
  int lim_max = 0;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int r = q0 + 4 * a + r4;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int h = 4 * hh + k;
        wv[a][4 * r4 + k] = (r < Q && h < Hi) ? w[((size_t)b * Q + r) * Hi + h] : 0.f;
      }
      lim[4 * a + r4] = r < Q ? (q_pos ? min(ne, (q_pos[(size_t)b * Q + r] + 1) >> 1) : ne) : 0;
      lim_max = max(lim_max, lim[4 * a + r4]);
    }

  const int e_begin = chunk * CH_ROWS;
  const int e_end = min(e_begin + CH_ROWS, cap);
  const uint16_t* kbase = K8 ? nullptr : key_cache + (size_t)b * cap * DI + 8 * hh;
  auto load = [&](int e, uint4 (&kv)[4]) {
    const int j = e + col;
    if (j < lim_max) {
      if constexpr (K8) {
        // dims 16ks + 8hh + [0, 8): 8 codes at that byte offset, scale of group ks / 2
        const size_t ke = (size_t)b * cap + (size_t)j;
        const uint8_t* kp = key8 + ke * DI + 8 * hh;
        const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(key8_scale + ke * 2);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint2 c = *reinterpret_cast<const uint2*>(kp + 16 * ks);
          kv[ks] = fp8x8_bf16(c.x, c.y, e8m0_float((sc2 >> (8 * (ks >> 1))) & 0xFFu));
        }
      } else {
        const uint16_t* kp = kbase + (size_t)j * DI;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kv[ks] = *reinterpret_cast<const uint4*>(kp + 16 * ks);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kv[ks] = make_uint4(0, 0, 0, 0);
    }
  };
  auto score = [&](int e, const uint4 (&kv)[4]) {
    const int j = e + col;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      // keys past every row's limit load as zeros and their scores are masked
      // below, so the chain runs unconditionally (no zeroed accumulator)
      floatx16 acc = mfma32_bf16(qa[a][0], kv[0], floatx16{});
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) acc = mfma32_bf16(qa[a][ks], kv[ks], acc);
      // this lane's heads 4hh..4hh+3 of the set's rows r4 = 0..3
      float ps[4];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) s += wv[a][4 * r4 + k] * fmaxf(acc[4 * r4 + k], 0.f);
        ps[r4] = s;
      }
      // the low lane finishes rows 0, 1 and the high lane rows 2, 3: each sends
      // its partial sums of the other's rows (swap: [0] = low lane's, [1] = high's)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float snd = hh ? ps[u] : ps[2 + u];
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(snd), __float_as_uint(snd), false, false);
        const int r4 = 2 * hh + u;
        float s = (hh ? ps[2 + u] : ps[u]) + __uint_as_float(hh ? pr[0] : pr[1]);
        s = j < lim[4 * a + r4] ? s : -__builtin_inff();
        // max over the 8 lanes of the block: quad xor 1, quad xor 2, half-row mirror
        s = fmaxf(s, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0xB1, 0xF, 0xF, false)));
        s = fmaxf(s, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x4E, 0xF, 0xF, false)));
        s = fmaxf(s, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x141, 0xF, 0xF, false)));
        const int r = q0 + 4 * a + r4;
        if ((col & 7) == 0 && r < Q && j < cap) scores[((size_t)b * Q + r) * n_out + (j >> 3)] = s;
      }
    }
  };
  uint4 k0[4], k1[4];
  int e = e_begin;
  if (e < e_end) load(e, k0);
  for (; e + 32 < e_end; e += 64) {
    load(e + 32, k1);
    score(e, k0);
    if (e + 64 < e_end) load(e + 64, k0);
    score(e + 32, k1);
  }
  if (e < e_end) score(e, k0);
}

// Two-level stage, coarse scores: a [Hi x 64] x [64 x G] contraction per query
// row on v_mfma_f32_16x16x32_bf16, as the fine indexer's: A = the row's
// indexer query (heads padded to 16), B = 16 group means, each mean (fp32 sum
// / present count) split into bf16 hi + lo (16 significant bits between them),
// so a 16-group tile takes 4 MFMAs.  The epilogue applies ReLU and the head
// weights and sums the heads; groups with no entry score -inf.  A row's group
// sums (G x 256 B, 256 KB at G = 1024) are spread over G / 64 workgroups of
// 64 groups (one tile per wave): one workgroup per row would stream them
// through a single CU.  grid: (ceil(G / 64), rows).
constexpr int COARSE_GROUPS_WG = 64;

__global__ __launch_bounds__(256) void coarse_scores_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const float* __restrict__ group_sum,
    const int32_t* __restrict__ n_entries, int Q, int Hi, int cap, float* __restrict__ gscore) {
  const int row = blockIdx.y, b = row / Q;
  const int G = cap / GROUP_ENTRIES;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int n = lane & 15;            // group within the tile / head row of A
  const int kg = lane >> 4;           // k-group: dims [8kg, 8kg + 8) of each 32-dim k-step
  const int g = blockIdx.x * COARSE_GROUPS_WG + wave * 16 + n;
  // this lane's group-sum dims 32ks + 8kg + [0, 8), ks = 0, 1 (all requested first)
  float4 gs[2][2];
  {
    const float4* src = reinterpret_cast<const float4*>(group_sum + ((size_t)b * G + min(g, G - 1)) * DI + 8 * kg);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) gs[ks][0] = src[8 * ks], gs[ks][1] = src[8 * ks + 1];
  }
  // A fragments: head n (< Hi), dims 32ks + 8kg + [0, 8)
  uint4 qa[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    qa[ks] = n < Hi ? *reinterpret_cast<const uint4*>(q_idx + ((size_t)row * Hi + n) * DI + 32 * ks + 8 * kg)
                    : make_uint4(0, 0, 0, 0);
  float wv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wv[i] = 4 * kg + i < Hi ? w[(size_t)row * Hi + 4 * kg + i] : 0.f;
  const int ne = min(n_entries[b], cap);
  const int cnt = g < G ? min(GROUP_ENTRIES, ne - g * GROUP_ENTRIES) : 0;
  const float inv = cnt > 0 ? 1.f / (float)cnt : 0.f;

  floatx4 acc = floatx4{};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const float v[8] = {gs[ks][0].x * inv, gs[ks][0].y * inv, gs[ks][0].z * inv, gs[ks][0].w * inv,
                        gs[ks][1].x * inv, gs[ks][1].y * inv, gs[ks][1].z * inv, gs[ks][1].w * inv};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t h0 = f32_to_bf16_rne(v[2 * k]), h1 = f32_to_bf16_rne(v[2 * k + 1]);
      const uint32_t l0 = f32_to_bf16_rne(v[2 * k] - __uint_as_float(h0 << 16));
      const uint32_t l1 = f32_to_bf16_rne(v[2 * k + 1] - __uint_as_float(h1 << 16));
      hi[k] = h0 | (h1 << 16);
      lo[k] = l0 | (l1 << 16);
    }
    acc = mfma16(qa[ks], make_uint4(hi[0], hi[1], hi[2], hi[3]), acc);
    acc = mfma16(qa[ks], make_uint4(lo[0], lo[1], lo[2], lo[3]), acc);
  }
  // acc[i]: head 4kg + i, group n
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) part += wv[i] * fmaxf(acc[i], 0.f);
  part = cross_rows_sum(part);
  if (kg == 0 && g < G) gscore[(size_t)row * G + g] = cnt > 0 ? part : -__builtin_inff();
}

template <bool K8>
static void launch_index_scores_t(const uint16_t* q_idx, const float* w, const KeyCache& k,
                                  const int32_t* n_entries, const int32_t* q_pos, int B, int Q, int Hi,
                                  int cap, const int32_t* gsel, int n_groups_sel, float* scores,
                                  hipStream_t stream) {
  const int rows = B * Q;
  if (gsel) {
    dim3 grid(n_groups_sel, rows);
    index_scores_kernel<CH_GROUP, K8><<<grid, 256, 0, stream>>>(
        q_idx, w, k.bf16, k.codes, k.scales, n_entries, q_pos, Q, Hi, cap, gsel, n_groups_sel,
        n_groups_sel * (CH_GROUP / BLOCK), scores);
  } else if (Q >= 16 && Hi <= 8) {
    // many rows per sequence: up to 64 rows share each key read
    dim3 grid(B * ((Q + ROWS_T - 1) / ROWS_T), (cap + CH_ROWS - 1) / CH_ROWS);
    index_rows_kernel<K8><<<grid, 256, 0, stream>>>(q_idx, w, k.bf16, k.codes, k.scales, n_entries, q_pos,
                                                    Q, Hi, cap, cap / BLOCK, scores);
  } else {
    dim3 grid((cap + CH_FLAT - 1) / CH_FLAT, rows);
    index_scores_kernel<CH_FLAT, K8><<<grid, 256, 0, stream>>>(
        q_idx, w, k.bf16, k.codes, k.scales, n_entries, q_pos, Q, Hi, cap, nullptr, 0, cap / BLOCK, scores);
  }
}

int launch_index_scores(const uint16_t* q_idx, const float* w, const KeyCache& keys,
                        const int32_t* n_entries, const int32_t* q_pos, int B, int Q, int Hi,
                        int cap, const int32_t* gsel, int n_groups_sel, float* scores,
                        hipStream_t stream) {
  if (keys.bf16)
    launch_index_scores_t<false>(q_idx, w, keys, n_entries, q_pos, B, Q, Hi, cap, gsel, n_groups_sel, scores,
                                 stream);
  else
    launch_index_scores_t<true>(q_idx, w, keys, n_entries, q_pos, B, Q, Hi, cap, gsel, n_groups_sel, scores,
                                stream);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_coarse_scores(const uint16_t* q_idx, const float* w, const float* group_sum,
                         const int32_t* n_entries, int B, int Q, int Hi, int cap, float* gscore, hipStream_t stream) {
  const int G = cap / GROUP_ENTRIES;
  if (G < 1) return -4;
  coarse_scores_kernel<<<dim3((G + COARSE_GROUPS_WG - 1) / COARSE_GROUPS_WG, B * Q), 256, 0, stream>>>(
      q_idx, w, group_sum, n_entries, Q, Hi, cap, gscore);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace csa2
