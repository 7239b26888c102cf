// Radix top-K selection core shared by the top-K kernels (a row of keys held
// in registers by one workgroup).  The rule, and how the passes run, are
// described in topk.hip.
#pragma once
#include "device.h"
#include <type_traits>

namespace csa2 {
namespace sel {


constexpr int HIST_BINS = 2048;
constexpr uint32_t RANK_MAX = 256;   // a boundary bin this small is ranked directly

// Wave-wide inclusive prefix sum: four DPP row shifts (1, 2, 4, 8) within each
// 16-lane row, then row broadcasts of lane 15 and lane 31.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
  return x;
}

// Exclusive scan of one value per thread across the block; *total = block sum.
template <int TPB>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sbuf, uint32_t* total) {
  constexpr int NW = TPB / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sbuf[wv] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = sbuf[w];
    off += w < wv ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}


// Two exclusive scans across the block in one pass (one pair of barriers).
template <int TPB>
__device__ __forceinline__ void block_excl_scan2(uint32_t v0, uint32_t v1, uint32_t (*sbuf2)[2], uint32_t* pre0,
                                                 uint32_t* pre1, uint32_t* tot0, uint32_t* tot1) {
  constexpr int NW = TPB / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t inc0 = wave_incl_scan(v0), inc1 = wave_incl_scan(v1);
  if (lane == 63) sbuf2[wv][0] = inc0, sbuf2[wv][1] = inc1;
  __syncthreads();
  uint32_t o0 = 0, o1 = 0, t0 = 0, t1 = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x0 = sbuf2[w][0], x1 = sbuf2[w][1];
    o0 += w < wv ? x0 : 0u;
    o1 += w < wv ? x1 : 0u;
    t0 += x0;
    t1 += x1;
  }
  __syncthreads();
  *pre0 = o0 + inc0 - v0;
  *pre1 = o1 + inc1 - v1;
  *tot0 = t0;
  *tot1 = t1;
}

// Selects the k largest of the row's keys (key[c] = score_key of position
// threadIdx.x * C + c, 0 = not a candidate) and writes their positions --
// mapped through gsel when given -- ascending to out (k slots, -1 padded) and
// their number to *count_out.  Every thread of the TPB-thread block must call it.
template <int TPB, int C, bool RANGE>
__device__ __forceinline__ void select_core(uint32_t (&key)[C], int n, int k, const int32_t* __restrict__ gsel,
                                            int n_gsel, int row, int32_t* __restrict__ out,
                                            int32_t* __restrict__ count_out) {
  constexpr int NW = TPB / 64;
  constexpr int BPT = HIST_BINS / TPB;      // histogram bins scanned per thread
  __shared__ uint32_t hist[HIST_BINS];
  __shared__ uint32_t sbuf[NW];
  __shared__ uint32_t sred[NW][5];
  __shared__ uint32_t sh_digit, sh_above, sh_cnt;
  __shared__ __align__(16) uint32_t rk_key[RANK_MAX];
  __shared__ uint32_t rk_n, sh_tau, sh_need;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int i0 = t * C;
  if (t == 0) rk_n = 0;
  // a thread's C keys lie in one 64-wide slice (C divides 64), so its group id
  // (two-level selection) is one load, issued before the passes
  static_assert(64 % C == 0, "a thread's keys must share one group");
  const int gid = (gsel != nullptr && i0 < n) ? gsel[(size_t)row * n_gsel + i0 / 64] : 0;

  bool all = false;               // every candidate is kept (block-uniform)
  bool ranked = false;            // tau and its tie count are in sh_tau, sh_need
  uint32_t prefix = 0, kleft = (uint32_t)k;
  int pos = 32;
  if constexpr (RANGE) {
    // candidate count and key range of the row, and the same over the
    // candidates scoring >= 0 (keys >= 0x80000000)
    uint32_t kmin = 0xffffffffu, kmax = 0u, nv = 0, kmin_nn = 0xffffffffu, n_nn = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      // selects, not branches (0 = not a candidate)
      const uint32_t x = key[c];
      const bool cand = x != 0u, nn = x >= 0x80000000u;
      kmin = min(kmin, cand ? x : 0xffffffffu);
      kmax = max(kmax, x);
      nv += cand ? 1u : 0u;
      kmin_nn = min(kmin_nn, nn ? x : 0xffffffffu);
      n_nn += nn ? 1u : 0u;
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    nv = wave_sum_u32(nv);
    kmin_nn = wave_min_u32(kmin_nn);
    n_nn = wave_sum_u32(n_nn);
    if (lane == 0) sred[wv][0] = kmin, sred[wv][1] = kmax, sred[wv][2] = nv, sred[wv][3] = kmin_nn,
                   sred[wv][4] = n_nn;
    __syncthreads();
    kmin = 0xffffffffu, kmax = 0u, nv = 0, kmin_nn = 0xffffffffu, n_nn = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      kmin = min(kmin, sred[w][0]);
      kmax = max(kmax, sred[w][1]);
      nv += sred[w][2];
      kmin_nn = min(kmin_nn, sred[w][3]);
      n_nn += sred[w][4];
    }
    all = nv <= (uint32_t)k;
    // with at least k candidates scoring >= 0 the k-th lies among them, so the
    // digits need only span their range: a row whose scores take both signs
    // otherwise covers the whole key space, and its first pass is coarse.  Keys
    // below the range can never be kept and count as non-candidates from here.
    if (!all && n_nn >= (uint32_t)k) kmin = kmin_nn;
    // from here on key[c] holds x = key - kmin + 1 for a candidate at or above
    // kmin (no wrap: kmin >= 1), 0 otherwise
#pragma unroll
    for (int c = 0; c < C; ++c) key[c] = key[c] >= kmin ? key[c] - kmin + 1u : 0u;
    pos = all ? 0 : 32 - __clz(kmax - kmin + 1u);
  }

  // radix select on x (x = key without RANGE), from bit pos - 1 down
#pragma unroll 1
  while (pos > 0) {
    const int sh = pos > 11 ? pos - 11 : 0;
    const int nb = 1 << (pos - sh);
    const uint32_t hmask = pos >= 32 ? 0u : (~0u << pos);   // bits already decided
    for (int i = t; i < nb; i += TPB) hist[i] = 0;
    for (int i = t; i < (int)RANK_MAX; i += TPB) rk_key[i] = 0;   // the rank step reads 4 at a time
    __syncthreads();
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint32_t x = key[c];
      if (x && (x & hmask) == prefix) atomicAdd(&hist[(x >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    // thread t owns the reversed bins BPT*t .. BPT*t + BPT - 1 (counted from the top)
    uint32_t h[BPT], hs = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int r = BPT * t + j;
      h[j] = r < nb ? hist[nb - 1 - r] : 0u;
      hs += h[j];
    }
    uint32_t tot;
    uint32_t before = block_excl_scan<TPB>(hs, sbuf, &tot);
    if (!RANGE && pos == 32 && tot <= kleft) {      // at most k candidates
      all = true;
      break;
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int r = BPT * t + j;
      if (r < nb && before < kleft && kleft <= before + h[j])
        sh_digit = nb - 1 - r, sh_above = before, sh_cnt = h[j];
      before += h[j];
    }
    __syncthreads();
    prefix |= sh_digit << sh;
    kleft -= sh_above;
    pos = sh;
    if (pos > 0 && sh_cnt <= RANK_MAX) {
      // rank step: the keys of the boundary bin go to LDS; lane j of wave 0
      // counts the keys above and at its own key, and the lane whose key is the
      // kleft-th largest of the bin publishes it (tau) and how many of its
      // equal keys are kept
      const uint32_t m2 = ~0u << pos;
      // one slot reservation per thread for all of its keys in the bin
      uint32_t nin = 0;
#pragma unroll
      for (int c = 0; c < C; ++c) nin += (key[c] && (key[c] & m2) == prefix) ? 1u : 0u;
      if (nin) {
        uint32_t slot = atomicAdd(&rk_n, nin);
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (key[c] && (key[c] & m2) == prefix) rk_key[slot++] = key[c];
      }
      __syncthreads();
      const uint32_t cnt = rk_n;
      if (cnt <= 64) {
        // one wave: lane j holds key j and reads the others from its neighbours
        if (wv == 0) {
          const uint32_t kj = (uint32_t)lane < cnt ? rk_key[lane] : 0u;
          uint32_t gt = 0, ge = 0;
          for (uint32_t i = 0; i < cnt; ++i) {
            const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)kj, (int)i);
            gt += ki > kj;
            ge += ki >= kj;
          }
          if ((uint32_t)lane < cnt && gt < kleft && kleft <= ge) sh_tau = kj, sh_need = kleft - gt;
        }
      } else {
        // thread t ranks key t of the bin against all of them (4-key LDS reads
        // every thread makes at the same address); equal keys publish the same
        // tau and count
        if ((uint32_t)t < cnt) {
          const uint32_t kj = rk_key[t];
          uint32_t gt = 0, ge = 0;
          const uint4* rk4 = reinterpret_cast<const uint4*>(rk_key);
          for (uint32_t i = 0; i < (cnt + 3) / 4; ++i) {
            const uint4 v = rk4[i];          // slots past cnt hold 0: never counted
            gt += (v.x > kj) + (v.y > kj) + (v.z > kj) + (v.w > kj);
            ge += (v.x >= kj) + (v.y >= kj) + (v.z >= kj) + (v.w >= kj);
          }
          if (gt < kleft && kleft <= ge) sh_tau = kj, sh_need = kleft - gt;
        }
      }
      __syncthreads();
      ranked = true;
      break;
    }
    if (pos > 0) {
      // a large boundary bin: its key range places the next digits (the bits
      // its keys share are skipped), or, when all its keys are equal, is tau
      const uint32_t m2 = ~0u << pos;
      uint32_t bmin = 0xffffffffu, bmax = 0u;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t x = key[c];
        if (x && (x & m2) == prefix) bmin = min(bmin, x), bmax = max(bmax, x);
      }
      bmin = wave_min_u32(bmin);
      bmax = wave_max_u32(bmax);
      if (lane == 0) sred[wv][0] = bmin, sred[wv][1] = bmax;
      __syncthreads();
      bmin = 0xffffffffu, bmax = 0u;
#pragma unroll
      for (int w = 0; w < NW; ++w) bmin = min(bmin, sred[w][0]), bmax = max(bmax, sred[w][1]);
      if (bmin == bmax) {
        if (t == 0) sh_tau = bmin, sh_need = kleft;
        __syncthreads();
        ranked = true;
        break;
      }
      pos = 32 - __clz(bmin ^ bmax);
      prefix = pos >= 32 ? 0u : (bmin & (~0u << pos));
    }
  }
  // keep x > tau, plus the first need_eq candidates (in id order) with x == tau;
  // tau >= 1 unless every candidate is kept, when tau = 0 keeps all x >= 1
  const uint32_t tau = all ? 0u : ranked ? sh_tau : prefix;
  const uint32_t need_eq = all ? 0u : ranked ? sh_need : kleft;

  // per-thread bit masks of the keys above tau and at tau (bit c = position i0 + c)
  typedef typename std::conditional<(C > 32), unsigned long long, uint32_t>::type mask_t;
  mask_t gtm = 0, eqm = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    gtm |= (mask_t)(key[c] > tau) << c;
    eqm |= (mask_t)(key[c] == tau) << c;
  }
  const uint32_t gt = (uint32_t)__builtin_popcountll((unsigned long long)gtm);
  const uint32_t eq = (uint32_t)__builtin_popcountll((unsigned long long)eqm);
  __shared__ uint32_t sbuf2[NW][2];
  uint32_t tot_gt, tot_eq, gt_pre, eq_pre;
  block_excl_scan2<TPB>(gt, eq, sbuf2, &gt_pre, &eq_pre, &tot_gt, &tot_eq);
  // of this thread's keys at tau, the lowest-position ones that the earlier
  // threads' ties leave room for are kept (counted up with compares only: a
  // clamped need_eq - eq_pre was folded into an unclamped subtract that also
  // stood in for min(eq_pre, need_eq) below)
  mask_t sel = gtm;
  uint32_t eq_seen = eq_pre;
  for (mask_t m = eqm; m != 0 && eq_seen < need_eq; m &= m - 1, ++eq_seen) sel |= m & (~m + 1);
  // ascending positions: the set bits from the lowest up
  uint32_t pos_out = gt_pre + min(eq_pre, need_eq);
  for (mask_t m = sel; m != 0; m &= m - 1) {
    const int c = __builtin_ctzll((unsigned long long)m);
    const int i = i0 + c;
    out[pos_out++] = gsel ? gid * 64 + (i & 63) : i;
  }
  const uint32_t total = tot_gt + min(tot_eq, need_eq);
  for (int i = (int)total + t; i < k; i += TPB) out[i] = -1;
  if (t == 0) *count_out = (int32_t)total;
}

}  // namespace sel
}  // namespace csa2
