// Top-K block selection per query row.
//
// The pages bound the selection at "up to 2,048 blocks of 8" per query
// (observer.broadside.tech card, Key ideas, "CSA2 with three static layer
// modes") and state no tie rule or order.  Rule used: candidates (finite
// scores) ordered by score descending, then block id ascending; keep the first
// min(K, #candidates); emit them ascending by block id, -1 padded, with a count.
//
// One workgroup per row, keys read once into registers (C per thread, fixed at
// compile time).  Exact radix select on order-preserving 32-bit keys, taken
// relative to the row's smallest candidate key lo: the digits of key - lo + 1
// start at the top bit of max - lo + 1, so the first 2048-bin histogram spreads
// over the range the row's scores actually occupy (a fixed top-11-bit digit
// puts a typical row into a handful of bins, and the LDS atomics on those few
// bins serialise).  Each pass fixes up to 11 more bits of the K-th largest
// key; once the bin holding it has at most 64 keys, those keys go to LDS and
// one wave ranks them directly instead of running further passes.  A larger
// bin's own key range places the next pass's digits (skipping the bits all its
// keys share), and a bin of equal keys ends the search (planted blocks of equal
// score pile up there).  Then a block-wide scan compacts the ids with key >
// tau, plus the lowest-id ties at tau, in id order.
#include "device.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int HIST_BINS = 2048;
constexpr uint32_t RANK_MAX = 64;   // a boundary bin this small is ranked directly

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

}  // namespace

// RANGE: digits relative to the row's key range (min/max reduction first);
// otherwise fixed digits from bit 31 (11 + 11 + 10 bits), which skips the
// reduction (short rows).
template <int TPB, int C, bool RANGE>
__global__ __launch_bounds__(TPB) void topk_kernel(const float* __restrict__ scores, int n, int k, int vec,
                                                   const int32_t* __restrict__ gsel, int n_gsel,
                                                   int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ count) {
  constexpr int NW = TPB / 64;
  constexpr int BPT = HIST_BINS / TPB;      // histogram bins scanned per thread
  __shared__ uint32_t hist[HIST_BINS];
  __shared__ uint32_t sbuf[NW];
  __shared__ uint32_t sred[NW][3];
  __shared__ uint32_t sh_digit, sh_above, sh_cnt;
  __shared__ uint32_t rk_key[RANK_MAX], rk_n, sh_tau, sh_need;
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const float* s = scores + (size_t)row * n;
  const int i0 = t * C;
  if (t == 0) rk_n = 0;

  uint32_t key[C];
#pragma unroll
  for (int c = 0; c < C; c += 4) {
    if (vec && i0 + c + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(s + i0 + c);
      key[c] = score_key(v.x), key[c + 1] = score_key(v.y);
      key[c + 2] = score_key(v.z), key[c + 3] = score_key(v.w);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) key[c + j] = i0 + c + j < n ? score_key(s[i0 + c + j]) : 0u;
    }
  }

  bool all = false;               // every candidate is kept (block-uniform)
  bool ranked = false;            // tau and its tie count are in sh_tau, sh_need
  uint32_t prefix = 0, kleft = (uint32_t)k;
  int pos = 32;
  if constexpr (RANGE) {
    // candidate count and key range of the row
    uint32_t kmin = 0xffffffffu, kmax = 0u, nv = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (key[c]) {
        kmin = min(kmin, key[c]);
        kmax = max(kmax, key[c]);
        ++nv;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
      nv += (uint32_t)__shfl_xor((int)nv, o, 64);
    }
    if (lane == 0) sred[wv][0] = kmin, sred[wv][1] = kmax, sred[wv][2] = nv;
    __syncthreads();
    kmin = 0xffffffffu, kmax = 0u, nv = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      kmin = min(kmin, sred[w][0]);
      kmax = max(kmax, sred[w][1]);
      nv += sred[w][2];
    }
    all = nv <= (uint32_t)k;
    // from here on key[c] holds x = key - kmin + 1 for a candidate (no wrap:
    // kmin >= 1), 0 for a non-candidate
#pragma unroll
    for (int c = 0; c < C; ++c) key[c] = key[c] ? key[c] - kmin + 1u : 0u;
    pos = all ? 0 : 32 - __clz(kmax - kmin + 1u);
  }

  // radix select on x (x = key without RANGE), from bit pos - 1 down
#pragma unroll 1
  while (pos > 0) {
    const int sh = pos > 11 ? pos - 11 : 0;
    const int nb = 1 << (pos - sh);
    const uint32_t hmask = pos >= 32 ? 0u : (~0u << pos);   // bits already decided
    for (int i = t; i < nb; i += TPB) hist[i] = 0;
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
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t x = key[c];
        if (x && (x & m2) == prefix) rk_key[atomicAdd(&rk_n, 1u)] = x;
      }
      __syncthreads();
      if (wv == 0) {
        const uint32_t cnt = rk_n;
        const uint32_t kj = (uint32_t)lane < cnt ? rk_key[lane] : 0u;
        uint32_t gt = 0, ge = 0;
        for (uint32_t i = 0; i < cnt; ++i) {
          const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)kj, (int)i);
          gt += ki > kj;
          ge += ki >= kj;
        }
        if ((uint32_t)lane < cnt && gt < kleft && kleft <= ge) sh_tau = kj, sh_need = kleft - gt;
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
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        bmin = min(bmin, (uint32_t)__shfl_xor((int)bmin, o, 64));
        bmax = max(bmax, (uint32_t)__shfl_xor((int)bmax, o, 64));
      }
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

  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    gt += key[c] > tau;
    eq += key[c] == tau;
  }
  uint32_t tot_gt, tot_eq;
  const uint32_t gt_pre = block_excl_scan<TPB>(gt, sbuf, &tot_gt);
  const uint32_t eq_pre = block_excl_scan<TPB>(eq, sbuf, &tot_eq);
  uint32_t pos_out = gt_pre + min(eq_pre, need_eq);
  uint32_t eq_seen = eq_pre;
  int32_t* out = idx + (size_t)row * k;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    bool sel = key[c] > tau;
    if (key[c] == tau) {
      sel = eq_seen < need_eq;
      ++eq_seen;
    }
    if (sel) {
      const int i = i0 + c;
      const int id = gsel ? gsel[(size_t)row * n_gsel + i / 64] * 64 + (i & 63) : i;
      out[pos_out++] = id;
    }
  }
  const uint32_t total = tot_gt + min(tot_eq, need_eq);
  for (int i = (int)total + t; i < k; i += TPB) out[i] = -1;
  if (t == 0) count[row] = (int32_t)total;
}

// n <= 65536.  Rows of up to 1024 scores run on 256 threads with fixed digits
// (one short pass); longer ones use range-relative digits, on 256 threads, or
// on 512-1024 when there are too few rows to fill the chip (there one row's
// latency is the cost: 32 rows of 4096 scores 8.4 -> 7.4 us on 512 threads).
int launch_topk(const float* scores, int rows, int n, int k, const int32_t* gsel, int n_gsel,
                int32_t* idx, int32_t* count, hipStream_t stream) {
  const int vec = (n % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
#define CSA2_TOPK(T, C, R) \
  topk_kernel<T, C, R><<<rows, T, 0, stream>>>(scores, n, k, vec, gsel, n_gsel, idx, count)
  if (n <= 256 * 4) CSA2_TOPK(256, 4, false);
  else if (n <= 512 * 8 && rows < 128) CSA2_TOPK(512, 8, true);
  else if (n <= 256 * 16) CSA2_TOPK(256, 16, true);
  else if (n <= 256 * 32) CSA2_TOPK(256, 32, true);
  else if (n <= 256 * 64 && rows >= 128) CSA2_TOPK(256, 64, true);
  else if (n <= 1024 * 16) CSA2_TOPK(1024, 16, true);
  else CSA2_TOPK(1024, 64, true);
#undef CSA2_TOPK
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace csa2
