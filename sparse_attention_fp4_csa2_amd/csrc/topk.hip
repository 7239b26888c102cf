// Top-K block selection per query row.
//
// The pages bound the selection at "up to 2,048 blocks of 8" per query
// (observer.broadside.tech card, Key ideas, "CSA2 with three static layer
// modes") and state no tie rule or order.  Rule used: candidates (finite
// scores) ordered by score descending, then block id ascending; keep the first
// min(K, #candidates); emit them ascending by block id, -1 padded, with a count.
//
// One 1024-thread workgroup per row: an exact radix select (11 + 11 + 10 bits)
// over order-preserving 32-bit keys finds the K-th largest key tau, then a
// block-wide scan compacts the ids with key > tau, plus the lowest-id ties at
// tau, in id order.  The keys are read once and stay in registers.
#include "device.h"
#include "launch.h"

namespace csa2 {

namespace {

constexpr int TPB = 1024;

// Exclusive scan of one value per thread across the 1024-thread block.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sbuf, uint32_t* total) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // inclusive scan inside the wave
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sbuf[wv] = x;
  __syncthreads();
  if (t < 64) {
    uint32_t s = t < TPB / 64 ? sbuf[t] : 0u;
    uint32_t inc = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = (uint32_t)__shfl_up((int)inc, o, 64);
      if (t >= o) inc += y;
    }
    if (t < TPB / 64) sbuf[32 + t] = inc - s;     // exclusive wave offsets
    if (t == TPB / 64 - 1) sbuf[63] = inc;         // block total
  }
  __syncthreads();
  const uint32_t res = x - v + sbuf[32 + wv];
  *total = sbuf[63];
  __syncthreads();
  return res;
}

}  // namespace

// Thread t holds the keys of positions [t*C, t*C + C) in registers (C fixed at
// compile time), so the scores are read from memory once.
template <int C>
__global__ __launch_bounds__(TPB) void topk_kernel(const float* __restrict__ scores, int n, int k,
                                                   const int32_t* __restrict__ gsel, int n_gsel,
                                                   int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ count) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sbuf[64];
  __shared__ uint32_t sh_digit, sh_above;
  const int row = blockIdx.x, t = threadIdx.x;
  const float* s = scores + (size_t)row * n;
  const int i0 = t * C;

  uint32_t key[C];
#pragma unroll
  for (int c = 0; c < C; ++c) key[c] = i0 + c < n ? score_key(s[i0 + c]) : 0u;

  uint32_t prefix = 0, kleft = (uint32_t)k;
  bool all = false;          // every candidate is selected
  const int shifts[3] = {21, 10, 0};
  const int nbits[3] = {11, 11, 10};
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass], nb = 1 << nbits[pass];
    const int hi_shift = sh + nbits[pass];          // bits above this digit are decided
    for (int i = t; i < nb; i += TPB) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool match = hi_shift >= 32 ? true : ((key[c] >> hi_shift) == (prefix >> hi_shift));
      if (key[c] != 0u && match) atomicAdd(&hist[(key[c] >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    // suffix counts from the top bin: thread t owns reversed bins 2t, 2t+1
    const int r0 = 2 * t, r1 = 2 * t + 1;
    const uint32_t h0 = r0 < nb ? hist[nb - 1 - r0] : 0u;
    const uint32_t h1 = r1 < nb ? hist[nb - 1 - r1] : 0u;
    uint32_t tot;
    const uint32_t before = block_exclusive_scan(h0 + h1, sbuf, &tot);
    if (pass == 0 && tot <= kleft) { all = true; break; }      // uniform: tot is block-wide
    if (r0 < nb && before < kleft && kleft <= before + h0) { sh_digit = nb - 1 - r0; sh_above = before; }
    if (r1 < nb && before + h0 < kleft && kleft <= before + h0 + h1) {
      sh_digit = nb - 1 - r1; sh_above = before + h0;
    }
    __syncthreads();
    prefix |= sh_digit << sh;
    kleft -= sh_above;
    __syncthreads();
  }
  const uint32_t tau = all ? 0u : prefix;            // select key > tau, plus need_eq ties at tau
  const uint32_t need_eq = all ? 0u : kleft;

  // compaction in id order
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    gt += key[c] > tau;
    eq += (key[c] == tau && tau != 0u);
  }
  uint32_t tot_gt, tot_eq;
  const uint32_t gt_pre = block_exclusive_scan(gt, sbuf, &tot_gt);
  const uint32_t eq_pre = block_exclusive_scan(eq, sbuf, &tot_eq);
  uint32_t pos = gt_pre + min(eq_pre, need_eq);
  uint32_t eq_seen = eq_pre;
  int32_t* out = idx + (size_t)row * k;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    bool sel = key[c] > tau;
    if (!sel && key[c] == tau && tau != 0u) {
      sel = eq_seen < need_eq;
      ++eq_seen;
    }
    if (sel) {
      const int i = i0 + c;
      const int id = gsel ? gsel[(size_t)row * n_gsel + i / 64] * 64 + (i & 63) : i;
      out[pos++] = id;
    }
  }
  const uint32_t total = tot_gt + min(tot_eq, need_eq);
  for (int i = (int)total + t; i < k; i += TPB) out[i] = -1;
  if (t == 0) count[row] = (int32_t)total;
}

int launch_topk(const float* scores, int rows, int n, int k, const int32_t* gsel, int n_gsel,
                int32_t* idx, int32_t* count, hipStream_t stream) {
  const int per = (n + TPB - 1) / TPB;
  if (per <= 1) topk_kernel<1><<<rows, TPB, 0, stream>>>(scores, n, k, gsel, n_gsel, idx, count);
  else if (per <= 4) topk_kernel<4><<<rows, TPB, 0, stream>>>(scores, n, k, gsel, n_gsel, idx, count);
  else if (per <= 8) topk_kernel<8><<<rows, TPB, 0, stream>>>(scores, n, k, gsel, n_gsel, idx, count);
  else if (per <= 16) topk_kernel<16><<<rows, TPB, 0, stream>>>(scores, n, k, gsel, n_gsel, idx, count);
  else topk_kernel<64><<<rows, TPB, 0, stream>>>(scores, n, k, gsel, n_gsel, idx, count);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace csa2
