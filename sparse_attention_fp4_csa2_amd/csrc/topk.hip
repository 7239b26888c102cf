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
// key; once the bin holding it has at most 1024 keys, those keys go to LDS and
// are ranked directly (one wave for up to 64, else every thread takes its share
// of the bin and counts the keys above it) instead of running further passes:
// rows whose scores span both signs cover the whole 32-bit key range, where
// the first 2048-bin pass leaves a few hundred keys with the K-th.  A larger
// bin's own key range places the next pass's digits (skipping the bits all its
// keys share), and a bin of equal keys ends the search (planted blocks of equal
// score pile up there).  Then a block-wide scan compacts the ids with key >
// tau, plus the lowest-id ties at tau, in id order.
#include "device.h"
#include "launch.h"
#include "select.h"

namespace csa2 {

// RANGE: digits relative to the row's key range (min/max reduction first);
// otherwise fixed digits from bit 31 (11 + 11 + 10 bits), which skips the
// reduction (short rows).
template <int TPB, int C, bool RANGE>
__global__ __launch_bounds__(TPB) void topk_kernel(const float* __restrict__ scores, int n, int k, int vec,
                                                   const int32_t* __restrict__ gsel, int n_gsel,
                                                   int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ count) {
  const int row = blockIdx.x, t = threadIdx.x;
  const float* s = scores + (size_t)row * n;
  const int i0 = t * C;

  // one decision per thread, so a full thread's vector loads are all in flight
  // before the first is used (a per-chunk branch waits on each in turn)
  uint32_t key[C];
  if (C >= 4 && vec && i0 + C <= n) {
    float4 v[C / 4 > 0 ? C / 4 : 1];
#pragma unroll
    for (int c = 0; c < C / 4; ++c) v[c] = reinterpret_cast<const float4*>(s + i0)[c];
#pragma unroll
    for (int c = 0; c < C / 4; ++c) {
      key[4 * c] = score_key(v[c].x), key[4 * c + 1] = score_key(v[c].y);
      key[4 * c + 2] = score_key(v[c].z), key[4 * c + 3] = score_key(v[c].w);
    }
  } else {
    float v[C];
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = i0 + c < n ? s[i0 + c] : -__builtin_inff();
#pragma unroll
    for (int c = 0; c < C; ++c) key[c] = score_key(v[c]);
  }

  sel::select_core<TPB, C, RANGE>(key, n, k, gsel, n_gsel, row, idx + (size_t)row * k, count + row);
}

// n <= 65536.  Rows of up to 1024 scores run on 256 threads, 4 scores each:
// with fixed digits (one short pass) when rows are many, with range-relative
// digits when they are too few to fill the chip (8 rows of 1024 coarse group
// scores, whose few exponents crowd fixed digits into a handful of bins; one
// score per thread on 1024 threads took 5.4 us there, 4 on 256 take 4.6 us).
// Longer rows use range-relative digits, on 256 threads, or on 512-1024 when
// rows are few (there one row's latency is the cost: 32 rows of 4096 scores
// 8.4 -> 7.4 us on 512 threads).
int launch_topk(const float* scores, int rows, int n, int k, const int32_t* gsel, int n_gsel,
                int32_t* idx, int32_t* count, hipStream_t stream) {
  const int vec = (n % 4 == 0) && (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
#define CSA2_TOPK(T, C, R) \
  topk_kernel<T, C, R><<<rows, T, 0, stream>>>(scores, n, k, vec, gsel, n_gsel, idx, count)
  if (n <= 1024 && rows < 128) CSA2_TOPK(256, 4, true);
  else if (n <= 256 * 4) CSA2_TOPK(256, 4, false);
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
