// csa2_index_topk without a caller workspace: for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The selection's scratch -- block scores,
// and for the two-level indexer the group scores and the kept groups -- lives
// in a file-scope device array of CSA2_INDEX_SCRATCH_BYTES, one copy per GPU,
// held until the process ends.  Nothing in it needs clearing between calls:
// every score the top-K reads is written by the scoring kernel of the same
// call first.  All calls on one GPU share that GPU's copy, so calls that
// overlap on one GPU (different streams, or threads without ordering) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/csa2.h"
#include "launch.h"

namespace {

constexpr size_t SCRATCH_BYTES = CSA2_INDEX_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_lock;
void* g_scratch[MAX_DEVICES];    // device address of `scratch` on each GPU, once looked up

// The current device's copy of `scratch` (looked up once per device, with that
// device current).  The name `scratch` is a host-side stand-in in host code:
// only this address may reach a kernel or a copy.
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return CSA2_ERR_LAUNCH;
  std::lock_guard<std::mutex> hold(g_lock);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CSA2_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CSA2_OK;
}

}  // namespace

extern "C" int csa2_index_topk_noalloc(const uint16_t* q_idx, const float* w, const uint16_t* key_cache,
                                       const float* group_sum, const int32_t* n_entries, const int32_t* q_pos,
                                       int B, int Q, int Hi, int cap, int top_k, int top_groups, int32_t* idx,
                                       int32_t* count, void* stream) {
  if (!key_cache) return CSA2_ERR_INVALID_ARG;
  if ((uintptr_t)key_cache % 16 != 0) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || Q <= 0 || cap <= 0 || top_groups < 0) return CSA2_ERR_INVALID_ARG;
  if (csa2_index_topk_ws(B, Q, cap, top_groups) > SCRATCH_BYTES) return CSA2_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const int rc = scratch_for_current_device(&ws);
  if (rc != CSA2_OK) return rc;
  const csa2::KeyCache keys{key_cache, nullptr, nullptr};
  return csa2::index_topk_run(q_idx, w, keys, group_sum, n_entries, q_pos, B, Q, Hi, cap, top_k, top_groups,
                              idx, count, ws, SCRATCH_BYTES, stream);
}
