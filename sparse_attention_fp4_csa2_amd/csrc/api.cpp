// C ABI of the CSA2 sparse-decode library: argument checks, workspace
// carving, and kernel launch sequencing.  Every check runs on the host before
// anything is enqueued; the library allocates nothing and keeps no state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa2.h"
#include "launch.h"

using namespace csa2;

namespace {

constexpr size_t WS_ALIGN = 256;

inline size_t align_up(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int launch_status(int rc) { return rc == 0 ? CSA2_OK : CSA2_ERR_LAUNCH; }

// Index/top-K workspace pieces.
struct IndexWs {
  size_t scores;      // fp32 [rows][n_score]
  size_t gscore;      // fp32 [rows][cap / 512]
  size_t gsel;        // int32 [rows][top_groups]
  size_t gcount;      // int32 [rows]
  size_t total;
};

IndexWs index_ws_layout(int B, int Q, int cap, int top_groups) {
  const size_t rows = (size_t)B * Q;
  IndexWs l{};
  const size_t n_score = top_groups > 0 ? (size_t)top_groups * CSA2_GROUP_BLOCKS : (size_t)cap / CSA2_BLOCK;
  size_t off = 0;
  l.scores = off; off += align_up(rows * n_score * sizeof(float));
  if (top_groups > 0) {
    l.gscore = off; off += align_up(rows * ((size_t)cap / 512) * sizeof(float));
    l.gsel = off; off += align_up(rows * (size_t)top_groups * sizeof(int32_t));
    l.gcount = off; off += align_up(rows * sizeof(int32_t));
  }
  l.total = off;
  return l;
}

// Split-K partials of the attention calls: fp16 o [rows][H][splits][512],
// int32 exponent and fp32 lse [rows][H][splits] (a (row, head)'s splits adjacent).
struct PartWs {
  size_t o16, oexp, lse, total;
};

PartWs part_ws_layout(int rows, int splits, int H) {
  const size_t n = (size_t)rows * splits * H;
  PartWs l{};
  size_t off = 0;
  l.o16 = off; off += align_up(n * CSA2_D * sizeof(uint16_t));
  l.oexp = off; off += align_up(n * sizeof(int32_t));
  l.lse = off; off += align_up(n * sizeof(float));
  l.total = off;
  return l;
}

// point p's split outputs at the partial buffers in ws
void set_partials(AttnParams& p, void* ws, const PartWs& l, int out_splits, int split_base) {
  char* base = static_cast<char*>(ws);
  p.o_out = nullptr;
  p.o16_out = reinterpret_cast<uint16_t*>(base + l.o16);
  p.oexp_out = reinterpret_cast<int32_t*>(base + l.oexp);
  p.lse_out = reinterpret_cast<float*>(base + l.lse);
  p.out_splits = out_splits;
  p.split_base = split_base;
}

int combine_partials(void* ws, const PartWs& l, int rows, int splits, int H, const float* o_ext,
                     const float* lse_ext, float* out, float* lse_out, hipStream_t st) {
  char* base = static_cast<char*>(ws);
  return launch_combine(reinterpret_cast<const uint16_t*>(base + l.o16),
                        reinterpret_cast<const int32_t*>(base + l.oexp),
                        reinterpret_cast<const float*>(base + l.lse), rows, splits, H, o_ext, lse_ext,
                        out, lse_out, st);
}

}  // namespace

extern "C" {

const char* csa2_status_str(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported configuration";
    case CSA2_ERR_WS_TOO_SMALL: return "workspace too small";
    case CSA2_ERR_LAUNCH: return "kernel launch failed";
    case CSA2_ERR_SCRATCH_LIMIT: return "request exceeds the static scratch";
    default: return "unknown status";
  }
}

int csa2_version(void) { return 10000; }

int csa2_append_fp4(const uint16_t* latent, const uint16_t* idx_key, const int32_t* start_entry,
                    int B, int n_new, int cap, uint8_t* cache, uint16_t* key_cache,
                    float* group_sum, void* stream) {
  if (!latent || !start_entry || !cache) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || n_new < 0 || cap <= 0 || cap % CSA2_BLOCK != 0) return CSA2_ERR_INVALID_ARG;
  if (!aligned(latent, 16) || !aligned(cache, 16)) return CSA2_ERR_INVALID_ARG;
  if ((idx_key == nullptr) != (key_cache == nullptr)) return CSA2_ERR_INVALID_ARG;
  if (idx_key && (!aligned(idx_key, 16) || !aligned(key_cache, 16))) return CSA2_ERR_INVALID_ARG;
  if (group_sum) {
    if (!idx_key) return CSA2_ERR_INVALID_ARG;
    if (cap % 512 != 0) return CSA2_ERR_UNSUPPORTED;
    if (!aligned(group_sum, 16)) return CSA2_ERR_INVALID_ARG;
  }
  if (n_new == 0) return CSA2_OK;
  return launch_status(launch_append(latent, idx_key, start_entry, B, n_new, cap, cache, key_cache,
                                     group_sum, as_stream(stream)));
}

size_t csa2_index_topk_ws(int B, int Q, int cap, int top_groups) {
  if (B <= 0 || Q <= 0 || cap <= 0) return 0;
  return index_ws_layout(B, Q, cap, top_groups).total;
}

}  // extern "C"

// The selection behind csa2_index_topk(_key8) and the no-allocation variant:
// argument checks, workspace carving, launches.
int csa2::index_topk_run(const uint16_t* q_idx, const float* w, const KeyCache& keys,
                      const float* group_sum, const int32_t* n_entries, const int32_t* q_pos,
                      int B, int Q, int Hi, int cap, int top_k, int top_groups,
                      int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  if (!q_idx || !w || !n_entries || !idx || !count) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || Q <= 0 || Hi <= 0 || cap <= 0 || top_k <= 0 || top_groups < 0)
    return CSA2_ERR_INVALID_ARG;
  if (cap % CSA2_BLOCK != 0 || top_k > cap / CSA2_BLOCK) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q_idx, 16)) return CSA2_ERR_INVALID_ARG;
  if (Hi > CSA2_MAX_INDEX_HEADS) return CSA2_ERR_UNSUPPORTED;
  if ((size_t)cap / CSA2_BLOCK > 65536) return CSA2_ERR_UNSUPPORTED;
  const IndexWs l = index_ws_layout(B, Q, cap, top_groups);
  if (!ws || ws_bytes < l.total) return CSA2_ERR_WS_TOO_SMALL;
  if (!aligned(ws, WS_ALIGN)) return CSA2_ERR_INVALID_ARG;
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + l.scores);
  hipStream_t st = as_stream(stream);
  const int rows = B * Q;
  if (top_groups == 0) {
    int rc = launch_index_scores(q_idx, w, keys, n_entries, q_pos, B, Q, Hi, cap, nullptr, 0, scores, st);
    if (rc) return CSA2_ERR_LAUNCH;
    return launch_status(launch_topk(scores, rows, cap / CSA2_BLOCK, top_k, nullptr, 0, idx, count, st));
  }
  // two-level
  if (!group_sum || q_pos) return CSA2_ERR_UNSUPPORTED;
  if (cap % 512 != 0) return CSA2_ERR_UNSUPPORTED;
  const int G = cap / 512;
  if (top_groups > G) return CSA2_ERR_INVALID_ARG;
  if ((size_t)top_groups * CSA2_GROUP_BLOCKS > 65536) return CSA2_ERR_UNSUPPORTED;
  int32_t* gsel = reinterpret_cast<int32_t*>(base + l.gsel);
  int32_t* gcount = reinterpret_cast<int32_t*>(base + l.gcount);
  float* gscore = reinterpret_cast<float*>(base + l.gscore);
  int rc = launch_coarse_scores(q_idx, w, group_sum, n_entries, B, Q, Hi, cap, gscore, st);
  if (!rc) rc = launch_topk(gscore, rows, G, top_groups, nullptr, 0, gsel, gcount, st);
  if (!rc) rc = launch_index_scores(q_idx, w, keys, n_entries, nullptr, B, Q, Hi, cap, gsel, top_groups,
                                    scores, st);
  if (!rc) rc = launch_topk(scores, rows, top_groups * CSA2_GROUP_BLOCKS, top_k, gsel, top_groups,
                            idx, count, st);
  return launch_status(rc);
}

extern "C" {

int csa2_index_topk(const uint16_t* q_idx, const float* w, const uint16_t* key_cache,
                    const float* group_sum, const int32_t* n_entries, const int32_t* q_pos,
                    int B, int Q, int Hi, int cap, int top_k, int top_groups,
                    int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  if (!key_cache) return CSA2_ERR_INVALID_ARG;
  if (!aligned(key_cache, 16)) return CSA2_ERR_INVALID_ARG;
  const KeyCache keys{key_cache, nullptr, nullptr};
  return csa2::index_topk_run(q_idx, w, keys, group_sum, n_entries, q_pos, B, Q, Hi, cap, top_k, top_groups,
                              idx, count, ws, ws_bytes, stream);
}

int csa2_index_topk_key8(const uint16_t* q_idx, const float* w, const uint8_t* key8,
                         const uint8_t* key8_scale, const float* group_sum, const int32_t* n_entries,
                         const int32_t* q_pos, int B, int Q, int Hi, int cap, int top_k, int top_groups,
                         int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  if (!key8 || !key8_scale) return CSA2_ERR_INVALID_ARG;
  if (!aligned(key8, 16) || !aligned(key8_scale, 4)) return CSA2_ERR_INVALID_ARG;
  const KeyCache keys{nullptr, key8, key8_scale};
  return csa2::index_topk_run(q_idx, w, keys, group_sum, n_entries, q_pos, B, Q, Hi, cap, top_k, top_groups,
                              idx, count, ws, ws_bytes, stream);
}

int csa2_append_key8(const uint16_t* latent, const uint16_t* idx_key, const int32_t* start_entry, int B,
                     int n_new, int cap, uint8_t* cache, uint8_t* key8, uint8_t* key8_scale, float* group_sum,
                     void* stream) {
  if (!idx_key || !start_entry || !key8 || !key8_scale) return CSA2_ERR_INVALID_ARG;
  if ((latent == nullptr) != (cache == nullptr)) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || n_new < 0 || cap <= 0 || cap % CSA2_BLOCK != 0) return CSA2_ERR_INVALID_ARG;
  if (!aligned(key8, 16) || !aligned(key8_scale, 4)) return CSA2_ERR_INVALID_ARG;
  if (latent && (!aligned(latent, 16) || !aligned(cache, 16))) return CSA2_ERR_INVALID_ARG;
  if (group_sum) {
    if (cap % 512 != 0) return CSA2_ERR_UNSUPPORTED;
    if (!aligned(group_sum, 16)) return CSA2_ERR_INVALID_ARG;
  }
  if (n_new == 0) return CSA2_OK;
  return launch_status(launch_append_key8(latent, idx_key, start_entry, B, n_new, cap, cache, key8, key8_scale,
                                          group_sum, as_stream(stream)));
}

int csa2_topk(const float* scores, int rows, int n, int k, int32_t* idx, int32_t* count,
              void* stream) {
  if (!scores || !idx || !count) return CSA2_ERR_INVALID_ARG;
  if (rows <= 0 || n <= 0 || k <= 0) return CSA2_ERR_INVALID_ARG;
  if (n > 65536) return CSA2_ERR_UNSUPPORTED;
  return launch_status(launch_topk(scores, rows, n, k, nullptr, 0, idx, count, as_stream(stream)));
}

size_t csa2_sparse_attn_ws(int B, int Q, int H, int top_k) {
  if (B <= 0 || Q <= 0 || H <= 0 || top_k <= 0) return 0;
  const int rows = B * Q;
  const int s = sparse_attn_splits(B, Q, H, top_k);
  if (s <= 1) return 0;
  return part_ws_layout(rows, s, H).total;
}

int csa2_sparse_attn(const uint16_t* q, const uint8_t* cache, const int32_t* idx,
                     const int32_t* count, const int32_t* n_entries, const int32_t* q_pos,
                     int B, int Q, int H, int cap, int top_k, float scale,
                     float* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !cache || !idx || !count || !n_entries || !o || !lse) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || Q <= 0 || H <= 0 || cap <= 0 || top_k <= 0) return CSA2_ERR_INVALID_ARG;
  if (cap % CSA2_BLOCK != 0 || !(scale > 0.f) || !isfinite(scale)) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(o, 16)) return CSA2_ERR_INVALID_ARG;
  if (H > CSA2_MAX_HEADS) return CSA2_ERR_UNSUPPORTED;
  if ((size_t)cap / CSA2_BLOCK * CSA2_RECORD_BYTES > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
  const int rows = B * Q;
  const int splits = sparse_attn_splits(B, Q, H, top_k);
  const size_t need = csa2_sparse_attn_ws(B, Q, H, top_k);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WS_TOO_SMALL;
  if (need > 0 && !aligned(ws, WS_ALIGN)) return CSA2_ERR_INVALID_ARG;
  AttnParams p{};
  p.q = q; p.cache = cache; p.idx = idx; p.count = count; p.n_entries = n_entries;
  p.top_k = top_k; p.cap = cap; p.q_pos = q_pos; p.Q = Q; p.H = H; p.rows = rows;
  p.splits = splits;
  p.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t st = as_stream(stream);
  if (splits == 1) {
    p.o_out = o; p.lse_out = lse; p.out_splits = 1; p.split_base = 0;
    return launch_status(launch_sparse_fp4(p, st));
  }
  const PartWs l = part_ws_layout(rows, splits, H);
  set_partials(p, ws, l, splits, 0);
  int rc = launch_sparse_fp4(p, st);
  if (!rc) rc = combine_partials(ws, l, rows, splits, H, nullptr, nullptr, o, lse, st);
  return launch_status(rc);
}

size_t csa2_swa_merge_ws(int B, int Q, int H, int W) {
  if (B <= 0 || Q <= 0 || H <= 0 || W <= 0) return 0;
  const int rows = B * Q;
  const int s = window_attn_splits(B, Q, H, W);
  return part_ws_layout(rows, s, H).total;
}

int csa2_swa_merge(const uint16_t* q, const uint16_t* swa_kv, const int32_t* swa_len,
                   const int32_t* swa_pos0, const int32_t* q_pos, int B, int Q, int H, int W,
                   int Lw, float scale, const float* o_sparse, const float* lse_sparse,
                   float* out, float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !swa_kv || !swa_len || !o_sparse || !lse_sparse || !out || !lse_out)
    return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || Q <= 0 || H <= 0 || W <= 0 || Lw <= 0) return CSA2_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(swa_kv, 16) || !aligned(o_sparse, 16) || !aligned(out, 16))
    return CSA2_ERR_INVALID_ARG;
  if (H > CSA2_MAX_HEADS) return CSA2_ERR_UNSUPPORTED;
  const size_t need = csa2_swa_merge_ws(B, Q, H, W);
  if (!ws || ws_bytes < need) return CSA2_ERR_WS_TOO_SMALL;
  if (!aligned(ws, WS_ALIGN)) return CSA2_ERR_INVALID_ARG;
  const int rows = B * Q;
  const int splits = window_attn_splits(B, Q, H, W);
  AttnParams p{};
  p.q = q; p.swa = swa_kv; p.swa_len = swa_len; p.swa_pos0 = swa_pos0; p.W = W; p.Lw = Lw;
  p.q_pos = q_pos; p.Q = Q; p.H = H; p.rows = rows; p.splits = splits;
  p.scale_log2 = scale * 1.4426950408889634f;
  const PartWs l = part_ws_layout(rows, splits, H);
  set_partials(p, ws, l, splits, 0);
  hipStream_t st = as_stream(stream);
  int rc = launch_window(p, st);
  if (!rc) rc = combine_partials(ws, l, rows, splits, H, o_sparse, lse_sparse, out, lse_out, st);
  return launch_status(rc);
}

// Window splits of a layer, shared by csa2_attend_layer and its two phases so
// that they write one split layout.  The window runs inside the sparse
// workgroups of the one launch (split s of each row and head group in the
// sparse workgroup of split s) when the sparse branch has at least one split
// per window tile (few rows: 8 decode rows over 1M-entry caches take 32
// sparse splits; measured there 36.4 -> 34.3 us) or when the window's own
// workgroups would each run more than 8 tiles, a long tail after the sparse
// ones (128 rows of 4 per sequence: 334.6 -> 326.5 us).  Otherwise it keeps
// its own split count and workgroups after the sparse ones: inline it cost
// up to ~1 us more there, plus a combine over more splits.
static bool layer_window_inline(int rows, int Q, int H, int s_sparse, int W) {
  // row tiles: the window on the same tiles, half the work of its own 32-head workgroups
  if (sparse_rows_per_tile(H, Q) > 1) return true;
  const int wt = (W + 31) / 32;
  const int s_own = window_splits(rows, H, wt);
  return s_sparse >= wt || (wt + s_own - 1) / s_own > 8;
}
static int layer_window_splits(int rows, int Q, int H, int s_sparse, int W) {
  const int wt = (W + 31) / 32;
  return layer_window_inline(rows, Q, H, s_sparse, W) ? (s_sparse < wt ? s_sparse : wt) : window_splits(rows, H, wt);
}

int csa2_attend_layer_launches(int B, int Q, int H, int top_k, int W) {
  if (B <= 0 || Q <= 0 || H <= 0 || top_k <= 0 || W <= 0) return 0;
  const int rows = B * Q;
  const int s_sparse = sparse_attn_splits(B, Q, H, top_k);
  return layer_window_inline(rows, Q, H, s_sparse, W) && s_sparse == 1 ? 1 : 2;
}

size_t csa2_attend_layer_ws(int B, int Q, int H, int top_k, int W) {
  if (B <= 0 || Q <= 0 || H <= 0 || top_k <= 0 || W <= 0) return 0;
  const int rows = B * Q;
  const int s_sparse = sparse_attn_splits(B, Q, H, top_k);
  return part_ws_layout(rows, s_sparse + layer_window_splits(rows, Q, H, s_sparse, W), H).total;
}

int csa2_attend_layer_window(const uint16_t* q, const uint16_t* swa_kv, const int32_t* swa_len,
                             const int32_t* swa_pos0, const int32_t* q_pos, int B, int Q, int H,
                             int top_k, int W, int Lw, float scale, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!q || !swa_kv || !swa_len) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || Q <= 0 || H <= 0 || top_k <= 0 || W <= 0 || Lw <= 0) return CSA2_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(swa_kv, 16)) return CSA2_ERR_INVALID_ARG;
  if (H > CSA2_MAX_HEADS) return CSA2_ERR_UNSUPPORTED;
  const size_t need = csa2_attend_layer_ws(B, Q, H, top_k, W);
  if (!ws || ws_bytes < need) return CSA2_ERR_WS_TOO_SMALL;
  if (!aligned(ws, WS_ALIGN)) return CSA2_ERR_INVALID_ARG;
  const int rows = B * Q;
  const int s_sparse = sparse_attn_splits(B, Q, H, top_k);
  const int s_window = layer_window_splits(rows, Q, H, s_sparse, W);
  const int total = s_sparse + s_window;
  if (total > 128) return CSA2_ERR_UNSUPPORTED;
  AttnParams pw{};
  pw.q = q; pw.swa = swa_kv; pw.swa_len = swa_len; pw.swa_pos0 = swa_pos0; pw.W = W; pw.Lw = Lw;
  pw.q_pos = q_pos; pw.Q = Q; pw.H = H; pw.rows = rows;
  pw.scale_log2 = scale * 1.4426950408889634f;
  pw.splits = s_window;
  set_partials(pw, ws, part_ws_layout(rows, total, H), total, s_sparse);
  return launch_status(launch_window(pw, as_stream(stream)));
}

int csa2_attend_layer_sparse(const uint16_t* q, const uint8_t* cache, const int32_t* idx,
                             const int32_t* count, const int32_t* n_entries, const int32_t* q_pos,
                             int B, int Q, int H, int cap, int top_k, int W, float scale,
                             float* out, float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !cache || !idx || !count || !n_entries || !out || !lse_out) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || Q <= 0 || H <= 0 || cap <= 0 || top_k <= 0 || W <= 0) return CSA2_ERR_INVALID_ARG;
  if (cap % CSA2_BLOCK != 0 || !(scale > 0.f) || !isfinite(scale)) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16)) return CSA2_ERR_INVALID_ARG;
  if (H > CSA2_MAX_HEADS) return CSA2_ERR_UNSUPPORTED;
  if ((size_t)cap / CSA2_BLOCK * CSA2_RECORD_BYTES > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
  const size_t need = csa2_attend_layer_ws(B, Q, H, top_k, W);
  if (!ws || ws_bytes < need) return CSA2_ERR_WS_TOO_SMALL;
  if (!aligned(ws, WS_ALIGN)) return CSA2_ERR_INVALID_ARG;
  const int rows = B * Q;
  const int s_sparse = sparse_attn_splits(B, Q, H, top_k);
  const int s_window = layer_window_splits(rows, Q, H, s_sparse, W);
  const int total = s_sparse + s_window;
  if (total > 128) return CSA2_ERR_UNSUPPORTED;
  const PartWs l = part_ws_layout(rows, total, H);
  hipStream_t st = as_stream(stream);
  AttnParams p{};
  p.q = q; p.cache = cache; p.idx = idx; p.count = count; p.n_entries = n_entries;
  p.top_k = top_k; p.cap = cap; p.q_pos = q_pos; p.Q = Q; p.H = H; p.rows = rows;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.splits = s_sparse;
  set_partials(p, ws, l, total, 0);
  int rc = launch_sparse_fp4(p, st);
  if (!rc) rc = combine_partials(ws, l, rows, total, H, nullptr, nullptr, out, lse_out, st);
  return launch_status(rc);
}

int csa2_attend_layer(const uint16_t* q, const uint8_t* cache, const int32_t* idx,
                      const int32_t* count, const int32_t* n_entries, const int32_t* q_pos,
                      const uint16_t* swa_kv, const int32_t* swa_len, const int32_t* swa_pos0,
                      int B, int Q, int H, int cap, int top_k, int W, int Lw, float scale,
                      float* out, float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !cache || !idx || !count || !n_entries || !swa_kv || !swa_len || !out || !lse_out)
    return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || Q <= 0 || H <= 0 || cap <= 0 || top_k <= 0 || W <= 0 || Lw <= 0)
    return CSA2_ERR_INVALID_ARG;
  if (cap % CSA2_BLOCK != 0 || !(scale > 0.f) || !isfinite(scale)) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(swa_kv, 16) || !aligned(out, 16))
    return CSA2_ERR_INVALID_ARG;
  if (H > CSA2_MAX_HEADS) return CSA2_ERR_UNSUPPORTED;
  if ((size_t)cap / CSA2_BLOCK * CSA2_RECORD_BYTES > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
  const size_t need = csa2_attend_layer_ws(B, Q, H, top_k, W);
  if (!ws || ws_bytes < need) return CSA2_ERR_WS_TOO_SMALL;
  if (!aligned(ws, WS_ALIGN)) return CSA2_ERR_INVALID_ARG;
  const int rows = B * Q;
  const int s_sparse = sparse_attn_splits(B, Q, H, top_k);
  const int s_window = layer_window_splits(rows, Q, H, s_sparse, W);
  const bool inl = layer_window_inline(rows, Q, H, s_sparse, W);
  // inline: sparse split s also runs window split s on the same softmax state,
  // so the layer leaves s_sparse partials (with one split, the output itself);
  // otherwise sparse -> splits [0, s_sparse), window -> [s_sparse, total)
  const int total = inl ? s_sparse : s_sparse + s_window;
  if (s_sparse + s_window > 128) return CSA2_ERR_UNSUPPORTED;
  const PartWs l = part_ws_layout(rows, total, H);
  hipStream_t st = as_stream(stream);
  AttnParams p{};
  p.q = q; p.cache = cache; p.idx = idx; p.count = count; p.n_entries = n_entries;
  p.top_k = top_k; p.cap = cap; p.q_pos = q_pos; p.Q = Q; p.H = H; p.rows = rows;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.splits = s_sparse;
  if (total == 1) {
    p.o_out = out; p.lse_out = lse_out; p.out_splits = 1; p.split_base = 0;
  } else {
    set_partials(p, ws, l, total, 0);
  }
  AttnParams pw = p;
  pw.cache = nullptr; pw.idx = nullptr; pw.count = nullptr; pw.n_entries = nullptr;
  pw.swa = swa_kv; pw.swa_len = swa_len; pw.swa_pos0 = swa_pos0; pw.W = W; pw.Lw = Lw;
  pw.splits = s_window; pw.split_base = s_sparse;
  int rc = launch_attend(p, pw, inl, st);   // both branches in one launch
  if (!rc && total > 1) rc = combine_partials(ws, l, rows, total, H, nullptr, nullptr, out, lse_out, st);
  return launch_status(rc);
}

}  // extern "C"
