// Internal launch entry points (host side of each .hip translation unit).
// Arguments are validated by the C-ABI layer before these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

int launch_append(const uint16_t* latent, const uint16_t* idx_key, const int32_t* start_entry,
                  int B, int n_new, int cap, uint8_t* cache, uint16_t* key_cache,
                  float* group_sum, hipStream_t stream);

// MXFP8 indexer keys (append.hip): E4M3 codes [B][cap][64] + E8M0 scales
// [B][cap][2], with the latent's records in the same launch when latent is
// not null; group sums (optional) of the dequantised keys
int launch_append_key8(const uint16_t* latent, const uint16_t* idx_key, const int32_t* start_entry, int B,
                       int n_new, int cap, uint8_t* cache, uint8_t* key8, uint8_t* key8_scale, float* group_sum,
                       hipStream_t stream);

// Indexer keys: bf16 [B][cap][64] (bf16 != nullptr) or MXFP8 (codes, scales).
struct KeyCache {
  const uint16_t* bf16;
  const uint8_t* codes;
  const uint8_t* scales;
};

// csa2_index_topk / _key8 after their pointer checks: argument checks against
// the sizes, workspace carving and the launches; returns a CSA2 status.
int index_topk_run(const uint16_t* q_idx, const float* w, const KeyCache& keys, const float* group_sum,
                   const int32_t* n_entries, const int32_t* q_pos, int B, int Q, int Hi, int cap, int top_k,
                   int top_groups, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);

// Block scores fp32 [rows][n_out]: flat (gsel == nullptr: n_out = cap/8) or
// restricted to the selected groups gsel [rows][n_groups_sel] (n_out = 64 per group).
int launch_index_scores(const uint16_t* q_idx, const float* w, const KeyCache& keys,
                        const int32_t* n_entries, const int32_t* q_pos, int B, int Q, int Hi,
                        int cap, const int32_t* gsel, int n_groups_sel, float* scores,
                        hipStream_t stream);

// Coarse scores of the two-level indexer: the score of every group from its
// group sums -> gscore [rows][cap / 512] (-inf for groups with no entry).
int launch_coarse_scores(const uint16_t* q_idx, const float* w, const float* group_sum,
                         const int32_t* n_entries, int B, int Q, int Hi, int cap, float* gscore, hipStream_t stream);

// Top-k per row of scores [rows][n] -> idx [rows][k] ascending, -1 padded, count [rows].
// With gsel != nullptr, position p maps to block gsel[row][p / 64] * 64 + p % 64.
int launch_topk(const float* scores, int rows, int n, int k, const int32_t* gsel, int n_gsel,
                int32_t* idx, int32_t* count, hipStream_t stream);

struct AttnParams {
  const uint16_t* q;        // [rows][H][512]
  // MXFP4 source
  const uint8_t* cache;     // [B][cap/8][2176]
  const int32_t* idx;       // [rows][top_k]
  const int32_t* count;     // [rows]
  const int32_t* n_entries; // [B]
  int top_k, cap;
  // bf16 window source
  const uint16_t* swa;      // [B][Lw][512]
  const int32_t* swa_len;   // [B]
  const int32_t* swa_pos0;  // [B] or null
  int W, Lw;
  // common
  const int32_t* q_pos;     // [rows] or null
  int Q, H, rows, splits;
  float scale_log2;         // scale * log2(e)
  // output: either the final fp32 o (o_out, one split) or split-K partials:
  // o16_out fp16 [rows][H][out_splits][512] with o = o16 * 2^oexp_out per
  // (row, split, head), so the partials take half the bytes of fp32
  float* o_out;             // [rows][H][512] final o, or null
  uint16_t* o16_out;        // [rows][H][out_splits][512] partial o, or null
  int32_t* oexp_out;        // [rows][H][out_splits] power-of-two exponent of o16_out
  float* lse_out;           // [rows][H][out_splits] (one split: the final [rows][H])
  int out_splits;           // split stride of the outputs (>= split_base + splits)
  int split_base;           // this launch writes splits [split_base, split_base + splits)
};

// bf16 window (attention.hip): 32-head workgroups, few tiles per row
int window_splits(int rows, int H, int n_tiles);
// split count of a window launch over B sequences of Q rows (row tiles as in the sparse kernel)
int window_attn_splits(int B, int Q, int H, int W);
int launch_window(const AttnParams& p, hipStream_t stream);
// MXFP4 selected blocks (sparse_fp4.hip): 32-head workgroups, two per CU
int sparse_fp4_splits(int rows, int H, int n_tiles, int stage);   // stage: block ids a split stages
// rows per tile (1, 2 or 4: with 16 or fewer heads, rows of a sequence share
// the tile's columns and its gathers) and the split count of a sparse launch
int sparse_rows_per_tile(int H, int Q);
int sparse_attn_splits(int B, int Q, int H, int top_k);
int launch_sparse_fp4(const AttnParams& p, hipStream_t stream);
// Both branches of a layer in one launch (sparse_fp4.hip); each writes its own
// partial splits.  inline_window: every sparse workgroup also runs the window
// split of its own index (needs pw.splits <= ps.splits, same rows and heads);
// otherwise the window's workgroups follow the sparse ones in the grid.
int launch_attend(const AttnParams& ps, const AttnParams& pw, bool inline_window, hipStream_t stream);

// Merge split partials (fp16 o, exponent, lse; and an optional fp32 extra
// branch) -> out [rows][H][512], lse [rows][H].
int launch_combine(const uint16_t* o16, const int32_t* oexp, const float* lse_part, int rows,
                   int splits, int H, const float* o_ext, const float* lse_ext, float* out,
                   float* lse_out, hipStream_t stream);

}  // namespace csa2
