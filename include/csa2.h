/*
 * csa2.h -- C ABI of the CSA2 sparse-decode attention library for MI355X (gfx950).
 *
 * The operation: compressed sparse attention over an FP4 global latent cache.
 * One 512-d latent per compressed entry is the key and the value for every
 * query head; each entry merges two adjacent raw positions (paper-digest.app,
 * "DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache Compression", Core
 * Mechanics, "Compressed along three axes").  An indexer selects up to 2048
 * blocks of 8 entries per query, every layer also attends its own sliding
 * window, and layers run in Full / Reindex / Reuse modes
 * (observer.broadside.tech card, same title, Key ideas, "CSA2 with three static
 * layer modes").  The cache is stored in FP4 (news.promptgoblins.ai, "DeepSeek
 * Releases V4.1 Flash with 4x KV Cache Compression ...", Details, "FP4 KVCache
 * precision"); the concrete format here is MXFP4 (OCP Microscaling v1.0:
 * E2M1 codes, one E8M0 scale per 32 values).
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers unless stated.  The caller owns
 *    every buffer, including workspaces sized by the *_ws() queries; the
 *    library allocates nothing and keeps no state, and calls are re-entrant.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; nothing is synchronised.
 *  - bfloat16 arrays are passed as uint16_t bit patterns.
 *  - Return value: CSA2_OK (0) or a negative status; argument checks run on
 *    the host before anything is enqueued, so on error nothing was launched.
 *    No exception or abort crosses the ABI.  Device data is not validated:
 *    block ids outside [0, cap/8) (e.g. the -1 padding) are skipped in-kernel.
 *
 * Byte layouts (fixed by this header):
 *  - Latent cache, per sequence: cap/8 block records of CSA2_RECORD_BYTES.
 *    Record of block b (entries 8b..8b+7): bytes [0,2048) = the 8 entries'
 *    packed codes, entry-major, 256 B each (byte k: code of dim 2k in the low
 *    nibble, dim 2k+1 in the high nibble; code = sign<<3 | E2M1 magnitude
 *    code); bytes [2048,2176) = the 8 entries' 16 E8M0 scale bytes,
 *    entry-major (scale g covers dims 32g..32g+31).
 *  - Indexer keys: bf16 [B][cap][64].  Group sums: fp32 [B][cap/512][64].
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_D 512              /* latent width (K = V)                     */
#define CSA2_DI 64              /* indexer key / query width                */
#define CSA2_BLOCK 8            /* entries per selection block              */
#define CSA2_GROUP_BLOCKS 64    /* blocks per coarse group (two-level)      */
#define CSA2_RECORD_BYTES 2176  /* bytes per block record                   */
#define CSA2_MAX_HEADS 128      /* attention heads per row                  */
#define CSA2_MAX_INDEX_HEADS 16 /* indexer heads                            */

enum {
    CSA2_OK = 0,
    CSA2_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misaligned buffer   */
    CSA2_ERR_UNSUPPORTED = -2,   /* valid but not supported by these kernels    */
    CSA2_ERR_WS_TOO_SMALL = -3,  /* workspace smaller than the *_ws() query      */
    CSA2_ERR_LAUNCH = -4,        /* the HIP runtime reported a launch error      */
    CSA2_ERR_SCRATCH_LIMIT = -5  /* needs more than a static scratch array holds */
};

/* Append n_new entries per sequence to the latent cache (MXFP4 quantise + pack).
 * Defined by: the global cache held in FP4 (news.promptgoblins.ai, Details,
 * "FP4 KVCache precision"; thelatestinai.com, Abstract), one entry per merged
 * pair of raw positions (paper-digest.app, Core Mechanics, "Compressed along
 * three axes"); the FP4 format is this library's choice, OCP MXFP4.
 * Encoding per 32-value group: amax = max |x|; sb = clamp(floor(log2 amax) - 2
 * + 127, 0, 254) (amax = 0 -> 0); codes = |x| / 2^(sb-127) rounded to the E2M1
 * grid {0,.5,1,1.5,2,3,4,6} to nearest, halfway cases to the even code, above 6
 * saturating; sign bit copied (also for zero magnitudes).  A group holding a
 * NaN/Inf gets sb = 255 and zero codes.
 *   latent      bf16 [B][n_new][512]
 *   idx_key     bf16 [B][n_new][64] or NULL; copied to key_cache when given
 *   start_entry int32 [B] (device): entry position of each sequence's first
 *               new entry; entries at positions >= cap are dropped
 *   cache       u8 [B][cap/8][2176]; key_cache bf16 [B][cap][64] or NULL
 *   group_sum   fp32 [B][cap/512][64] or NULL (needs idx_key and cap % 512 ==
 *               0): every 512-entry group the call writes into is recomputed
 *               as the sum of the keys its 512 key_cache slots hold after the
 *               call (slots holding no entry must be zero, as in a
 *               zero-initialised cache), so an overwritten entry counts once,
 *               with its new key.  The sum is formed in fp64 and rounded once
 *               to fp32: exact up to that rounding for keys of ordinary range.
 * Bytes of records not covered by new entries are left untouched.  Errors:
 * CSA2_ERR_INVALID_ARG for a null latent / start_entry / cache, bad sizes,
 * 16-byte misalignment, or idx_key without key_cache (or the reverse). */
int csa2_append_fp4(const uint16_t* latent, const uint16_t* idx_key, const int32_t* start_entry,
                    int B, int n_new, int cap, uint8_t* cache, uint16_t* key_cache,
                    float* group_sum, void* stream);

/* Indexer + top-K block selection for B*Q query rows.
 * Defined by: the sparse indexer that picks up to 2048 blocks of 8 entries per
 * query, rescored per layer in Reindex mode, two-level ("hierarchical") to trim
 * decoder indexing (observer.broadside.tech card, Key ideas, "CSA2 with three
 * static layer modes").  The pages print no score formula; the one below is
 * this library's reading.
 * Entry score e_j = sum_h w_h * max(0, q_h . k_j) (fp32 accumulation); block
 * score = max over the block's present (j < n_entries[b]) and visible entries;
 * a block with none is not a candidate.  Visibility: with q_pos, entry j is
 * visible to raw position t iff 2j+1 <= t; without, all present entries are.
 * Keeps the top_k candidates by (score desc, block id asc) and writes them
 * ascending, padded with -1, plus their count.
 * Two-level (top_groups > 0, needs group_sum, q_pos == NULL): group g = blocks
 * [64g, 64g+64) scores its mean key (group_sum / present count, formed in fp32
 * and taken into the scoring MFMA as bf16 hi + lo: about 16 significant bits);
 * the best top_groups groups are kept, and blocks are scored only inside them.
 *   q_idx bf16 [B][Q][Hi][64]; w fp32 [B][Q][Hi]; key_cache bf16 [B][cap][64]
 *   n_entries int32 [B]; q_pos int32 [B][Q] or NULL
 *   idx int32 [B][Q][top_k]; count int32 [B][Q]
 *   ws: >= csa2_index_topk_ws(B, Q, cap, top_groups) bytes, 256-B aligned */
int csa2_index_topk(const uint16_t* q_idx, const float* w, const uint16_t* key_cache,
                    const float* group_sum, const int32_t* n_entries, const int32_t* q_pos,
                    int B, int Q, int Hi, int cap, int top_k, int top_groups,
                    int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);
size_t csa2_index_topk_ws(int B, int Q, int cap, int top_groups);

/* csa2_index_topk for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, rule, outputs and errors as csa2_index_topk, without ws /
 * ws_bytes: the selection's scratch is a static device array of
 * CSA2_INDEX_SCRATCH_BYTES per GPU (held until the process ends), and the call
 * allocates nothing.  A call whose csa2_index_topk_ws(B, Q, cap, top_groups)
 * exceeds it returns CSA2_ERR_SCRATCH_LIMIT before anything is enqueued (8 MiB
 * covers 2M block scores: every decode workload here; a 4096-row prefill does
 * not fit).  The scratch used is the current device's (the stream must belong
 * to it); nothing in it needs clearing between calls.  Calls that overlap on one
 * GPU (other streams, or unordered host threads) share that scratch and race:
 * order them. */
#define CSA2_INDEX_SCRATCH_BYTES ((size_t)8 << 20)
int csa2_index_topk_noalloc(const uint16_t* q_idx, const float* w, const uint16_t* key_cache,
                            const float* group_sum, const int32_t* n_entries, const int32_t* q_pos,
                            int B, int Q, int Hi, int cap, int top_k, int top_groups,
                            int32_t* idx, int32_t* count, void* stream);

/* Lower-precision indexer key cache: the keys in MXFP8 (OCP Microscaling
 * v1.0, E4M3 elements -- bias 7, subnormals, largest finite 448, no
 * infinities -- with one E8M0 scale per 32 dims), half the bytes of bf16.
 * The pages give the indexer no precision (observer.broadside.tech card, Key
 * ideas, "CSA2 with three static layer modes"); the latent stays MXFP4.
 * Encoding of a 32-dim group x: sb = clamp(floor(log2 max|x|) - 8 + 127, 0,
 * 254) (0 for an all-zero group), code = sign<<7 | E4M3 magnitude of
 * |x| / 2^(sb-127) rounded to nearest, ties to the even code, above 448
 * saturating to 448 (0x7E).
 *
 * csa2_append_key8: quantises n_new new keys per sequence (bf16 idx_key
 * [B][n_new][64]) into entries start_entry[b] .. of key8 u8 [B][cap][64]
 * (byte d = dim d; 16-B aligned) and key8_scale u8 [B][cap][2] (byte g for
 * dims 32g..32g+31; 4-B aligned), and, when group_sum fp32 [B][cap/512][64] is
 * not NULL (cap % 512 == 0), recomputes every group it writes into as the sum
 * of the dequantised keys its 512 slots hold, as csa2_append_fp4 does.  With latent
 * and cache (both or neither) it also writes the latent's MXFP4 records as
 * csa2_append_fp4 does, in the same launch.  Entries at or beyond cap are
 * skipped.
 *
 * csa2_index_topk_key8: csa2_index_topk on such a cache (the scores use the
 * dequantised keys, exact in bf16, against the bf16 query); same outputs,
 * workspace (csa2_index_topk_ws) and errors. */
int csa2_append_key8(const uint16_t* latent, const uint16_t* idx_key, const int32_t* start_entry, int B,
                     int n_new, int cap, uint8_t* cache, uint8_t* key8, uint8_t* key8_scale, float* group_sum,
                     void* stream);
int csa2_index_topk_key8(const uint16_t* q_idx, const float* w, const uint8_t* key8,
                         const uint8_t* key8_scale, const float* group_sum, const int32_t* n_entries,
                         const int32_t* q_pos, int B, int Q, int Hi, int cap, int top_k, int top_groups,
                         int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);

/* Top-K of precomputed scores (the selection step of csa2_index_topk).
 * scores fp32 [rows][n]; -inf or NaN marks a non-candidate.  Same rule and
 * output format as csa2_index_topk: idx int32 [rows][k] ascending, -1 padded;
 * count int32 [rows].  n <= 65536. */
int csa2_topk(const float* scores, int rows, int n, int k, int32_t* idx, int32_t* count,
              void* stream);

/* Sparse multi-head attention over the selected blocks of the latent cache.
 * Defined by: one 512-d latent per entry is the key and the value of every
 * query head (paper-digest.app, Core Mechanics, "Compressed along three
 * axes"), attended over the selected blocks only (observer.broadside.tech
 * card, Key ideas, "CSA2 with three static layer modes").
 * For each row r = (b, q) and head h: z_j = scale * (q_h . V_j) over the
 * present, visible entries j of the blocks idx[r][0..count[r]); V_j = the
 * dequantised entry; o = softmax(z) V (fp32), lse = log sum exp z.  An empty
 * selection gives o = 0, lse = -inf.  q . K runs on the scaled FP4 x FP6 MFMA
 * (each 32-dim block of the query split into three E2M3 terms that carry it to
 * within 2^-11.9 of the block's largest value, fp32 accumulation); a wave whose
 * query blocks spread too far for that (fewer than half of a block's values
 * within 2^5 of its largest) runs q . K on bf16 MFMAs instead, with the codes
 * dequantised to bf16 (exact) against the bf16 query.  The softmax weights are
 * rounded to fp16 before the value product with V in fp16.
 * With 16 or fewer heads (one GPU's share of heads split across GPUs) and
 * Q >= 2, 2 (H <= 16) or 4 (H <= 8) consecutive rows of a sequence share each
 * attention tile: the tile attends the union of their selections, every block
 * gathered and dequantised once for all of them, and each row still sees only
 * its own blocks, count and causal limit (the results are those of one row
 * at a time, up to rounding order; a row that lists a block twice counts it
 * twice, as it does alone).
 *   q bf16 [B][Q][H][512]; cache as above; idx int32 [B][Q][top_k];
 *   count int32 [B][Q]; n_entries int32 [B]; q_pos int32 [B][Q] or NULL
 *   o fp32 [B][Q][H][512]; lse fp32 [B][Q][H] (natural log)
 *   ws: >= csa2_sparse_attn_ws(B, Q, H, top_k) bytes (split-K partials) */
int csa2_sparse_attn(const uint16_t* q, const uint8_t* cache, const int32_t* idx,
                     const int32_t* count, const int32_t* n_entries, const int32_t* q_pos,
                     int B, int Q, int H, int cap, int top_k, float scale,
                     float* o, float* lse, void* ws, size_t ws_bytes, void* stream);
size_t csa2_sparse_attn_ws(int B, int Q, int H, int top_k);

/* Sliding-window branch and log-sum-exp merge with the sparse branch.
 * Defined by: every layer keeps its own query and sliding-window KV
 * (observer.broadside.tech card, Key ideas, "CSA2 with three static layer
 * modes"; the window is named in the paper-digest.app Terminology); the merge
 * is the log-sum-exp combination of the two branches.  Beyond the four-call
 * outline, this call also takes swa_pos0 (raw position of slot 0, so causal
 * rows can sit inside the window) and a workspace for its split-K partials.
 * Window slot i of sequence b holds raw position swa_pos0[b] + i (swa_pos0
 * NULL = 0), for i < swa_len[b] <= Lw.  The query at raw position t (q_pos, or
 * NULL = the newest held token) attends positions [t-W+1, t] that are held.
 * Branch (o_w, lse_w) is computed as in csa2_sparse_attn (K = V = bf16
 * window tokens), then out = e^(lse_s-L) o_s + e^(lse_w-L) o_w with
 * L = logaddexp(lse_s, lse_w) (both -inf: out = 0, L = -inf).
 *   swa_kv bf16 [B][Lw][512]; o_sparse/out fp32 [B][Q][H][512] (may alias);
 *   lse_sparse/lse_out fp32 [B][Q][H] (may alias)
 *   ws: >= csa2_swa_merge_ws(B, Q, H, W) bytes */
int csa2_swa_merge(const uint16_t* q, const uint16_t* swa_kv, const int32_t* swa_len,
                   const int32_t* swa_pos0, const int32_t* q_pos, int B, int Q, int H, int W,
                   int Lw, float scale, const float* o_sparse, const float* lse_sparse,
                   float* out, float* lse_out, void* ws, size_t ws_bytes, void* stream);
size_t csa2_swa_merge_ws(int B, int Q, int H, int W);

/* One attention layer in a single call: the sparse branch of csa2_sparse_attn
 * and the window branch of csa2_swa_merge, merged by log-sum-exp (which is one
 * softmax over the selected entries and the window tokens together).  Both
 * branches run in one launch and write split-K partials into ws (where a
 * workgroup runs a window split after its sparse split, it continues the same
 * softmax and leaves one partial for both), then one combine pass produces
 * out / lse_out; with a single partial per (row, head) the launch writes
 * out / lse_out itself and no combine runs.  No intermediate sparse-only
 * output exists.  Arguments as in the two calls above (q_pos also fixes the
 * window, swa_pos0 NULL = 0).
 *   out fp32 [B][Q][H][512]; lse_out fp32 [B][Q][H]
 *   ws: >= csa2_attend_layer_ws(B, Q, H, top_k, W) bytes */
int csa2_attend_layer(const uint16_t* q, const uint8_t* cache, const int32_t* idx,
                      const int32_t* count, const int32_t* n_entries, const int32_t* q_pos,
                      const uint16_t* swa_kv, const int32_t* swa_len, const int32_t* swa_pos0,
                      int B, int Q, int H, int cap, int top_k, int W, int Lw, float scale,
                      float* out, float* lse_out, void* ws, size_t ws_bytes, void* stream);
size_t csa2_attend_layer_ws(int B, int Q, int H, int top_k, int W);
/* Kernel launches csa2_attend_layer makes for these sizes (1 or 2; 0 for
 * invalid sizes): a report for callers that count launches per layer. */
int csa2_attend_layer_launches(int B, int Q, int H, int top_k, int W);

/* csa2_attend_layer in two phases, so that the window branch -- which needs no
 * selection -- can run on a second stream while the indexer and top-K run.
 * The results are identical to csa2_attend_layer's (same kernels, same split
 * slots in ws).
 * Phase 1, csa2_attend_layer_window: the window branch's split-K partials into
 * ws (a workspace of csa2_attend_layer_ws(B, Q, H, top_k, W) bytes).
 * Phase 2, csa2_attend_layer_sparse: the sparse branch's partials into the same
 * ws, then the combine of both into out / lse_out.  Phase 1 on the same ws must
 * be complete before phase 2 starts on its stream: the caller orders them
 * (same stream, or an event recorded after phase 1 and waited on by phase 2's
 * stream).  Phase 2 must also complete before phase 1 of a later call reuses
 * ws.  Arguments as in csa2_attend_layer; top_k and W must match between the
 * two phases (they fix the split layout of ws). */
int csa2_attend_layer_window(const uint16_t* q, const uint16_t* swa_kv, const int32_t* swa_len,
                             const int32_t* swa_pos0, const int32_t* q_pos, int B, int Q, int H,
                             int top_k, int W, int Lw, float scale, void* ws, size_t ws_bytes,
                             void* stream);
int csa2_attend_layer_sparse(const uint16_t* q, const uint8_t* cache, const int32_t* idx,
                             const int32_t* count, const int32_t* n_entries, const int32_t* q_pos,
                             int B, int Q, int H, int cap, int top_k, int W, float scale,
                             float* out, float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* Human-readable name of a status code (static string, host). */
const char* csa2_status_str(int status);
/* Library version: major * 10000 + minor * 100 + patch. */
int csa2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
