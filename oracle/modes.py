"""Cross-layer modes and one decode row of the whole path (oracle; test infrastructure).

The pages define three static layer modes ([card] Key ideas, "CSA2 with three
static layer modes"):
  Full    -- the layer makes the global KV and indexes it;
  Reindex -- the layer reuses an earlier layer's KV but rescores it with its own
             indexer query;
  Reuse   -- the layer reuses both the KV and the earlier layer's top-K indices.
Every layer keeps its own attention query and its own sliding-window KV.

Here a "row" is one query token of one sequence.  ``select_blocks`` is the
indexer + top-K step (flat, or two-level when ``top_groups`` is given);
``attend_row`` is sparse attention + window branch + merge.
"""

import numpy as np

from . import attention, indexer, topk


def select_blocks(q_idx, w, keys, n_entries, k, q_pos=None, top_groups=None, n_blocks=None):
    """Indexer + top-K for one row -> (idx int32 [k], count).

    Flat: block scores over every block.  Two-level: coarse group scores, keep the
    top ``top_groups`` groups, score only their blocks, then top-K among those.
    """
    keys = np.asarray(keys)
    nb = n_blocks if n_blocks is not None else (keys.shape[0] + indexer.BLOCK - 1) // indexer.BLOCK
    if not top_groups:
        s = indexer.block_scores(q_idx, w, keys, n_entries, q_pos, n_blocks=nb)
        return topk.select(s, k)
    n_groups = (nb + indexer.GROUP_BLOCKS - 1) // indexer.GROUP_BLOCKS
    gs = indexer.group_scores(q_idx, w, keys, n_entries, n_groups=n_groups)
    gsel, gcount = topk.select(gs, top_groups)
    cand = indexer.blocks_of_groups(gsel[:gcount])
    cand = cand[cand < nb]
    full = indexer.block_scores(q_idx, w, keys, n_entries, q_pos, n_blocks=nb)
    s = np.full(nb, -np.inf)
    s[cand] = full[cand]
    return topk.select(s, k)


def attend_row(q, cache, idx, count, n_entries, swa, swa_len, W,
               q_pos=None, swa_pos0=0, scale=attention.SCALE_512):
    """Sparse branch + window branch + LSE merge for one row -> (out [H][512], lse [H])."""
    o_s, l_s = attention.sparse_attention(q, cache, idx, count, n_entries, q_pos, scale)
    o_w, l_w = attention.window_attention(q, swa, swa_len, W, swa_pos0, q_pos, scale)
    return attention.merge(o_s, l_s, o_w, l_w)


def full_layer(q, q_idx, w, keys, cache, n_entries, k, swa, swa_len, W, top_groups=None):
    """Full mode for one decode row: index own keys, select, attend, merge -> (idx, count, out, lse)."""
    idx, count = select_blocks(q_idx, w, keys, n_entries, k, top_groups=top_groups,
                               n_blocks=np.asarray(cache).shape[0])
    out, lse = attend_row(q, cache, idx, count, n_entries, swa, swa_len, W)
    return idx, count, out, lse


def reindex_layer(q, q_idx, w, keys, cache, n_entries, k, swa, swa_len, W, top_groups=None):
    """Reindex mode: the same KV and indexer keys, the layer's own indexer query."""
    return full_layer(q, q_idx, w, keys, cache, n_entries, k, swa, swa_len, W, top_groups)


def reuse_layer(q, prev_idx, prev_count, cache, n_entries, swa, swa_len, W):
    """Reuse mode: the earlier layer's indices unchanged, own query and window."""
    idx = np.asarray(prev_idx, dtype=np.int32).copy()
    out, lse = attend_row(q, cache, idx, prev_count, n_entries, swa, swa_len, W)
    return idx, prev_count, out, lse
