"""Sparse indexer: entry scores, block scores, two-level group stage (oracle; test infrastructure).

The pages say a sparse indexer picks "up to 2,048 blocks of 8" for attention,
that each layer may rescore with its own indexer query (Reindex mode), and that
a hierarchical indexer trims decoder indexing ([card] Key ideas, "CSA2 with
three static layer modes").  They give no score formula.  Readings taken:

* Indexer keys are a separate bfloat16 [N][64] array per sequence (one row per
  compressed entry); the query side has Hi heads of 64 dims plus one float32
  weight per head.
* Entry score  e_j = sum_h w_h * max(0, q_h . k_j)   (no extra scale factor).
* Block b holds entries [8b, 8b+8).  Its score is the max of e_j over the
  entries that are present (j < n_entries) and visible to the query; a block
  with no such entry is not a candidate (score -inf here).
* Visibility (causal, prefill only): entry j merges raw positions 2j and 2j+1
  ([digest] Core Mechanics: two adjacent positions per entry), so it is visible
  to the query at raw position t iff 2j + 1 <= t.  Without a query position
  every present entry is visible (decode: the query is the newest token).
* Two-level stage: group g = blocks [64g, 64g+64) = entries [512g, 512g+512).
  Its coarse key is the arithmetic mean of the group's present entries' keys;
  its coarse score is the entry-score formula applied to that mean.  The top
  ``top_groups`` groups are kept (same tie rule as blocks) and block scores are
  taken only inside them.

All arithmetic in float64.
"""

import numpy as np

from . import bf16

BLOCK = 8
GROUP_BLOCKS = 64
GROUP_ENTRIES = BLOCK * GROUP_BLOCKS   # 512


def entry_scores(q_idx, w, keys):
    """e_j = sum_h w_h * relu(q_h . k_j).

    q_idx [Hi][64], w [Hi], keys [N][64] (float64 or bf16 bits) -> [N] float64.
    """
    q = _f64(q_idx)
    k = _f64(keys)
    w = np.asarray(w, dtype=np.float64)
    dots = k @ q.T                         # [N][Hi]
    return np.maximum(dots, 0.0) @ w       # [N]


def visible_mask(n_total, n_entries, q_pos=None):
    """Entries j < n_total that are present (j < n_entries) and visible to raw position q_pos."""
    j = np.arange(n_total)
    m = j < n_entries
    if q_pos is not None:
        m &= (2 * j + 1) <= q_pos
    return m


def block_scores(q_idx, w, keys, n_entries, q_pos=None, n_blocks=None):
    """Block scores [nb] float64: max of visible present entry scores per block of 8, else -inf.

    ``keys`` covers at least the present entries; ``n_blocks`` (default
    ceil(len(keys)/8)) sets the length of the result.
    """
    k = _f64(keys)
    n_total = k.shape[0]
    nb = n_blocks if n_blocks is not None else (n_total + BLOCK - 1) // BLOCK
    e = np.full(nb * BLOCK, -np.inf)
    vis = visible_mask(min(n_total, nb * BLOCK), n_entries, q_pos)
    idx = np.nonzero(vis)[0]
    if idx.size:
        e[idx] = entry_scores(q_idx, w, k[idx])
    return e.reshape(nb, BLOCK).max(axis=1)


def group_means(keys, n_entries, n_groups=None):
    """Mean indexer key per group of 512 entries over its present entries -> ([G][64], present[G])."""
    k = _f64(keys)
    G = n_groups if n_groups is not None else (k.shape[0] + GROUP_ENTRIES - 1) // GROUP_ENTRIES
    means = np.zeros((G, k.shape[1]))
    present = np.zeros(G, dtype=bool)
    for g in range(G):
        lo = g * GROUP_ENTRIES
        hi = min(lo + GROUP_ENTRIES, n_entries)
        if hi > lo:
            means[g] = k[lo:hi].mean(axis=0)
            present[g] = True
    return means, present


def group_scores(q_idx, w, keys, n_entries, n_groups=None):
    """Coarse score per group [G]: entry-score formula on the group's mean key; -inf if empty."""
    means, present = group_means(keys, n_entries, n_groups)
    s = entry_scores(q_idx, w, means)
    return np.where(present, s, -np.inf)


def blocks_of_groups(groups):
    """Block ids covered by the given group ids, ascending within each group."""
    groups = np.asarray(groups, dtype=np.int64)
    groups = groups[groups >= 0]
    return (groups[:, None] * GROUP_BLOCKS + np.arange(GROUP_BLOCKS)[None, :]).reshape(-1)


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16.to_f64(a)
    return a.astype(np.float64)
