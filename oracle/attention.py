"""Sparse attention over the selected MXFP4 latent, sliding window, LSE merge (oracle; test infrastructure).

What the pages fix: one 512-d latent per compressed entry is shared as key and
value by all query heads ([digest] Core Mechanics, "Compressed along three
axes", channel axis); attention reads only the top-K selected blocks of 8
entries, and every layer also keeps its own query and sliding-window KV ([card]
Key ideas, "CSA2 with three static layer modes"; [digest] Terminology, SWA).
They give no formula.  Readings taken:

* Each head h has a 512-d latent-space query q_h (the up-projection of a full
  model is outside this path); K_j = V_j = dequant(entry j).
* Logit z_j = s * (q_h . K_j) with s = 1/sqrt(512); no bias, no rotary term,
  no attention sink.
* Softmax over the selected, present, visible entries; o_h = sum_j p_j V_j,
  lse_h = log sum_j exp(z_j).  An empty selection gives o = 0, lse = -inf.
* Sliding window: the last W raw tokens, bfloat16, K = V, same scale.  Window
  slot i of a sequence holds raw position pos0 + i; the query at raw position t
  sees positions [t - W + 1, t] among the held ones.  Without a query position
  the query is the newest held token.
* The two branches are joined by a log-sum-exp merge, which equals one softmax
  over the union of both key sets (tokens that sit in both the window and a
  selected entry are counted in both branches).

All arithmetic in float64.
"""

import numpy as np

from . import bf16, mxfp4

SCALE_512 = 1.0 / np.sqrt(512.0)


def attend(q, kv, scale):
    """Softmax attention of queries q [H][D] over keys = values kv [n][D].

    Returns (o [H][D], lse [H]); n == 0 gives o = 0, lse = -inf.
    """
    q = _f64(q)
    kv = _f64(kv)
    H, D = q.shape
    if kv.shape[0] == 0:
        return np.zeros((H, D)), np.full(H, -np.inf)
    z = scale * (q @ kv.T)                    # [H][n]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ kv) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def selected_entries(idx, count, n_entries, q_pos=None, n_blocks=None):
    """Entry ids attended for one query: the present, visible entries of the selected blocks.

    Block ids outside [0, n_blocks) (the -1 padding) are skipped.
    """
    idx = np.asarray(idx, dtype=np.int64)[:count]
    if n_blocks is not None:
        idx = idx[(idx >= 0) & (idx < n_blocks)]
    else:
        idx = idx[idx >= 0]
    ent = (idx[:, None] * mxfp4.BLOCK + np.arange(mxfp4.BLOCK)[None, :]).reshape(-1)
    keep = ent < n_entries
    if q_pos is not None:
        keep &= (2 * ent + 1) <= q_pos
    return ent[keep]


def sparse_attention(q, cache, idx, count, n_entries, q_pos=None, scale=SCALE_512):
    """One query row: q [H][512] over the selected blocks of a record cache -> (o, lse)."""
    ent = selected_entries(idx, count, n_entries, q_pos, n_blocks=np.asarray(cache).shape[0])
    kv = mxfp4.read_entries(cache, ent) if ent.size else np.zeros((0, mxfp4.D))
    return attend(q, kv, scale)


def window_positions(swa_len, W, pos0=0, q_pos=None):
    """Slots of the window buffer visible to the query (ascending)."""
    if q_pos is None:
        q_pos = pos0 + swa_len - 1
    lo = max(q_pos - W + 1, pos0)
    hi = min(q_pos, pos0 + swa_len - 1)
    if hi < lo:
        return np.zeros(0, dtype=np.int64)
    return np.arange(lo, hi + 1) - pos0


def window_attention(q, swa, swa_len, W, pos0=0, q_pos=None, scale=SCALE_512):
    """Sliding-window branch: q [H][512] over bf16 window tokens swa [Lw][512] -> (o, lse)."""
    slots = window_positions(swa_len, W, pos0, q_pos)
    kv = _f64(np.asarray(swa)[slots]) if slots.size else np.zeros((0, np.asarray(swa).shape[-1]))
    return attend(q, kv, scale)


def merge(o1, lse1, o2, lse2):
    """Log-sum-exp merge of two attention branches.

    L = log(exp(lse1) + exp(lse2)); out = exp(lse1 - L) o1 + exp(lse2 - L) o2.
    Both -inf gives out = 0, L = -inf.
    """
    o1, o2 = _f64(o1), _f64(o2)
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    L = np.logaddexp(lse1, lse2)
    fin = np.isfinite(L)
    Ls = np.where(fin, L, 0.0)
    a1 = np.where(fin, np.exp(lse1 - Ls), 0.0)
    a2 = np.where(fin, np.exp(lse2 - Ls), 0.0)
    out = a1[..., None] * o1 + a2[..., None] * o2
    return out, L


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16.to_f64(a)
    return a.astype(np.float64)
