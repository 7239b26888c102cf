"""Top-K block selection (oracle; test infrastructure).

The pages say the indexer keeps "up to 2,048 blocks of 8" per query ([card] Key
ideas, "CSA2 with three static layer modes").  They state no tie rule, no order
and no padding.  Readings taken:

* Candidates are the blocks with a finite score (a block with no present and
  visible entry is not a candidate).
* Order candidates by score descending, then block id ascending (ties go to the
  lower block id); keep the first min(K, #candidates).
* Output the kept block ids sorted ascending in an int32 row of length K, padded
  with -1, plus the count of kept blocks.
"""

import numpy as np


def select(scores, k):
    """scores [n] (float, -inf = not a candidate) -> (idx int32 [k], count int)."""
    s = np.asarray(scores)
    cand = np.nonzero(np.isfinite(s))[0]
    # primary key: score descending; secondary: id ascending (lexsort: last key is primary)
    order = cand[np.lexsort((cand, -s[cand]))]
    kept = np.sort(order[:k])
    out = np.full(k, -1, dtype=np.int32)
    out[:kept.size] = kept
    return out, int(kept.size)


def gap_at_rank(scores, k):
    """Score difference between rank k and rank k+1 among candidates (inf if <= k candidates)."""
    s = np.asarray(scores, dtype=np.float64)
    c = np.sort(s[np.isfinite(s)])[::-1]
    if c.size <= k:
        return np.inf
    return float(c[k - 1] - c[k])
