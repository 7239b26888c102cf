"""Sharded-context emulation on the CPU: how the path splits one sequence's
cache over P devices, checked against the unsharded result with the oracle.

Each shard holds a contiguous range of whole blocks (whole 64-block groups for
the two-level selection). It scores its blocks and keeps its local top-K as
(score, global block id) pairs; the pairs of all shards are merged by the same
rule as one top-K (score descending, lower id first), which is exact because
every block of the global top-K has fewer than K blocks above it in its own
shard too. Each shard then attends the selected blocks it holds and emits
(o, lse); folding those with the log-sum-exp merge gives the attention over
the whole selection. The two-level selection needs one exchange more: the
shards' local top groups are merged into the global top groups first, and
each shard fine-scores only the selected groups it holds.
"""

import numpy as np
import pytest

from oracle import attention, indexer, modes, mxfp4, topk
from synth import normal_bf16, rng_for

BLOCK = 8
GROUP_BLOCKS = 64


def _inputs(seed, n, hi=8, h=4):
    rng = rng_for(seed)
    keys = normal_bf16(rng, (n, 64))
    q_idx = normal_bf16(rng, (hi, 64))
    w = rng.uniform(0.25, 1.0, hi).astype(np.float32)
    lat = normal_bf16(rng, (n, 512))
    q = normal_bf16(rng, (h, 512))
    return keys, q_idx, w, lat, q


def _shard_ranges(nb, p, unit=1):
    """P contiguous block ranges [b0, b1), sized in the ratio 1 : 2 : ... : P
    (uneven on purpose), cut at multiples of `unit` blocks; none is empty."""
    units = -(-nb // unit)
    wts = np.arange(1, p + 1, dtype=np.float64)
    cuts = np.concatenate([[0], np.round(np.cumsum(wts) / wts.sum() * units)]).astype(int)
    for i in range(1, p + 1):
        cuts[i] = max(cuts[i], cuts[i - 1] + 1)
    cuts[-1] = units
    assert np.all(np.diff(cuts) > 0)
    return [(int(a) * unit, min(int(b) * unit, nb)) for a, b in zip(cuts[:-1], cuts[1:])]


def _merge_pairs(scores, ids, k):
    """Top-k of (score, global id) pairs by the top-K rule -> ascending ids, count."""
    scores = np.asarray(scores, np.float64)
    ids = np.asarray(ids, np.int64)
    order = np.lexsort((ids, -scores))[:k]
    kept = np.sort(ids[order])
    out = np.full(k, -1, np.int64)
    out[:kept.size] = kept
    return out, int(kept.size)


def _local_topk(q_idx, w, keys, n, b0, b1, k, allowed=None):
    """A shard's local top-K over its blocks [b0, b1) -> (scores, global ids)."""
    e0, e1 = b0 * BLOCK, min(b1 * BLOCK, n)
    bs = indexer.block_scores(q_idx, w, keys[e0:e1], e1 - e0, n_blocks=b1 - b0)
    if allowed is not None:
        bs = np.where(allowed[b0:b1], bs, -np.inf)
    idx, c = topk.select(bs, k)
    local = idx[:c].astype(np.int64)
    return bs[local], local + b0


@pytest.mark.parametrize("n,k,p", [(4096, 64, 2), (4101, 100, 3), (3000, 300, 4), (2049, 40, 5)])
def test_local_topk_merge_equals_global_topk(n, k, p):
    keys, q_idx, w, _, _ = _inputs(11 * n + p, n)
    nb = -(-n // BLOCK)
    ranges = _shard_ranges(nb, p)
    shard_of = lambda b: next(i for i, (b0, b1) in enumerate(ranges) if b0 <= b < b1)   # noqa: E731
    # a tie at the boundary across shards: the k-th ranked block's keys copied
    # into an unselected full block of another shard, so ranks k and k+1 share a
    # score and the lower id must win in the merge as in the global top-K
    bs0 = indexer.block_scores(q_idx, w, keys, n, n_blocks=nb)
    order = np.argsort(-bs0, kind="stable")
    kth = int(order[k - 1])
    dst = next(int(b) for b in order[k:] if shard_of(int(b)) != shard_of(kth) and (b + 1) * BLOCK <= n)
    keys[dst * BLOCK:(dst + 1) * BLOCK] = keys[kth * BLOCK:(kth + 1) * BLOCK]
    bs1 = indexer.block_scores(q_idx, w, keys, n, n_blocks=nb)
    assert bs1[dst] == bs1[kth] and topk.gap_at_rank(bs1, k) == 0.0
    exp, c = topk.select(bs1, k)

    sc, ids = [], []
    for b0, b1 in ranges:
        s, g = _local_topk(q_idx, w, keys, n, b0, b1, k)
        sc.append(s)
        ids.append(g)
    got, gc = _merge_pairs(np.concatenate(sc), np.concatenate(ids), k)
    assert gc == c
    assert np.array_equal(got, exp.astype(np.int64))


@pytest.mark.parametrize("n,k,p,groups", [(8 * 512, 96, 2, 3), (8 * 512 + 100, 130, 3, 4)])
def test_two_level_sharded_selection_equals_global(n, k, p, groups):
    keys, q_idx, w, _, _ = _inputs(23 * n + p, n)
    nb = -(-n // BLOCK)
    n_groups = -(-nb // GROUP_BLOCKS)
    exp, c = modes.select_blocks(q_idx, w, keys, n, k, top_groups=groups, n_blocks=nb)

    ranges = _shard_ranges(nb, p, unit=GROUP_BLOCKS)
    # exchange 1: each shard's local top groups (score, global group id), merged
    gs_all = indexer.group_scores(q_idx, w, keys, n, n_groups=n_groups)
    sc, ids = [], []
    for b0, b1 in ranges:
        g0, g1 = b0 // GROUP_BLOCKS, -(-b1 // GROUP_BLOCKS)
        local = gs_all[g0:g1]            # a shard sees only its own groups' sums
        li, lc = topk.select(local, groups)
        sc.append(local[li[:lc]])
        ids.append(li[:lc].astype(np.int64) + g0)
    gsel, gc = _merge_pairs(np.concatenate(sc), np.concatenate(ids), groups)
    allowed = np.zeros(nb, bool)
    allowed[indexer.blocks_of_groups(gsel[:gc])[indexer.blocks_of_groups(gsel[:gc]) < nb]] = True
    # exchange 2: fine top-K inside the selected groups each shard holds, merged
    sc, ids = [], []
    for b0, b1 in ranges:
        s, g = _local_topk(q_idx, w, keys, n, b0, b1, k, allowed=allowed)
        sc.append(s)
        ids.append(g)
    got, fc = _merge_pairs(np.concatenate(sc), np.concatenate(ids), k)
    assert fc == c
    assert np.array_equal(got, exp.astype(np.int64))


@pytest.mark.parametrize("n,k,p", [(2048, 64, 2), (2053, 90, 3), (1500, 187, 4)])
def test_lse_combine_of_shard_attention_equals_global(n, k, p):
    keys, q_idx, w, lat, q = _inputs(37 * n + p, n)
    nb = -(-n // BLOCK)
    cache = mxfp4.build_records(lat, nb * BLOCK)
    idx, c = topk.select(indexer.block_scores(q_idx, w, keys, n, n_blocks=nb), k)
    o_ref, lse_ref = attention.sparse_attention(q, cache, idx, c, n)

    o, lse = None, None
    for b0, b1 in _shard_ranges(nb, p):
        mine = idx[:c][(idx[:c] >= b0) & (idx[:c] < b1)] - b0
        local = np.full(k, -1, np.int32)
        local[:mine.size] = mine
        n_local = min(b1 * BLOCK, n) - b0 * BLOCK
        op, lp = attention.sparse_attention(q, cache[b0:b1], local, mine.size, n_local)
        o, lse = (op, lp) if o is None else attention.merge(o, lse, op, lp)
    assert np.allclose(lse, lse_ref, rtol=0, atol=1e-12)
    assert np.allclose(o, o_ref, rtol=1e-12, atol=1e-13)


def test_shard_holding_no_selected_block_is_the_identity():
    n, k = 1024, 16
    keys, q_idx, w, lat, q = _inputs(5, n)
    nb = n // BLOCK
    cache = mxfp4.build_records(lat, n)
    idx, c = topk.select(indexer.block_scores(q_idx, w, keys, n, n_blocks=nb), k)
    o_ref, lse_ref = attention.sparse_attention(q, cache, idx, c, n)
    empty = np.full(k, -1, np.int32)
    oe, le = attention.sparse_attention(q, cache[:1], empty, 0, 8)
    assert np.all(np.isneginf(le))
    o, lse = attention.merge(o_ref, lse_ref, oe, le)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
