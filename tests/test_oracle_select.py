"""Pins for the oracle's indexer, two-level group stage and top-K (CPU only)."""

import math

import numpy as np
import pytest

from oracle import indexer, modes, topk
from synth import normal_bf16, rng_for, bf16_to_f32
from tests import pins


def _small(seed, n=45, hi=3):
    rng = rng_for(seed)
    q = normal_bf16(rng, (hi, 64))
    w = rng.standard_normal(hi).astype(np.float32)
    k = normal_bf16(rng, (n, 64))
    return q, w, k


def test_entry_scores_vs_loops():
    q, w, k = _small(1)
    e = indexer.entry_scores(q, w, k)
    qf, kf = bf16_to_f32(q), bf16_to_f32(k)
    for j in range(k.shape[0]):
        assert e[j] == pytest.approx(pins.entry_score_loops(qf, w, kf[j]), rel=1e-12, abs=1e-12)


def test_entry_scores_special_cases():
    q, w, k = _small(2, hi=1)
    onehot = np.zeros((64, 64))
    onehot[np.arange(64), np.arange(64)] = 1.0
    e = indexer.entry_scores(q, np.array([1.0]), onehot)
    assert np.array_equal(e, np.maximum(bf16_to_f32(q[0]).astype(np.float64), 0))
    assert (indexer.entry_scores(q, np.array([0.0]), k) == 0).all()
    # positive homogeneity in the key
    q3, w3, k3 = _small(3)
    base = indexer.entry_scores(q3, w3, k3)
    assert np.allclose(indexer.entry_scores(q3, w3, 2.5 * bf16_to_f32(k3)), 2.5 * base, rtol=1e-12)
    # a negative weight on a head subtracts that head's ReLU term
    e_pos = indexer.entry_scores(q3, np.abs(w3), k3)
    assert (e_pos >= 0).all()


def test_block_scores_vs_loops_with_visibility():
    q, w, k = _small(4, n=45)
    for n_entries, q_pos in [(45, None), (41, None), (45, 37), (45, 0), (3, None)]:
        s = indexer.block_scores(q, w, k, n_entries, q_pos, n_blocks=7)
        qf, kf = bf16_to_f32(q), bf16_to_f32(k)
        for b in range(7):
            vals = []
            for j in range(8 * b, 8 * b + 8):
                if j < min(n_entries, 45) and (q_pos is None or 2 * j + 1 <= q_pos):
                    vals.append(pins.entry_score_loops(qf, w, kf[j]))
            if vals:
                assert s[b] == pytest.approx(max(vals), rel=1e-12, abs=1e-12)
            else:
                assert s[b] == -math.inf


def test_causal_visibility_rule():
    # entry j covers raw positions 2j and 2j+1: visible to t iff 2j+1 <= t
    m = indexer.visible_mask(6, 6, q_pos=4)
    assert m.tolist() == [True, True, False, False, False, False]
    m = indexer.visible_mask(6, 6, q_pos=5)
    assert m.tolist() == [True, True, True, False, False, False]


def test_group_means_vs_loops():
    rng = rng_for(5)
    k = normal_bf16(rng, (1100, 64))
    means, present = indexer.group_means(k, 1100, n_groups=4)
    kf = bf16_to_f32(k).astype(np.float64)
    assert present.tolist() == [True, True, True, False]
    for g, (lo, hi) in enumerate([(0, 512), (512, 1024), (1024, 1100)]):
        exp = [sum(kf[j, d] for j in range(lo, hi)) / (hi - lo) for d in range(64)]
        assert np.allclose(means[g], exp, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("k", [1, 5, 13, 40, 64])
def test_topk_vs_pairwise_rank(k):
    rng = rng_for(100 + k)
    s = rng.integers(0, 12, size=50).astype(np.float64)   # many ties
    s[rng.choice(50, 7, replace=False)] = -np.inf           # non-candidates
    idx, count = topk.select(s, k)
    exp = pins.topk_pairwise(s, k)
    assert count == len(exp)
    assert idx[:count].tolist() == exp                       # ascending ids
    assert (idx[count:] == -1).all()


def test_topk_invariants_and_all_selected():
    rng = rng_for(9)
    s = rng.standard_normal(300)
    idx, count = topk.select(s, 64)
    sel = idx[:count]
    uns = np.setdiff1d(np.arange(300), sel)
    assert count == 64 and s[sel].min() >= s[uns].max()
    assert np.all(np.diff(sel) > 0)
    idx2, c2 = topk.select(s, 500)
    assert c2 == 300 and np.array_equal(idx2[:300], np.arange(300)) and (idx2[300:] == -1).all()
    # equal scores: the lowest ids win
    idx3, c3 = topk.select(np.zeros(10), 4)
    assert idx3.tolist() == [0, 1, 2, 3] and c3 == 4


def test_two_level_with_all_groups_equals_flat():
    rng = rng_for(12)
    n = 3000
    q = normal_bf16(rng, (4, 64))
    w = rng.standard_normal(4).astype(np.float32)
    k = normal_bf16(rng, (n, 64))
    flat = modes.select_blocks(q, w, k, n, 40)
    groups = (n + 511) // 512
    two = modes.select_blocks(q, w, k, n, 40, top_groups=groups)
    assert np.array_equal(flat[0], two[0]) and flat[1] == two[1]
    # restricting to fewer groups only ever picks blocks inside the kept groups
    gs = indexer.group_scores(q, w, k, n)
    gsel, gc = topk.select(gs, 2)
    part, pc = modes.select_blocks(q, w, k, n, 40, top_groups=2)
    assert set((part[:pc] // 64).tolist()) <= set(gsel[:gc].tolist())


def test_two_level_group_stage_vs_loops():
    rng = rng_for(13)
    n = 1600
    q = normal_bf16(rng, (2, 64))
    w = np.array([0.7, -0.4], dtype=np.float32)
    k = normal_bf16(rng, (n, 64))
    gs = indexer.group_scores(q, w, k, n)
    qf, kf = bf16_to_f32(q), bf16_to_f32(k).astype(np.float64)
    for g in range(4):
        lo, hi = 512 * g, min(512 * g + 512, n)
        mean = kf[lo:hi].mean(axis=0)
        assert gs[g] == pytest.approx(pins.entry_score_loops(qf, w, mean), rel=1e-10)
