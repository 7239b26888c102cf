"""Checks of the seeded input generator against the oracle (CPU only)."""

import numpy as np
import torch

from oracle import indexer, modes, topk
from synth import CONFIGS, bf16_rne, decode_inputs, normal_bf16, prefill_inputs, rng_for


def test_bf16_rne_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.00390625, 1.01171875, -2.0078125, 0.0]          # exact halfway cases
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_rne(x), ref)


def test_seeded_determinism():
    a = normal_bf16(rng_for(5), (3, 100))
    b = normal_bf16(rng_for(5), (3, 100))
    assert a.tobytes() == b.tobytes()


def test_tiny_dominant_plant_gap_and_selection():
    cfg = CONFIGS["tiny"]
    x = decode_inputs(cfg)
    s = indexer.block_scores(x.q_idx[0, 0], x.w[0, 0], x.keys[0], cfg.N)
    assert topk.gap_at_rank(s, cfg.K) >= 1e-2
    idx, c = topk.select(s, cfg.K)
    assert c == cfg.K and np.array_equal(idx, x.planted[0])


def test_tiny_tight_plant_gap():
    cfg = CONFIGS["tiny"]
    holder = {}

    def score_fn(b):
        return lambda keys: indexer.entry_scores(holder["x"].q_idx[b, 0], holder["x"].w[b, 0], keys)

    # generate once without a plant to get the query, then plant tightly on the same draw
    x = decode_inputs(cfg, plant=None)
    holder["x"] = x
    from synth import plant_tight
    keys = x.keys[0].copy()
    plant_tight(keys, cfg.N, x.q_idx[0, 0], x.w[0, 0], np.arange(0, 256, 8), rng_for(1), score_fn(0))
    s = indexer.block_scores(x.q_idx[0, 0], x.w[0, 0], keys, cfg.N)
    gap = topk.gap_at_rank(s, 32)
    srt = np.sort(s)[::-1]
    assert gap >= 1e-2
    assert srt[31] - srt[32] < 5.0          # tight: just above the best unplanted block
    idx, c = topk.select(s, 32)
    assert np.array_equal(idx, np.arange(0, 256, 8))


def test_two_level_plant_gap_small():
    # a scaled-down two-level case: 32 groups, keep 4, K 64 inside them
    from synth.configs import Config
    cfg = Config("small2", B=1, Q=1, H=4, N=32 * 512, Hi=8, K=64, W=16, top_groups=4, seed=77)
    x = decode_inputs(cfg)
    gs = indexer.group_scores(x.q_idx[0, 0], x.w[0, 0], x.keys[0], cfg.N)
    assert topk.gap_at_rank(gs, 4) >= 1e-2
    idx, c = modes.select_blocks(x.q_idx[0, 0], x.w[0, 0], x.keys[0], cfg.N, cfg.K, top_groups=4)
    assert np.array_equal(idx, x.planted[0])


def test_prefill_generator_shapes_and_gap_on_sample_rows():
    from synth.configs import Config
    cfg = Config("smallpf", B=1, Q=64, H=4, N=4096 + 32, Hi=4, K=32, W=16, prior=4096, seed=5)
    x = prefill_inputs(cfg)
    assert x["latent"].shape == (1, 4096 + 32, 512) and x["q_pos"].shape == (1, 64)
    for r in (0, 17, 63):
        s = indexer.block_scores(x["q_idx"][0, r], x["w"][0, r], x["keys"][0], 4096 + 32,
                                 q_pos=int(x["q_pos"][0, r]))
        assert topk.gap_at_rank(s, 32) >= 1e-2


def test_specdec_rows_positions_window_and_plants():
    # draft rows: consecutive raw positions after the cache, a window that holds
    # exactly W tokens for each row, and row 0's plant still the top-K of every row
    from oracle import indexer, topk
    from synth import specdec_inputs
    from synth.configs import Config
    cfg = Config("t", B=2, Q=4, H=16, N=2048, Hi=4, K=32, W=128, seed=7)
    x = specdec_inputs(cfg)
    assert (x.q_pos == 2 * cfg.N + np.arange(cfg.Q)).all()
    assert (x.swa_len == cfg.W + cfg.Q - 1).all() and x.swa.shape[1] == cfg.W + cfg.Q - 1
    for b in range(cfg.B):
        for r in range(cfg.Q):
            t = int(x.q_pos[b, r])
            lo, hi = max(t - cfg.W + 1, int(x.swa_pos0[b])), min(t, int(x.swa_pos0[b]) + int(x.swa_len[b]) - 1)
            assert hi - lo + 1 == cfg.W
            s = indexer.block_scores(x.q_idx[b, r], x.w[b, r], x.keys[b], cfg.N, q_pos=t, n_blocks=cfg.nb)
            assert topk.gap_at_rank(s, cfg.K) >= 1e-2
            sel, c = topk.select(s, cfg.K)
            assert c == cfg.K and np.array_equal(sel, np.sort(x.planted[b]))
