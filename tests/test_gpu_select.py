"""GPU parity: csa2_topk and csa2_index_topk selected block indices vs the oracle."""

import numpy as np
import pytest
import torch

from oracle import indexer, modes, topk
from synth import CONFIGS, decode_inputs, normal_bf16, plant_tight, rng_for, bf16_rne
from synth.configs import Config
from tests.gpu_util import dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _lib():
    from sparse_attention_fp4_csa2_amd import _lib
    return _lib


def gpu_topk(scores, k):
    lib = _lib()
    s = dev(scores.astype(np.float32))
    rows = scores.shape[0]
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    lib.topk(s, k, idx, cnt)
    torch.cuda.synchronize()
    return host(idx), host(cnt)


@pytest.mark.parametrize("n,k", [(256, 32), (4096, 2048), (2502, 700), (8448, 2048), (16384, 2048),
                                 (37, 64), (1000, 1), (65536, 2048)])
def test_topk_from_scores_bit_exact_with_ties(n, k):
    rng = rng_for(n * 7 + k)
    rows = 10
    s = np.empty((rows, n), dtype=np.float32)
    s[0] = rng.standard_normal(n)
    s[1] = rng.integers(-3, 4, size=n)                 # heavy ties, negatives, zeros
    s[2] = 1.5                                          # all equal
    s[3] = rng.standard_normal(n)
    s[3, rng.choice(n, n // 3, replace=False)] = -np.inf   # non-candidates
    s[4] = -np.inf
    s[4, :min(n, 5)] = [0.0, -0.0, 2.0, -1.0, 2.0][:min(n, 5)]   # fewer candidates than k
    s[5] = np.float32(1e30) * rng.standard_normal(n).astype(np.float32)
    s[5, ::5] = np.nan                                  # NaN = non-candidate
    s[6] = rng.choice(np.array([0.0, -0.0], np.float32), n)   # +0 and -0 tie; rank k among them
    s[6, rng.choice(n, max(1, min(n, k) // 2), replace=False)] = 1.0
    # a few equal keys straddling rank k amid distinct ones: the bin holding
    # the k-th key is small, so the kernel ranks it directly
    s[7] = rng.standard_normal(n)
    order = np.argsort(-s[7].astype(np.float64), kind="stable")
    lo, hi = max(0, min(n, k) - 4), min(n, k + 3)
    s[7, order[lo:hi]] = s[7, order[lo]]
    # planted-like rows: one score shared by exactly k blocks (then by k + 5),
    # far above the rest, beside a few negatives: the boundary bin is one value
    for r, extra in ((8, 0), (9, 5)):
        s[r] = rng.standard_normal(n) * 20.0
        s[r, rng.choice(n, min(n, k + extra), replace=False)] = 317.9581
    got, cnt = gpu_topk(s, k)
    for r in range(rows):
        ref_in = np.where(np.isnan(s[r]), -np.inf, s[r]).astype(np.float64)
        exp, c = topk.select(ref_in, k)
        assert cnt[r] == c, (r, cnt[r], c)
        assert np.array_equal(got[r], exp), f"row {r}"


def _index_gpu(x, cfg, n_entries, top_groups=0, q_pos=None, group_sum=None):
    lib = _lib()
    B, Q = x["q_idx"].shape[:2]
    cap = x["cap"]
    keys = np.zeros((B, cap, 64), dtype=np.uint16)
    keys[:, :x["keys"].shape[1]] = x["keys"]
    kc = dev_bf16(keys)
    gs = None
    if top_groups:
        gs = torch.zeros(B, cap // 512, 64, dtype=torch.float32, device="cuda")
        kf = (keys.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        for b in range(B):
            ne = int(n_entries[b])
            for g in range((ne + 511) // 512):
                gs[b, g] = torch.from_numpy(kf[b, 512 * g:min(512 * g + 512, ne)].sum(0).astype(np.float32))
    idx = torch.full((B, Q, cfg.K), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Q), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(lib.index_topk_ws(B, Q, cap, top_groups), 256), dtype=torch.uint8, device="cuda")
    lib.index_topk(dev_bf16(x["q_idx"]), dev(x["w"]), kc, dev(np.asarray(n_entries, np.int32)),
                   cfg.K, idx, cnt, ws, group_sum=gs, q_pos=None if q_pos is None else dev(q_pos),
                   top_groups=top_groups)
    torch.cuda.synchronize()
    if x.get("want_scores"):
        # flat call: the workspace starts with the fp32 block scores [rows][cap/8]
        sc = host(ws[:B * Q * (cap // 8) * 4].view(torch.float32)).reshape(B, Q, cap // 8)
        return host(idx), host(cnt), sc
    return host(idx), host(cnt)


def test_tiny_tight_plant_indices_bit_exact():
    cfg = CONFIGS["tiny"]
    x = decode_inputs(cfg, plant=None)
    keys = x.keys[0]
    plant_tight(keys, cfg.N, x.q_idx[0, 0], x.w[0, 0], np.arange(3, 256, 8), rng_for(2),
                lambda k: indexer.entry_scores(x.q_idx[0, 0], x.w[0, 0], k))
    s = indexer.block_scores(x.q_idx[0, 0], x.w[0, 0], keys, cfg.N)
    assert topk.gap_at_rank(s, cfg.K) >= 1e-2
    got, cnt = _index_gpu(dict(q_idx=x.q_idx, w=x.w, keys=x.keys, cap=cfg.N), cfg, x.n_entries)
    exp, c = topk.select(s, cfg.K)
    assert cnt[0, 0] == c and np.array_equal(got[0, 0], exp)


def test_unplanted_random_selection_is_valid():
    # no gap: the GPU's choice must still be a valid top-K under the oracle's fp64 scores
    cfg = Config("r", B=3, Q=1, H=16, N=3000, Hi=8, K=100, W=16, seed=5)
    x = decode_inputs(cfg, plant=None)
    ne = np.array([3000, 2999, 1234], np.int32)
    cap = 3000 + (8 - 3000 % 8) % 8
    got, cnt = _index_gpu(dict(q_idx=x.q_idx, w=x.w, keys=x.keys, cap=cap), cfg, ne)
    for b in range(3):
        s = indexer.block_scores(x.q_idx[b, 0], x.w[b, 0], x.keys[b], int(ne[b]), n_blocks=cap // 8)
        sel = got[b, 0, :cnt[b, 0]]
        assert cnt[b, 0] == min(cfg.K, np.isfinite(s).sum())
        assert np.all(np.diff(sel) > 0) and (got[b, 0, cnt[b, 0]:] == -1).all()
        uns = np.setdiff1d(np.nonzero(np.isfinite(s))[0], sel)
        eps = 1e-3 * max(1.0, np.abs(s[np.isfinite(s)]).max())
        assert s[sel].min() >= s[uns].max() - eps


def test_ragged_and_causal_rows_bit_exact():
    # Q = 3 query rows per sequence at different raw positions (causal visibility)
    cfg = Config("c", B=2, Q=3, H=16, N=2048, Hi=4, K=24, W=16, seed=9)
    rng = rng_for(9)
    keys = normal_bf16(rng, (2, 2048, 64))
    q_idx = normal_bf16(rng, (2, 3, 4, 64))
    w = rng.standard_normal((2, 3, 4)).astype(np.float32)
    w[..., 0] = np.abs(w[..., 0]) + 0.5
    ne = np.array([2048, 1501], np.int32)
    q_pos = np.array([[4095, 1001, 17], [3001, 2400, 640]], np.int32)
    for b in range(2):
        for r in range(3):
            nvis = min(int(ne[b]), (int(q_pos[b, r]) + 1) // 2)
            nbv = nvis // 8
            if nbv <= 24:
                continue                        # every visible block is selected anyway
            blocks = np.sort(rng.choice(nbv, 24, replace=False))
            plant_tight(keys[b], nvis, q_idx[b, r], w[b, r], blocks, rng,
                        lambda k, b=b, r=r: indexer.entry_scores(q_idx[b, r], w[b, r], k), margin=2.0)
    got, cnt = _index_gpu(dict(q_idx=q_idx, w=w, keys=keys, cap=2048), cfg, ne, q_pos=q_pos)
    for b in range(2):
        for r in range(3):
            s = indexer.block_scores(q_idx[b, r], w[b, r], keys[b], int(ne[b]), q_pos=int(q_pos[b, r]),
                                     n_blocks=256)
            exp, c = topk.select(s, 24)
            if topk.gap_at_rank(s, 24) >= 1e-2:
                assert cnt[b, r] == c and np.array_equal(got[b, r], exp), (b, r)
            else:
                sel = got[b, r, :cnt[b, r]]
                uns = np.setdiff1d(np.nonzero(np.isfinite(s))[0], sel)
                assert s[sel].min() >= s[uns].max() - 1e-3 * np.abs(s[np.isfinite(s)]).max()


def test_two_level_small_bit_exact_and_all_groups_equals_flat():
    cfg = Config("t", B=2, Q=1, H=16, N=32 * 512, Hi=8, K=64, W=16, top_groups=4, seed=77)
    x = decode_inputs(cfg)
    ne = x.n_entries
    d = dict(q_idx=x.q_idx, w=x.w, keys=x.keys, cap=cfg.N)
    got, cnt = _index_gpu(d, cfg, ne, top_groups=4)
    for b in range(2):
        gs = indexer.group_scores(x.q_idx[b, 0], x.w[b, 0], x.keys[b], cfg.N)
        assert topk.gap_at_rank(gs, 4) >= 1e-2
        exp, c = modes.select_blocks(x.q_idx[b, 0], x.w[b, 0], x.keys[b], cfg.N, cfg.K, top_groups=4)
        assert cnt[b, 0] == c and np.array_equal(got[b, 0], exp), b
    # keeping every group reduces to the flat selection
    got_all, cnt_all = _index_gpu(d, cfg, ne, top_groups=32)
    got_flat, cnt_flat = _index_gpu(d, cfg, ne)
    assert np.array_equal(got_all, got_flat) and np.array_equal(cnt_all, cnt_flat)


@pytest.mark.parametrize("hi,Q", [(8, 40), (5, 40), (8, 150)])
def test_many_rows_per_sequence_scores_and_selection(hi, Q):
    # causal query rows of the multi-row MFMA indexer (64-row workgroups of four
    # 16-row waves): 40 rows leave one wave partly filled and one empty, 150
    # rows take two full workgroups and a ragged third; block scores compared
    # value by value
    B, cap, K = 2, 4096 + 512, 64
    cfg = Config("m", B=B, Q=Q, H=16, N=cap, Hi=hi, K=K, W=16, seed=21)
    rng = rng_for(21 + hi + Q)
    keys = normal_bf16(rng, (B, cap, 64))
    q_idx = normal_bf16(rng, (B, Q, hi, 64))
    w = rng.standard_normal((B, Q, hi)).astype(np.float32)
    ne = np.array([cap, 3001], np.int32)
    q_pos = np.sort(rng.integers(0, 2 * cap + 64, size=(B, Q)), axis=1).astype(np.int32)
    q_pos[0, 0], q_pos[1, -1] = 0, 2 * cap + 63           # nothing visible / everything visible
    got, cnt, sc = _index_gpu(dict(q_idx=q_idx, w=w, keys=keys, cap=cap, want_scores=True), cfg, ne,
                              q_pos=q_pos)
    worst = 0.0
    for b in range(B):
        for r in range(Q):
            s = indexer.block_scores(q_idx[b, r], w[b, r], keys[b], int(ne[b]), q_pos=int(q_pos[b, r]),
                                     n_blocks=cap // 8)
            fin = np.isfinite(s)
            assert np.array_equal(np.isfinite(sc[b, r]), fin), (b, r)
            if fin.any():
                scale = max(1.0, np.abs(s[fin]).max())
                worst = max(worst, np.abs(sc[b, r][fin] - s[fin]).max() / scale)
            exp, c = topk.select(s, K)
            assert cnt[b, r] == c, (b, r)
            if topk.gap_at_rank(s, K) >= 1e-2:
                assert np.array_equal(got[b, r], exp), (b, r)
            elif c:
                sel = got[b, r, :c]
                uns = np.setdiff1d(np.nonzero(fin)[0], sel)
                if uns.size:
                    assert s[sel].min() >= s[uns].max() - 1e-4 * np.abs(s[fin]).max()
    print(f"[parity] multi-row block scores: max|err|/max|s| = {worst:.2e}")
    assert worst < 1e-5
