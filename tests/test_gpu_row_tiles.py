"""GPU parity: row tiles (16 or fewer heads), where 2 or 4 rows of a sequence
share the attention tile's 32 columns and attend the union of their selections.

Each row must still see exactly its own selection (its blocks, its causal
limit, its count): checked against the fp64 oracle row by row, at the same bar
as the single-row tiles (max|err| <= 1e-2 x RMS, lse within 1e-3).  Covered:
overlapping and disjoint selections, ragged and empty counts, out-of-range ids,
causal rows, a short last group, duplicate ids and caches too large for the
union's bitmap (both run the rows' lists one after the other), the one-call
layer with its window branch, and the standalone window call on row tiles.
"""

import numpy as np
import pytest
import torch

from oracle import modes, mxfp4
from synth import normal_bf16, rng_for
from tests.gpu_util import assert_close_rms, assert_lse_close, dev, dev_bf16, host
from tests.test_gpu_attention import SCALE, gpu_cache, gpu_layer, gpu_sparse, oracle_rows

pytestmark = pytest.mark.gpu


def _lib():
    from sparse_attention_fp4_csa2_amd import _lib
    return _lib


def _selections(rng, B, Q, nb, K, shared, extra):
    """Per row: `shared` blocks common to its sequence plus `extra` of its own, ascending."""
    idx = np.full((B, Q, K), -1, np.int32)
    count = np.zeros((B, Q), np.int32)
    for b in range(B):
        common = rng.choice(nb, shared, replace=False)
        for r in range(Q):
            own = rng.choice(np.setdiff1d(np.arange(nb), common), extra, replace=False)
            sel = np.sort(np.concatenate([common, own]))[:K]
            idx[b, r, :sel.size] = sel
            count[b, r] = sel.size
    return idx, count


@pytest.mark.parametrize("H,Q", [(16, 2), (16, 3), (16, 5), (12, 4), (8, 4), (8, 3), (4, 6)])
def test_row_tiles_sparse_matches_oracle(H, Q):
    rng = rng_for(700 + 10 * H + Q)
    B, N, K = 2, 1200, 48
    lat = normal_bf16(rng, (B, N, 512))
    q = normal_bf16(rng, (B, Q, H, 512))
    ne = np.array([1200, 1195], np.int32)
    idx, count = _selections(rng, B, Q, 149, K, shared=30, extra=14)
    count[0, Q - 1] = 0                       # an empty row
    count[1, 0] = 17                          # a ragged row (ids past its count are ignored)
    idx[1, 1 % Q, 2] = 100000                 # out of range: skipped
    idx[1, 1 % Q] = np.sort(idx[1, 1 % Q])
    # sequence 0: every row sees the whole cache; sequence 1: causal rows that
    # see only part of it (entry j is visible to raw position t iff 2j + 1 <= t)
    q_pos = np.stack([2 * N + np.arange(Q), 900 + 151 * np.arange(Q)]).astype(np.int32)
    cache = gpu_cache(lat, N)
    cache_np = np.stack([mxfp4.build_records(lat[b], N) for b in range(B)])
    o, l = gpu_sparse(q, cache, idx, count, ne, q_pos=q_pos)
    ro, rl = oracle_rows(q, cache_np, idx, count, ne, q_pos)
    assert_close_rms(o, ro)
    assert_lse_close(l, rl)
    assert (o[0, Q - 1] == 0).all() and np.isneginf(l[0, Q - 1]).all(), "empty row"


def test_row_tiles_disjoint_and_identical_selections():
    # rows of one tile with disjoint selections (the union is twice a row's)
    # and with identical ones (the union is one row's)
    rng = rng_for(731)
    B, Q, H, N, K = 2, 4, 16, 2048, 64
    lat = normal_bf16(rng, (B, N, 512))
    q = normal_bf16(rng, (B, Q, H, 512))
    perm = rng.permutation(N // 8)
    idx = np.zeros((B, Q, K), np.int32)
    for r in range(Q):
        idx[0, r] = np.sort(perm[r * K:(r + 1) * K])
        idx[1, r] = np.sort(perm[:K])
    count = np.full((B, Q), K, np.int32)
    ne = np.full(B, N, np.int32)
    cache = gpu_cache(lat, N)
    cache_np = np.stack([mxfp4.build_records(lat[b], N) for b in range(B)])
    o, l = gpu_sparse(q, cache, idx, count, ne)
    ro, rl = oracle_rows(q, cache_np, idx, count, ne)
    assert_close_rms(o, ro)
    assert_lse_close(l, rl)


def test_row_tiles_duplicate_ids_count_twice():
    # a row listing a block twice attends its entries twice (as the oracle and
    # the single-row tiles do); the tile then runs its rows' lists in turn
    rng = rng_for(732)
    B, Q, H, N, K = 1, 4, 16, 1024, 24
    lat = normal_bf16(rng, (B, N, 512))
    q = normal_bf16(rng, (B, Q, H, 512))
    idx, count = _selections(rng, B, Q, N // 8, K, shared=12, extra=12)
    idx[0, 2, 5] = idx[0, 2, 4]               # a duplicate in row 2
    ne = np.full(B, N, np.int32)
    cache = gpu_cache(lat, N)
    cache_np = np.stack([mxfp4.build_records(lat[0], N)])
    o, l = gpu_sparse(q, cache, idx, count, ne)
    ro, rl = oracle_rows(q, cache_np, idx, count, ne)
    assert_close_rms(o, ro)
    assert_lse_close(l, rl)


def test_row_tiles_cache_beyond_the_bitmap():
    # 4 rows per tile (8 heads): the union's bitmap covers 65536 blocks; a
    # cache of 65544 blocks runs the rows' lists in turn.  Only two chunks of
    # the cache hold data (the rest stays zero: present entries of value 0).
    rng = rng_for(733)
    lib = _lib()
    Q, H, K = 4, 8, 40
    nb = 65544
    cap = nb * 8
    chunks = [(0, 1024), (cap - 1088, 1088)]
    cache = torch.zeros(1, nb, 2176, dtype=torch.uint8, device="cuda")
    cache_np = np.zeros((nb, 2176), np.uint8)
    for start, n in chunks:
        lat = normal_bf16(rng, (1, n, 512))
        lib.append_fp4(dev_bf16(lat), dev(np.array([start], np.int32)), cache)
        mxfp4.write_records(cache_np, lat[0], start)
    blocks = np.concatenate([np.arange(0, 128), np.arange(nb - 136, nb), rng.choice(nb, 64, replace=False)])
    idx = np.stack([np.sort(rng.choice(np.unique(blocks), K, replace=False)) for _ in range(Q)])[None].astype(np.int32)
    count = np.full((1, Q), K, np.int32)
    q = normal_bf16(rng, (1, Q, H, 512))
    o, l = gpu_sparse(q, cache, idx, count, np.array([cap], np.int32))
    torch.cuda.synchronize()
    ro, rl = oracle_rows(q, cache_np[None], idx, count, np.array([cap]))
    assert_close_rms(o, ro)
    assert_lse_close(l, rl)


@pytest.mark.parametrize("H,Q", [(16, 4), (8, 5)])
def test_row_tiles_attend_layer(H, Q):
    # draft rows after the cache (each row sees every entry and its own
    # window of W tokens), in the one-call layer
    rng = rng_for(740 + H)
    B, N, K, W = 3, 2048, 64, 128
    lat = normal_bf16(rng, (B, N, 512))
    cache = gpu_cache(lat, N)
    cache_np = [mxfp4.build_records(lat[b], N) for b in range(B)]
    q = normal_bf16(rng, (B, Q, H, 512))
    Lw = W + Q - 1
    swa = normal_bf16(rng, (B, Lw, 512))
    swa_len = np.full(B, Lw, np.int32)
    pos0 = 2 * N - W + 1
    q_pos = np.broadcast_to(2 * N + np.arange(Q, dtype=np.int32), (B, Q)).copy()
    idx, count = _selections(rng, B, Q, N // 8, K, shared=50, extra=14)
    count[2, 1] = 0
    ne = np.full(B, N, np.int32)
    out, lse = gpu_layer(q, cache, idx, count, ne, swa, swa_len, W, swa_pos0=np.full(B, pos0), q_pos=q_pos)
    for b in range(B):
        for r in range(Q):
            ro, rl = modes.attend_row(q[b, r], cache_np[b], idx[b, r], int(count[b, r]), N, swa[b], Lw, W,
                                      q_pos=int(q_pos[b, r]), swa_pos0=pos0)
            assert_close_rms(out[b, r], ro, what=f"row ({b}, {r})")
            assert_lse_close(lse[b, r], rl)


@pytest.mark.parametrize("H,Q", [(16, 3), (8, 4)])
def test_row_tiles_swa_merge(H, Q):
    # the standalone window call on row tiles: causal rows of one sequence at
    # different positions (their windows overlap only in part), one sequence
    # with a short window; merged with the oracle's sparse branch
    rng = rng_for(760 + H)
    B, N, K, W, Lw = 2, 1024, 24, 96, 160
    lat = normal_bf16(rng, (B, N, 512))
    cache_np = [mxfp4.build_records(lat[b], N) for b in range(B)]
    q = normal_bf16(rng, (B, Q, H, 512))
    swa = normal_bf16(rng, (B, Lw, 512))
    swa_len = np.array([Lw, 40], np.int32)
    pos0 = np.array([2 * N - 100, 2 * N - 30], np.int32)
    q_pos = np.stack([2 * N - 100 + 37 * np.arange(Q) + 50, 2 * N - 30 + np.arange(Q) + 5]).astype(np.int32)
    idx, count = _selections(rng, B, Q, N // 8, K, shared=12, extra=12)
    o_s = np.zeros((B, Q, H, 512))
    l_s = np.zeros((B, Q, H))
    for b in range(B):
        for r in range(Q):
            o1, l1 = oracle_rows(q[b:b + 1, r:r + 1], cache_np[b][None], idx[b:b + 1, r:r + 1],
                                 count[b:b + 1, r:r + 1], [N], q_pos[b:b + 1, r:r + 1])
            o_s[b, r], l_s[b, r] = o1[0, 0], l1[0, 0]
    from tests.test_gpu_attention import gpu_swa
    out, lse = gpu_swa(q, swa, swa_len, W, o_s, l_s, swa_pos0=pos0, q_pos=q_pos)
    for b in range(B):
        for r in range(Q):
            ro, rl = modes.attend_row(q[b, r], cache_np[b], idx[b, r], int(count[b, r]), N, swa[b],
                                      int(swa_len[b]), W, q_pos=int(q_pos[b, r]), swa_pos0=int(pos0[b]))
            assert_close_rms(out[b, r], ro, what=f"row ({b}, {r})")
            assert_lse_close(lse[b, r], rl)
