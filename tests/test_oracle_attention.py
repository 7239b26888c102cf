"""Pins for the oracle's sparse attention, window branch, merge and modes (CPU only)."""

import math

import numpy as np
import pytest

from oracle import attention, modes, mxfp4
from synth import normal_bf16, rng_for, bf16_to_f32
from tests import pins

S = 1.0 / math.sqrt(512.0)


def _cache(seed, n, cap=None):
    rng = rng_for(seed)
    lat = normal_bf16(rng, (n, 512))
    cap = cap or ((n + 7) // 8) * 8
    return lat, mxfp4.build_records(lat, cap)


def test_all_blocks_selected_equals_dense_loops():
    lat, cache = _cache(1, 21)                 # 3 blocks, last one partial
    rng = rng_for(2)
    q = normal_bf16(rng, (3, 512))
    idx = np.array([2, 0, 1, -1], dtype=np.int32)
    o, lse = attention.sparse_attention(q, cache, idx, 3, n_entries=21)
    kv = mxfp4.quantize_dequantize(lat)
    o2, lse2 = pins.dense_attention_loops(bf16_to_f32(q).astype(float).tolist(), kv.tolist(), S)
    assert np.allclose(o, o2, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, lse2, rtol=1e-12)


def test_softmax_weights_sum_to_one_and_single_entry():
    lat, cache = _cache(3, 16)
    rng = rng_for(4)
    q = normal_bf16(rng, (2, 512))
    qf = bf16_to_f32(q).astype(np.float64)
    kv = mxfp4.quantize_dequantize(lat)
    z = S * qf @ kv.T
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert abs(p.sum(1) - 1).max() < 1e-12
    # V = identity-like probe: o . e_d recovers sum_j p_j kv_jd
    o, _ = attention.attend(q, kv, S)
    assert np.allclose(o, p @ kv, rtol=1e-12)
    # one present entry in the selected block
    o1, l1 = attention.sparse_attention(q, cache, np.array([1]), 1, n_entries=9)
    assert np.array_equal(o1, np.broadcast_to(kv[8], o1.shape))
    assert np.allclose(l1, S * qf @ kv[8], rtol=1e-12)


def test_identical_keys_and_zero_query():
    rng = rng_for(5)
    v = bf16_to_f32(normal_bf16(rng, (1, 512))).astype(np.float64)
    kv = np.repeat(v, 7, axis=0)
    q = normal_bf16(rng, (4, 512))
    o, lse = attention.attend(q, kv, S)
    assert np.allclose(o, np.broadcast_to(v, o.shape), rtol=1e-12)
    kv2 = bf16_to_f32(normal_bf16(rng, (9, 512))).astype(np.float64)
    o0, l0 = attention.attend(np.zeros((2, 512)), kv2, S)
    assert np.allclose(o0, kv2.mean(0), rtol=1e-12)
    assert np.allclose(l0, math.log(9))


def test_index_permutation_invariance_and_padding():
    lat, cache = _cache(6, 64)
    q = normal_bf16(rng_for(7), (4, 512))
    a = attention.sparse_attention(q, cache, np.array([1, 3, 6, -1, -1]), 3, 64)
    b = attention.sparse_attention(q, cache, np.array([6, 1, 3, -1, -1]), 3, 64)
    assert np.allclose(a[0], b[0], rtol=1e-12) and np.allclose(a[1], b[1], rtol=1e-12)


def test_empty_selection():
    lat, cache = _cache(8, 16)
    q = normal_bf16(rng_for(9), (2, 512))
    o, l = attention.sparse_attention(q, cache, np.full(4, -1), 0, 16)
    assert (o == 0).all() and (l == -np.inf).all()


def test_causal_visibility_in_attention():
    lat, cache = _cache(10, 16)
    q = normal_bf16(rng_for(11), (2, 512))
    kv = mxfp4.quantize_dequantize(lat)
    # raw position 9 sees entries with 2j+1 <= 9 -> j <= 4
    o, l = attention.sparse_attention(q, cache, np.array([0, 1]), 2, 16, q_pos=9)
    o2, l2 = attention.attend(q, kv[:5], S)
    assert np.allclose(o, o2, rtol=1e-12) and np.allclose(l, l2, rtol=1e-12)


def test_merge_equals_joint_softmax():
    rng = rng_for(12)
    q = normal_bf16(rng, (3, 512))
    a = bf16_to_f32(normal_bf16(rng, (10, 512))).astype(np.float64)
    b = bf16_to_f32(normal_bf16(rng, (6, 512))).astype(np.float64)
    oa, la = attention.attend(q, a, S)
    ob, lb = attention.attend(q, b, S)
    om, lm = attention.merge(oa, la, ob, lb)
    oj, lj = pins.dense_attention_loops(bf16_to_f32(q).astype(float).tolist(),
                                        np.concatenate([a, b]).tolist(), S)
    assert np.allclose(om, oj, rtol=1e-10, atol=1e-12) and np.allclose(lm, lj, rtol=1e-12)
    # empty branch is the identity
    e_o, e_l = np.zeros_like(oa), np.full(3, -np.inf)
    o1, l1 = attention.merge(oa, la, e_o, e_l)
    assert np.allclose(o1, oa, rtol=1e-14) and np.allclose(l1, la)
    o2, l2 = attention.merge(e_o, e_l, e_o, e_l)
    assert (o2 == 0).all() and (l2 == -np.inf).all()
    # associativity over three parts
    c = bf16_to_f32(normal_bf16(rng, (5, 512))).astype(np.float64)
    oc, lc = attention.attend(q, c, S)
    x = attention.merge(*attention.merge(oa, la, ob, lb), oc, lc)
    y = attention.merge(oa, la, *attention.merge(ob, lb, oc, lc))
    assert np.allclose(x[0], y[0], rtol=1e-12) and np.allclose(x[1], y[1], rtol=1e-12)


def test_window_positions():
    assert attention.window_positions(512, 128).tolist() == list(range(384, 512))
    assert attention.window_positions(50, 128).tolist() == list(range(50))
    # causal: buffer holds raw positions 100..139, query at raw 120, window 8 -> 113..120
    assert attention.window_positions(40, 8, pos0=100, q_pos=120).tolist() == list(range(13, 21))
    assert attention.window_positions(40, 8, pos0=100, q_pos=102).tolist() == [0, 1, 2]


def test_modes_reuse_identity_and_reindex_equals_full():
    rng = rng_for(14)
    n = 256
    lat = normal_bf16(rng, (n, 512))
    cache = mxfp4.build_records(lat, n)
    keys = normal_bf16(rng, (n, 64))
    swa = normal_bf16(rng, (16, 512))
    q1, q2 = normal_bf16(rng, (4, 512)), normal_bf16(rng, (4, 512))
    qi = normal_bf16(rng, (2, 64))
    w = np.array([1.0, 0.5], np.float32)
    i1, c1, o1, l1 = modes.full_layer(q1, qi, w, keys, cache, n, 5, swa, 16, 8)
    i2, c2, o2, l2 = modes.reindex_layer(q1, qi, w, keys, cache, n, 5, swa, 16, 8)
    assert np.array_equal(i1, i2) and c1 == c2 and np.array_equal(o1, o2)
    i3, c3, o3, l3 = modes.reuse_layer(q2, i1, c1, cache, n, swa, 16, 8)
    assert i3.tobytes() == i1.tobytes() and c3 == c1
    # Reuse output = the same attention with the layer's own query
    o4, l4 = modes.attend_row(q2, cache, i1, c1, n, swa, 16, 8)
    assert np.array_equal(o3, o4)
