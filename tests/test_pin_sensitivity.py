"""Plant plausible mistakes in copies of oracle routines (CPU only) and check the pins catch them."""

import math

import numpy as np

from oracle import attention, indexer, mxfp4, topk
from synth import bf16_to_f32, normal_bf16, rng_for
from tests import pins

SWEEP_ROWS = np.arange(0, 65280, 7)          # a spread subset keeps this fast


def _encode_with(round_fn=None, scale_fn=None, keep_sign_on_zero=True):
    def enc(bits):
        bits = np.asarray(bits, dtype=np.uint16)
        g = bits.reshape(bits.shape[:-1] + (16, 32))
        x = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        amax = np.abs(x).max(-1)
        sb = (scale_fn or mxfp4.scale_byte)(amax)
        X = np.ldexp(1.0, sb - 127)
        mag = (round_fn or mxfp4.round_magnitude)(np.abs(x) / X[..., None])
        sign = ((g >> 15) & 1).astype(np.uint8)
        if not keep_sign_on_zero:
            sign = np.where(mag == 0, 0, sign).astype(np.uint8)
        code = (sign << 3) | mag
        return code.reshape(bits.shape), sb.astype(np.uint8)
    return enc


def test_sweep_accepts_oracle():
    assert not pins.check_encode_sweep(mxfp4.encode_values, rows=SWEEP_ROWS)


def test_sweep_catches_ties_away_from_zero():
    def round_half_up(a):
        return np.searchsorted(mxfp4._MID, a, side="right").astype(np.uint8)
    assert pins.check_encode_sweep(_encode_with(round_fn=round_half_up), rows=SWEEP_ROWS)


def test_sweep_catches_ceil_scale_rule():
    def ceil_rule(amax):
        # non-saturating variant: smallest scale with amax / X <= 6
        e = np.ceil(np.log2(np.where(amax > 0, amax, 1) / 6.0)).astype(np.int64)
        return np.where(amax > 0, np.clip(e + 127, 0, 254), 0)
    assert pins.check_encode_sweep(_encode_with(scale_fn=ceil_rule), rows=SWEEP_ROWS)


def test_sweep_catches_dropped_negative_zero_sign():
    assert pins.check_encode_sweep(_encode_with(keep_sign_on_zero=False), rows=SWEEP_ROWS)


def test_sweep_catches_no_saturation():
    def no_sat(a):
        c = mxfp4.round_magnitude(a)
        return np.where(a > 6, 0, c).astype(np.uint8)
    assert pins.check_encode_sweep(_encode_with(round_fn=no_sat), rows=SWEEP_ROWS)


def test_dense_pin_catches_attention_mistakes():
    rng = rng_for(1)
    q = normal_bf16(rng, (2, 512))
    kv = bf16_to_f32(normal_bf16(rng, (6, 512))).astype(np.float64)
    ref_o, ref_l = pins.dense_attention_loops(bf16_to_f32(q).astype(float).tolist(), kv.tolist(),
                                              attention.SCALE_512)
    good_o, good_l = attention.attend(q, kv, attention.SCALE_512)
    assert np.allclose(good_o, ref_o, rtol=1e-10)
    # missing 1/sqrt(d) scale
    bad_o, _ = attention.attend(q, kv, 1.0)
    assert not np.allclose(bad_o, ref_o, rtol=1e-3)
    # lse without the max term
    qf = bf16_to_f32(q).astype(np.float64)
    z = attention.SCALE_512 * qf @ kv.T
    bad_l = np.log(np.exp(z - z.max(1, keepdims=True)).sum(1))
    assert not np.allclose(bad_l, ref_l, rtol=1e-3)


def test_loop_pin_catches_indexer_mistakes():
    rng = rng_for(2)
    q = normal_bf16(rng, (3, 64))
    w = np.array([0.9, -1.2, 0.4], np.float32)
    k = normal_bf16(rng, (32, 64))
    qf, kf = bf16_to_f32(q), bf16_to_f32(k)
    ref = np.array([pins.entry_score_loops(qf, w, kf[j]) for j in range(32)])
    assert np.allclose(indexer.entry_scores(q, w, k), ref, rtol=1e-12)
    no_relu = (kf.astype(np.float64) @ qf.T.astype(np.float64)) @ w.astype(np.float64)
    assert not np.allclose(no_relu, ref, rtol=1e-6)
    relu_after = np.maximum((kf.astype(np.float64) @ qf.T.astype(np.float64)) @ w, 0)
    assert not np.allclose(relu_after, ref, rtol=1e-6)


def test_pairwise_pin_catches_wrong_tie_rule():
    s = np.array([3, 1, 3, 2, 3, 0, 3], dtype=np.float64)
    exp = pins.topk_pairwise(s, 2)
    got, c = topk.select(s, 2)
    assert got[:c].tolist() == exp == [0, 2]
    order = sorted(range(7), key=lambda b: (-s[b], -b))       # ties to the higher id
    assert sorted(order[:2]) != exp
    assert math.isinf(topk.gap_at_rank(np.array([1.0, 2.0]), 2))
