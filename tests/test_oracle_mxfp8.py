"""Pins for the oracle's MXFP8 (E4M3) indexer-key encoding (CPU only).

The E4M3 element format (bias 7, subnormals, 448 as the largest finite value,
S.1111.111 as NaN, no infinities), the E8M0 scale and round-to-nearest-even come
from the OCP Microscaling Formats (MX) v1.0 specification and the OCP 8-bit
floating point specification, cited by name; the pages give the indexer no
precision (observer.broadside.tech card, Key ideas, "CSA2 with three static
layer modes").
"""

import numpy as np

from oracle import bf16, mxfp8
from synth import normal_bf16, rng_for


def _bits(vals):
    """float values (exactly representable in bf16) -> bf16 bit patterns."""
    f = np.asarray(vals, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16.to_f64(b), np.asarray(vals, dtype=np.float64)), "not bf16-exact"
    return b


def _key(group0, group1):
    """A 64-d key from two 32-value groups (short lists are zero-padded)."""
    k = np.zeros(64)
    k[:len(group0)] = group0
    k[32:32 + len(group1)] = group1
    return _bits(k)


def test_spec_values():
    # OCP FP8 E4M3: S.0000.001 = 2^-9 (min subnormal), S.0000.111 = 0.875 * 2^-6
    # (max subnormal), S.0001.000 = 2^-6 (min normal), S.0111.000 = 1,
    # S.1111.110 = 448 (max normal), S.1111.111 = NaN, sign bit 7
    v = mxfp8.code_value(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x40, 0x30, 0x77, 0x7E,
                                   0x80, 0xB8, 0xFE], np.uint8))
    assert np.array_equal(v, [0.0, 2.0 ** -9, 0.875 * 2.0 ** -6, 2.0 ** -6, 1.0, 1.5, 2.0, 0.5, 240.0,
                              448.0, -0.0, -1.0, -448.0])
    assert np.signbit(v[10])
    assert np.isnan(mxfp8.code_value(np.array([0x7F, 0xFF], np.uint8))).all()


def test_grid_structure():
    m = mxfp8.MAG
    assert len(m) == 127 and m[0] == 0.0 and m[-1] == 448.0
    assert (np.diff(m) > 0).all()
    # spacing 2^-9 through the subnormals and the first binade, then doubling per binade
    d = np.diff(m)
    assert (d[:8] == 2.0 ** -9).all()
    for e in range(1, 16):        # binade e: codes 8e .. 8e + 7, step 2^(e - 10)
        assert (d[8 * e:8 * e + 8] == 2.0 ** (e - 10)).all(), e


def test_every_code_round_trips():
    # groups scaled by X = 1 (largest value 256: floor(log2) = 8, byte 127);
    # every E4M3 magnitude and its negative encode to its own code
    mags = mxfp8.MAG
    for lo in range(0, 127, 31):
        vals = np.concatenate([[256.0], mags[lo:lo + 31]])
        k = _key(vals, -vals)
        codes, sb = mxfp8.encode_keys(k)
        assert list(sb) == [127, 127]
        want = np.concatenate([[0x78], np.arange(lo, lo + len(vals) - 1)]).astype(np.uint8)
        assert np.array_equal(codes[:len(vals)], want)
        assert np.array_equal(codes[32:32 + len(vals)], want | 0x80)
        assert np.array_equal(mxfp8.decode_keys(codes, sb)[:len(vals)], vals)


def test_ties_to_even_and_saturation():
    # X = 1 groups: halfway points go to the even code, above 448 saturates
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
             (1.09375, 0x39), (304.0, 0x7A), (450.0, 0x7E), (464.0, 0x7E), (480.0, 0x7E),
             (510.0, 0x7E), (300.0, 0x79)]
    vals = [256.0] + [c[0] for c in cases]
    codes, sb = mxfp8.encode_keys(_key(vals, []))
    assert sb[0] == 127
    assert list(codes[1:len(vals)]) == [c[1] for c in cases]


def test_scale_rule():
    # byte = floor(log2 amax) - 8 + 127, clamped to [0, 254]; 0 for an all-zero group
    for amax, want in [(1.0, 119), (0.75, 118), (1.5, 119), (256.0, 127), (510.0, 127), (512.0, 128),
                       (2.0 ** 100, 219), (2.0 ** -133, 0), (2.0 ** -120, 0), (2.0 ** -118, 1)]:
        _, sb = mxfp8.encode_keys(_key([amax], [0.0]))
        assert sb[0] == want, (amax, sb[0])
        assert sb[1] == 0
    # the smallest bf16 subnormal with the clamped scale: 2^-133 / 2^-127 = 2^-6
    codes, _ = mxfp8.encode_keys(_key([2.0 ** -133], []))
    assert codes[0] == 0x08


def test_sign_of_zero():
    codes, sb = mxfp8.encode_keys(_key([-0.0, 1.0, -2.0 ** -20], [-0.0]))
    assert codes[0] == 0x80 and codes[2] == 0x80 and codes[32] == 0x80
    assert sb[1] == 0


def test_error_bound_random_keys():
    rng = rng_for(808)
    k = normal_bf16(rng, (2000, 64))
    x = bf16.to_f64(k)
    codes, sb = mxfp8.encode_keys(k)
    d = mxfp8.decode_keys(codes, sb)
    X = np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), 32, axis=-1)
    a = np.abs(x) / X
    sat = a > 448
    assert np.array_equal(d[sat], np.sign(x[sat]) * 448 * X[sat])
    err = np.abs(d - x)
    # half a unit in the last place: 2^-4 relative for normals, 2^-10 absolute below 2^-6
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * X)
    assert (err[~sat] <= bound[~sat]).all()
    # and the chosen grid value is a nearest one: neither neighbour is closer
    c = (codes & 0x7F).astype(np.int64)[~sat]
    aa = a[~sat]
    dist = np.abs(mxfp8.MAG[c] - aa)
    assert (dist <= np.abs(mxfp8.MAG[np.minimum(c + 1, 126)] - aa)).all()
    assert (dist <= np.abs(mxfp8.MAG[np.maximum(c - 1, 0)] - aa)).all()


def _pins_fail(encode):
    """Run the fixed-case pins above against an encoder; return True if any fails."""
    try:
        cases = [(1.0625, 0x38), (1.1875, 0x3A), (480.0, 0x7E), (300.0, 0x79)]
        vals = [256.0] + [c[0] for c in cases]
        codes, sb = encode(_key(vals, [-0.0]))
        ok = sb[0] == 127 and list(codes[1:len(vals)]) == [c[1] for c in cases] and codes[32] == 0x80
        _, sb2 = encode(_key([1.5], []))
        ok = ok and sb2[0] == 119
        return not ok
    except Exception:
        return True


def _encoder(round_fn=None, scale_fn=None, keep_sign_on_zero=True):
    def enc(bits):
        g = np.asarray(bits, np.uint16).reshape(2, 32)
        x = bf16.to_f64(g)
        sb = (scale_fn or mxfp8.scale_byte)(np.abs(x).max(-1))
        mag = (round_fn or mxfp8.round_magnitude)(np.abs(x) / np.ldexp(1.0, sb - 127)[:, None])
        sign = ((g >> 15) & 1).astype(np.uint8)
        if not keep_sign_on_zero:
            sign = np.where(mag == 0, 0, sign).astype(np.uint8)
        return ((sign << 7) | mag).reshape(64).astype(np.uint8), sb.astype(np.uint8)
    return enc


def test_pins_accept_oracle_and_catch_planted_mistakes():
    assert not _pins_fail(mxfp8.encode_keys)
    assert not _pins_fail(_encoder())
    half_up = lambda a: np.minimum(np.searchsorted(mxfp8._MID, a, side="right"), 126).astype(np.uint8)
    no_sat = lambda a: np.where(a > 448, 127, mxfp8.round_magnitude(a)).astype(np.uint8)
    truncate = lambda a: np.maximum(np.searchsorted(mxfp8.MAG, a, side="right") - 1, 0).astype(np.uint8)
    minus7 = lambda amax: np.where(amax > 0, np.clip(np.frexp(amax)[1] - 1 - 7 + 127, 0, 254), 0)
    for bad in (_encoder(round_fn=half_up), _encoder(round_fn=no_sat), _encoder(round_fn=truncate),
                _encoder(scale_fn=minus7), _encoder(keep_sign_on_zero=False)):
        assert _pins_fail(bad)
