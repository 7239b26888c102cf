"""Pins for the oracle's MXFP4 encoding (CPU only).

The E2M1 value table, the E8M0 scale rule and round-to-nearest-even come from
the OCP Microscaling Formats (MX) v1.0 specification, cited by name; the pages
only say "FP4" (news.promptgoblins.ai summary, Details: "FP4 KVCache
precision").
"""

import numpy as np
import pytest

from oracle import mxfp4
from tests import pins


def test_page_constants_golden():
    """Structural numbers the pages print, from tests/golden/page_constants.txt."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "page_constants.txt")
    vals = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = int(v)
    assert mxfp4.D == vals["latent_dim"]
    assert mxfp4.BLOCK == vals["block_entries"]
    from oracle import indexer
    assert indexer.BLOCK == vals["block_entries"]
    assert vals["positions_per_entry"] == 2


def test_e2m1_table_roundtrip_all_16_codes():
    # decode every code at scale 2**s (planted by 6*2**s in the group) and re-encode
    for s in (-3, 0, 5):
        X = 2.0 ** s
        vals = [pins.E2M1_TABLE[c & 7] * X * (-1.0 if c & 8 else 1.0) for c in range(16)]
        row = np.zeros((1, 512), dtype=np.uint16)
        row[0, 0] = pins.f32_to_bf16_bits(6.0 * X)
        for c in range(16):
            row[0, 1 + c] = pins.f32_to_bf16_bits(vals[c])
        codes, sb = mxfp4.encode_values(row)
        assert sb[0, 0] == s + 127
        assert codes[0, 0] == 7
        for c in range(16):
            assert codes[0, 1 + c] == c, (s, c)
        dec = mxfp4.decode_values(codes, sb)
        for c in range(16):
            assert dec[0, 1 + c] == vals[c]
            assert np.signbit(dec[0, 1 + c]) == bool(c & 8) or vals[c] != 0


def test_decode_table_matches_spec():
    codes = np.zeros((1, 512), dtype=np.uint8)
    codes[0, :16] = np.arange(16)
    sb = np.full((1, 16), 127, dtype=np.uint8)
    dec = mxfp4.decode_values(codes, sb)
    for c in range(16):
        exp = pins.E2M1_TABLE[c & 7] * (-1 if c & 8 else 1)
        assert dec[0, c] == exp


@pytest.mark.parametrize("s", [0, -2, 7])
def test_exhaustive_bf16_sweep(s):
    bad = pins.check_encode_sweep(mxfp4.encode_values, pin_exponent=s)
    assert not bad, bad


def test_tie_points_and_saturation_closed_form():
    # at scale 1 (amax pinned to 6): halfway points go to the even code, >6 saturates
    cases = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
             (0.203125, 0), (0.30078125, 1), (2.59375, 5), (5.5, 7), (6.0, 7)]
    row = np.zeros((1, 512), dtype=np.uint16)
    row[0, 0] = pins.f32_to_bf16_bits(6.0)
    for i, (v, _) in enumerate(cases):
        row[0, 1 + i] = pins.f32_to_bf16_bits(float(np.float32(v)))
        row[0, 16 + i] = pins.f32_to_bf16_bits(-float(np.float32(v)))
    codes, sb = mxfp4.encode_values(row)
    assert sb[0, 0] == 127
    for i, (v, c) in enumerate(cases):
        assert codes[0, 1 + i] == c, v
        assert codes[0, 16 + i] == c | 8, v
    # amax in (6, 8) keeps scale 1 and saturates the largest values to 6
    row2 = np.zeros((1, 512), dtype=np.uint16)
    row2[0, 0] = pins.f32_to_bf16_bits(7.5)
    codes2, sb2 = mxfp4.encode_values(row2)
    assert sb2[0, 0] == 127 and codes2[0, 0] == 7


def test_scale_equivariance_and_sign_symmetry():
    from synth import normal_bf16, rng_for
    x = normal_bf16(rng_for(7), (64, 512))
    codes, sb = mxfp4.encode_values(x)
    for k in (-5, 3):
        xk = pins_scale(x, k)
        ck, sk = mxfp4.encode_values(xk)
        assert np.array_equal(ck, codes)
        assert np.array_equal(sk.astype(int), sb.astype(int) + k)
    neg = x ^ np.uint16(0x8000)
    cn, sn = mxfp4.encode_values(neg)
    assert np.array_equal(sn, sb)
    assert np.array_equal(cn, codes ^ np.uint8(8))


def pins_scale(bits, k):
    """Multiply bf16 values by 2**k exactly (exponent field add, values stay normal)."""
    b = bits.astype(np.int32)
    exp = (b >> 7) & 0xFF
    assert ((exp == 0) | ((exp + k > 0) & (exp + k < 255))).all()
    out = np.where(exp == 0, b, b + (k << 7))
    return out.astype(np.uint16)


def test_error_bound():
    from synth import normal_bf16, rng_for
    x = normal_bf16(rng_for(11), (256, 512))
    codes, sb = mxfp4.encode_values(x)
    xf = pins_f64(x).reshape(256, 16, 32)
    dq = mxfp4.decode_values(codes, sb).reshape(256, 16, 32)
    X = np.ldexp(1.0, sb.astype(np.int64) - 127)[..., None]
    v = np.abs(xf) / X
    half_step = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    unsat = v <= 6
    err = np.abs(xf - dq) / X
    assert (err[unsat] <= half_step[unsat]).all()
    # saturated values land on 6
    assert (np.abs(dq[~unsat]) == 6 * np.broadcast_to(X, dq.shape)[~unsat]).all()


def pins_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_zero_and_nonfinite_groups():
    row = np.zeros((1, 512), dtype=np.uint16)
    row[0, 32:64] = 0x8000                     # -0.0 group
    row[0, 64] = 0x7F80                        # +inf in group 2
    row[0, 96] = 0x7FC0                        # NaN in group 3
    row[0, 128] = 0x0001                       # smallest bf16 subnormal in group 4
    codes, sb = mxfp4.encode_values(row)
    assert sb[0, 0] == 0 and (codes[0, :32] == 0).all()
    assert sb[0, 1] == 0 and (codes[0, 32:64] == 8).all()
    assert sb[0, 2] == 255 and (codes[0, 64:96] == 0).all()
    assert sb[0, 3] == 255 and (codes[0, 96:128] == 0).all()
    # 2**-133: floor(log2) = -133 -> sb clamps to 0, value/2**-127 = 2**-6 rounds to 0
    assert sb[0, 4] == 0 and codes[0, 128] == 0


def test_largest_finite_scale_is_252_and_dequant_exact_in_bf16():
    row = np.zeros((1, 512), dtype=np.uint16)
    row[0, 0] = 0x7F7F                         # largest finite bf16
    codes, sb = mxfp4.encode_values(row)
    assert sb[0, 0] == 252 and codes[0, 0] == 7
    # every code x every producible scale byte is exactly representable in bf16
    for s in range(0, 253):
        for c in range(8):
            v = pins.E2M1_TABLE[c] * 2.0 ** (s - 127)
            f = np.float32(v)
            assert float(f) == v
            b = np.array([f], dtype=np.float32).view(np.uint32)[0]
            assert (b & 0xFFFF) == 0, (s, c)


def test_record_layout_and_packing():
    from synth import normal_bf16, rng_for
    lat = normal_bf16(rng_for(3), (21, 512))          # 2 full blocks + a partial one
    cache = mxfp4.build_records(lat, cap=32)
    assert cache.shape == (4, 2176)
    codes, sb = mxfp4.encode_values(lat)
    for j in range(21):
        b, r = divmod(j, 8)
        packed = cache[b, 256 * r:256 * r + 256]
        # low nibble = even dim, high nibble = odd dim
        assert np.array_equal(packed & 0xF, codes[j, 0::2])
        assert np.array_equal(packed >> 4, codes[j, 1::2])
        assert np.array_equal(cache[b, 2048 + 16 * r:2048 + 16 * r + 16], sb[j])
    # untouched tail of the partial block and the empty block stay zero
    assert (cache[2, 256 * 5:2048] == 0).all() and (cache[2, 2048 + 16 * 5:] == 0).all()
    assert (cache[3] == 0).all()
    dec = mxfp4.read_entries(cache, np.arange(21))
    assert np.array_equal(dec, mxfp4.quantize_dequantize(lat))
