"""MXFP8 (E4M3) encode / decode of the 64-d indexer keys (oracle; test infrastructure).

A lower-precision variant of the indexer key cache.  The pages store the global
latent in FP4 ([card] Key ideas, "FP4 global KV, trained that way"; [news]
Details, "FP4 KVCache precision") and name the indexer ([card] Key ideas, "CSA2
with three static layer modes") without giving its precision; the default key
cache holds the keys in bfloat16.  This variant keeps them in 8-bit
microscaling form, halving the bytes the (memory-bound) indexer reads.  Readings
taken here (choices, listed in the design notes):

* Variant: MXFP8 with E4M3 elements as in the OCP Microscaling Formats (MX) v1.0
  specification -- 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
  exponent field 0 holds the subnormals m * 2**-9; exponent field 15 with
  mantissa 7 is NaN (there are no infinities); the largest finite magnitude is
  448 = 1.75 * 2**8; one E8M0 (power-of-two) scale per 32 consecutive values.
* Scale: E = floor(log2(amax)) over the 32 values, scale byte
  sb = clamp(E - 8 + 127, 0, 254) (8 = exponent of the largest E4M3 normal),
  scale X = 2**(sb - 127).  amax == 0 gives sb = 0.
* Rounding of |x|/X to the E4M3 grid: nearest value, exact halfway cases go to
  the code whose lowest (mantissa) bit is 0; magnitudes above 448 saturate to
  448 (|x|/X lies below 512, so only the group's largest values can).
* Sign: bit 7 of the code is the sign bit of x, also when the magnitude rounds
  to 0.
* Layout: codes [entry][64] (byte d holds dim d), scales [entry][2] (byte g
  for dims 32g .. 32g + 31).

Inputs are bfloat16 and the scale is a power of two, so x / X and every
comparison below are exact in float64.
"""

import numpy as np

from . import bf16

DI = 64                  # indexer key width
GROUP = 32               # values per E8M0 scale
NGROUPS = DI // GROUP    # 2 scales per key
E4M3_MAX = 448.0


def _magnitudes():
    """Value of each 7-bit magnitude code 0..126 (code 127 is NaN)."""
    c = np.arange(127, dtype=np.int64)
    e, m = c >> 3, c & 7
    sub = np.ldexp(m.astype(np.float64), -9)                       # e == 0: m * 2**-9
    nrm = np.ldexp(1.0 + m.astype(np.float64) / 8.0, (e - 7).astype(np.int64))
    return np.where(e == 0, sub, nrm)


MAG = _magnitudes()                          # strictly increasing, MAG[126] = 448
_MID = (MAG[:-1] + MAG[1:]) / 2.0            # halfway points between neighbours


def code_value(codes):
    """E4M3 codes (uint8) -> float64 values; 0x7F and 0xFF decode to NaN."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = (codes & np.uint8(0x7F)).astype(np.int64)
    v = MAG[np.minimum(mag, 126)]
    v = np.where(mag == 127, np.nan, v)
    return np.where(codes >> np.uint8(7), -v, v)


def scale_byte(amax):
    """E8M0 scale byte for a group with largest magnitude ``amax`` (float64 array).

    floor(log2(amax)) is read off the binary exponent (frexp): amax = m * 2**e
    with m in [0.5, 1) gives floor(log2 amax) = e - 1.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    E = e.astype(np.int64) - 1
    sb = np.clip(E - 8 + 127, 0, 254)
    return np.where(amax > 0, sb, 0).astype(np.int64)


def round_magnitude(a):
    """Round magnitudes ``a`` (>= 0, float64, already divided by the scale) to codes 0..126.

    Nearest grid value; an exact halfway case takes the even code; a > 448
    saturates to code 126.
    """
    a = np.asarray(a, dtype=np.float64)
    # a lies in (MID[c-1], MID[c]]: nearest is code c unless a sits on MID[c]
    c = np.searchsorted(_MID, a, side="left")
    on_mid = (c < len(_MID)) & (_MID[np.minimum(c, len(_MID) - 1)] == a)
    c = np.where(on_mid & (c % 2 == 1), c + 1, c)
    return np.minimum(c, 126).astype(np.uint8)


def encode_keys(bits):
    """bfloat16 keys ``bits`` [..., 64] (uint16) -> (codes [..., 64] u8, sb [..., 2] u8)."""
    bits = np.asarray(bits, dtype=np.uint16)
    assert bits.shape[-1] == DI
    lead = bits.shape[:-1]
    g = bits.reshape(lead + (NGROUPS, GROUP))
    x = bf16.to_f64(g)
    assert np.isfinite(x).all(), "indexer keys must be finite"
    ax = np.abs(x)
    sb = scale_byte(ax.max(axis=-1))
    X = np.ldexp(1.0, sb - 127)
    mag = round_magnitude(ax / X[..., None])
    sign = ((g >> np.uint16(15)) & np.uint16(1)).astype(np.uint8)
    code = (sign << np.uint8(7)) | mag
    return code.reshape(lead + (DI,)).astype(np.uint8), sb.astype(np.uint8)


def decode_keys(codes, sb):
    """codes [..., 64] + scale bytes [..., 2] -> float64 keys [..., 64]."""
    codes = np.asarray(codes, dtype=np.uint8)
    sb = np.asarray(sb, dtype=np.int64)
    lead = codes.shape[:-1]
    v = code_value(codes.reshape(lead + (NGROUPS, GROUP)))
    v = v * np.ldexp(1.0, sb - 127)[..., None]
    return v.reshape(lead + (DI,))


def quantize_dequantize(bits):
    """Round trip bfloat16 keys [..., 64] through MXFP8 -> float64."""
    return decode_keys(*encode_keys(bits))
