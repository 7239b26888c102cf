"""MXFP4 encode / decode of the 512-d latent cache entries (oracle; test infrastructure).

The pages say the global KV cache is stored in 4-bit floating point
([news] Details, "FP4 KVCache precision"; [abstract]; [card] Key ideas, "FP4
global KV, trained that way") and that one 512-d latent per entry serves as key
and value for every head ([digest] Core Mechanics, "Compressed along three
axes").  They do not name the FP4 variant, the scaling, the rounding or the byte
layout.  Readings taken here (all of them choices, listed in the design notes):

* Variant: MXFP4 as in the OCP Microscaling Formats (MX) v1.0 specification --
  FP4 E2M1 elements, one E8M0 (power-of-two) scale per 32 consecutive values.
  E2M1 magnitudes, by 3-bit code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* Scale: E = floor(log2(amax)) over the 32 values, scale byte
  sb = clamp(E - 2 + 127, 0, 254) (2 = exponent of the largest E2M1 value 6),
  scale X = 2**(sb - 127).  amax == 0 gives sb = 0.
* Rounding of |x|/X to the E2M1 grid: nearest value, exact halfway cases go to
  the code whose lowest (mantissa) bit is 0; magnitudes above 6 saturate to 6.
* Sign: bit 3 of the code is the sign bit of x, also when the magnitude rounds
  to 0 (so -0.0 and tiny negatives give code 0x8).
* A group holding a NaN or an infinity gets sb = 255 (the E8M0 NaN) and all
  codes 0.  Never produced for finite inputs.
* Packing: byte k of an entry holds code[2k] in the low nibble and code[2k+1]
  in the high nibble (256 bytes per 512-value entry).
* Block record (8 entries = one selection block): bytes [0, 2048) hold the 8
  entries' packed codes, entry-major (256 B each); bytes [2048, 2176) hold the
  8 entries' 16 scale bytes, entry-major (16 B each).  2176 B per block.

Every step is exact: inputs are bfloat16, the scale is a power of two, so x / X
and all comparisons are exact in float64.
"""

import numpy as np

from . import bf16

D = 512                  # latent width
GROUP = 32               # values per E8M0 scale
NGROUPS = D // GROUP     # 16 scales per entry
ENTRY_CODE_BYTES = D // 2          # 256
BLOCK = 8                # entries per selection block
RECORD_BYTES = BLOCK * (ENTRY_CODE_BYTES + NGROUPS)   # 2176
SCALE_OFFSET = BLOCK * ENTRY_CODE_BYTES               # 2048

# E2M1 magnitudes by 3-bit code (OCP MX v1.0, FP4 E2M1 element table).
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
# Halfway points between neighbouring grid values.
_MID = (E2M1[:-1] + E2M1[1:]) / 2.0   # 0.25 0.75 1.25 1.75 2.5 3.5 5.0


def scale_byte(amax):
    """E8M0 scale byte for a group with largest magnitude ``amax`` (float64 array).

    floor(log2(amax)) is read off the binary exponent (frexp), never a floating
    log2: amax = m * 2**e with m in [0.5, 1) gives floor(log2 amax) = e - 1.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    E = e.astype(np.int64) - 1
    sb = np.clip(E - 2 + 127, 0, 254)
    return np.where(amax > 0, sb, 0).astype(np.int64)


def round_magnitude(a):
    """Round magnitudes ``a`` (>= 0, float64, already divided by the scale) to E2M1 codes 0..7.

    Nearest grid value; an exact halfway case takes the even code; a > 6 saturates
    to code 7 (value 6).
    """
    a = np.asarray(a, dtype=np.float64)
    # number of halfway points strictly below a: a lies in (MID[c-1], MID[c]],
    # whose nearest grid value is code c unless a sits exactly on MID[c].
    c = np.searchsorted(_MID, a, side="left")
    on_mid = (c < len(_MID)) & (_MID[np.minimum(c, len(_MID) - 1)] == a)
    # tie between codes c and c+1: keep the one with mantissa bit 0
    c = np.where(on_mid & (c % 2 == 1), c + 1, c)
    return c.astype(np.uint8)       # a > 5 gives 7 (a > 6 saturates to 6)


def encode_values(bits):
    """Encode bfloat16 values ``bits`` [..., 512] (uint16) -> (codes [..., 512] u8, sb [..., 16] u8).

    ``codes`` are unpacked 4-bit codes (sign << 3 | magnitude code).
    """
    bits = np.asarray(bits, dtype=np.uint16)
    assert bits.shape[-1] == D
    lead = bits.shape[:-1]
    g = bits.reshape(lead + (NGROUPS, GROUP))
    x = bf16.to_f64(g)
    nonfinite = ~np.isfinite(x).all(axis=-1)                 # [..., 16]
    ax = np.where(np.isfinite(x), np.abs(x), 0.0)
    amax = ax.max(axis=-1)
    sb = scale_byte(amax)
    X = np.ldexp(1.0, sb - 127)                               # exact powers of two
    a = ax / X[..., None]                                     # exact division
    mag = round_magnitude(a)
    sign = ((g >> np.uint16(15)) & np.uint16(1)).astype(np.uint8)
    code = (sign << np.uint8(3)) | mag
    code = np.where(nonfinite[..., None], np.uint8(0), code).astype(np.uint8)
    sb = np.where(nonfinite, 255, sb).astype(np.uint8)
    return code.reshape(lead + (D,)), sb


def pack_codes(codes):
    """Unpacked codes [..., 512] -> packed bytes [..., 256] (even value in the low nibble)."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes[..., 0::2] & np.uint8(0xF)
    hi = codes[..., 1::2] & np.uint8(0xF)
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack_codes(packed):
    """Packed bytes [..., 256] -> codes [..., 512]."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (D,), dtype=np.uint8)
    out[..., 0::2] = packed & np.uint8(0xF)
    out[..., 1::2] = packed >> np.uint8(4)
    return out


def decode_values(codes, sb):
    """codes [..., 512] + scale bytes [..., 16] -> float64 values [..., 512].

    value = (-1)**s * E2M1[mag] * 2**(sb - 127); sb == 255 decodes to NaN.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    sb = np.asarray(sb, dtype=np.int64)
    lead = codes.shape[:-1]
    c = codes.reshape(lead + (NGROUPS, GROUP))
    mag = E2M1[(c & 7).astype(np.int64)]
    sgn = np.where((c >> 3) & 1, -1.0, 1.0)
    X = np.ldexp(1.0, sb - 127)[..., None]
    v = sgn * mag * X
    v = np.where((sb == 255)[..., None], np.nan, v)
    return v.reshape(lead + (D,))


def build_records(latent_bits, cap):
    """Encode entries [n][512] (bf16 bits) into a zero-filled block-record cache [cap/8][2176] u8.

    Entries n..cap-1 stay zero (the caller zero-fills an empty cache).
    """
    latent_bits = np.asarray(latent_bits, dtype=np.uint16)
    n = latent_bits.shape[0]
    assert cap % BLOCK == 0 and n <= cap
    cache = np.zeros((cap // BLOCK, RECORD_BYTES), dtype=np.uint8)
    write_records(cache, latent_bits, 0)
    return cache


def write_records(cache, latent_bits, start):
    """Encode entries and store them at entry positions start.. of a record cache (in place)."""
    codes, sb = encode_values(latent_bits)
    packed = pack_codes(codes)
    for i in range(latent_bits.shape[0]):
        j = start + i
        blk, r = divmod(j, BLOCK)
        cache[blk, r * ENTRY_CODE_BYTES:(r + 1) * ENTRY_CODE_BYTES] = packed[i]
        cache[blk, SCALE_OFFSET + r * NGROUPS:SCALE_OFFSET + (r + 1) * NGROUPS] = sb[i]
    return cache


def read_entries(cache, entries):
    """Decode entry ids ``entries`` of a record cache -> float64 [len][512]."""
    cache = np.asarray(cache, dtype=np.uint8)
    entries = np.asarray(entries, dtype=np.int64)
    blk, r = np.divmod(entries, BLOCK)
    code_off = r[:, None] * ENTRY_CODE_BYTES + np.arange(ENTRY_CODE_BYTES)[None, :]
    sc_off = SCALE_OFFSET + r[:, None] * NGROUPS + np.arange(NGROUPS)[None, :]
    packed = cache[blk[:, None], code_off]
    sb = cache[blk[:, None], sc_off]
    return decode_values(unpack_codes(packed), sb)


def quantize_dequantize(latent_bits):
    """Round trip float64 values of bf16 entries [..., 512] through MXFP4."""
    codes, sb = encode_values(latent_bits)
    return decode_values(codes, sb)
