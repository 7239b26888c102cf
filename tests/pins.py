"""Independent checks ("pins") for the oracle, written as functions of the routine under test.

Each check takes the oracle routine as an argument so that ``test_pin_sensitivity``
can hand it deliberately broken variants (a dropped term, a wrong sign, a wrong
tie rule) and confirm that the check fails.  The checks use methods other than
the oracle's own: brute-force nearest-value search, float.hex() exponents,
explicit Python loops, pairwise rank counting.
"""

import math

import numpy as np

# FP4 E2M1 element magnitudes by 3-bit code, from the OCP Microscaling Formats
# (MX) v1.0 specification's E2M1 table (sign bit is bit 3 of the 4-bit code).
E2M1_TABLE = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}


def f32_to_bf16_bits(x):
    """Truncating float -> bfloat16 bits for values known to be exact in bfloat16."""
    b = np.array([x], dtype=np.float32).view(np.uint32)[0]
    assert (b & 0xFFFF) == 0, x
    return np.uint16(b >> 16)


def bf16_bits_to_float(b):
    return float(np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0])


def floor_log2_hex(a):
    """floor(log2 a) for a > 0 read from float.hex() (independent of frexp)."""
    h = float(a).hex()            # '0x1.8p+2' or '0x0.0000000000001p-1022'
    mant, exp = h.split("p")
    e = int(exp)
    lead = mant[2] if not mant.startswith("-") else mant[3]
    if lead == "1":
        return e
    # subnormal double: count the position of the leading 1 in the fraction
    frac = mant.split(".")[1]
    bits = bin(int(frac, 16))[2:].zfill(len(frac) * 4)
    return e - (bits.index("1") + 1)


def nearest_code_bruteforce(v):
    """E2M1 magnitude code for v >= 0: argmin |v - grid|, exact ties to the even code, >6 -> 7."""
    if v > 6.0:
        return 7
    best, best_d = None, None
    for c in range(8):
        d = abs(v - E2M1_TABLE[c])
        if best is None or d < best_d or (d == best_d and c % 2 == 0 and best % 2 == 1):
            best, best_d = c, d
    return best


def expected_group_encoding(values):
    """Brute-force MXFP4 encoding of one 32-value group given as Python floats."""
    if any(not math.isfinite(v) for v in values):
        return [0] * len(values), 255
    amax = max(abs(v) for v in values)
    if amax == 0:
        sb = 0
    else:
        sb = min(max(floor_log2_hex(amax) - 2 + 127, 0), 254)
    X = 2.0 ** (sb - 127)
    codes = []
    for v in values:
        s = 1 if math.copysign(1.0, v) < 0 else 0
        codes.append((s << 3) | nearest_code_bruteforce(abs(v) / X))
    return codes, sb


def check_encode_sweep(encode_values, pin_exponent=0, rows=None):
    """All finite bfloat16 patterns as x_1 in groups whose other values pin amax >= 6*2**s.

    ``encode_values(bits [n][512]) -> (codes [n][512], sb [n][16])``.  Each row
    holds x_0 = 6*2**s in dim 0, the swept value in dim 1, and a fixed pattern
    elsewhere; the result is compared with ``expected_group_encoding``.
    """
    s = pin_exponent
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (all_bits.astype(np.uint32) << 16).view(np.float32)
    fin = np.isfinite(vals)
    sweep = all_bits[fin]
    if rows is not None:
        sweep = sweep[rows]
    n = sweep.size
    block = np.zeros((n, 512), dtype=np.uint16)
    pin = f32_to_bf16_bits(6.0 * 2.0 ** s)
    block[:, 0] = pin
    block[:, 1] = sweep
    # other groups: a ramp of exact small values, so every group is exercised
    ramp = np.array([f32_to_bf16_bits(v) for v in (0.0, -0.0, 0.5, 1.5, -3.0, 0.75, 5.0, -6.0)],
                    dtype=np.uint16)
    block[:, 32:] = np.tile(ramp, (512 - 32) // 8)
    codes, sb = encode_values(block)
    bad = []
    # group 0 per row
    for i in range(n):
        grp = [bf16_bits_to_float(b) for b in block[i, :32]]
        ec, esb = expected_group_encoding(grp)
        if int(sb[i, 0]) != esb or [int(c) for c in codes[i, :32]] != ec:
            bad.append((hex(int(sweep[i])), int(sb[i, 0]), esb))
            if len(bad) > 5:
                break
    # one representative row for the other groups (identical in every row)
    for g in range(1, 16):
        grp = [bf16_bits_to_float(b) for b in block[0, 32 * g:32 * g + 32]]
        ec, esb = expected_group_encoding(grp)
        if int(sb[0, g]) != esb or [int(c) for c in codes[0, 32 * g:32 * g + 32]] != ec:
            bad.append(("group", g))
    return bad


def dense_attention_loops(q, kv, scale):
    """Plain-loop softmax attention (Python floats, math.exp): q [H][D], kv [n][D]."""
    H, D = len(q), len(q[0])
    o = [[0.0] * D for _ in range(H)]
    lse = [-math.inf] * H
    n = len(kv)
    for h in range(H):
        if n == 0:
            continue
        z = [scale * sum(q[h][d] * kv[j][d] for d in range(D)) for j in range(n)]
        m = max(z)
        e = [math.exp(zj - m) for zj in z]
        l = sum(e)
        for d in range(D):
            o[h][d] = sum(e[j] * kv[j][d] for j in range(n)) / l
        lse[h] = m + math.log(l)
    return np.array(o), np.array(lse)


def entry_score_loops(q_idx, w, key):
    """sum_h w_h * max(0, sum_d q_hd k_d) with Python loops."""
    tot = 0.0
    for h in range(len(q_idx)):
        dot = 0.0
        for d in range(len(key)):
            dot += float(q_idx[h][d]) * float(key[d])
        tot += float(w[h]) * (dot if dot > 0 else 0.0)
    return tot


def topk_pairwise(scores, k):
    """Selected set by rank counting: b is kept iff fewer than k candidates beat it.

    c beats b iff s_c > s_b, or s_c == s_b and c < b.  O(n^2).
    """
    s = list(scores)
    n = len(s)
    kept = []
    for b in range(n):
        if not math.isfinite(s[b]):
            continue
        better = 0
        for c in range(n):
            if c != b and math.isfinite(s[c]) and (s[c] > s[b] or (s[c] == s[b] and c < b)):
                better += 1
        if better < k:
            kept.append(b)
    return kept
