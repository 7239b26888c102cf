"""GPU parity: csa2_append_fp4 packed bytes must equal the oracle's bit for bit."""

import numpy as np
import pytest
import torch

from oracle import indexer, mxfp4, mxfp8
from synth import CONFIGS, normal_bf16, rng_for
from tests import pins
from tests.gpu_util import dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _lib():
    from sparse_attention_fp4_csa2_amd import _lib
    return _lib


def _append(latent, cap, start=None, keys=None, with_groups=False, cache=None, key_cache=None,
            gsum=None):
    lib = _lib()
    B, n = latent.shape[0], latent.shape[1]
    if cache is None:
        cache = torch.zeros(B, cap // 8, 2176, dtype=torch.uint8, device="cuda")
    if keys is not None and key_cache is None:
        key_cache = torch.zeros(B, cap, 64, dtype=torch.bfloat16, device="cuda")
    if with_groups and gsum is None:
        gsum = torch.zeros(B, cap // 512, 64, dtype=torch.float32, device="cuda")
    st = dev(np.zeros(B, np.int32) if start is None else np.asarray(start, np.int32))
    lib.append_fp4(dev_bf16(latent), st, cache,
                   idx_key=dev_bf16(keys) if keys is not None else None,
                   key_cache=key_cache if keys is not None else None, group_sum=gsum)
    torch.cuda.synchronize()
    return cache, key_cache, gsum


def test_tiny_cache_bytes_bit_exact():
    cfg = CONFIGS["tiny"]
    lat = normal_bf16(rng_for(cfg.seed), (1, cfg.N, 512))
    cache, _, _ = _append(lat, cfg.N)
    ref = mxfp4.build_records(lat[0], cfg.N)
    got = host(cache)[0]
    assert np.array_equal(got, ref), f"{(got != ref).sum()} bytes differ"


def test_exhaustive_bf16_sweep_bit_exact():
    # every finite bf16 pattern as x_1 of a group pinned by x_0 = 6 * 2**s, at three scales
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (all_bits.astype(np.uint32) << 16).view(np.float32)
    sweep = all_bits[np.isfinite(vals)]
    for s in (0, -2, 7):
        rows = np.zeros((sweep.size, 512), dtype=np.uint16)
        rows[:, 0] = pins.f32_to_bf16_bits(6.0 * 2.0 ** s)
        rows[:, 1] = sweep
        rows[:, 33] = sweep                         # group 1: amax = |x| itself
        cap = ((sweep.size + 7) // 8) * 8
        cache, _, _ = _append(rows[None], cap)
        ref = mxfp4.build_records(rows, cap)
        got = host(cache)[0]
        assert np.array_equal(got, ref), f"s={s}: {(got != ref).sum()} bytes differ"


def test_special_groups_bit_exact():
    row = np.zeros((8, 512), dtype=np.uint16)
    row[0, 32:64] = 0x8000                    # -0.0
    row[0, 64] = 0x7F80                       # +inf
    row[0, 96] = 0x7FC0                       # NaN
    row[0, 128] = 0x0001                      # smallest subnormal
    row[0, 160:192] = np.arange(32) + 1       # subnormal ramp
    row[1, :] = 0x7F7F                        # largest finite
    row[2, :] = 0xFF7F                        # most negative finite
    row[3, ::2] = 0x0080                      # smallest normal
    row[4] = normal_bf16(rng_for(4), (512,))
    row[5] = (normal_bf16(rng_for(5), (512,)).astype(np.uint32) & 0x807F).astype(np.uint16)  # subnormals
    cache, _, _ = _append(row[None], 8)
    ref = mxfp4.build_records(row, 8)
    assert np.array_equal(host(cache)[0], ref)


def _oracle_group_sums(keys_u16, n_entries, cap):
    """fp32 group sums the GPU must hold: the oracle's group mean times the present count."""
    means, present = indexer.group_means(keys_u16, n_entries, n_groups=cap // 512)
    cnt = np.clip(n_entries - 512 * np.arange(cap // 512), 0, 512)
    return (means * cnt[:, None]).astype(np.float32), present


def test_ragged_appends_keys_and_group_sums():
    # append, overwrite the tail across a group boundary, overwrite inside a
    # group, run past capacity: each touched group's sum is recomputed from the
    # keys the cache holds, so an overwritten key counts once, with its new value
    rng = rng_for(21)
    B, cap = 4, 2048
    first = normal_bf16(rng, (B, 700, 512))
    kfirst = normal_bf16(rng, (B, 700, 64))
    cache, kc, gs = _append(first, cap, start=[0] * B, keys=kfirst, with_groups=True)
    second = normal_bf16(rng, (B, 37, 512))
    ksecond = normal_bf16(rng, (B, 37, 64))
    starts = [700, 500, 2040, 100]
    _append(second, cap, start=starts, keys=ksecond, with_groups=True, cache=cache,
            key_cache=kc, gsum=gs)
    got = host(cache)
    gotk = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    gsum = host(gs)
    for b in range(B):
        lat = np.zeros((cap, 512), dtype=np.uint16)
        keys = np.zeros((cap, 64), dtype=np.uint16)
        written = np.zeros(cap, dtype=bool)
        lat[:700], keys[:700], written[:700] = first[b], kfirst[b], True
        s = starts[b]
        n2 = min(37, cap - s)
        lat[s:s + n2], keys[s:s + n2], written[s:s + n2] = second[b, :n2], ksecond[b, :n2], True
        ref = np.zeros((cap // 8, 2176), dtype=np.uint8)
        for lo, hi in _runs(written):
            mxfp4.write_records(ref, lat[lo:hi], lo)
        assert np.array_equal(got[b], ref), f"seq {b}"
        assert np.array_equal(gotk[b][written], keys[written])
        n_ent = int(np.nonzero(written)[0].max()) + 1
        exp, _ = _oracle_group_sums(keys[:n_ent], n_ent, cap)
        assert np.array_equal(gsum[b], exp), f"seq {b}: group sums differ at " \
            f"{np.argwhere(gsum[b] != exp)[:4].tolist()}"


def test_repeated_overwrites_keep_group_sums():
    # the decode step rewrites one entry again and again: its group's sum must
    # stay the sum of the keys held (bf16 and MXFP8 key caches)
    rng = rng_for(22)
    B, cap, n = 2, 1024, 1000
    lat = normal_bf16(rng, (B, n, 512))
    keys = normal_bf16(rng, (B, n, 64))
    cache, kc, gs = _append(lat, cap, keys=keys, with_groups=True)
    lib = _lib()
    k8 = torch.zeros(B, cap, 64, dtype=torch.uint8, device="cuda")
    ks = torch.zeros(B, cap, 2, dtype=torch.uint8, device="cuda")
    gs8 = torch.zeros(B, cap // 512, 64, dtype=torch.float32, device="cuda")
    lib.append_key8(dev_bf16(keys), dev(np.zeros(B, np.int32)), k8, ks, group_sum=gs8)
    last = dev(np.full(B, n - 1, np.int32))
    new_lat, new_key = dev_bf16(lat[:, n - 1:]), dev_bf16(keys[:, n - 1:])
    for _ in range(200):
        lib.append_fp4(new_lat, last, cache, idx_key=new_key, key_cache=kc, group_sum=gs)
        lib.append_key8(new_key, last, k8, ks, group_sum=gs8)
    torch.cuda.synchronize()
    for b in range(B):
        exp, _ = _oracle_group_sums(keys[b], n, cap)
        assert np.array_equal(host(gs)[b], exp), f"bf16 keys, seq {b}"
        deq = mxfp8.quantize_dequantize(keys[b])
        exp8, _ = _oracle_group_sums(deq, n, cap)
        assert np.array_equal(host(gs8)[b], exp8), f"MXFP8 keys, seq {b}"


def _runs(mask):
    out, j, n = [], 0, len(mask)
    while j < n:
        if mask[j]:
            k = j
            while k < n and mask[k]:
                k += 1
            out.append((j, k))
            j = k
        else:
            j += 1
    return out


def test_decode_single_entry_append():
    # decode: one new entry per sequence at each sequence's own position
    rng = rng_for(31)
    B, cap = 4, 64
    base = normal_bf16(rng, (B, 20, 512))
    cache, _, _ = _append(base, cap)
    new = normal_bf16(rng, (B, 1, 512))
    starts = [20, 5, 63, 64]
    _append(new, cap, start=starts, cache=cache)
    got = host(cache)
    for b in range(B):
        lat = base[b].copy()
        ref = mxfp4.build_records(lat, cap)
        if starts[b] < cap:
            mxfp4.write_records(ref, new[b], starts[b])
        assert np.array_equal(got[b], ref), b
