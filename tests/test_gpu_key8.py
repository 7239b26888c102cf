"""GPU parity of the MXFP8 indexer key cache: csa2_append_key8 bytes bit-exact with
the oracle's encoding, group sums, and csa2_index_topk_key8 scores / selections
against the oracle indexer on the dequantised keys."""

import numpy as np
import pytest
import torch

from oracle import indexer, mxfp8, topk
from synth import normal_bf16, rng_for
from tests import pins
from tests.gpu_util import dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _lib():
    from sparse_attention_fp4_csa2_amd import _lib
    return _lib


def _append_key8(keys, cap, start=None, with_groups=False, key8=None, ks=None, gsum=None):
    lib = _lib()
    B = keys.shape[0]
    if key8 is None:
        key8 = torch.zeros(B, cap, 64, dtype=torch.uint8, device="cuda")
        ks = torch.zeros(B, cap, 2, dtype=torch.uint8, device="cuda")
    if with_groups and gsum is None:
        gsum = torch.zeros(B, cap // 512, 64, dtype=torch.float32, device="cuda")
    st = dev(np.zeros(B, np.int32) if start is None else np.asarray(start, np.int32))
    lib.append_key8(dev_bf16(keys), st, key8, ks, group_sum=gsum)
    torch.cuda.synchronize()
    return key8, ks, gsum


def test_append_key8_sweep_bit_exact():
    # every finite bf16 pattern as dim 1 of a key whose group 0 is pinned by
    # dim 0 = 256 * 2^s (scale byte 127 + s), and as the whole of group 1 (its
    # own scale), at three scales
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (all_bits.astype(np.uint32) << 16).view(np.float32)
    sweep = all_bits[np.isfinite(vals)]
    for s in (0, -30, 40):
        keys = np.zeros((sweep.size, 64), dtype=np.uint16)
        keys[:, 0] = pins.f32_to_bf16_bits(256.0 * 2.0 ** s)
        keys[:, 1] = sweep
        keys[:, 32] = sweep
        keys[:, 40] = sweep ^ np.uint16(0x8000)
        cap = ((sweep.size + 7) // 8) * 8
        k8, ks, _ = _append_key8(keys[None], cap)
        codes, sb = mxfp8.encode_keys(keys)
        got_c, got_s = host(k8)[0, :sweep.size], host(ks)[0, :sweep.size]
        assert np.array_equal(got_s, sb), f"s={s}: {(got_s != sb).sum()} scale bytes differ"
        assert np.array_equal(got_c, codes), f"s={s}: {(got_c != codes).sum()} code bytes differ"


def test_append_key8_special_keys_and_group_sums():
    rng = rng_for(88)
    B, cap = 2, 2048
    keys = normal_bf16(rng, (B, 600, 64))
    keys[0, 0] = 0                                  # all-zero key
    keys[0, 1] = 0x8000                             # all -0.0
    keys[0, 2, :32] = 0x0001                        # smallest subnormal group
    keys[0, 3] = 0x7F7F                             # largest finite
    keys[1, 4] = (keys[1, 4].astype(np.uint32) & 0x807F).astype(np.uint16)   # subnormals
    k8, ks, gs = _append_key8(keys, cap, with_groups=True)
    more = normal_bf16(rng, (B, 37, 64))
    starts = [600, 2030]                            # append; run past capacity
    _append_key8(more, cap, start=starts, with_groups=True, key8=k8, ks=ks, gsum=gs)
    got_c, got_s, got_g = host(k8), host(ks), host(gs)
    for b in range(B):
        ref = np.zeros((cap, 64), dtype=np.uint16)
        written = np.zeros(cap, dtype=bool)
        ref[:600], written[:600] = keys[b], True
        n2 = min(37, cap - starts[b])
        ref[starts[b]:starts[b] + n2], written[starts[b]:starts[b] + n2] = more[b, :n2], True
        codes, sb = mxfp8.encode_keys(ref[written])
        assert np.array_equal(got_c[b][written], codes), b
        assert np.array_equal(got_s[b][written], sb), b
        assert not got_c[b][~written].any() and not got_s[b][~written].any()
        # group sums of the dequantised keys, every appended key once
        deq = mxfp8.decode_keys(codes, sb)
        exp = np.zeros((cap // 512, 64))
        for j, v in zip(np.nonzero(written)[0], deq):
            exp[j // 512] += v
        fin = np.isfinite(exp)
        assert np.allclose(got_g[b][fin], exp[fin], rtol=1e-5, atol=1e-3)


def test_append_key8_with_latent_one_launch_bit_exact():
    # latent records and MXFP8 keys written by one call: the records equal the
    # oracle's MXFP4 encoding, the keys its MXFP8 encoding (ragged start, one
    # sequence running past capacity)
    from oracle import mxfp4
    lib = _lib()
    rng = rng_for(89)
    B, cap, n = 2, 1024, 300
    lat = normal_bf16(rng, (B, n, 512))
    keys = normal_bf16(rng, (B, n, 64))
    cache = torch.zeros(B, cap // 8, 2176, dtype=torch.uint8, device="cuda")
    key8 = torch.zeros(B, cap, 64, dtype=torch.uint8, device="cuda")
    ks = torch.zeros(B, cap, 2, dtype=torch.uint8, device="cuda")
    starts = [5, cap - 100]
    lib.append_key8(dev_bf16(keys), dev(np.array(starts, np.int32)), key8, ks, latent=dev_bf16(lat), cache=cache)
    torch.cuda.synchronize()
    for b in range(B):
        m = min(n, cap - starts[b])
        ref = np.zeros((cap // 8, 2176), dtype=np.uint8)
        mxfp4.write_records(ref, lat[b, :m], starts[b])
        assert np.array_equal(host(cache)[b], ref), b
        codes, sb = mxfp8.encode_keys(keys[b, :m])
        assert np.array_equal(host(key8)[b, starts[b]:starts[b] + m], codes), b
        assert np.array_equal(host(ks)[b, starts[b]:starts[b] + m], sb), b


def _index_key8(keys, q_idx, w, n_entries, cap, K, q_pos=None, top_groups=0):
    lib = _lib()
    B, Q = q_idx.shape[:2]
    k8, ks, gs = _append_key8(keys, cap, with_groups=top_groups > 0)
    idx = torch.full((B, Q, K), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Q), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(lib.index_topk_ws(B, Q, cap, top_groups), 256), dtype=torch.uint8, device="cuda")
    lib.index_topk_key8(dev_bf16(q_idx), dev(w), k8, ks, dev(np.asarray(n_entries, np.int32)), K, idx, cnt,
                        ws, group_sum=gs, q_pos=None if q_pos is None else dev(q_pos), top_groups=top_groups)
    torch.cuda.synchronize()
    sc = None
    if top_groups == 0:
        sc = host(ws[:B * Q * (cap // 8) * 4].view(torch.float32)).reshape(B, Q, cap // 8)
    return host(idx), host(cnt), sc, host(k8), host(ks)


def _check_rows(got, cnt, sc, keys_f, q_idx, w, n_entries, cap, K, q_pos=None):
    worst = 0.0
    B, Q = q_idx.shape[:2]
    for b in range(B):
        for r in range(Q):
            qp = None if q_pos is None else int(q_pos[b, r])
            s = indexer.block_scores(q_idx[b, r], w[b, r], keys_f[b], int(n_entries[b]), q_pos=qp,
                                     n_blocks=cap // 8)
            fin = np.isfinite(s)
            assert np.array_equal(np.isfinite(sc[b, r]), fin), (b, r)
            if fin.any():
                scale = max(np.abs(s[fin]).max(), 1e-300)
                worst = max(worst, np.abs(sc[b, r][fin] - s[fin]).max() / scale)
            exp, c = topk.select(s, K)
            assert cnt[b, r] == c, (b, r)
            smax = np.abs(s[fin]).max() if fin.any() else 0.0
            if topk.gap_at_rank(s, K) >= 1e-2 * smax:
                assert np.array_equal(got[b, r], exp), (b, r)
    return worst


@pytest.mark.parametrize("Q,Hi", [(1, 8), (40, 8), (150, 8), (1, 5), (40, 5)])
def test_index_topk_key8_scores_and_selection(Q, Hi):
    # Q = 1: the per-row decode kernel; 40 and 150 causal rows: the multi-row
    # MFMA kernel (a partly filled workgroup; two full ones and a ragged one);
    # Hi = 5 leaves padded head rows in both
    rng = rng_for(90 + Q + Hi)
    B, cap, K = 2, 4096 + 512, 64
    keys = normal_bf16(rng, (B, cap, 64))
    # sequence 1: keys scaled far from 1 in two ranges (E8M0 bytes ~27 and ~187)
    kf = (keys[1].astype(np.uint32) << 16).view(np.float32)
    kf[:2048] *= np.float32(2.0 ** -100)
    kf[2048:] *= np.float32(2.0 ** 60)
    keys[1] = (kf.view(np.uint32) >> 16).astype(np.uint16)
    q_idx = normal_bf16(rng, (B, Q, Hi, 64))
    w = rng.standard_normal((B, Q, Hi)).astype(np.float32)
    ne = np.array([cap, 3001], np.int32)
    q_pos = None
    if Q > 1:
        q_pos = np.sort(rng.integers(0, 2 * cap + 64, size=(B, Q)), axis=1).astype(np.int32)
        q_pos[0, 0], q_pos[1, -1] = 0, 2 * cap + 63
    got, cnt, sc, k8, ks = _index_key8(keys, q_idx, w, ne, cap, K, q_pos=q_pos)
    codes, sb = mxfp8.encode_keys(keys)             # the oracle's own encoding ...
    assert np.array_equal(k8, codes) and np.array_equal(ks, sb)   # ... which the GPU's bytes match
    keys_f = mxfp8.decode_keys(codes, sb)
    worst = _check_rows(got, cnt, sc, keys_f, q_idx, w, ne, cap, K, q_pos)
    print(f"[parity] MXFP8-key block scores (Q={Q}, Hi={Hi}): max|err|/max|s| = {worst:.2e}")
    assert worst < 1e-5


def test_index_topk_key8_two_level_equals_flat_when_all_groups_kept():
    rng = rng_for(97)
    B, cap, K, Hi = 2, 8192, 128, 8
    keys = normal_bf16(rng, (B, cap, 64))
    q_idx = normal_bf16(rng, (B, 1, Hi, 64))
    w = np.abs(rng.standard_normal((B, 1, Hi))).astype(np.float32)
    ne = np.array([cap, 5000], np.int32)
    got_all, cnt_all, _, _, _ = _index_key8(keys, q_idx, w, ne, cap, K, top_groups=cap // 512)
    got_flat, cnt_flat, _, _, _ = _index_key8(keys, q_idx, w, ne, cap, K)
    assert np.array_equal(cnt_all, cnt_flat)
    assert np.array_equal(got_all, got_flat)
