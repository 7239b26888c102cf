"""GPU parity: csa2_sparse_attn and csa2_swa_merge vs the fp64 oracle.

Bar: attention outputs within max|err| <= 1e-2 * RMS(oracle output) over the
call's whole output; lse within 1e-3 absolute; exact dequantisation checked bit
for bit through single-entry attention (softmax weight 1, o = V exactly).
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, modes, mxfp4
from synth import CONFIGS, bf16_rne, bf16_to_f32, decode_inputs, normal_bf16, rng_for
from tests.gpu_util import assert_close_rms, assert_lse_close, dev, dev_bf16, host

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(512.0)


def _lib():
    from sparse_attention_fp4_csa2_amd import _lib
    return _lib


def gpu_cache(latent, cap):
    lib = _lib()
    B = latent.shape[0]
    cache = torch.zeros(B, cap // 8, 2176, dtype=torch.uint8, device="cuda")
    lib.append_fp4(dev_bf16(latent), dev(np.zeros(B, np.int32)), cache)
    return cache


def gpu_sparse(q, cache, idx, count, n_entries, q_pos=None, scale=SCALE):
    lib = _lib()
    B, Q, H = q.shape[:3]
    K = idx.shape[-1]
    o = torch.full((B, Q, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((max(lib.sparse_attn_ws(B, Q, H, K), 256),), 255, dtype=torch.uint8, device="cuda")
    lib.sparse_attn(dev_bf16(q), cache, dev(np.asarray(idx, np.int32)), dev(np.asarray(count, np.int32)),
                    dev(np.asarray(n_entries, np.int32)), scale, o, lse, ws=ws,
                    q_pos=None if q_pos is None else dev(np.asarray(q_pos, np.int32)))
    torch.cuda.synchronize()
    return host(o), host(lse)


def gpu_swa(q, swa, swa_len, W, o_s, lse_s, swa_pos0=None, q_pos=None, alias=False):
    lib = _lib()
    B, Q, H = q.shape[:3]
    o_sd, l_sd = dev(o_s.astype(np.float32)), dev(lse_s.astype(np.float32))
    if alias:
        out, lse_out = o_sd, l_sd
    else:
        out = torch.full_like(o_sd, float("nan"))
        lse_out = torch.full_like(l_sd, float("nan"))
    ws = torch.empty(lib.swa_merge_ws(B, Q, H, W), dtype=torch.uint8, device="cuda")
    lib.swa_merge(dev_bf16(q), dev_bf16(swa), dev(np.asarray(swa_len, np.int32)), W, SCALE,
                  o_sd, l_sd, out, lse_out, ws,
                  swa_pos0=None if swa_pos0 is None else dev(np.asarray(swa_pos0, np.int32)),
                  q_pos=None if q_pos is None else dev(np.asarray(q_pos, np.int32)))
    torch.cuda.synchronize()
    return host(out), host(lse_out)


def oracle_rows(q, cache_np, idx, count, n_entries, q_pos=None):
    B, Q, H = q.shape[:3]
    o = np.zeros((B, Q, H, 512))
    l = np.zeros((B, Q, H))
    for b in range(B):
        for r in range(Q):
            o[b, r], l[b, r] = attention.sparse_attention(
                q[b, r], cache_np[b], idx[b, r], count[b, r], n_entries[b],
                None if q_pos is None else int(q_pos[b, r]))
    return o, l


def test_tiny_sparse_attention():
    cfg = CONFIGS["tiny"]
    x = decode_inputs(cfg)
    cache_np = np.stack([mxfp4.build_records(x.latent[0], cfg.N)])
    idx = np.stack([x.planted[0]])[:, None, :].astype(np.int32)
    count = np.array([[cfg.K]], np.int32)
    o, l = gpu_sparse(x.q, gpu_cache(x.latent, cfg.N), idx, count, x.n_entries)
    ro, rl = oracle_rows(x.q, cache_np, idx, count, x.n_entries)
    assert_close_rms(o, ro)
    assert_lse_close(l, rl)


@pytest.mark.parametrize("H", [16, 40, 64, 128])
def test_head_counts_and_ragged_selection(H):
    rng = rng_for(100 + H)
    B, N, K = 3, 1200, 40
    lat = normal_bf16(rng, (B, N, 512))
    q = normal_bf16(rng, (B, 1, H, 512))
    ne = np.array([1200, 1195, 333], np.int32)
    idx = np.full((B, 1, K), -1, np.int32)
    count = np.array([[K], [17], [0]], np.int32)
    for b in range(B):
        nbp = (ne[b] + 7) // 8
        sel = np.sort(rng.choice(nbp, min(count[b, 0], nbp), replace=False))
        idx[b, 0, :sel.size] = sel
    idx[0, 0, 5] = 149          # last (partial for seq 1) block id, keep sorted-ness irrelevant
    idx[1, 0, 3] = 100000       # out of range: skipped
    cache = gpu_cache(lat, N)
    cache_np = np.stack([mxfp4.build_records(lat[b], N) for b in range(B)])
    o, l = gpu_sparse(q, cache, idx, count, ne)
    ro, rl = oracle_rows(q, cache_np, idx, count, ne)
    assert_close_rms(o, ro)
    assert_lse_close(l, rl)
    # empty selection: o = 0, lse = -inf
    assert (o[2] == 0).all() and np.isneginf(l[2]).all()


def test_all_blocks_selected_equals_dense():
    rng = rng_for(7)
    N = 520
    lat = normal_bf16(rng, (1, N, 512))
    q = normal_bf16(rng, (1, 1, 64, 512))
    idx = np.arange(N // 8, dtype=np.int32)[None, None]
    o, l = gpu_sparse(q, gpu_cache(lat, N), idx, np.array([[N // 8]]), np.array([N]))
    kv = mxfp4.quantize_dequantize(lat[0])
    ro, rl = attention.attend(q[0, 0], kv, SCALE)
    assert_close_rms(o[0, 0], ro)
    assert_lse_close(l[0, 0], rl)


def _single_entry_cache(sbs_per_seq):
    codes = np.tile(np.arange(16, dtype=np.uint8), 32)               # every code in every group
    packed = mxfp4.pack_codes(codes[None])[0]
    B = len(sbs_per_seq)
    cache_np = np.zeros((B, 1, 2176), np.uint8)
    for b in range(B):
        cache_np[b, 0, :256] = packed
        cache_np[b, 0, 2048:2064] = sbs_per_seq[b]
    return cache_np


def test_dequant_exact_all_codes_and_scales_via_single_entry():
    # one present entry per sequence: softmax weight 1, so o equals the dequantised entry.
    # Every code meets every scale byte the encoder can produce (0..252); the 4 scale
    # groups a wave owns (128 dims) stay within 3 of each other, as in real data.
    B = 16
    sbs = (list(range(253)) + [252] * 3)
    cache_np = _single_entry_cache([sbs[16 * b:16 * b + 16] for b in range(B)])
    q = np.zeros((B, 1, 16, 512), np.uint16)
    o, l = gpu_sparse(q, dev(cache_np), np.zeros((B, 1, 1), np.int32), np.ones((B, 1), np.int32),
                      np.ones(B, np.int32))
    for b in range(B):
        exp = mxfp4.read_entries(cache_np[b], [0])[0]
        assert np.array_equal(o[b, 0, 0].astype(np.float64), exp), b
        assert (o[b, 0] == o[b, 0, 0]).all()
    assert np.allclose(l, 0.0)


def test_dequant_wide_scale_spread_within_tolerance():
    # scale bytes 125 apart inside one 128-dim slice: values far below the slice's largest
    # scale may flush toward zero in the fp16 value path; the output stays within the bar
    sbs = [[252, 127, 127, 127] * 4, [130, 3, 60, 127] * 4, [0, 40, 80, 120] * 4]
    cache_np = _single_entry_cache(sbs)
    B = len(sbs)
    q = np.zeros((B, 1, 16, 512), np.uint16)
    o, l = gpu_sparse(q, dev(cache_np), np.zeros((B, 1, 1), np.int32), np.ones((B, 1), np.int32),
                      np.ones(B, np.int32))
    for b in range(B):
        exp = mxfp4.read_entries(cache_np[b], [0])[0]
        assert_close_rms(o[b, 0, 0], exp)


def test_causal_rows_visibility():
    rng = rng_for(12)
    N, Q, H, K = 256, 4, 64, 12
    lat = normal_bf16(rng, (1, N, 512))
    q = normal_bf16(rng, (1, Q, H, 512))
    q_pos = np.array([[511, 300, 40, 0]], np.int32)
    idx = np.tile(np.sort(rng.choice(32, K, replace=False)).astype(np.int32), (1, Q, 1))
    idx[0, 2, :3] = [0, 1, 2]
    idx[0, 2] = np.sort(idx[0, 2])
    count = np.full((1, Q), K, np.int32)
    o, l = gpu_sparse(q, gpu_cache(lat, N), idx, count, np.array([N]), q_pos=q_pos)
    ro, rl = oracle_rows(q, np.stack([mxfp4.build_records(lat[0], N)]), idx, count, np.array([N]), q_pos)
    assert_close_rms(o, ro)
    assert_lse_close(l, rl)


@pytest.mark.parametrize("alias", [False, True])
def test_swa_merge_decode(alias):
    rng = rng_for(13)
    B, H, W, Lw = 3, 64, 128, 160
    q = normal_bf16(rng, (B, 1, H, 512))
    swa = normal_bf16(rng, (B, Lw, 512))
    swa_len = np.array([160, 128, 7], np.int32)
    o_s = rng.standard_normal((B, 1, H, 512)) * 0.05
    lse_s = rng.standard_normal((B, 1, H)) + 3.0
    lse_s[2, 0, :5] = -np.inf
    o_s[2, 0, :5] = 0
    out, lo = gpu_swa(q, swa, swa_len, W, o_s, lse_s, alias=alias)
    ro = np.zeros_like(o_s)
    rl = np.zeros_like(lse_s)
    for b in range(B):
        ow, lw = attention.window_attention(q[b, 0], swa[b], int(swa_len[b]), W)
        ro[b, 0], rl[b, 0] = attention.merge(o_s[b, 0].astype(np.float32), lse_s[b, 0].astype(np.float32), ow, lw)
    assert_close_rms(out, ro)
    assert_lse_close(lo, rl)


def test_swa_merge_causal_positions():
    rng = rng_for(14)
    B, Q, H, W = 1, 5, 16, 8
    Lw = 40
    q = normal_bf16(rng, (B, Q, H, 512))
    swa = normal_bf16(rng, (B, Lw, 512))
    pos0 = np.array([100], np.int32)
    q_pos = np.array([[100, 103, 120, 139, 99]], np.int32)   # last one sees nothing held
    o_s = np.zeros((B, Q, H, 512))
    lse_s = np.full((B, Q, H), -np.inf)
    out, lo = gpu_swa(q, swa, [Lw], W, o_s, lse_s, swa_pos0=pos0, q_pos=q_pos)
    for r in range(Q):
        ow, lw = attention.window_attention(q[0, r], swa[0], Lw, W, 100, int(q_pos[0, r]))
        ro, rl = attention.merge(o_s[0, r], lse_s[0, r], ow, lw)
        if np.isfinite(rl).any():
            assert_close_rms(out[0, r], ro)
        else:
            assert (out[0, r] == 0).all()
        assert_lse_close(lo[0, r], rl)


def test_end_to_end_tiny_full_and_reuse_layers():
    from sparse_attention_fp4_csa2_amd import modes as gm
    cfg = CONFIGS["tiny"]
    x = decode_inputs(cfg)
    cache = gm.LatentCache.empty(1, cfg.N)
    cache.append(dev_bf16(x.latent), dev_bf16(x.keys))
    buf = gm.LayerBuffers(1, 1, cfg.H, cfg.N, cfg.K, cfg.W)
    swa_len = dev(x.swa_len)
    idx, count = gm.run_layer("F", buf, cache, dev_bf16(x.q), dev_bf16(x.swa), swa_len,
                              q_idx=dev_bf16(x.q_idx), w=dev(x.w))
    torch.cuda.synchronize()
    cache_np = mxfp4.build_records(x.latent[0], cfg.N)
    ri, rc, ro, rl = modes.full_layer(x.q[0, 0], x.q_idx[0, 0], x.w[0, 0], x.keys[0], cache_np,
                                      cfg.N, cfg.K, x.swa[0], cfg.W, cfg.W)
    assert np.array_equal(host(idx)[0, 0], ri) and host(count)[0, 0] == rc
    assert_close_rms(host(buf.out)[0, 0], ro)
    assert_lse_close(host(buf.lse_out)[0, 0], rl)
    # Reuse layer with its own query and window: indices passed through untouched
    rng = rng_for(99)
    q2, swa2 = normal_bf16(rng, (1, 1, cfg.H, 512)), normal_bf16(rng, (1, cfg.W, 512))
    before = host(idx).copy()
    buf2 = gm.LayerBuffers(1, 1, cfg.H, cfg.N, cfg.K, cfg.W)
    i2, c2 = gm.run_layer("U", buf2, cache, dev_bf16(q2), dev_bf16(swa2), swa_len, prev=(idx, count))
    torch.cuda.synchronize()
    assert host(i2).tobytes() == before.tobytes()
    _, _, ro2, rl2 = modes.reuse_layer(q2[0, 0], ri, rc, cache_np, cfg.N, swa2[0], cfg.W, cfg.W)
    assert_close_rms(host(buf2.out)[0, 0], ro2)


def test_repeat_runs_bitwise_identical():
    cfg = CONFIGS["tiny"]
    x = decode_inputs(cfg)
    cache = gpu_cache(x.latent, cfg.N)
    idx = np.stack([x.planted[0]])[:, None, :].astype(np.int32)
    outs = [gpu_sparse(x.q, cache, idx, np.array([[cfg.K]]), x.n_entries) for _ in range(5)]
    for o, l in outs[1:]:
        assert o.tobytes() == outs[0][0].tobytes() and l.tobytes() == outs[0][1].tobytes()


def gpu_layer(q, cache, idx, count, n_entries, swa, swa_len, W, swa_pos0=None, q_pos=None, ws=None):
    lib = _lib()
    B, Q, H = q.shape[:3]
    out = torch.full((B, Q, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = torch.empty(lib.attend_layer_ws(B, Q, H, idx.shape[-1], W), dtype=torch.uint8, device="cuda")
    lib.attend_layer(dev_bf16(q), cache, dev(np.ascontiguousarray(idx, np.int32)),
                     dev(np.asarray(count, np.int32)), dev(np.asarray(n_entries, np.int32)), dev_bf16(swa),
                     dev(np.asarray(swa_len, np.int32)), W, SCALE, out, lse, ws,
                     swa_pos0=None if swa_pos0 is None else dev(np.asarray(swa_pos0, np.int32)),
                     q_pos=None if q_pos is None else dev(np.asarray(q_pos, np.int32)))
    torch.cuda.synchronize()
    return host(out), host(lse)


@pytest.mark.parametrize("H", [16, 40, 64, 128])
def test_attend_layer_decode_matches_joint_softmax(H):
    # one call: sparse branch + window branch, checked against the oracle's
    # sparse attention, window attention and merge (= one softmax over both sets)
    rng = rng_for(30 + H)
    B, N, K, W, Lw = 3, 2048, 64, 128, 160
    latent = normal_bf16(rng, (B, N, 512))
    cache = gpu_cache(latent, N)
    cache_np = [mxfp4.build_records(latent[b], N) for b in range(B)]
    q = normal_bf16(rng, (B, 1, H, 512))
    swa = normal_bf16(rng, (B, Lw, 512))
    swa_len = np.array([160, 128, 9], np.int32)
    n_entries = np.array([2048, 1999, 2048], np.int32)
    idx = np.full((B, 1, K), -1, np.int32)
    count = np.array([[K], [37], [0]], np.int32)             # full, ragged, empty selection
    for b in range(B):
        c = int(count[b, 0])
        if c:
            idx[b, 0, :c] = np.sort(rng.choice(N // 8, c, replace=False))
    out, lse = gpu_layer(q, cache, idx, count, n_entries, swa, swa_len, W)
    ro = np.zeros((B, 1, H, 512))
    rl = np.zeros((B, 1, H))
    for b in range(B):
        ro[b, 0], rl[b, 0] = modes.attend_row(q[b, 0], cache_np[b], idx[b, 0], int(count[b, 0]),
                                              int(n_entries[b]), swa[b], int(swa_len[b]), W)
    assert_close_rms(out, ro)
    assert_lse_close(lse, rl)


@pytest.mark.parametrize("B,N,K,W", [(4, 2048, 64, 128),     # few rows: window inside the sparse workgroups
                                     (32, 1024, 64, 512)])   # 32 rows: window workgroups after the sparse ones
def test_attend_layer_empty_branches(B, N, K, W):
    # rows cycle through: both branches, empty window, empty selection, both
    # empty (nothing visible: out 0, lse -inf); the merge must take a lone
    # branch unchanged and the empty row must stay exactly zero
    rng = rng_for(50 + B)
    H, Lw = 64, W
    latent = normal_bf16(rng, (B, N, 512))
    cache = gpu_cache(latent, N)
    cache_np = [mxfp4.build_records(latent[b], N) for b in range(B)]
    q = normal_bf16(rng, (B, 1, H, 512))
    swa = normal_bf16(rng, (B, Lw, 512))
    swa_len = np.array([[Lw, 0, W // 2 + 3, 0][b % 4] for b in range(B)], np.int32)
    count = np.array([[[K], [K - 5], [0], [0]][b % 4] for b in range(B)], np.int32)
    n_entries = np.full(B, N, np.int32)
    idx = np.full((B, 1, K), -1, np.int32)
    for b in range(B):
        c = int(count[b, 0])
        idx[b, 0, :c] = np.sort(rng.choice(N // 8, c, replace=False))
    out, lse = gpu_layer(q, cache, idx, count, n_entries, swa, swa_len, W)
    ro = np.zeros((B, 1, H, 512))
    rl = np.zeros((B, 1, H))
    for b in range(B):
        ro[b, 0], rl[b, 0] = modes.attend_row(q[b, 0], cache_np[b], idx[b, 0], int(count[b, 0]), N,
                                              swa[b], int(swa_len[b]), W)
    assert_close_rms(out, ro)
    assert_lse_close(lse, rl)
    for b in range(3, B, 4):
        assert (out[b] == 0).all() and np.isneginf(lse[b]).all(), f"row {b}: nothing visible"


def test_attend_layer_causal_rows():
    rng = rng_for(41)
    B, Q, H, N, K, W = 1, 6, 64, 4096, 96, 32
    latent = normal_bf16(rng, (B, N, 512))
    cache = gpu_cache(latent, N)
    cache_np = mxfp4.build_records(latent[0], N)
    q = normal_bf16(rng, (B, Q, H, 512))
    pos0 = 2 * N - 40
    Lw = 80
    swa = normal_bf16(rng, (B, Lw, 512))
    q_pos = np.array([[2 * N - 40, 2 * N - 20, 2 * N - 1, 2 * N + 30, 3000, 2 * N + 39]], np.int32)
    idx = np.stack([np.sort(rng.choice(N // 8, K, replace=False)) for _ in range(Q)])[None].astype(np.int32)
    count = np.full((B, Q), K, np.int32)
    out, lse = gpu_layer(q, cache, idx, count, [N], swa, [Lw], W, swa_pos0=[pos0], q_pos=q_pos)
    for r in range(Q):
        ro, rl = modes.attend_row(q[0, r], cache_np, idx[0, r], K, N, swa[0], Lw, W,
                                  q_pos=int(q_pos[0, r]), swa_pos0=pos0)
        assert_close_rms(out[0, r], ro, what=f"row {r}")
        assert_lse_close(lse[0, r], rl)


@pytest.mark.parametrize("H", [64, 16])   # 16 heads: rows 0-1 share a row tile, row 2 is a short group
def test_two_phase_layer_on_two_streams_matches_one_call(H):
    # csa2_attend_layer_window on a second stream + csa2_attend_layer_sparse on
    # the first (joined by an event) against csa2_attend_layer and the oracle;
    # twice in a row on one workspace, the second call with other queries.  The
    # one launch folds the window into the sparse workgroups' softmax (one
    # partial per split) where the phases keep a partial per branch, so the two
    # agree to rounding, not bit for bit; both meet the bar against the oracle
    lib = _lib()
    rng = rng_for(52)
    B, Q, N, K, W, Lw = 2, 3, 4096, 128, 96, 96
    latent = normal_bf16(rng, (B, N, 512))
    cache = gpu_cache(latent, N)
    cache_np = [mxfp4.build_records(latent[b], N) for b in range(B)]
    swa = normal_bf16(rng, (B, Lw, 512))
    pos0 = [2 * N - 60, 2 * N - 90]
    q_pos = np.array([[2 * N - 50, 2 * N - 10, 2 * N + 20], [2 * N - 90, 2 * N - 1, 2 * N + 5]], np.int32)
    idx = np.stack([np.sort(rng.choice(N // 8, K, replace=False)) for _ in range(B * Q)])
    idx = idx.reshape(B, Q, K).astype(np.int32)
    count = np.array([[K, 50, 0], [K, K, 7]], np.int32)
    n_entries = np.array([N, N - 100], np.int32)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ws = torch.empty(lib.attend_layer_ws(B, Q, H, K, W), dtype=torch.uint8, device="cuda")
    d_idx, d_cnt, d_n = dev(idx), dev(count), dev(n_entries)
    d_swa, d_len, d_pos0, d_qpos = dev_bf16(swa), dev(np.array([Lw, Lw], np.int32)), dev(np.array(pos0, np.int32)), dev(q_pos)
    for call in range(2):
        q = normal_bf16(rng, (B, Q, H, 512))
        ref_o, ref_l = gpu_layer(q, cache, idx, count, n_entries, swa, [Lw, Lw], W, swa_pos0=pos0, q_pos=q_pos)
        d_q = dev_bf16(q)
        out = torch.full((B, Q, H, 512), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device="cuda")
        side.wait_stream(main)
        lib.attend_layer_window(d_q, d_swa, d_len, K, W, SCALE, ws, swa_pos0=d_pos0, q_pos=d_qpos, stream=side)
        done = torch.cuda.Event()
        done.record(side)
        main.wait_event(done)
        lib.attend_layer_sparse(d_q, cache, d_idx, d_cnt, d_n, W, SCALE, out, lse, ws, q_pos=d_qpos, stream=main)
        torch.cuda.synchronize()
        got_o, got_l = host(out), host(lse)
        assert_close_rms(got_o, ref_o, what=f"call {call}: two phases vs one call")
        assert_lse_close(got_l, ref_l, tol=1e-4)
        for b in range(B):
            for r in range(Q):
                ro, rl = modes.attend_row(q[b, r], cache_np[b], idx[b, r], int(count[b, r]), int(n_entries[b]),
                                          swa[b], Lw, W, q_pos=int(q_pos[b, r]), swa_pos0=pos0[b])
                assert_close_rms(got_o[b, r], ro, what=f"call {call} row {b},{r}: two phases")
                assert_close_rms(ref_o[b, r], ro, what=f"call {call} row {b},{r}: one call")
                assert_lse_close(got_l[b, r], rl)


@pytest.mark.parametrize("B,H", [(2, 64), (8, 40)])
def test_one_launch_layer_reuses_its_workspace(B, H):
    # the library keeps no state between calls: three calls in a row on one
    # workspace (other queries, the last with fewer rows) give the bytes of
    # calls on fresh workspaces.  B = 8 puts the window inside the sparse
    # workgroups; H = 40 leaves a partly filled head group.
    lib = _lib()
    rng = rng_for(61 + B)
    Q, N, K, W, Lw = 1, 8192, 256, 128, 128
    cache = gpu_cache(normal_bf16(rng, (B, N, 512)), N)
    swa = normal_bf16(rng, (B, Lw, 512))
    idx = np.stack([np.sort(rng.choice(N // 8, K, replace=False)) for _ in range(B * Q)]).reshape(B, Q, K)
    count = np.full((B, Q), K, np.int32)
    count[0, 0] = 100
    n_entries = np.full(B, N, np.int32)
    ws = torch.empty(lib.attend_layer_ws(B, Q, H, K, W), dtype=torch.uint8, device="cuda")
    for call, b in enumerate((B, B, B - 1)):
        q = normal_bf16(rng, (b, Q, H, 512))
        args = (cache[:b], idx[:b].astype(np.int32), count[:b], n_entries[:b], swa[:b], [Lw] * b, W)
        o1, l1 = gpu_layer(q, *args, ws=ws)
        o2, l2 = gpu_layer(q, *args)
        assert np.isfinite(o1).all(), call
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"call {call}"


def test_run_layer_side_stream_matches_one_stream():
    # modes.run_layer with the window branch forked onto a second stream (the
    # two-phase calls) against the one-stream call (one launch), for a Full and
    # a Reuse layer: the same selection bit for bit, the outputs to rounding (the
    # one launch may fold the window into the sparse partials)
    from sparse_attention_fp4_csa2_amd import modes as gm
    cfg = CONFIGS["tiny"]
    x = decode_inputs(cfg)
    cache = gm.LatentCache.empty(cfg.B, cfg.N)
    cache.append(dev_bf16(x.latent), dev_bf16(x.keys))
    q, swa, swa_len = dev_bf16(x.q), dev_bf16(x.swa), dev(np.asarray(x.swa_len, np.int32))
    qi, w = dev_bf16(x.q_idx), dev(x.w)
    side = torch.cuda.Stream()
    res = []
    for s in (None, side):
        bf = gm.LayerBuffers(cfg.B, cfg.Q, cfg.H, cfg.N, cfg.K, cfg.W)
        bu = gm.LayerBuffers(cfg.B, cfg.Q, cfg.H, cfg.N, cfg.K, cfg.W)
        prev = gm.run_layer("F", bf, cache, q, swa, swa_len, q_idx=qi, w=w, side_stream=s)
        gm.run_layer("U", bu, cache, q, swa, swa_len, prev=prev, side_stream=s)
        torch.cuda.synchronize()
        res.append([host(t) for t in (bf.idx, bf.count, bf.out, bf.lse_out, bu.out, bu.lse_out)])
    (i1, c1, o1, l1, u1, m1), (i2, c2, o2, l2, u2, m2) = res
    assert np.array_equal(i1, i2) and np.array_equal(c1, c2)
    for a, b, what in ((o1, o2, "Full out"), (u1, u2, "Reuse out")):
        assert_close_rms(b, a, what=f"side stream vs one stream: {what}")
    for a, b in ((l1, l2), (m1, m2)):
        assert_lse_close(b, a, tol=1e-4)


def _scale_bf16(bits, k):
    """bf16 bit patterns times 2^k, exactly (nonzero normals whose exponent stays in range)."""
    b = np.asarray(bits, np.uint16).astype(np.int32)
    e = (b >> 7) & 0xFF
    assert ((e == 0) | ((e + k >= 1) & (e + k <= 254))).all()
    return np.where(e != 0, b + (k << 7), b).astype(np.uint16)


def test_attend_layer_extreme_magnitudes():
    # values near 2^100 and near 2^-100 in either branch: the split-K partials
    # (fp16 relative to a per-head power of two) and the combine keep them;
    # logits stay O(1) by scaling the query the other way
    rng = rng_for(61)
    B, H, N, K, W, Lw = 3, 64, 2048, 96, 128, 128
    lat = normal_bf16(rng, (B, N, 512))
    q = normal_bf16(rng, (B, 1, H, 512))
    swa = normal_bf16(rng, (B, Lw, 512))
    ks = [(100, -100, -60), (-100, 100, -100), (0, 0, 0)]        # (latent, query, window) exponents
    for b, (kl, kq, kw) in enumerate(ks):
        lat[b], q[b], swa[b] = _scale_bf16(lat[b], kl), _scale_bf16(q[b], kq), _scale_bf16(swa[b], kw)
    cache = gpu_cache(lat, N)
    cache_np = [mxfp4.build_records(lat[b], N) for b in range(B)]
    idx = np.stack([np.sort(rng.choice(N // 8, K, replace=False)) for _ in range(B)])[:, None].astype(np.int32)
    count = np.full((B, 1), K, np.int32)
    out, lse = gpu_layer(q, cache, idx, count, np.full(B, N, np.int32), swa, np.full(B, Lw, np.int32), W)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    for b in range(B):
        ro, rl = modes.attend_row(q[b, 0], cache_np[b], idx[b, 0], K, N, swa[b], Lw, W)
        assert_close_rms(out[b, 0], ro, what=f"row {b} (2^{ks[b]})")
        assert_lse_close(lse[b, 0], rl)


@pytest.mark.parametrize("factor", [16, 64, 256, 1024, 4096])
def test_outlier_query_channels(factor):
    # one channel per 32-dim block of every head's query at `factor` times the
    # rest (H 64, K 2048 blocks = 16384 entries): the scaled MFMA keeps its sums
    # to ~15 bits below the largest product, so a block this wide loses its
    # bulk's share of q.K there; from about 2^5 x a wave switches to bf16 Q.K
    # (exactly dequantised codes against the bf16 query); the output must stay
    # within the bar
    rng = rng_for(300 + factor)
    B, N, H, K = 2, 20000, 64, 2048
    lat = normal_bf16(rng, (B, N, 512))
    qf = bf16_to_f32(normal_bf16(rng, (B, 1, H, 512))).reshape(B, 1, H, 16, 32)
    cols = rng.integers(0, 32, size=(B, 1, H, 16))
    np.put_along_axis(qf, cols[..., None], np.take_along_axis(qf, cols[..., None], -1) * factor, -1)
    if factor >= 1024:
        # logits that large leave one entry per head; scale the whole query down so
        # the softmax keeps many entries and the bulk channels decide their order
        qf = qf * np.float32(64.0 / factor)
    q = bf16_rne(qf.reshape(B, 1, H, 512))
    nbp = (N + 7) // 8
    idx = np.stack([np.sort(rng.choice(nbp, K, replace=False)) for _ in range(B)])[:, None].astype(np.int32)
    count = np.full((B, 1), K, np.int32)
    ne = np.full(B, N, np.int32)
    o, l = gpu_sparse(q, gpu_cache(lat, N), idx, count, ne)
    cache_np = np.stack([mxfp4.build_records(lat[b], N) for b in range(B)])
    ro, rl = oracle_rows(q, cache_np, idx, count, ne)
    assert_close_rms(o, ro, what=f"outlier x{factor} out")
    # logits here reach ~60 (the outlier channels dominate q.K): the lse bound
    # takes a part relative to their size; the output bar above is unchanged
    assert_lse_close(l, rl, rel=1e-4)


def test_outlier_query_mixed_waves():
    # outliers only in dims 0..127 of head group 0 (wave 0 of those workgroups
    # takes the bf16 form, the other waves and head group 1 stay FP6), several
    # splits, ragged counts
    rng = rng_for(310)
    B, N, H, K = 3, 9000, 64, 600
    lat = normal_bf16(rng, (B, N, 512))
    qf = bf16_to_f32(normal_bf16(rng, (B, 1, H, 512)))
    qf[:, :, :32, 0:128:32] *= np.float32(2048.0)
    q = bf16_rne(qf)
    nbp = (N + 7) // 8
    count = np.array([[K], [311], [1]], np.int32)
    idx = np.full((B, 1, K), -1, np.int32)
    for b in range(B):
        idx[b, 0, :count[b, 0]] = np.sort(rng.choice(nbp, count[b, 0], replace=False))
    ne = np.full(B, N, np.int32)
    o, l = gpu_sparse(q, gpu_cache(lat, N), idx, count, ne)
    cache_np = np.stack([mxfp4.build_records(lat[b], N) for b in range(B)])
    ro, rl = oracle_rows(q, cache_np, idx, count, ne)
    assert_close_rms(o, ro, what="mixed FP6 / bf16 waves out")
    assert_lse_close(l, rl, rel=1e-4)
