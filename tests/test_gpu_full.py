"""GPU parity at full workload sizes, in the launch configuration bench.py times.

Each test builds a workload exactly as ``bench.py --config <name>`` does (same
seeded inputs, same buffers, same calls), runs its step twice, and checks the
results against the fp64 oracle:

* selected block ids and counts: bit-exact on every row whose oracle score gap
  at rank K (and at rank top_groups for the two-level indexer) is >= 1e-2;
  other rows must be a valid top-K (every selected block scores at least as
  high as every unselected candidate, up to fp32 score rounding);
* attention + window + merge outputs: max|err| <= 1e-2 * RMS over the checked
  rows, with the oracle attending the block ids the GPU selected;
* record bytes of the appended entries and of sampled selected blocks: exact.
"""

import numpy as np
import pytest
import torch

from oracle import indexer, modes as om, mxfp4, mxfp8, topk
from tests.gpu_util import assert_close_rms, assert_lse_close, host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
GAP = 1e-2


def _workload(name, key_format="bf16"):
    import bench
    print(f"[full] building {name} ({key_format} indexer keys)", flush=True)
    cfg, host_in, wl = bench.make_workload(name, key_format=key_format)
    wl.step()
    wl.step()
    torch.cuda.synchronize()
    return cfg, host_in, wl


def _records_of(latent_seq, blocks, nb):
    """Oracle record cache holding just ``blocks``."""
    cache = np.zeros((nb, mxfp4.RECORD_BYTES), dtype=np.uint8)
    n = latent_seq.shape[0]
    for b in np.asarray(blocks, dtype=np.int64):
        if 0 <= b < nb:
            lo, hi = 8 * int(b), min(8 * int(b) + 8, n)
            if hi > lo:
                mxfp4.write_records(cache, latent_seq[lo:hi], lo)
    return cache


def _check_selection(got_idx, got_cnt, scores, k, what, cand_mask=None):
    """Exact when the gap at rank k is clear, else a valid top-k.  Returns True if exact was asserted."""
    s = np.asarray(scores, dtype=np.float64)
    if cand_mask is not None:
        s = np.where(cand_mask, s, -np.inf)
    ref_idx, ref_cnt = topk.select(s, k)
    gap = topk.gap_at_rank(s, k)
    if gap >= GAP:
        assert got_cnt == ref_cnt, f"{what}: count {got_cnt} != {ref_cnt}"
        assert np.array_equal(got_idx, ref_idx), f"{what}: block ids differ (gap {gap:.3g})"
        return True
    sel = got_idx[:got_cnt]
    assert got_cnt == ref_cnt, f"{what}: count {got_cnt} != {ref_cnt}"
    assert np.all(np.diff(sel) > 0), f"{what}: ids not strictly ascending"
    assert np.all(got_idx[got_cnt:] == -1), f"{what}: padding is not -1"
    assert np.isfinite(s[sel]).all(), f"{what}: a selected block is not a candidate"
    rest = np.setdiff1d(np.nonzero(np.isfinite(s))[0], sel)
    if rest.size and sel.size:
        tol = 1e-5 * max(1.0, np.abs(s[np.isfinite(s)]).max())
        assert s[sel].min() >= s[rest].max() - tol, f"{what}: not a valid top-{k}"
    return False


def _decode_checks(cfg, x, layers, wl, rows, keys=None):
    """rows: sequences to check; every query row of each (cfg.Q per sequence).

    keys: the indexer keys the oracle scores (default: the bf16 keys)."""
    keys = x.keys if keys is None else keys
    nb = cfg.cap // 8
    N = cfg.N
    Q = cfg.Q
    qpos = (lambda b, r: None) if x.q_pos is None else (lambda b, r: int(x.q_pos[b, r]))
    p0 = (lambda b: 0) if x.swa_pos0 is None else (lambda b: int(x.swa_pos0[b]))
    prev_sel = prev_buf = None
    exact = 0
    for li, (L, D) in enumerate(zip(layers, wl.layers)):
        buf = D["buf"]
        idx, cnt = host(buf.idx), host(buf.count)            # [B][Q][K], [B][Q]
        out, lse = host(buf.out), host(buf.lse_out)
        if L.mode in ("F", "R"):
            for b in range(x.latent.shape[0]):
                for r in range(Q):
                    s = indexer.block_scores(L.q_idx[b, r], L.w[b, r], keys[b], N, q_pos=qpos(b, r),
                                             n_blocks=nb)
                    mask = None
                    if cfg.top_groups:
                        gs = indexer.group_scores(L.q_idx[b, r], L.w[b, r], keys[b], N, n_groups=nb // 64)
                        assert topk.gap_at_rank(gs, cfg.top_groups) >= GAP, "generator gap at the group rank"
                        gsel, gc = topk.select(gs, cfg.top_groups)
                        mask = np.zeros(nb, dtype=bool)
                        mask[indexer.blocks_of_groups(gsel[:gc])] = True
                    exact += _check_selection(idx[b, r], int(cnt[b, r]), s, cfg.K, f"layer {li} row {b}.{r}", mask)
            sel = (idx, cnt)
            buf_used = buf
        else:
            # Reuse: the layer attends the earlier layer's buffers themselves (its own
            # idx/count buffers stay unused); they must still hold what was checked
            assert prev_sel is not None
            src = prev_buf
            same = np.array_equal(host(src.idx), prev_sel[0]) and np.array_equal(host(src.count), prev_sel[1])
            assert same, "Reuse layer changed the index buffer it was given"
            sel = prev_sel
            buf_used = src
        ref_o, ref_l, got_o, got_l = [], [], [], []
        for b in rows:
            for r in range(Q):
                rec = _records_of(x.latent[b], sel[0][b, r, :sel[1][b, r]], nb)
                ro, rl = om.attend_row(L.q[b, r], rec, sel[0][b, r], int(sel[1][b, r]), N, L.swa[b],
                                       int(x.swa_len[b]), cfg.W, q_pos=qpos(b, r), swa_pos0=p0(b))
                ref_o.append(ro), ref_l.append(rl), got_o.append(out[b, r]), got_l.append(lse[b, r])
        assert_close_rms(np.stack(got_o), np.stack(ref_o), what=f"{cfg.name} layer {li} ({L.mode}) out")
        assert_lse_close(np.stack(got_l), np.stack(ref_l))
        prev_sel = sel
        prev_buf = buf_used
    print(f"[full] {cfg.name}: {exact} exact selections", flush=True)
    # appended entry (position N-1) and a few selected blocks: record bytes exact
    rec_gpu = wl.cache.records
    rng = np.random.default_rng(5)
    for b in rows[:4]:
        blocks = np.unique(np.concatenate([[(N - 1) // 8], rng.choice(prev_sel[0][b, 0, :prev_sel[1][b, 0]], 8)]))
        ref = _records_of(x.latent[b], blocks, nb)
        got = host(rec_gpu[b, torch.from_numpy(blocks).cuda()])
        assert np.array_equal(got, ref[blocks]), f"row {b}: record bytes differ"


@pytest.mark.timeout(600)
def test_decode64k_full_size():
    cfg, (x, layers), wl = _workload("decode64k")
    _decode_checks(cfg, x, layers, wl, rows=list(range(cfg.B)))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["decode64k", "decode1m"])
def test_mxfp8_key_cache_full_size(name):
    # the whole step on the MXFP8 indexer key cache (flat, and two-level with
    # the group sums of the dequantised keys); the oracle scores the keys
    # through its own MXFP8 encoding
    cfg, (x, layers), wl = _workload(name, key_format="mxfp8")
    _decode_checks(cfg, x, layers, wl, rows=list(range(cfg.B)), keys=mxfp8.quantize_dequantize(x.keys))


@pytest.mark.timeout(600)
def test_decode1m_two_level_full_size():
    # the bench's step loop (its decode append rewrites entry N-1 every step)
    # for 1000 more steps: the group sums must still be the sums of the keys the
    # cache holds, and the two-level selection the oracle's
    cfg, (x, layers), wl = _workload("decode1m")
    for _ in range(1000):
        wl.step()
    torch.cuda.synchronize()
    got = host(wl.cache.group_sum)
    G = cfg.cap // 512
    for b in range(cfg.B):
        means, _ = indexer.group_means(x.keys[b], int(x.n_entries[b]), n_groups=G)
        cnt = np.clip(int(x.n_entries[b]) - 512 * np.arange(G), 0, 512)
        exp = (means * cnt[:, None]).astype(np.float32)
        assert np.array_equal(got[b], exp), f"seq {b}: group sums differ after 1002 steps"
    _decode_checks(cfg, x, layers, wl, rows=list(range(cfg.B)))


@pytest.mark.timeout(600)
def test_layers128k_full_reindex_reuse():
    cfg, (x, layers), wl = _workload("layers128k")
    rows = sorted(set([0, cfg.B - 1] + list(np.random.default_rng(3).choice(cfg.B, 6, replace=False))))
    _decode_checks(cfg, x, layers, wl, rows=rows)


@pytest.mark.timeout(600)
def test_specdec64k_draft_rows_full_size():
    # 4 rows per sequence at consecutive positions (a token and 3 drafts), each
    # with its own selection, causal window and attention
    cfg, (x, layers), wl = _workload("specdec64k")
    _decode_checks(cfg, x, layers, wl, rows=list(range(0, cfg.B, 4)))


@pytest.mark.timeout(600)
def test_prefill_sampled_rows():
    _prefill_checks("prefill", sorted(set([0, 4095] + list(np.random.default_rng(4).choice(4096, 62,
                                                                                           replace=False)))))


@pytest.mark.timeout(600)
def test_row_tiles_full_size():
    # the head-sharded workloads, where rows share attention tiles: draft rows
    # (every sequence's 4 rows checked in 8 sequences) and prefill (both rows
    # of 31 sampled tiles, and the first and last rows)
    cfg, (x, layers), wl = _workload("specdec64k_h16")
    _decode_checks(cfg, x, layers, wl, rows=list(range(0, cfg.B, 4)))
    del wl
    torch.cuda.empty_cache()
    pairs = np.random.default_rng(6).choice(2048, 31, replace=False)
    _prefill_checks("prefill_h16", sorted(set([0, 4095] + [int(r) for k in pairs for r in (2 * k, 2 * k + 1)])))


def _prefill_checks(name, rows):
    cfg, p, wl = _workload(name)
    Q = p["q"].shape[1]
    N, prior = int(p["n_entries"][0]), int(p["prior"])
    nb = cfg.cap // 8
    idx, cnt = host(wl.buf.idx)[0], host(wl.buf.count)[0]
    out, lse = host(wl.buf.out)[0], host(wl.buf.lse_out)[0]
    exact = 0
    ref_o, ref_l = [], []
    for r in rows:
        t = int(p["q_pos"][0, r])
        s = indexer.block_scores(p["q_idx"][0, r], p["w"][0, r], p["keys"][0], N, q_pos=t, n_blocks=nb)
        exact += _check_selection(idx[r], int(cnt[r]), s, cfg.K, f"prefill row {r}")
        rec = _records_of(p["latent"][0], idx[r, :cnt[r]], nb)
        ro, rl = om.attend_row(p["q"][0, r], rec, idx[r], int(cnt[r]), N, p["swa"][0], int(p["swa_len"][0]),
                               cfg.W, q_pos=t, swa_pos0=int(p["swa_pos0"][0]))
        ref_o.append(ro), ref_l.append(rl)
    print(f"[full] {name}: {exact} of {len(rows)} sampled rows exact", flush=True)
    assert_close_rms(out[rows], np.stack(ref_o), what=f"{name} out")
    assert_lse_close(lse[rows], np.stack(ref_l))
    # the chunk's appended records, all 256 blocks: exact bytes
    blocks = np.arange(prior // 8, N // 8)
    ref = _records_of(p["latent"][0], blocks, nb)
    got = host(wl.cache.records[0, prior // 8:N // 8])
    assert np.array_equal(got, ref[blocks]), "chunk record bytes differ"
