"""Benchmark: CSA2 sparse attention over an MXFP4 latent cache on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  decode    csa2_append_fp4 (one new entry per sequence) -> per layer:
            csa2_index_topk (Full / Reindex) -> csa2_attend_layer (sparse branch +
            sliding window, merged by one log-sum-exp combine)
  prefill   csa2_append_fp4 (the chunk's 2048 entries) -> csa2_index_topk (causal,
            every query row) -> csa2_attend_layer (causal window)
All calls run on one stream: running the window branch on a second stream
beside the indexer (csa2_attend_layer_window / _sparse) measured no faster,
as the two contend for HBM and CUs.

Default workload (--config decode1m): decode at 1M raw positions, 8 sequences,
64 heads, 524288 MXFP4 entries = 65536 blocks of 8 per sequence, two-level
8 x 64 indexer keeping 256 of 1024 groups of 64 blocks, top-K 2048, window 512;
seeded N(0,1) bf16 inputs with planted relevant groups and blocks.  decode64k
and layers128k are timed after it and carried in the same line
(``other_workloads``); --config selects any single workload (tiny, decode64k,
decode1m, layers128k, prefill, specdec64k: decode64k's cache with 4 query rows
per sequence, a token and 3 drafts verified in one pass).

Prints ONE JSON line.  `value` = query rows per second (decode queries/s, or
prefill tokens/s) over cold steps: each timed step starts after a 1 GiB scratch
read, so L2 and the 256 MB last-level cache hold none of the workload (HIP
events on the library's stream bracket the step itself); `warm_value` times the
same steps back to back.  `roofline` covers csa2_attend_layer, the attention
call the step makes (the one-launch sparse + window kernel and its combine;
MFMA-bound at 64 heads): algorithmic FLOPs = 4 * H * 512 per attended entry or
window token, over the call's mean cold time.  `cpu_baseline` times the NumPy
fp64 oracle on a bounded sample of rows on the host cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn decode queries/s and TB/s FP4 KV read; % of HBM/MFMA roofline"
PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0
RECORD = 2176
# HBM bytes per csa2_attend_layer call (attend_kernel + its combine) from
# rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs, with the hash of the kernel
# sources they were taken on
KERNEL_SRCS = [os.path.join(ROOT, "sparse_attention_fp4_csa2_amd", "csrc", f)
               for f in ("sparse_fp4.hip", "attention.hip", "window_body.h", "device.h")]


def traffic_file(config):
    return os.path.join(ROOT, "profiles", f"traffic_attend_layer_{config}.json")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode1m",
                    choices=["tiny", "decode64k", "decode1m", "layers128k", "prefill", "specdec64k",
                             "specdec64k_h16", "prefill_h16"])
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads timed after the headline one and carried in the same "
                         "JSON line (default for decode1m: decode64k,layers128k; '' for none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--index-keys", default="bf16", choices=["bf16", "mxfp8"],
                    help="indexer key cache: bf16 (the workload's definition) or the lower-precision "
                         "MXFP8 variant")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed steps for this long (seconds) before the warm-up steps, so the GPU "
                         "clocks reach their steady state (they ramp over the first ~30 ms of work)")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="reps of the cold per-call timings (a 1 GiB read before each evicts L2 and the "
                         "256 MB last-level cache)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak reference runs")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run a plain fp32 copy kernel over this many bytes "
                         "(the calibration point for rocprofv3 FETCH_SIZE / WRITE_SIZE runs)")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="no GPU work: turn rocprofv3 CSV output into a profile summary on stdout. "
                         "'trace KERNEL_TRACE_CSV BENCH_JSON' (per-kernel durations, markdown), "
                         "'traffic FETCH_CSV WRITE_CSV COPY_BYTES' (HBM bytes per csa2_attend_layer "
                         "call, JSON), 'counters COUNTER_CSV' (SQ counters per kernel, markdown); "
                         "--config names the workload, --command the commands that made the input")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize: a command that produced the input (recorded verbatim)")
    return ap.parse_args(argv)


# ---------------------------------------------------------------------------
# workloads (device state + one step), shared with the full-size parity tests


class Key8Index:
    """The same selection on the MXFP8 indexer key cache (csa2_append_key8 +
    csa2_index_topk_key8): a timed call beside the step, not part of it."""

    def __init__(self, lib, keys, cap, B, Q, K, top_groups, device="cuda"):
        import torch
        self.lib, self.K, self.top_groups = lib, K, top_groups
        self.key8 = torch.zeros(B, cap, 64, dtype=torch.uint8, device=device)
        self.scale = torch.zeros(B, cap, 2, dtype=torch.uint8, device=device)
        self.gsum = (torch.zeros(B, cap // 512, 64, dtype=torch.float32, device=device)
                     if top_groups else None)
        lib.append_key8(keys, torch.zeros(B, dtype=torch.int32, device=device), self.key8, self.scale,
                        group_sum=self.gsum)
        self.idx = torch.empty(B, Q, K, dtype=torch.int32, device=device)
        self.count = torch.empty(B, Q, dtype=torch.int32, device=device)
        self.ws = torch.empty(max(lib.index_topk_ws(B, Q, cap, top_groups), 256), dtype=torch.uint8,
                              device=device)

    def call(self, q_idx, w, n_entries, q_pos, stream):
        self.lib.index_topk_key8(q_idx, w, self.key8, self.scale, n_entries, self.K, self.idx, self.count,
                                 self.ws, group_sum=self.gsum, q_pos=q_pos, top_groups=self.top_groups,
                                 stream=stream)


class DecodeWorkload:
    """Decode: B sequences, one query row each, through the layers of ``cfg.layers``."""

    def __init__(self, cfg, x, layers, device="cuda", key_format="bf16"):
        import torch
        from sparse_attention_fp4_csa2_amd import _lib, modes
        self.torch, self._lib, self.modes = torch, _lib, modes
        self.cfg, self.x, self.layer_inputs = cfg, x, layers
        B, N = x.latent.shape[0], cfg.N
        self.B, self.rows = B, B * cfg.Q
        self.cache = modes.LatentCache.empty(B, cfg.cap, device, with_groups=bool(cfg.top_groups),
                                             key_format=key_format)
        self.cache.append(_bf(x.latent, device), _bf(x.keys, device))
        self.key8 = (Key8Index(_lib, _bf(x.keys, device), cfg.cap, B, cfg.Q, cfg.K, cfg.top_groups, device)
                     if key_format == "bf16" else None)
        self.swa_len = torch.from_numpy(x.swa_len).to(device)
        self.layers = []
        for L in layers:
            buf = modes.LayerBuffers(B, cfg.Q, cfg.H, cfg.cap, cfg.K, cfg.W,
                                     top_groups=cfg.top_groups, device=device)
            self.layers.append(dict(
                mode=L.mode, buf=buf, q=_bf(L.q, device), swa=_bf(L.swa, device),
                q_idx=_bf(L.q_idx, device) if L.q_idx is not None else None,
                w=torch.from_numpy(L.w).to(device) if L.w is not None else None))
        # decode append: one new entry per sequence, rewritten at the last held
        # position so every step sees the same cache
        self.new_lat = _bf(x.latent[:, N - 1:N], device)
        self.new_key = _bf(x.keys[:, N - 1:N], device)
        self.start = torch.full((B,), N - 1, dtype=torch.int32, device=device)
        # several rows per sequence (draft verification): their raw positions
        self.q_pos = None if x.q_pos is None else torch.from_numpy(x.q_pos).to(device)
        self.swa_pos0 = None if x.swa_pos0 is None else torch.from_numpy(x.swa_pos0).to(device)
        self.stream = torch.cuda.current_stream()

    def append(self):
        self.cache.write(self.new_lat, self.new_key, self.start, stream=self.stream)

    def step(self):
        self.append()
        prev = None
        for L in self.layers:
            prev = self.modes.run_layer(L["mode"], L["buf"], self.cache, L["q"], L["swa"],
                                        self.swa_len, q_idx=L["q_idx"], w=L["w"], prev=prev,
                                        stream=self.stream, q_pos=self.q_pos, swa_pos0=self.swa_pos0)

    def calls(self):
        """name -> (callable, launches per step) for the per-call breakdown."""
        L0 = self.layers[0]
        buf = L0["buf"]
        m, lib, s = self.modes, self._lib, self.stream
        n_index = sum(1 for L in self.layers if L["mode"] in ("F", "R"))
        return {
            "append": (self.append, 1),
            "index_topk": (lambda: m.index(buf, self.cache, L0["q_idx"], L0["w"], q_pos=self.q_pos, stream=s),
                           n_index),
            "attend_layer": (lambda: m.attend(buf, self.cache, L0["q"], L0["swa"], self.swa_len,
                                              swa_pos0=self.swa_pos0, q_pos=self.q_pos, stream=s),
                             len(self.layers)),
            # the two branches as separate calls (not part of the step; sparse_attn is the roofline unit)
            "sparse_attn": (self.sparse_attn_call, 0),
            **({"index_topk_key8": (lambda: self.key8.call(L0["q_idx"], L0["w"], self.cache.n_entries,
                                                            self.q_pos, s), 0)} if self.key8 else {}),
            "swa_merge": (lambda: lib.swa_merge(L0["q"], L0["swa"], self.swa_len, self.cfg.W, m.SCALE,
                                                buf.o, buf.lse, buf.out, buf.lse_out, buf.ws_swa,
                                                swa_pos0=self.swa_pos0, q_pos=self.q_pos, stream=s), 0),
        }

    def sparse_attn_call(self):
        L0 = self.layers[0]
        buf = L0["buf"]
        self._lib.sparse_attn(L0["q"], self.cache.records, buf.idx, buf.count, self.cache.n_entries,
                              self.modes.SCALE, buf.o, buf.lse, ws=buf.ws_attn, q_pos=self.q_pos,
                              stream=self.stream)

    def attended_entries(self):
        """Selected visible entries summed over rows, for the first layer's selection."""
        counts = self.layers[0]["buf"].count.cpu().numpy()
        return int(counts.sum()) * 8

    def window_tokens(self):
        """Window tokens attended, summed over rows (one layer)."""
        x = self.x
        p0 = np.zeros(self.B, np.int64) if x.swa_pos0 is None else x.swa_pos0.astype(np.int64)
        last = p0 + x.swa_len.astype(np.int64) - 1
        t = np.repeat(last[:, None], self.cfg.Q, 1) if x.q_pos is None else x.q_pos.astype(np.int64)
        lo = np.maximum(t - self.cfg.W + 1, p0[:, None])
        hi = np.minimum(t, last[:, None])
        return int(np.clip(hi - lo + 1, 0, None).sum())


class PrefillWorkload:
    """Chunked prefill: Q query tokens after ``prior`` cached entries, causal everywhere."""

    def __init__(self, cfg, p, device="cuda", key_format="bf16"):
        import torch
        from sparse_attention_fp4_csa2_amd import _lib, modes
        self.torch, self._lib, self.modes = torch, _lib, modes
        self.cfg, self.p = cfg, p
        N, prior = int(p["n_entries"][0]), int(p["prior"])
        Q = p["q"].shape[1]
        self.B, self.rows = 1, Q
        self.cache = modes.LatentCache.empty(1, cfg.cap, device, key_format=key_format)
        self.cache.append(_bf(p["latent"], device), _bf(p["keys"], device))
        self.key8 = Key8Index(_lib, _bf(p["keys"], device), cfg.cap, 1, Q, cfg.K, 0, device) \
            if key_format == "bf16" else None
        self.buf = modes.LayerBuffers(1, Q, cfg.H, cfg.cap, cfg.K, cfg.W, device=device)
        self.q = _bf(p["q"], device)
        self.q_idx = _bf(p["q_idx"], device)
        self.w = torch.from_numpy(p["w"]).to(device)
        self.q_pos = torch.from_numpy(p["q_pos"]).to(device)
        self.swa = _bf(p["swa"], device)
        self.swa_len = torch.from_numpy(p["swa_len"]).to(device)
        self.swa_pos0 = torch.from_numpy(p["swa_pos0"]).to(device)
        # the chunk's entries, rewritten in place each step
        self.chunk_lat = _bf(p["latent"][:, prior:N], device)
        self.chunk_key = _bf(p["keys"][:, prior:N], device)
        self.start = torch.full((1,), prior, dtype=torch.int32, device=device)
        self.stream = torch.cuda.current_stream()

    def append(self):
        self.cache.write(self.chunk_lat, self.chunk_key, self.start, stream=self.stream)

    def index(self):
        self.modes.index(self.buf, self.cache, self.q_idx, self.w, q_pos=self.q_pos, stream=self.stream)

    def sparse_attn_call(self):
        b = self.buf
        self._lib.sparse_attn(self.q, self.cache.records, b.idx, b.count, self.cache.n_entries,
                              self.modes.SCALE, b.o, b.lse, ws=b.ws_attn, q_pos=self.q_pos,
                              stream=self.stream)

    def swa_call(self):
        b = self.buf
        self._lib.swa_merge(self.q, self.swa, self.swa_len, self.cfg.W, self.modes.SCALE, b.o, b.lse,
                            b.out, b.lse_out, b.ws_swa, swa_pos0=self.swa_pos0, q_pos=self.q_pos,
                            stream=self.stream)

    def attend_call(self):
        self.modes.attend(self.buf, self.cache, self.q, self.swa, self.swa_len, swa_pos0=self.swa_pos0,
                          q_pos=self.q_pos, stream=self.stream)

    def step(self):
        self.append()
        self.index()
        self.attend_call()

    def calls(self):
        return {"append": (self.append, 1), "index_topk": (self.index, 1),
                "attend_layer": (self.attend_call, 1),
                "sparse_attn": (self.sparse_attn_call, 0), "swa_merge": (self.swa_call, 0),
                **({"index_topk_key8": (lambda: self.key8.call(self.q_idx, self.w, self.cache.n_entries,
                                                                self.q_pos, self.stream), 0)}
                   if self.key8 else {})}

    def attended_entries(self):
        """Visible entries of the selected blocks summed over rows (causal masking counted)."""
        idx = self.buf.idx.cpu().numpy()[0]
        cnt = self.buf.count.cpu().numpy()[0]
        qpos = self.p["q_pos"][0]
        n = int(self.p["n_entries"][0])
        total = 0
        for r in range(idx.shape[0]):
            blk = idx[r, :cnt[r]].astype(np.int64)
            ent = blk[:, None] * 8 + np.arange(8)[None, :]
            total += int(((ent < n) & (2 * ent + 1 <= qpos[r])).sum())
        return total

    def window_tokens(self):
        """Window tokens attended, summed over query rows (causal)."""
        p0 = int(self.p["swa_pos0"][0])
        last = p0 + int(self.p["swa_len"][0]) - 1
        t = self.p["q_pos"][0].astype(np.int64)
        lo = np.maximum(t - self.cfg.W + 1, p0)
        hi = np.minimum(t, last)
        return int(np.clip(hi - lo + 1, 0, None).sum())


def _bf(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def make_workload(name, device="cuda", key_format="bf16"):
    """(cfg, host inputs, workload) for a named config, as bench.py times it."""
    from synth import CONFIGS, decode_inputs, layers_inputs, prefill_inputs, specdec_inputs
    from synth.gen import LayerInputs
    cfg = CONFIGS[name]
    if cfg.prior:
        p = prefill_inputs(cfg)
        return cfg, p, PrefillWorkload(cfg, p, device, key_format)
    if len(cfg.layers) > 1:
        x, layers = layers_inputs(cfg)
    else:
        x = specdec_inputs(cfg) if cfg.Q > 1 else decode_inputs(cfg)
        layers = [LayerInputs("F", x.q, x.q_idx, x.w, x.swa, x.planted)]
    return cfg, (x, layers), DecodeWorkload(cfg, x, layers, device, key_format)


# ---------------------------------------------------------------------------


def _workload_for(name, index_keys):
    import torch
    t0 = time.time()
    cfg, host_in, wl = make_workload(name, key_format=index_keys)
    torch.cuda.synchronize()
    return cfg, host_in, wl, time.time() - t0


def measure(name, args):
    """Time one workload: cold steps (the headline form), warm steps, per-call
    breakdowns, the attention call against the MFMA roofline.  Returns
    (cfg, host inputs, workload, result dict)."""
    import torch
    cfg, host_in, wl, gen_s = _workload_for(name, args.index_keys)
    stream = wl.stream
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731

    # settle: the same step, untimed, until the clocks have ramped up
    t_settle = time.time()
    while time.time() - t_settle < args.settle_s:
        for _ in range(10):
            wl.step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()

    # timed: exactly `steps` cold steps.  Each starts after a 1 GiB scratch
    # read (L2 and the 256 MB last-level cache then hold clean scratch lines,
    # not the workload; a write would leave dirty lines whose write-back would
    # run into the timed step); HIP events on the library's stream bracket the
    # step alone.
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(scratch, dim=0, out=flush_out)

    flush()
    pairs = []
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush()
        a, b = ev(), ev()
        a.record(stream)
        wl.step()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    cold_steps = [a.elapsed_time(b) for a, b in pairs]
    ms_cold = float(np.mean(cold_steps))

    # warm: the same number of steps back to back (inputs partly stay in the
    # last-level cache between steps)
    a, b = ev(), ev()
    a.record(stream)
    for _ in range(args.steps):
        wl.step()
    b.record(stream)
    torch.cuda.synchronize()
    ms_warm = a.elapsed_time(b) / args.steps

    def warm_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def cold_ms(fn, reps):
        ts = []
        for i in range(reps):
            flush()
            a, b = ev(), ev()
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.mean(ts))

    reps = max(args.steps, 10)
    breakdown, cold_bd, per_step = {}, {}, {}
    for cname, (fn, n) in wl.calls().items():
        breakdown[cname] = warm_ms(fn, reps)
        per_step[cname] = n
        if n > 0 or cname == "sparse_attn":
            cold_bd[cname] = cold_ms(fn, max(args.cold_reps, 1))
    wl.step()
    torch.cuda.synchronize()
    n_ent = wl.attended_entries()
    rows = wl.rows
    win = wl.window_tokens()
    flops_layer = 4.0 * cfg.H * 512 * (n_ent + win)
    flops_sparse = 4.0 * cfg.H * 512 * n_ent
    t_layer, t_layer_warm = cold_bd["attend_layer"], breakdown["attend_layer"]
    t_sparse = cold_bd["sparse_attn"]
    tf = lambda fl, ms: fl / (ms * 1e-3) / 1e12    # noqa: E731

    # top-K on unplanted scores: the selection call's top-K over N(0,1) scores of
    # the step's shape (rows x candidates), i.e. a boundary inside a dense
    # score distribution rather than under a planted set
    n_cand = cfg.top_groups * 64 if cfg.top_groups else cfg.cap // 8
    g = torch.Generator(device="cuda").manual_seed(cfg.seed)
    rnd = torch.randn(rows, n_cand, device="cuda", generator=g)
    t_idx = torch.empty(rows, cfg.K, dtype=torch.int32, device="cuda")
    t_cnt = torch.empty(rows, dtype=torch.int32, device="cuda")
    topk_random = warm_ms(lambda: wl._lib.topk(rnd, cfg.K, t_idx, t_cnt, stream=stream), reps)
    del rnd, scratch, flush_out

    prefill = cfg.prior > 0
    res = {
        "value": round(rows / (ms_cold * 1e-3), 1),
        "unit": "tokens/s" if prefill else "queries/s",
        "ms_per_step": round(ms_cold, 4),
        "warm_value": round(rows / (ms_warm * 1e-3), 1),
        "warm_ms_per_step": round(ms_warm, 4),
        "config": workload_config(cfg, rows, args.index_keys),
        "fp4_kv_read_TBps": round(n_ent * 272 / (t_layer * 1e-3) / 1e12, 3),
        "cold_breakdown_ms": {k: round(v, 4) for k, v in cold_bd.items()},
        "breakdown_ms": {k: round(v, 4) for k, v in breakdown.items()},
        "launches_per_step": per_step,
        "kernels_per_layer": kernels_per_layer(cfg, wl._lib),
        "topk_unplanted_ms": round(topk_random, 4),
        "roofline": {"kernel": "csa2_attend_layer (attend_kernel: sparse + window branches; then the combine "
                               "unless one partial per (row, head) remains)",
                     "bound": "mfma", "achieved": round(tf(flops_layer, t_layer), 2),
                     "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf(flops_layer, t_layer) / PEAK_FP16_TFLOPS, 4),
                     "traffic": stored_traffic(name),
                     "flops_per_launch": flops_layer,
                     "timing": "cold (1 GiB scratch read before each call), mean",
                     "achieved_warm": round(tf(flops_layer, t_layer_warm), 2),
                     "frac_warm": round(tf(flops_layer, t_layer_warm) / PEAK_FP16_TFLOPS, 4)},
        "roofline_sparse_attn": {"kernel": "csa2_sparse_attn (sparse branch alone + combine)",
                                 "achieved": round(tf(flops_sparse, t_sparse), 2), "unit": "TFLOP/s",
                                 "frac": round(tf(flops_sparse, t_sparse) / PEAK_FP16_TFLOPS, 4),
                                 "timing": "cold, mean"},
        "setup_s": round(gen_s, 1),
    }
    if not prefill:
        kb = 128 if args.index_keys == "bf16" else 66     # key bytes: bf16, or MXFP8 codes + scales
        idx_bytes = wl.B * cfg.N * kb if not cfg.top_groups else \
            wl.B * (cfg.cap // 512 * 256 + cfg.top_groups * 512 * kb)
        res["indexer_GBps"] = round(idx_bytes / (cold_bd["index_topk"] * 1e-3) / 1e9, 1)
        if "index_topk_key8" in breakdown:
            idx8_bytes = wl.B * cfg.N * 66 if not cfg.top_groups else \
                wl.B * (cfg.cap // 512 * 256 + cfg.top_groups * 512 * 66)
            res["indexer_key8_GBps_warm"] = round(idx8_bytes / (breakdown["index_topk_key8"] * 1e-3) / 1e9, 1)
    if len(cfg.layers) > 1:
        res["reuse_saving_ms"] = round(cold_bd["index_topk"] * cfg.layers.count("U"), 4)
    return cfg, host_in, wl, res


def main():
    args = parse()
    if args.summarize:
        sys.exit(summarize(args))
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence/row with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_fp4_csa2_amd import _lib
    _lib.load()
    also = args.also
    if also is None:
        also = "decode64k,layers128k" if args.config == "decode1m" else ""
    also = [c for c in also.split(",") if c and c != args.config]

    cfg, host_in, wl, res = measure(args.config, args)
    stream = wl.stream
    peaks = None if args.no_peaks else measured_peaks(torch, stream)
    cpu = None if args.no_cpu else cpu_baseline(cfg, host_in, args.cpu_seconds)
    del wl, host_in
    torch.cuda.empty_cache()

    others = {}
    for name in also:
        _, _, w2, r2 = measure(name, args)
        others[name] = {k: r2[k] for k in ("value", "unit", "ms_per_step", "warm_value", "warm_ms_per_step",
                                           "cold_breakdown_ms", "topk_unplanted_ms") if k in r2}
        others[name]["workload"] = r2["config"]["workload"]
        others[name]["roofline_frac"] = r2["roofline"]["frac"]
        others[name]["roofline_frac_warm"] = r2["roofline"]["frac_warm"]
        del w2
        torch.cuda.empty_cache()

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    result = {
        "metric": METRIC,
        "value": res["value"],
        "unit": res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4xfp6 Q.K / fp16 P.V",
        "data": "synthetic (seeded N(0,1) bf16, planted relevant blocks with distinct scores)",
        "config": res["config"],
        "timing": ("value: cold steps (each after a 1 GiB scratch read that evicts L2 and the last-level "
                   "cache; HIP events around the step); warm_value: the same steps back to back"),
        "compute": ("Q.K on the scaled FP4 x FP6 MFMA (query split into three E2M3 terms; bf16 MFMA on exactly "
                    "dequantised codes for query blocks with outlier channels), P.V on fp16 MFMA with the "
                    "MXFP4 values dequantised to fp16, fp32 accumulate; window in bf16"),
    }
    for k, v in res.items():
        if k not in result and k not in ("value", "unit", "ms_per_step"):
            result[k] = v
    if peaks is not None:
        result["measured_peaks"] = peaks
        result["roofline"]["frac_of_measured_gemm"] = round(result["roofline"]["achieved"] /
                                                            peaks["bf16_gemm_TFLOPs"], 4)
    if others:
        result["other_workloads"] = others
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def measured_peaks(torch, stream):
    """Reference rates measured in the same session: a 1 GiB fp32 copy (read +
    write bytes over time) and a dense 8192^3 bf16 GEMM through torch.matmul
    (the vendor GEMM library); medians of 10 runs each."""
    def med(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = med(lambda: dst.copy_(src))
    del src, dst
    n = 8192
    a = torch.ones((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.ones((n, n), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    t_mm = med(lambda: torch.matmul(a, b, out=c))
    del a, b, c
    return {"copy_GBps": round(2 * (1 << 30) / (t_copy * 1e-3) / 1e9, 1),
            "bf16_gemm_TFLOPs": round(2.0 * n ** 3 / (t_mm * 1e-3) / 1e12, 1)}


def kernels_per_layer(cfg, lib=None):
    """Kernel launches of one layer's attention path, by layer mode (append not included).

    csa2_index_topk launches the indexer and the top-K (two-level: coarse scores,
    group top-K, fine scores, top-K); csa2_attend_layer launches both branches
    in one kernel, then a combine unless that kernel leaves a single partial
    per (row, head) (the library reports which).  Reuse layers run only the
    latter."""
    index = 4 if cfg.top_groups else 2
    attend = lib.attend_layer_launches(cfg.B, cfg.Q, cfg.H, cfg.K, cfg.W) if lib is not None else 2
    modes = sorted(set(cfg.layers)) if not cfg.prior else ["F"]
    return {m: (index + attend if m in ("F", "R") else attend) for m in modes}


def workload_config(cfg, rows, index_keys="bf16"):
    if cfg.prior:
        desc = (f"prefill: {cfg.Q} query tokens after {cfg.prior} cached entries (+{cfg.Q // 2} "
                f"appended), H {cfg.H}, indexer {cfg.Hi}x64, top-K {cfg.K} per row, window {cfg.W}, causal"
                + (f", query rows in runs of {cfg.q_run} per indexer direction" if cfg.q_run > 1 else ""))
    else:
        desc = (f"{cfg.name}: decode, B {cfg.B}, H {cfg.H}, {cfg.N} MXFP4 entries/seq "
                f"({cfg.N // 8} blocks of 8), indexer {cfg.Hi}x64"
                + (f" two-level ({cfg.top_groups} of {cfg.cap // 512} groups)" if cfg.top_groups else "")
                + f", top-K {cfg.K}, window {cfg.W}"
                + (f", layers {'/'.join(cfg.layers)}" if len(cfg.layers) > 1 else "")
                + (f", {cfg.Q} rows per sequence (1 + {cfg.Q - 1} drafts verified together)"
                   if cfg.Q > 1 else ""))
    if index_keys != "bf16":
        desc += f", {index_keys.upper()} indexer keys"
    return {"workload": desc, "global_batch": rows, "seq_len": 2 * cfg.N, "parallelism": "single GPU"}


def kernel_digest():
    """SHA-256 over the sources of the csa2_sparse_attn kernels (attention + combine)."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def stored_traffic(config):
    """Measured HBM bytes per csa2_sparse_attn call, or None once the kernel source changed."""
    path = traffic_file(config)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    digest = kernel_digest()
    if rec.get("kernel_sources_sha256") != digest:
        return None
    return rec.get("bytes_per_call")


# ---------------------------------------------------------------------------
# rocprofv3 output -> the profile summaries kept with the sources

_CALL_OF_COMBINE = {"attend_kernel": "csa2_attend_layer", "sparse_fp4_kernel": "csa2_sparse_attn",
                    "window_kernel": "csa2_swa_merge"}


def _csa2_base(name):
    """csa2 kernel name without namespace and argument list; the attention
    and window kernels also without their rows-per-tile template argument (a
    workload runs one of each)."""
    base = name.split("(")[0].replace("void ", "").strip()
    if not base.startswith("csa2::"):
        return None
    base = base[len("csa2::"):]
    if base.startswith(("attend_kernel<", "sparse_fp4_kernel<", "window_kernel<")):
        base = base.split("<")[0]
    return base


def _kernel_label(name, prev_csa2):
    """Short label of a dispatch: csa2 kernels without namespace and argument
    list, the bf16- and MXFP8-key indexers told apart, combine_kernel named by
    the call it closes (the csa2 kernel dispatched before it)."""
    base = _csa2_base(name)
    if base is None:
        return None
    if base.startswith("index_scores_kernel") or base.startswith("index_rows_kernel"):
        base += " (MXFP8 keys)" if base.rstrip(">").endswith("true") else " (bf16 keys)"
    if base == "combine_kernel":
        base += f" ({_CALL_OF_COMBINE.get(prev_csa2, 'csa2_attend_layer')})"
    return base


def _labelled(rows):
    """rows: (name, start_ns, end_ns, extra) sorted by start -> (label, cold, dur_us, extra).
    A dispatch is cold when it runs in the same back-to-back burst as a
    preceding 1 GiB flush read (no idle gap above 15 us since it)."""
    out, prev_csa2, cold, last_end = [], None, False, None
    for name, st, en, extra in rows:
        if last_end is not None and st - last_end > 15000:
            cold = False
        last_end = en if last_end is None else max(last_end, en)
        if "reduce_kernel" in name:
            cold = True
            continue
        lab = _kernel_label(name, prev_csa2)
        if lab is None:
            continue
        prev_csa2 = _csa2_base(name)
        out.append((lab, cold, (en - st) / 1000.0, extra))
    return out


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _commands_block(args):
    return "\n".join(args.command) if args.command else "(not recorded)"


def summarize(args):
    from synth import CONFIGS
    kind, inputs = args.summarize[0], args.summarize[1:]
    cfg_desc = workload_config(CONFIGS[args.config], None, args.index_keys)["workload"]
    if kind == "trace":
        rows = _read_csv(inputs[0])
        disp = sorted(((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"]), None)
                       for r in rows), key=lambda x: x[1])
        lab = _labelled(disp)
        bench = json.loads(open(inputs[1]).read().strip().splitlines()[-1]) if len(inputs) > 1 else None
        by = {}
        for k, cold, d, _ in lab:
            by.setdefault(k, {"cold": [], "warm": []})["cold" if cold else "warm"].append(d)
        lines = [f"# Kernel trace: {cfg_desc}", "", "Commands (repository root on the GPU host as `$REPO`):",
                 "", "```", _commands_block(args), "```", "",
                 "Per-dispatch durations from the kernel-trace CSV, split into cold dispatches (in the "
                 "back-to-back burst after a 1 GiB scratch read that evicts L2 and the last-level cache) "
                 "and warm ones (the rest: settle, warm-up and back-to-back loops).  `combine_kernel` is "
                 "named by the call it closes; torch's own kernels are left out.", "",
                 "| kernel | warm n | warm median µs | warm mean µs | cold n | cold mean µs | min µs |",
                 "|---|---|---|---|---|---|---|"]
        order = sorted(by.items(), key=lambda kv: -sum(kv[1]["warm"] + kv[1]["cold"]))
        for k, v in order:
            w, c = v["warm"], v["cold"]
            fmt = lambda x: f"{x:.2f}" if x is not None else "-"   # noqa: E731
            lines.append(f"| {k} | {len(w)} | {fmt(float(np.median(w)) if w else None)} | "
                         f"{fmt(float(np.mean(w)) if w else None)} | {len(c)} | "
                         f"{fmt(float(np.mean(c)) if c else None)} | {min(w + c):.2f} |")
        att = [v for v in (by.get("attend_kernel"), by.get("combine_kernel (csa2_attend_layer)")) if v]
        if by.get("attend_kernel") and bench is not None:
            wm = sum(float(np.median(a["warm"])) for a in att)
            cm = sum(float(np.mean(a["cold"])) for a in att) if all(a["cold"] for a in att) else None
            ev_w = bench.get("breakdown_ms", {}).get("attend_layer")
            ev_c = bench.get("cold_breakdown_ms", {}).get("attend_layer")
            lines += ["", "The roofline's unit, one `csa2_attend_layer` call = `attend_kernel`"
                      + (" + its `combine_kernel`" if len(att) > 1 else " (one launch: no combine)") + ":", "",
                      f"- warm: trace medians {wm:.2f} µs; the traced run's own HIP-event time per call "
                      f"{ev_w * 1000:.2f} µs" if ev_w is not None else f"- warm: trace medians {wm:.2f} µs"]
            if cm is not None:
                lines.append(f"- cold: trace means {cm:.2f} µs; HIP events {ev_c * 1000:.2f} µs "
                             "(the roofline's `achieved` divides by this one)" if ev_c is not None
                             else f"- cold: trace means {cm:.2f} µs")
        if bench is not None:
            keep = {k: bench[k] for k in ("value", "unit", "ms_per_step", "warm_value", "warm_ms_per_step",
                                          "cold_breakdown_ms", "breakdown_ms", "roofline") if k in bench}
            lines += ["", "The traced bench.py run's line (profiling slows it; the figures above are from "
                      "the trace itself):", "", "```", json.dumps(keep), "```"]
        print("\n".join(lines))
        return 0
    if kind == "traffic":
        copy_bytes = int(inputs[2])
        per = {}
        for counter, path in (("FETCH_SIZE", inputs[0]), ("WRITE_SIZE", inputs[1])):
            rows = [r for r in _read_csv(path) if r["Counter_Name"] == counter]
            disp = sorted(((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                            float(r["Counter_Value"])) for r in rows), key=lambda x: x[1])
            vals = {}
            for k, _, _, v in _labelled(disp):
                vals.setdefault(k, []).append(v)
            # the calibration copy: the largest MulFunctor dispatches (bench.py runs it 3 times)
            muls = [float(r["Counter_Value"]) for r in rows if "MulFunctor" in r["Kernel_Name"]]
            copy = [v for v in muls if v >= 0.5 * max(muls)] if muls else []
            if not copy:
                print(f"no calibration copy kernel in {path}", file=sys.stderr)
                return 1
            vals["copy"] = copy
            per[counter] = {k: float(np.median(v)) for k, v in vals.items()}
        f_fac = copy_bytes / 1024.0 / per["FETCH_SIZE"]["copy"]
        w_fac = copy_bytes / 1024.0 / per["WRITE_SIZE"]["copy"]
        # the call's launches (the combine is absent when the launch leaves one partial)
        call = [k for k in ("attend_kernel", "combine_kernel (csa2_attend_layer)") if k in per["FETCH_SIZE"]]
        fetch = sum(per["FETCH_SIZE"][k] for k in call) * 1024 * f_fac
        write = sum(per["WRITE_SIZE"][k] for k in call) * 1024 * w_fac
        cfg = CONFIGS[args.config]
        rec = {"kernel": "csa2_attend_layer call = " + " + ".join(k.split(" (")[0] for k in call),
               "workload": cfg_desc, "kernel_sources_sha256": kernel_digest(),
               "bytes_per_call": int(round(fetch + write)), "fetch_bytes_per_call": int(round(fetch)),
               "write_bytes_per_call": int(round(write)),
               "selected_record_bytes_per_call": int(2176 * cfg.K * (cfg.B * cfg.Q)),
               "median_KiB_per_dispatch": {c: {k: round(v, 1) for k, v in d.items()} for c, d in per.items()},
               "calibration": {"copy_kernel": f"torch.mul(src, 1.0, out=dst) over {copy_bytes} bytes of fp32 "
                                              f"(reads and writes {copy_bytes} bytes)",
                               "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
               "commands": args.command}
        print(json.dumps(rec, indent=1))
        return 0
    if kind == "counters":
        rows = _read_csv(inputs[0])
        by_disp = {}
        for r in rows:
            key = int(r["Dispatch_Id"])
            d = by_disp.setdefault(key, {"name": r["Kernel_Name"], "st": int(r["Start_Timestamp"]),
                                         "en": int(r["End_Timestamp"]), "c": {}})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        disp = sorted(((d["name"], d["st"], d["en"], d["c"]) for d in by_disp.values()), key=lambda x: x[1])
        per = {}
        for k, _, _, c in _labelled(disp):
            per.setdefault(k, []).append(c)
        names = sorted({cn for v in per.values() for c in v for cn in c})
        lines = [f"# SQ counters: {cfg_desc}", "", "Commands (repository root on the GPU host as `$REPO`):",
                 "", "```", _commands_block(args), "```", "",
                 "Per-dispatch counter sums, median over the dispatches of each kernel (the bulk cache "
                 "fill at setup is one dispatch of the append kernel and does not move its median).  "
                 "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8), per "
                 "dispatch, median: GRBM_GUI_ACTIVE sums the 8 XCDs' busy clocks, so /8 is the "
                 "kernel's duration in clocks.  SQ_VALU_MFMA_BUSY_CYCLES counts the matrix pipe's busy "
                 "clocks: 32 per 32 x 32 MFMA and 16 per 16 x 16 one in these kernels.", "",
                 "| kernel | n | MFMA busy | " + " | ".join(names) + " |",
                 "|---|---|---|" + "---|" * len(names)]
        def med(v):
            return float(np.median(v)) if v else 0.0
        for k, v in sorted(per.items(), key=lambda kv: -med([c.get("GRBM_GUI_ACTIVE", 0) for c in kv[1]])
                           * len(kv[1])):
            busy = [c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024.0 * c["GRBM_GUI_ACTIVE"] / 8.0) for c in v
                    if c.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in c]
            lines.append(f"| {k} | {len(v)} | {med(busy):.3f} | "
                         + " | ".join(f"{med([c.get(cn, 0.0) for c in v]):.4g}" for cn in names) + " |")
        print("\n".join(lines))
        return 0
    print(f"unknown summary kind {kind}", file=sys.stderr)
    return 2


# ---------------------------------------------------------------------------
# oracle baseline


def _oracle_records(latent_seq, blocks, nb):
    """Record cache holding only the given blocks (built through the oracle's encoder)."""
    from oracle import mxfp4
    cache = np.zeros((nb, RECORD), dtype=np.uint8)
    n = latent_seq.shape[0]
    for b in np.asarray(blocks, dtype=np.int64):
        if 0 <= b < nb:
            lo, hi = 8 * int(b), min(8 * int(b) + 8, n)
            if hi > lo:
                mxfp4.write_records(cache, latent_seq[lo:hi], lo)
    return cache


def cpu_baseline(cfg, host_in, budget_s):
    """Time the fp64 oracle on a bounded sample of rows (whole step per row).

    Timed: indexer + top-K (Full / Reindex layers) and attention + window +
    merge for every layer.  Not timed: building the record bytes of the
    selected blocks, which stand for cache contents written at append time.
    """
    from oracle import modes as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    nb = cfg.cap // 8
    done, elapsed = 0, 0.0
    if cfg.prior:
        p = host_in
        Q = p["q"].shape[1]
        N = int(p["n_entries"][0])
        order = np.random.default_rng(0).permutation(Q)
        for r in order:
            t = time.perf_counter()
            idx, cnt = om.select_blocks(p["q_idx"][0, r], p["w"][0, r], p["keys"][0], N, cfg.K,
                                        q_pos=int(p["q_pos"][0, r]), n_blocks=nb)
            elapsed += time.perf_counter() - t
            rec = _oracle_records(p["latent"][0], idx[:cnt], nb)
            t = time.perf_counter()
            om.attend_row(p["q"][0, r], rec, idx, cnt, N, p["swa"][0], int(p["swa_len"][0]), cfg.W,
                          q_pos=int(p["q_pos"][0, r]), swa_pos0=int(p["swa_pos0"][0]))
            elapsed += time.perf_counter() - t
            done += 1
            if elapsed >= budget_s:
                break
        unit, total = "tokens/s", Q
        what = "index + top-K + attention + window merge per query token, causal"
    else:
        x, layers = host_in
        rows = [(b, r) for b in range(x.latent.shape[0]) for r in range(cfg.Q)]
        total = len(rows)
        # the rows in turn, again from the first while the budget lasts (a
        # workload of few rows, as decode1m's 8, takes under 2 s once)
        for b, r in (rows[i % total] for i in range(1 << 30)):
            qp = None if x.q_pos is None else int(x.q_pos[b, r])
            p0 = 0 if x.swa_pos0 is None else int(x.swa_pos0[b])
            prev = None
            for L in layers:
                if L.mode in ("F", "R"):
                    t = time.perf_counter()
                    idx, cnt = om.select_blocks(L.q_idx[b, r], L.w[b, r], x.keys[b], int(x.n_entries[b]),
                                                cfg.K, q_pos=qp, top_groups=cfg.top_groups or None,
                                                n_blocks=nb)
                    elapsed += time.perf_counter() - t
                else:
                    idx, cnt = prev
                rec = _oracle_records(x.latent[b], idx[:cnt], nb)
                t = time.perf_counter()
                om.attend_row(L.q[b, r], rec, idx, cnt, int(x.n_entries[b]), L.swa[b], int(x.swa_len[b]),
                              cfg.W, q_pos=qp, swa_pos0=p0)
                elapsed += time.perf_counter() - t
                prev = (idx, cnt)
            done += 1
            if elapsed >= budget_s:
                break
        unit = "queries/s"
        what = (f"index + top-K + attention + window merge per row, {len(layers)} layer(s) "
                f"{''.join(L.mode for L in layers)}")
    sample = (f"{done} of {total} rows of {cfg.name}" if done <= total else
              f"{done} row computations over the {total} rows of {cfg.name} (each row {done / total:.1f} times)")
    return {"value": round(done / elapsed, 3), "unit": unit, "cores": cores, "blas_threads": threads,
            "kind": "oracle", "sample": f"{sample} ({what}; fp64 NumPy), {elapsed:.1f} s"}


if __name__ == "__main__":
    main()
