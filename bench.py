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
Default workload (--config decode64k): decode at 64K context, 32 sequences, 64
heads, 32768 MXFP4 entries = 4096 blocks of 8 per sequence, 8 x 64 indexer,
top-K 2048, window 512; seeded N(0,1) bf16 inputs with planted relevant blocks.
Other configs (decode1m, layers128k, prefill, specdec64k, tiny) time the same
step shape on their own workloads; specdec64k is decode64k's cache with 4 query
rows per sequence at consecutive positions (a token and 3 drafts verified in
one pass).

Prints ONE JSON line.  `value` = query rows per second (decode queries/s, or
prefill tokens/s).  `roofline` covers csa2_sparse_attn (attention kernel + its
split-K combine; MFMA-bound at 64 heads): algorithmic FLOPs = 4 * H * 512 per
selected visible entry, over the call's mean time from HIP events recorded on
the stream the library launches on.  `cpu_baseline` times the NumPy fp64
oracle on a bounded sample of rows on the host cores.
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
# HBM bytes per csa2_sparse_attn call from rocprofv3 FETCH_SIZE / WRITE_SIZE
# counter runs, with the hash of the kernel source they were taken on
KERNEL_SRCS = [os.path.join(ROOT, "sparse_attention_fp4_csa2_amd", "csrc", f)
               for f in ("sparse_fp4.hip", "attention.hip")]


def traffic_file(config):
    return os.path.join(ROOT, "profiles", f"traffic_sparse_attn_{config}.json")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode64k",
                    choices=["tiny", "decode64k", "decode1m", "layers128k", "prefill", "specdec64k"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--index-keys", default="bf16", choices=["bf16", "mxfp8"],
                    help="indexer key cache: bf16 (the workload's definition) or the lower-precision "
                         "MXFP8 variant")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed steps for this long (seconds) before the warm-up steps, so the GPU "
                         "clocks reach their steady state (they ramp over the first ~30 ms of work)")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="reps of the cold timings (a 1 GiB write before each evicts L2 and the 256 MB "
                         "last-level cache); 0 skips them")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak reference runs")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run a plain fp32 copy kernel over this many bytes "
                         "(the calibration point for rocprofv3 FETCH_SIZE / WRITE_SIZE runs)")
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


def _bf(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def make_workload(name, device="cuda", key_format="bf16"):
    """(cfg, host inputs, workload) for a named config, as bench.py times it."""
    from synth import CONFIGS, decode_inputs, layers_inputs, prefill_inputs, specdec_inputs
    from synth.gen import LayerInputs
    cfg = CONFIGS[name]
    if name == "prefill":
        p = prefill_inputs(cfg)
        return cfg, p, PrefillWorkload(cfg, p, device, key_format)
    if len(cfg.layers) > 1:
        x, layers = layers_inputs(cfg)
    else:
        x = specdec_inputs(cfg) if cfg.Q > 1 else decode_inputs(cfg)
        layers = [LayerInputs("F", x.q, x.q_idx, x.w, x.swa, x.planted)]
    return cfg, (x, layers), DecodeWorkload(cfg, x, layers, device, key_format)


# ---------------------------------------------------------------------------


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence/row with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_fp4_csa2_amd import _lib
    _lib.load()
    t0 = time.time()
    cfg, host_in, wl = make_workload(args.config, key_format=args.index_keys)
    gen_s = time.time() - t0
    stream = wl.stream
    torch.cuda.synchronize()

    # settle: the same step, untimed, until the clocks have ramped up
    t_settle = time.time()
    while time.time() - t_settle < args.settle_s:
        for _ in range(10):
            wl.step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        wl.step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-call breakdown on the same stream (events bracket repeated calls)
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    reps = max(args.steps, 10)
    breakdown, per_step = {}, {}
    for name, (fn, n) in wl.calls().items():
        breakdown[name] = timed(fn, reps)
        per_step[name] = n
    t_attn = breakdown["sparse_attn"]
    wl.step()
    torch.cuda.synchronize()
    n_ent = wl.attended_entries()
    flops_attn = 4.0 * cfg.H * n_ent * 512
    attn_tflops = flops_attn / (t_attn * 1e-3) / 1e12
    kv_tbps = n_ent * 272 / (t_attn * 1e-3) / 1e12

    # cold: every timed call starts with L2 and the last-level cache holding a
    # 1 GiB scratch write instead of the workload's data (median of the reps)
    cold = None
    if args.cold_reps > 0:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

        def cold_ms(fn):
            ts = []
            for i in range(args.cold_reps):
                scratch.fill_(float(i))
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            return float(np.median(ts))

        cold = {"step": round(cold_ms(wl.step), 4), "sparse_attn": round(cold_ms(wl.sparse_attn_call), 4)}
        del scratch
    peaks = None if args.no_peaks else measured_peaks(torch, stream)

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    rows = wl.rows
    prefill = args.config == "prefill"
    result = {
        "metric": METRIC,
        "value": round(rows / (ms_step * 1e-3), 1),
        "unit": "tokens/s" if prefill else "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) bf16, planted relevant blocks)",
        "config": workload_config(cfg, rows, args.index_keys),
        "fp4_kv_read_TBps": round(kv_tbps, 3),
        "breakdown_ms": {k: round(v, 4) for k, v in breakdown.items()},
        "launches_per_step": per_step,
        "kernels_per_layer": kernels_per_layer(cfg),
        "compute": ("Q.K on the scaled FP4 x FP6 MFMA (query split into three E2M3 terms), P.V on fp16 MFMA "
                    "with the MXFP4 values dequantised to fp16, fp32 accumulate; window in bf16"),
        "roofline": {"kernel": "csa2_sparse_attn (attention + split-K combine)", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_FP16_TFLOPS, 4),
                     "traffic": stored_traffic(args.config),
                     "flops_per_launch": flops_attn},
        "setup_s": round(gen_s, 1),
    }
    if cold is not None:
        result["cold_ms"] = cold
        result["cold_value"] = round(rows / (cold["step"] * 1e-3), 1)
    if peaks is not None:
        result["measured_peaks"] = peaks
        result["roofline"]["frac_of_measured_gemm"] = round(attn_tflops / peaks["bf16_gemm_TFLOPs"], 4)
    if not prefill:
        kb = 128 if args.index_keys == "bf16" else 66     # key bytes: bf16, or MXFP8 codes + scales
        idx_bytes = wl.B * cfg.N * kb if not cfg.top_groups else \
            wl.B * (cfg.cap // 512 * 256 + cfg.top_groups * 512 * kb)
        result["indexer_GBps"] = round(idx_bytes / (breakdown["index_topk"] * 1e-3) / 1e9, 1)
        if "index_topk_key8" in breakdown:
            # the same call on the MXFP8 key cache: 64 code bytes + 2 scale bytes per key
            idx8_bytes = wl.B * cfg.N * 66 if not cfg.top_groups else \
                wl.B * (cfg.cap // 512 * 256 + cfg.top_groups * 512 * 66)
            result["indexer_key8_GBps"] = round(idx8_bytes / (breakdown["index_topk_key8"] * 1e-3) / 1e9, 1)
    if len(cfg.layers) > 1:
        result["reuse_saving_ms"] = round(breakdown["index_topk"] * cfg.layers.count("U"), 4)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg, host_in, args.cpu_seconds)
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


def kernels_per_layer(cfg):
    """Kernel launches of one layer's attention path, by layer mode (append not included).

    csa2_index_topk launches the indexer and the top-K (two-level: coarse scores,
    group top-K, fine scores, top-K); csa2_attend_layer always launches two
    (both branches in one kernel, then the combine).  Reuse layers run only
    the latter."""
    index = 4 if cfg.top_groups else 2
    modes = sorted(set(cfg.layers)) if cfg.name != "prefill" else ["F"]
    return {m: (index + 2 if m in ("F", "R") else 2) for m in modes}


def workload_config(cfg, rows, index_keys="bf16"):
    if cfg.name == "prefill":
        desc = (f"prefill: {cfg.Q} query tokens after {cfg.prior} cached entries (+{cfg.Q // 2} "
                f"appended), H {cfg.H}, indexer {cfg.Hi}x64, top-K {cfg.K} per row, window {cfg.W}, causal")
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
    nb = cfg.cap // 8
    done, elapsed = 0, 0.0
    if cfg.name == "prefill":
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
        for b, r in rows:
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
    return {"value": round(done / elapsed, 3), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{done} of {total} rows of {cfg.name} ({what}; fp64 NumPy), {elapsed:.1f} s"}


if __name__ == "__main__":
    main()
