"""Benchmark: CSA2 sparse-decode step over an MXFP4 latent cache on one MI355X.

One step = the whole hot path for one decode token of every sequence:
  csa2_append_fp4 (one new entry per sequence) -> csa2_index_topk (indexer +
  top-K blocks) -> csa2_sparse_attn (gather + dequant + 64-head attention,
  split-K) -> csa2_swa_merge (sliding window + log-sum-exp merge).
Default workload: decode at 64K context (32 sequences, 64 heads, 32768 MXFP4
entries = 4096 blocks of 8 per sequence, 8 x 64 indexer, top-K 2048, window
512), seeded synthetic N(0,1) inputs with planted relevant blocks.

Prints ONE JSON line.  `value` = decode queries/s (rows / step time).  The
`roofline` object covers the dominant call, csa2_sparse_attn (MFMA-bound at 64
heads): algorithmic FLOPs = 4 * H * (8 * K) * 512 per row, timed with HIP
events on the stream the library launches on.  `cpu_baseline` times the NumPy
fp64 oracle on a bounded sample of rows on the host cores.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn decode queries/s and TB/s FP4 KV read; % of HBM/MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBPS = 8000.0
# HBM bytes per csa2_sparse_attn call from rocprofv3 FETCH_SIZE / WRITE_SIZE
# counter runs, with the hash of the kernel source they were taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sparse_attn_decode64k.json")
KERNEL_SRC = os.path.join(ROOT, "sparse_attention_fp4_csa2_amd", "csrc", "attention.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode64k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, run a plain fp32 copy kernel over this many bytes "
                         "(the calibration point for rocprofv3 FETCH_SIZE / WRITE_SIZE runs)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence/row with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_fp4_csa2_amd import _lib, modes
    from synth import CONFIGS, decode_inputs

    _lib.load()
    cfg = CONFIGS[args.config]
    if cfg.Q != 1 or cfg.layers != "F":
        sys.exit(f"bench.py times single-layer decode workloads; {cfg.name} is not one")
    dev = "cuda"
    t0 = time.time()
    x = decode_inputs(cfg)
    gen_s = time.time() - t0

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    B, H, K, W, N = cfg.B, cfg.H, cfg.K, cfg.W, cfg.N
    cap = cfg.cap
    cache = modes.LatentCache.empty(B, cap, dev, with_groups=bool(cfg.top_groups))
    cache.append(bf(x.latent), bf(x.keys))
    q, q_idx, w = bf(x.q), bf(x.q_idx), torch.from_numpy(x.w).to(dev)
    swa, swa_len = bf(x.swa), torch.from_numpy(x.swa_len).to(dev)
    buf = modes.LayerBuffers(B, 1, H, cap, K, W, top_groups=cfg.top_groups, device=dev)
    # decode append: one new entry per sequence, written at the last held position
    new_lat = bf(x.latent[:, N - 1:N])
    new_key = bf(x.keys[:, N - 1:N])
    start = torch.full((B,), N - 1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step():
        _lib.append_fp4(new_lat, start, cache.records, idx_key=new_key, key_cache=cache.keys,
                        group_sum=None, stream=stream)
        modes.index(buf, cache, q_idx, w, stream=stream)
        modes.attend(buf, cache, q, swa, swa_len, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
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
    t_index = timed(lambda: modes.index(buf, cache, q_idx, w, stream=stream), reps)
    t_attn = timed(lambda: _lib.sparse_attn(q, cache.records, buf.idx, buf.count, cache.n_entries,
                                            modes.SCALE, buf.o, buf.lse, ws=buf.ws_attn,
                                            stream=stream), reps)
    t_swa = timed(lambda: _lib.swa_merge(q, swa, swa_len, W, modes.SCALE, buf.o, buf.lse, buf.out,
                                         buf.lse_out, buf.ws_swa, stream=stream), reps)
    t_append = timed(lambda: _lib.append_fp4(new_lat, start, cache.records, idx_key=new_key,
                                             key_cache=cache.keys, stream=stream), reps)

    counts = buf.count.cpu().numpy()
    n_sel_entries = int(counts.sum()) * 8
    flops_attn = 4.0 * H * n_sel_entries * 512
    attn_tflops = flops_attn / (t_attn * 1e-3) / 1e12
    kv_bytes = n_sel_entries * 272
    kv_tbps = kv_bytes / (t_attn * 1e-3) / 1e12
    idx_bytes = B * N * 128
    idx_gbps = idx_bytes / (t_index * 1e-3) / 1e9

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    traffic = stored_traffic()

    result = {
        "metric": METRIC,
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) bf16, planted relevant blocks)",
        "config": {"workload": f"{cfg.name}: decode, B {B}, H {H}, {N} MXFP4 entries/seq "
                               f"({N // 8} blocks of 8), indexer {cfg.Hi}x64, top-K {K}, window {W}",
                   "global_batch": B, "seq_len": 2 * N, "parallelism": "single GPU"},
        "fp4_kv_read_TBps": round(kv_tbps, 3),
        "breakdown_ms": {"append": round(t_append, 4), "index_topk": round(t_index, 4),
                         "sparse_attn": round(t_attn, 4), "swa_merge": round(t_swa, 4)},
        "indexer_GBps": round(idx_gbps, 1),
        "compute": "MXFP4 cache dequantised to fp16 for fp16 MFMA, fp32 accumulate; window in bf16",
        "roofline": {"kernel": "csa2_sparse_attn (attention + split-K combine)", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": flops_attn},
        "setup_s": round(gen_s, 1),
    }

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def stored_traffic():
    """Measured HBM bytes per csa2_sparse_attn call, or None once the kernel source changed."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    digest = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if rec.get("attention_hip_sha256") != digest:
        return None
    return rec.get("bytes_per_call")


def cpu_baseline(cfg, x, budget_s):
    """Time the fp64 oracle on a bounded sample of decode rows (whole step per row)."""
    from oracle import modes as omodes, mxfp4
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    done, elapsed = 0, 0.0
    for b in range(cfg.B):
        rec = mxfp4.build_records(x.latent[b], cfg.cap)       # cache contents (not timed)
        t = time.perf_counter()
        omodes.full_layer(x.q[b, 0], x.q_idx[b, 0], x.w[b, 0], x.keys[b], rec, cfg.N, cfg.K,
                          x.swa[b], int(x.swa_len[b]), cfg.W, top_groups=cfg.top_groups or None)
        elapsed += time.perf_counter() - t
        done += 1
        if elapsed >= budget_s:
            break
    return {"value": round(done / elapsed, 3), "unit": "queries/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {cfg.B} rows of {cfg.name} (index + top-K + attention + window merge "
                      f"per row, fp64 NumPy), {elapsed:.1f} s"}


if __name__ == "__main__":
    main()
