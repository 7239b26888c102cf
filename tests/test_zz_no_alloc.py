"""GPU: csa2_index_topk_noalloc (selection scratch in a static per-GPU array)
gives the bytes of csa2_index_topk (caller workspace), call after call."""

import numpy as np
import pytest
import torch

from synth import CONFIGS, decode_inputs, normal_bf16, rng_for
from tests.gpu_util import dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _lib():
    from sparse_attention_fp4_csa2_amd import _lib
    return _lib


def _cache(keys, cap, with_groups):
    lib = _lib()
    B, n = keys.shape[0], keys.shape[1]
    lat = torch.zeros(B, n, 512, dtype=torch.bfloat16, device="cuda")
    rec = torch.zeros(B, cap // 8, 2176, dtype=torch.uint8, device="cuda")
    kc = torch.zeros(B, cap, 64, dtype=torch.bfloat16, device="cuda")
    gs = torch.zeros(B, cap // 512, 64, dtype=torch.float32, device="cuda") if with_groups else None
    lib.append_fp4(lat, dev(np.zeros(B, np.int32)), rec, idx_key=dev_bf16(keys), key_cache=kc, group_sum=gs)
    return kc, gs


def _both(keys, q_idx, w, n_entries, cap, K, top_groups=0):
    lib = _lib()
    B, Q = q_idx.shape[0], q_idx.shape[1]
    kc, gs = _cache(keys, cap, top_groups > 0)
    qd, wd, ne = dev_bf16(q_idx), dev(w), dev(np.asarray(n_entries, np.int32))
    idx_a = torch.full((B, Q, K), -7, dtype=torch.int32, device="cuda")
    cnt_a = torch.full((B, Q), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(lib.index_topk_ws(B, Q, cap, top_groups), 256), dtype=torch.uint8, device="cuda")
    lib.index_topk(qd, wd, kc, ne, K, idx_a, cnt_a, ws, group_sum=gs, top_groups=top_groups)
    idx_b = torch.full_like(idx_a, -9)
    cnt_b = torch.full_like(cnt_a, -9)
    lib.index_topk_noalloc(qd, wd, kc, ne, K, idx_b, cnt_b, group_sum=gs, top_groups=top_groups)
    torch.cuda.synchronize()
    return host(idx_a), host(cnt_a), host(idx_b), host(cnt_b)


def test_noalloc_matches_workspace_call_twice_in_a_row():
    rng = rng_for(4242)
    # first call: 16 rows over 8192-entry caches (flat, 1024 blocks, K 256)
    B, N, K = 16, 8192, 256
    keys = normal_bf16(rng, (B, N, 64))
    q_idx = normal_bf16(rng, (B, 1, 8, 64))
    w = rng.standard_normal((B, 1, 8), dtype=np.float32)
    ne = rng.integers(N // 2, N + 1, size=B).astype(np.int32)
    ia, ca, ib, cb = _both(keys, q_idx, w, ne, N, K)
    assert np.array_equal(ca, cb) and np.array_equal(ia, ib), "first call differs"
    # second call, smaller: 3 rows over 2048 entries, the two-level stage on
    # (4 groups, 2 kept), K 40 -- the scratch still holds the first call's scores
    B2, N2, K2 = 3, 2048, 40
    keys2 = normal_bf16(rng, (B2, N2, 64))
    q2 = normal_bf16(rng, (B2, 1, 8, 64))
    w2 = rng.standard_normal((B2, 1, 8), dtype=np.float32)
    ia, ca, ib, cb = _both(keys2, q2, w2, [2048, 1500, 9], N2, K2, top_groups=2)
    assert np.array_equal(ca, cb) and np.array_equal(ia, ib), "second call differs"


def test_noalloc_decode64k_rows():
    # the decode64k workload's selection (32 rows x 4096 blocks, K 2048): 512 KB of scratch
    cfg = CONFIGS["decode64k"]
    x = decode_inputs(cfg, batches=4)
    ia, ca, ib, cb = _both(x.keys, x.q_idx, x.w, x.n_entries, cfg.cap, cfg.K)
    assert np.array_equal(ca, cb) and np.array_equal(ia, ib)


def test_noalloc_rejects_requests_beyond_the_scratch():
    import ctypes
    lib = _lib().load()
    fake = ctypes.c_void_p(4096)      # never dereferenced: the size check fails first
    # 4096 rows x 8192 blocks of fp32 scores = 128 MiB > 8 MiB
    rc = lib.csa2_index_topk_noalloc(fake, fake, fake, None, fake, None, 1, 4096, 8, 65536, 2048, 0,
                                     fake, fake, None)
    assert rc == -5
    assert lib.csa2_status_str(-5) == b"request exceeds the static scratch"
