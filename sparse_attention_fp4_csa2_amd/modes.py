"""Cross-layer modes composed from the four library calls (host orchestration only).

The pages define three static layer modes (observer.broadside.tech card, Key
ideas, "CSA2 with three static layer modes"): Full makes the global KV and
indexes it; Reindex reuses an earlier layer's KV but rescores it with the
layer's own indexer query; Reuse reuses both the KV and the earlier layer's
top-K indices.  Every layer has its own query and its own sliding window.
Here a mode is just which calls run: Full/Reindex = csa2_index_topk +
csa2_sparse_attn + csa2_swa_merge; Reuse = the last two on the earlier
layer's index buffer, passed unchanged.
"""

import math
from dataclasses import dataclass

import torch

from . import _lib

SCALE = 1.0 / math.sqrt(512.0)


@dataclass
class LatentCache:
    """Device state shared by the layers: MXFP4 records, indexer keys, group sums.

    The indexer keys are bf16 (``keys``) or, in the lower-precision key cache,
    MXFP8 (``key8`` E4M3 codes + ``key8_scale`` E8M0 scales; ``keys`` is None).
    """
    records: torch.Tensor     # u8 [B][cap/8][2176]
    keys: torch.Tensor        # bf16 [B][cap][64], or None
    group_sum: torch.Tensor   # fp32 [B][cap/512][64] or None
    n_entries: torch.Tensor   # int32 [B]
    key8: torch.Tensor = None        # u8 [B][cap][64]
    key8_scale: torch.Tensor = None  # u8 [B][cap][2]

    @property
    def cap(self):
        return self.records.shape[1] * _lib.BLOCK

    @staticmethod
    def empty(B, cap, device="cuda", with_groups=False, key_format="bf16"):
        if key_format not in ("bf16", "mxfp8"):
            raise ValueError(f"unknown key format {key_format!r}")
        rec = torch.zeros(B, cap // 8, _lib.RECORD_BYTES, dtype=torch.uint8, device=device)
        gs = torch.zeros(B, cap // 512, 64, dtype=torch.float32, device=device) if with_groups else None
        n = torch.zeros(B, dtype=torch.int32, device=device)
        if key_format == "bf16":
            return LatentCache(rec, torch.zeros(B, cap, 64, dtype=torch.bfloat16, device=device), gs, n)
        return LatentCache(rec, None, gs, n, torch.zeros(B, cap, 64, dtype=torch.uint8, device=device),
                           torch.zeros(B, cap, 2, dtype=torch.uint8, device=device))

    def write(self, latent, keys, start, stream=None):
        """Write n_new entries per sequence at entries start[b] .. (start int32 [B] on the device)."""
        if self.key8 is None:
            _lib.append_fp4(latent, start, self.records, idx_key=keys, key_cache=self.keys,
                            group_sum=self.group_sum, stream=stream)
        else:
            _lib.append_key8(keys, start, self.key8, self.key8_scale, group_sum=self.group_sum, latent=latent,
                             cache=self.records, stream=stream)

    def append(self, latent, keys, stream=None):
        """Append n_new entries per sequence at each sequence's current end."""
        self.write(latent, keys, self.n_entries.clone(), stream=stream)
        self.n_entries += latent.shape[1]


class LayerBuffers:
    """Per-layer outputs and workspaces, sized once (the calls themselves allocate nothing)."""

    def __init__(self, B, Q, H, cap, top_k, W, top_groups=0, device="cuda"):
        self.B, self.Q, self.H, self.cap, self.top_k, self.W = B, Q, H, cap, top_k, W
        self.top_groups = top_groups
        dev = device
        self.idx = torch.empty(B, Q, top_k, dtype=torch.int32, device=dev)
        self.count = torch.empty(B, Q, dtype=torch.int32, device=dev)
        self.o = torch.empty(B, Q, H, 512, dtype=torch.float32, device=dev)
        self.lse = torch.empty(B, Q, H, dtype=torch.float32, device=dev)
        self.out = torch.empty(B, Q, H, 512, dtype=torch.float32, device=dev)
        self.lse_out = torch.empty(B, Q, H, dtype=torch.float32, device=dev)
        self.ws_index = _ws(_lib.index_topk_ws(B, Q, cap, top_groups), dev)
        self.ws_attn = _ws(_lib.sparse_attn_ws(B, Q, H, top_k), dev)
        self.ws_swa = _ws(_lib.swa_merge_ws(B, Q, H, W), dev)
        self.ws_layer = _ws(_lib.attend_layer_ws(B, Q, H, top_k, W), dev)
        self.window_done = torch.cuda.Event() if torch.device(dev).type == "cuda" else None


def _ws(nbytes, dev):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def index(buf, cache, q_idx, w, q_pos=None, stream=None):
    gs = cache.group_sum if buf.top_groups else None
    if cache.key8 is None:
        _lib.index_topk(q_idx, w, cache.keys, cache.n_entries, buf.top_k, buf.idx, buf.count,
                        buf.ws_index, group_sum=gs, q_pos=q_pos, top_groups=buf.top_groups, stream=stream)
    else:
        _lib.index_topk_key8(q_idx, w, cache.key8, cache.key8_scale, cache.n_entries, buf.top_k, buf.idx,
                             buf.count, buf.ws_index, group_sum=gs, q_pos=q_pos, top_groups=buf.top_groups,
                             stream=stream)


def attend(buf, cache, q, swa, swa_len, idx=None, count=None, swa_pos0=None, q_pos=None,
           scale=SCALE, stream=None, fused=True):
    """Sparse + window branches merged into buf.out / buf.lse_out.

    fused=True: one csa2_attend_layer call (one combine over both branches'
    split-K partials).  fused=False: csa2_sparse_attn (buf.o, buf.lse) then
    csa2_swa_merge.
    """
    idx = buf.idx if idx is None else idx
    count = buf.count if count is None else count
    if fused:
        _lib.attend_layer(q, cache.records, idx, count, cache.n_entries, swa, swa_len, buf.W, scale,
                          buf.out, buf.lse_out, buf.ws_layer, swa_pos0=swa_pos0, q_pos=q_pos,
                          stream=stream)
        return
    _lib.sparse_attn(q, cache.records, idx, count, cache.n_entries, scale, buf.o, buf.lse,
                     ws=buf.ws_attn, q_pos=q_pos, stream=stream)
    _lib.swa_merge(q, swa, swa_len, buf.W, scale, buf.o, buf.lse, buf.out, buf.lse_out,
                   buf.ws_swa, swa_pos0=swa_pos0, q_pos=q_pos, stream=stream)


def run_layer(mode, buf, cache, q, swa, swa_len, q_idx=None, w=None, prev=None, stream=None,
              side_stream=None, q_pos=None, swa_pos0=None):
    """One decode layer.  mode: "F" (Full), "R" (Reindex) or "U" (Reuse, needs ``prev``).

    q_pos / swa_pos0: raw positions of the query rows and of window slot 0
    (several rows per sequence, e.g. draft tokens verified together); None =
    every row is the newest token.

    side_stream: run the window branch there (phase 1 of csa2_attend_layer),
    forked after the work already on ``stream`` and joined before the sparse
    branch, so it overlaps the indexer and top-K.  Same results either way.

    Returns the (idx, count) this layer attended; for Reuse they are ``prev``'s
    buffers themselves, untouched.
    """
    if mode not in ("F", "R", "U"):
        raise ValueError(f"unknown mode {mode!r}")
    if mode == "U" and prev is None:
        raise ValueError("Reuse needs the earlier layer's (idx, count)")
    main = stream if stream is not None else torch.cuda.current_stream()
    if side_stream is not None:
        side_stream.wait_stream(main)
        _lib.attend_layer_window(q, swa, swa_len, buf.top_k, buf.W, SCALE, buf.ws_layer,
                                 swa_pos0=swa_pos0, q_pos=q_pos, stream=side_stream)
        buf.window_done.record(side_stream)
    if mode in ("F", "R"):
        index(buf, cache, q_idx, w, q_pos=q_pos, stream=main)
        idx, count = buf.idx, buf.count
    else:
        idx, count = prev
    if side_stream is not None:
        main.wait_event(buf.window_done)
        _lib.attend_layer_sparse(q, cache.records, idx, count, cache.n_entries, buf.W, SCALE, buf.out,
                                 buf.lse_out, buf.ws_layer, q_pos=q_pos, stream=main)
    else:
        attend(buf, cache, q, swa, swa_len, idx=idx, count=count, swa_pos0=swa_pos0, q_pos=q_pos,
               stream=main)
    return idx, count
