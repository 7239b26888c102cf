"""ctypes binding of libcsa2.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module turns
torch tensors into device pointers and the current HIP stream, calls the C ABI
declared in include/csa2.h, and raises on a non-zero status.  There is no CPU
fallback: without the built library every call raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

CSA2_OK = 0
D, DI, BLOCK, RECORD_BYTES, GROUP_ENTRIES = 512, 64, 8, 2176, 512

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_F = ctypes.c_float

_SIGS = {
    "csa2_append_fp4": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P]),
    "csa2_index_topk": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "csa2_index_topk_ws": (_SZ, [_I, _I, _I, _I]),
    "csa2_index_topk_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "csa2_append_key8": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P]),
    "csa2_index_topk_key8": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "csa2_topk": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "csa2_sparse_attn": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _SZ, _P]),
    "csa2_sparse_attn_ws": (_SZ, [_I, _I, _I, _I]),
    "csa2_swa_merge": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _SZ, _P]),
    "csa2_swa_merge_ws": (_SZ, [_I, _I, _I, _I]),
    "csa2_attend_layer": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                               _P, _P, _P, _SZ, _P]),
    "csa2_attend_layer_ws": (_SZ, [_I, _I, _I, _I, _I]),
    "csa2_attend_layer_launches": (_I, [_I, _I, _I, _I, _I]),
    "csa2_attend_layer_window": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "csa2_attend_layer_sparse": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P,
                                      _SZ, _P]),
    "csa2_status_str": (ctypes.c_char_p, [_I]),
    "csa2_version": (_I, []),
}

_lib = None


class Csa2Error(RuntimeError):
    pass


def load(path=LIB_PATH):
    """Load the library (once) and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise Csa2Error(f"{path} is not built; run `python -m sparse_attention_fp4_csa2_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc, what):
    if rc != CSA2_OK:
        msg = load().csa2_status_str(rc).decode()
        raise Csa2Error(f"{what} failed: {msg} ({rc})")


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# bf16 inputs are carried as torch.bfloat16 (or int16/uint16 views of the bits)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _bf16_ptr(t, name):
    if t is None:
        return None
    if t.dtype not in _BF16:
        raise TypeError(f"{name} must be bfloat16 bits, got {t.dtype}")
    return _ptr(t, None, name)


def append_fp4(latent, start_entry, cache, idx_key=None, key_cache=None, group_sum=None,
               stream=None):
    """csa2_append_fp4: latent bf16 [B][n_new][512] -> cache u8 [B][cap/8][2176] (in place)."""
    lib = load()
    B, n_new = latent.shape[0], latent.shape[1]
    cap = cache.shape[1] * BLOCK
    rc = lib.csa2_append_fp4(_bf16_ptr(latent, "latent"), _bf16_ptr(idx_key, "idx_key"),
                             _ptr(start_entry, torch.int32, "start_entry"), B, n_new, cap,
                             _ptr(cache, torch.uint8, "cache"), _bf16_ptr(key_cache, "key_cache"),
                             _ptr(group_sum, torch.float32, "group_sum"), _stream(stream))
    _check(rc, "csa2_append_fp4")


def index_topk_ws(B, Q, cap, top_groups=0):
    return load().csa2_index_topk_ws(B, Q, cap, top_groups)


def index_topk(q_idx, w, key_cache, n_entries, top_k, idx, count, ws, group_sum=None,
               q_pos=None, top_groups=0, stream=None):
    """csa2_index_topk: q_idx bf16 [B][Q][Hi][64], w fp32 [B][Q][Hi] -> idx/count (in place)."""
    lib = load()
    B, Q, Hi = q_idx.shape[0], q_idx.shape[1], q_idx.shape[2]
    cap = key_cache.shape[1]
    rc = lib.csa2_index_topk(_bf16_ptr(q_idx, "q_idx"), _ptr(w, torch.float32, "w"),
                             _bf16_ptr(key_cache, "key_cache"), _ptr(group_sum, torch.float32, "group_sum"),
                             _ptr(n_entries, torch.int32, "n_entries"), _ptr(q_pos, torch.int32, "q_pos"),
                             B, Q, Hi, cap, top_k, top_groups,
                             _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"),
                             _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "csa2_index_topk")


def index_topk_noalloc(q_idx, w, key_cache, n_entries, top_k, idx, count, group_sum=None, q_pos=None,
                       top_groups=0, stream=None):
    """csa2_index_topk_noalloc: csa2_index_topk with its scratch in the library's static per-GPU array."""
    lib = load()
    B, Q, Hi = q_idx.shape[0], q_idx.shape[1], q_idx.shape[2]
    cap = key_cache.shape[1]
    rc = lib.csa2_index_topk_noalloc(_bf16_ptr(q_idx, "q_idx"), _ptr(w, torch.float32, "w"),
                                     _bf16_ptr(key_cache, "key_cache"), _ptr(group_sum, torch.float32, "group_sum"),
                                     _ptr(n_entries, torch.int32, "n_entries"), _ptr(q_pos, torch.int32, "q_pos"),
                                     B, Q, Hi, cap, top_k, top_groups,
                                     _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"),
                                     _stream(stream))
    _check(rc, "csa2_index_topk_noalloc")


def append_key8(idx_key, start_entry, key8, key8_scale, group_sum=None, latent=None, cache=None, stream=None):
    """csa2_append_key8: keys bf16 [B][n_new][64] -> key8 u8 [B][cap][64], key8_scale u8 [B][cap][2]
    (and, with latent bf16 [B][n_new][512] and cache u8 [B][cap/8][2176], the latent's records)."""
    lib = load()
    B, n_new = idx_key.shape[0], idx_key.shape[1]
    cap = key8.shape[1]
    rc = lib.csa2_append_key8(_bf16_ptr(latent, "latent"), _bf16_ptr(idx_key, "idx_key"),
                              _ptr(start_entry, torch.int32, "start_entry"), B, n_new, cap,
                              _ptr(cache, torch.uint8, "cache"), _ptr(key8, torch.uint8, "key8"),
                              _ptr(key8_scale, torch.uint8, "key8_scale"),
                              _ptr(group_sum, torch.float32, "group_sum"), _stream(stream))
    _check(rc, "csa2_append_key8")


def index_topk_key8(q_idx, w, key8, key8_scale, n_entries, top_k, idx, count, ws, group_sum=None,
                    q_pos=None, top_groups=0, stream=None):
    """csa2_index_topk_key8: as index_topk, on an MXFP8 key cache (key8, key8_scale)."""
    lib = load()
    B, Q, Hi = q_idx.shape[0], q_idx.shape[1], q_idx.shape[2]
    cap = key8.shape[1]
    rc = lib.csa2_index_topk_key8(_bf16_ptr(q_idx, "q_idx"), _ptr(w, torch.float32, "w"),
                                  _ptr(key8, torch.uint8, "key8"), _ptr(key8_scale, torch.uint8, "key8_scale"),
                                  _ptr(group_sum, torch.float32, "group_sum"),
                                  _ptr(n_entries, torch.int32, "n_entries"), _ptr(q_pos, torch.int32, "q_pos"),
                                  B, Q, Hi, cap, top_k, top_groups,
                                  _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"),
                                  _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "csa2_index_topk_key8")


def topk(scores, k, idx, count, stream=None):
    """csa2_topk: scores fp32 [rows][n] -> idx int32 [rows][k], count int32 [rows] (in place)."""
    lib = load()
    rows, n = scores.shape
    rc = lib.csa2_topk(_ptr(scores, torch.float32, "scores"), rows, n, k,
                       _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"), _stream(stream))
    _check(rc, "csa2_topk")


def sparse_attn_ws(B, Q, H, top_k):
    return load().csa2_sparse_attn_ws(B, Q, H, top_k)


def sparse_attn(q, cache, idx, count, n_entries, scale, o, lse, ws=None, q_pos=None, stream=None):
    """csa2_sparse_attn: q bf16 [B][Q][H][512] -> o fp32 [B][Q][H][512], lse fp32 [B][Q][H]."""
    lib = load()
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    cap = cache.shape[1] * BLOCK
    top_k = idx.shape[-1]
    ws_ptr = _ptr(ws, None, "ws") if ws is not None and ws.numel() else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    rc = lib.csa2_sparse_attn(_bf16_ptr(q, "q"), _ptr(cache, torch.uint8, "cache"),
                              _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"),
                              _ptr(n_entries, torch.int32, "n_entries"), _ptr(q_pos, torch.int32, "q_pos"),
                              B, Q, H, cap, top_k, float(scale),
                              _ptr(o, torch.float32, "o"), _ptr(lse, torch.float32, "lse"),
                              ws_ptr, ws_bytes, _stream(stream))
    _check(rc, "csa2_sparse_attn")


def swa_merge_ws(B, Q, H, W):
    return load().csa2_swa_merge_ws(B, Q, H, W)


def swa_merge(q, swa_kv, swa_len, W, scale, o_sparse, lse_sparse, out, lse_out, ws,
              swa_pos0=None, q_pos=None, stream=None):
    """csa2_swa_merge: window branch + LSE merge -> out fp32 [B][Q][H][512], lse_out [B][Q][H]."""
    lib = load()
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    Lw = swa_kv.shape[1]
    rc = lib.csa2_swa_merge(_bf16_ptr(q, "q"), _bf16_ptr(swa_kv, "swa_kv"),
                            _ptr(swa_len, torch.int32, "swa_len"), _ptr(swa_pos0, torch.int32, "swa_pos0"),
                            _ptr(q_pos, torch.int32, "q_pos"), B, Q, H, W, Lw, float(scale),
                            _ptr(o_sparse, torch.float32, "o_sparse"), _ptr(lse_sparse, torch.float32, "lse_sparse"),
                            _ptr(out, torch.float32, "out"), _ptr(lse_out, torch.float32, "lse_out"),
                            _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "csa2_swa_merge")


def attend_layer_ws(B, Q, H, top_k, W):
    return load().csa2_attend_layer_ws(B, Q, H, top_k, W)


def attend_layer_launches(B, Q, H, top_k, W):
    return load().csa2_attend_layer_launches(B, Q, H, top_k, W)


def attend_layer(q, cache, idx, count, n_entries, swa_kv, swa_len, W, scale, out, lse_out, ws,
                 swa_pos0=None, q_pos=None, stream=None):
    """csa2_attend_layer: sparse branch + window branch merged -> out fp32 [B][Q][H][512], lse_out."""
    lib = load()
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    cap = cache.shape[1] * BLOCK
    top_k = idx.shape[-1]
    Lw = swa_kv.shape[1]
    rc = lib.csa2_attend_layer(_bf16_ptr(q, "q"), _ptr(cache, torch.uint8, "cache"),
                               _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"),
                               _ptr(n_entries, torch.int32, "n_entries"), _ptr(q_pos, torch.int32, "q_pos"),
                               _bf16_ptr(swa_kv, "swa_kv"), _ptr(swa_len, torch.int32, "swa_len"),
                               _ptr(swa_pos0, torch.int32, "swa_pos0"), B, Q, H, cap, top_k, W, Lw,
                               float(scale), _ptr(out, torch.float32, "out"),
                               _ptr(lse_out, torch.float32, "lse_out"), _ptr(ws, None, "ws"),
                               ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "csa2_attend_layer")


def attend_layer_window(q, swa_kv, swa_len, top_k, W, scale, ws, swa_pos0=None, q_pos=None,
                        stream=None):
    """csa2_attend_layer_window: the window branch's split-K partials into ws (phase 1)."""
    lib = load()
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    Lw = swa_kv.shape[1]
    rc = lib.csa2_attend_layer_window(_bf16_ptr(q, "q"), _bf16_ptr(swa_kv, "swa_kv"),
                                      _ptr(swa_len, torch.int32, "swa_len"),
                                      _ptr(swa_pos0, torch.int32, "swa_pos0"),
                                      _ptr(q_pos, torch.int32, "q_pos"), B, Q, H, top_k, W, Lw,
                                      float(scale), _ptr(ws, None, "ws"), ws.numel() * ws.element_size(),
                                      _stream(stream))
    _check(rc, "csa2_attend_layer_window")


def attend_layer_sparse(q, cache, idx, count, n_entries, W, scale, out, lse_out, ws, q_pos=None,
                        stream=None):
    """csa2_attend_layer_sparse: sparse partials into ws, then the combine of both (phase 2)."""
    lib = load()
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    cap = cache.shape[1] * BLOCK
    top_k = idx.shape[-1]
    rc = lib.csa2_attend_layer_sparse(_bf16_ptr(q, "q"), _ptr(cache, torch.uint8, "cache"),
                                      _ptr(idx, torch.int32, "idx"), _ptr(count, torch.int32, "count"),
                                      _ptr(n_entries, torch.int32, "n_entries"),
                                      _ptr(q_pos, torch.int32, "q_pos"), B, Q, H, cap, top_k, W,
                                      float(scale), _ptr(out, torch.float32, "out"),
                                      _ptr(lse_out, torch.float32, "lse_out"), _ptr(ws, None, "ws"),
                                      ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "csa2_attend_layer_sparse")


def version():
    return load().csa2_version()
