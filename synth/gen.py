"""Seeded generators for the synthetic workloads (no arithmetic of the method here).

All float inputs are drawn as float32 N(0, 1) from NumPy's PCG64 and rounded to
bfloat16 with round-to-nearest-even; indexer weights stay float32.  Planting
only edits indexer keys (never the latent): one entry of each planted block gets
the key c_r * q_h* (h* = the indexer head with the largest weight, c_r a
multiplier of its own between c and 2c), so that block's score stands clear of
the unplanted ones and the planted scores are spread, not one shared value.  ``plant_tight`` instead puts
the planted scores just above the best unplanted block, using a scoring
function supplied by the caller.
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rng_for", "bf16_rne", "bf16_to_f32", "normal_bf16", "DecodeInputs",
    "decode_inputs", "choose_blocks", "plant_dominant", "plant_tight",
    "plant_groups", "layer_query", "prefill_inputs", "LayerInputs", "layers_inputs",
    "specdec_inputs",
]

D = 512
DI = 64


def rng_for(seed):
    return np.random.Generator(np.random.PCG64(seed))


def bf16_rne(x):
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng, shape, chunk=1 << 22):
    """N(0,1) float32 draws rounded to bfloat16.

    Chunk i of ``chunk`` values is drawn from its own PCG64 stream, seeded by
    the i-th 63-bit integer drawn from ``rng``; chunks are filled by a thread
    pool (the draws are the same for any number of threads).
    """
    size = int(np.prod(shape))
    out = np.empty(size, dtype=np.uint16)
    n_chunks = max(1, (size + chunk - 1) // chunk)
    seeds = rng.integers(0, 2 ** 63 - 1, size=n_chunks, dtype=np.int64)

    def fill(i):
        s, e = i * chunk, min(size, (i + 1) * chunk)
        if e > s:
            g = np.random.Generator(np.random.PCG64(int(seeds[i])))
            out[s:e] = bf16_rne(g.standard_normal(e - s, dtype=np.float32))

    if n_chunks == 1:
        fill(0)
    else:
        workers = max(1, min(8, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def _positive_weights(rng, shape):
    """float32 N(0,1) weights, redrawn per row until at least one entry is positive."""
    w = rng.standard_normal(shape, dtype=np.float32)
    flat = w.reshape(-1, shape[-1])
    for r in range(flat.shape[0]):
        while flat[r].max() <= 0:
            flat[r] = rng.standard_normal(shape[-1], dtype=np.float32)
    return flat.reshape(shape)


@dataclass
class DecodeInputs:
    latent: np.ndarray      # u16 [B][N][512]  entries to append to the MXFP4 cache
    keys: np.ndarray        # u16 [B][N][64]   indexer keys, one per entry
    q: np.ndarray           # u16 [B][Q][H][512]
    q_idx: np.ndarray       # u16 [B][Q][Hi][64]
    w: np.ndarray           # f32 [B][Q][Hi]
    swa: np.ndarray         # u16 [B][W][512]  sliding-window tokens (K = V)
    swa_len: np.ndarray     # i32 [B]
    n_entries: np.ndarray   # i32 [B]
    planted: list = field(default_factory=list)   # per sequence: planted block ids
    q_pos: np.ndarray = None     # i32 [B][Q] raw position of each query row (None: newest)
    swa_pos0: np.ndarray = None  # i32 [B] raw position of window slot 0 (None: 0)


def choose_blocks(rng, nb_present, count, exclude=None, pool=None):
    """``count`` distinct block ids drawn from ``pool`` (default all present blocks) minus ``exclude``."""
    cand = np.arange(nb_present) if pool is None else np.asarray(pool)
    if exclude is not None and len(exclude):
        cand = np.setdiff1d(cand, np.asarray(exclude))
    count = min(count, cand.size)
    return np.sort(rng.choice(cand, size=count, replace=False))


def _lead_head(w_row):
    return int(np.argmax(np.asarray(w_row)))


def _entry_in_block(rng, blk, n_entries):
    hi = min(8, n_entries - 8 * blk)
    return 8 * blk + int(rng.integers(0, hi))


def plant_dominant(keys, n_entries, q_idx_row, w_row, blocks, rng, c=3.0, spread=1.0):
    """In place: one present entry of each block in ``blocks`` gets key bf16(c_r * q_h*).

    The planted blocks take distinct multipliers c_r = c * (1 + spread * r / n) for
    r = 0 .. n-1 in a seeded random order, so their scores (positively
    homogeneous in the key) spread over [c, c * (1 + spread)) times the score of
    q_h* instead of sharing one value.  The key is rounded to bf16 (a relative
    step of 2^-8 .. 2^-7), so runs of about n / (2^7 spread) .. n / (2^8 spread)
    neighbouring multipliers share one key and tie.
    """
    h = _lead_head(w_row)
    u = bf16_to_f32(q_idx_row[h])
    blocks = np.asarray(blocks)
    n = max(len(blocks), 1)
    for r, b in enumerate(rng.permutation(blocks)):
        key = bf16_rne(np.float32(c * (1.0 + spread * r / n)) * u)
        keys[_entry_in_block(rng, int(b), n_entries)] = key
    return blocks


def plant_tight(keys, n_entries, q_idx_row, w_row, blocks, rng, score_fn, margin=0.5, step=0.01):
    """In place: planted blocks score a little above the best unplanted block.

    ``score_fn(keys_u16 [n][64]) -> float64 [n]`` gives entry scores for this row.
    Planted block r (in the given order) gets one entry with key bf16(c_r * q_h*)
    where c_r = (T + margin + step * r) / score(q_h*) and T is the best score of
    any entry outside the planted blocks.  The caller checks the resulting gap.
    """
    blocks = np.asarray(blocks)
    n = int(n_entries)
    s = np.asarray(score_fn(keys[:n]), dtype=np.float64)
    planted_entry = np.zeros(n, dtype=bool)
    for b in blocks:
        planted_entry[8 * b: min(8 * b + 8, n)] = True
    T = s[~planted_entry].max() if (~planted_entry).any() else 0.0
    order = np.argsort(-np.asarray(w_row))
    for h in order:
        u = bf16_to_f32(q_idx_row[h])
        su = float(score_fn(bf16_rne(u)[None, :])[0])
        if su > 0:
            break
    else:
        raise ValueError("no indexer head gives a positive planted score")
    for r, b in enumerate(rng.permutation(blocks)):
        c = np.float32((max(T, 0.0) + margin + step * r) / su)
        keys[_entry_in_block(rng, int(b), n)] = bf16_rne(c * u)
    return blocks


def plant_groups(keys, n_entries, q_idx_row, w_row, groups, mu=1.0):
    """In place: every present key of each group (512 entries) gets mu * q_h* / 8 added."""
    h = _lead_head(w_row)
    u = bf16_to_f32(q_idx_row[h]) * np.float32(mu / 8.0)
    for g in groups:
        lo, hi = 512 * int(g), min(512 * int(g) + 512, int(n_entries))
        if hi > lo:
            keys[lo:hi] = bf16_rne(bf16_to_f32(keys[lo:hi]) + u[None, :])
    return np.asarray(groups)


def layer_query(rng, B, Q, H, Hi):
    """One layer's own attention query and indexer query/weights."""
    q = normal_bf16(rng, (B, Q, H, D))
    q_idx = normal_bf16(rng, (B, Q, Hi, DI))
    w = _positive_weights(rng, (B, Q, Hi))
    return q, q_idx, w


def decode_inputs(cfg, seed=None, plant="dominant", score_fn=None, n_entries=None,
                  batches=None, c=3.0):
    """Inputs for a decode workload (Q rows per sequence attend the whole cache).

    plant: "dominant" (scores far above the rest), "tight" (needs ``score_fn(b)``
    returning a per-sequence entry-score function), or None (no plant).
    ``n_entries`` overrides the per-sequence entry counts (ragged caches);
    ``batches`` limits generation to the first ``batches`` sequences.
    """
    rng = rng_for(cfg.seed if seed is None else seed)
    B = cfg.B if batches is None else batches
    N = cfg.N
    ne = np.full(B, N, dtype=np.int32) if n_entries is None else np.asarray(n_entries, np.int32)
    latent = normal_bf16(rng, (B, N, D))
    keys = normal_bf16(rng, (B, N, DI))
    q, q_idx, w = layer_query(rng, B, cfg.Q, cfg.H, cfg.Hi)
    swa = normal_bf16(rng, (B, cfg.W, D))
    swa_len = np.full(B, cfg.W, dtype=np.int32)
    planted = []
    for b in range(B):
        nbp = (int(ne[b]) + 7) // 8
        if cfg.top_groups:
            ngp = (int(ne[b]) + 511) // 512
            groups = choose_blocks(rng, ngp, cfg.top_groups)
            plant_groups(keys[b], ne[b], q_idx[b, 0], w[b, 0], groups)
            pool = (groups[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
            pool = pool[pool < nbp]
        else:
            pool = None
        if plant is None:
            planted.append(np.zeros(0, dtype=np.int64))
            continue
        blocks = choose_blocks(rng, nbp, cfg.K, pool=pool)
        if plant == "dominant":
            plant_dominant(keys[b], ne[b], q_idx[b, 0], w[b, 0], blocks, rng, c=c)
        elif plant == "tight":
            plant_tight(keys[b], ne[b], q_idx[b, 0], w[b, 0], blocks, rng, score_fn(b))
        else:
            raise ValueError(plant)
        planted.append(blocks)
    return DecodeInputs(latent, keys, q, q_idx, w, swa, swa_len, ne, planted)


def specdec_inputs(cfg, seed=None, c=3.0, jitter=0.05):
    """Decode with draft verification: Q = 1 + drafts query rows per sequence.

    The rows sit at raw positions 2N .. 2N + Q - 1 (the tokens after the cached
    ones; every cached entry is visible to all of them).  Row 0 is drawn and
    planted as in decode_inputs; the draft rows' indexer queries are row 0's
    plus N(0, jitter^2) noise and share its weights (neighbouring tokens ask for
    much the same context), so the plant stands for every row.  The window holds
    raw positions [2N - W + 1, 2N + Q - 1], the drafts included, so each row
    sees exactly W window tokens.
    """
    x = decode_inputs(cfg, seed=seed, c=c)
    rng = rng_for((cfg.seed if seed is None else seed) + 104729)
    B, Q, N, W = x.q.shape[0], cfg.Q, cfg.N, cfg.W
    q_idx, w = x.q_idx.copy(), x.w.copy()
    base = bf16_to_f32(q_idx[:, 0])
    for r in range(1, Q):
        noise = rng.standard_normal(base.shape, dtype=np.float32) * np.float32(jitter)
        q_idx[:, r] = bf16_rne(base + noise)
        w[:, r] = w[:, 0]
    swa = np.concatenate([x.swa, normal_bf16(rng, (B, Q - 1, D))], axis=1)
    swa_len = np.full(B, W + Q - 1, dtype=np.int32)
    q_pos = np.broadcast_to(2 * N + np.arange(Q, dtype=np.int32), (B, Q)).copy()
    swa_pos0 = np.full(B, 2 * N - W + 1, dtype=np.int32)
    return DecodeInputs(x.latent, x.keys, x.q, q_idx, w, swa, swa_len, x.n_entries, x.planted,
                        q_pos=q_pos, swa_pos0=swa_pos0)


def prefill_inputs(cfg, seed=None, q_rows=None, n_dirs=4, c=3.0, beta=1.0):
    """Inputs for a causal chunk: cfg.prior entries already cached, then cfg.Q new raw tokens.

    The Q query tokens sit at raw positions 2*prior .. 2*prior + Q - 1; the chunk
    adds Q/2 new entries.  Queries are split into ``n_dirs`` groups (row r in
    group (r // cfg.q_run) % n_dirs: runs of q_run consecutive rows); group d's
    indexer queries share a direction v_d (q_idx = z + beta * v_d), and 2048
    blocks per group among the prior blocks get one key bf16(c * v_d).  Returns
    a dict of arrays; ``q_rows`` limits the query rows generated (all positions
    are kept so the cache is the same).
    """
    rng = rng_for(cfg.seed if seed is None else seed)
    Q = cfg.Q
    prior = cfg.prior
    N = prior + Q // 2
    latent = normal_bf16(rng, (1, N, D))
    keys = normal_bf16(rng, (1, N, DI))
    dirs = normal_bf16(rng, (n_dirs, DI))
    z = rng.standard_normal((Q, cfg.Hi, DI), dtype=np.float32)
    group = (np.arange(Q) // max(int(cfg.q_run), 1)) % n_dirs
    qf = z + np.float32(beta) * bf16_to_f32(dirs)[group][:, None, :]
    q_idx = bf16_rne(qf)[None]
    w = np.abs(rng.standard_normal((1, Q, cfg.Hi), dtype=np.float32)) + np.float32(0.1)
    q = normal_bf16(rng, (1, Q, cfg.H, D))
    nb_prior = prior // 8
    planted = []
    used = np.zeros(0, dtype=np.int64)
    for d in range(n_dirs):
        blocks = choose_blocks(rng, nb_prior, cfg.K, exclude=used)
        used = np.concatenate([used, blocks])
        v = bf16_to_f32(dirs[d])
        # distinct multipliers per planted block, as in plant_dominant
        for r, b in enumerate(rng.permutation(blocks)):
            key = bf16_rne(np.float32(c * (1.0 + r / len(blocks))) * v)
            keys[0, _entry_in_block(rng, int(b), prior)] = key
        planted.append(blocks)
    swa_total = cfg.W + Q
    swa_pos0 = 2 * prior - cfg.W
    swa = normal_bf16(rng, (1, swa_total, D))
    q_pos = (2 * prior + np.arange(Q)).astype(np.int32)[None]
    if q_rows is not None:
        sel = np.asarray(q_rows)
        q, q_idx, w, q_pos = q[:, sel], q_idx[:, sel], w[:, sel], q_pos[:, sel]
    return dict(latent=latent, keys=keys, q=q, q_idx=q_idx, w=w, q_pos=q_pos,
                swa=swa, swa_len=np.array([swa_total], np.int32),
                swa_pos0=np.array([swa_pos0], np.int32), prior=prior,
                n_entries=np.array([N], np.int32), planted=planted)


@dataclass
class LayerInputs:
    mode: str               # "F" Full, "R" Reindex, "U" Reuse
    q: np.ndarray           # u16 [B][Q][H][512]  the layer's own attention query
    q_idx: np.ndarray       # u16 [B][Q][Hi][64]  own indexer query (F, R), else None
    w: np.ndarray           # f32 [B][Q][Hi]      own indexer weights (F, R), else None
    swa: np.ndarray         # u16 [B][W][512]     own sliding window
    planted: list = field(default_factory=list)


def layers_inputs(cfg, seed=None, c=3.0):
    """Shared cache + one LayerInputs per letter of ``cfg.layers`` (e.g. "FRUU").

    The first layer uses the decode_inputs draw (its plant included).  Every
    later layer draws its own query and window; a Reindex layer also draws its
    own indexer query and plants its own K blocks (one key c * q_h* each, blocks
    disjoint from the earlier plants) into the shared keys.
    """
    base = cfg.seed if seed is None else seed
    x = decode_inputs(cfg, seed=base, c=c)
    rng = rng_for(base + 7919)
    layers = []
    used = [np.asarray(p) for p in x.planted]
    for i, mode in enumerate(cfg.layers):
        if i == 0:
            if mode != "F":
                raise ValueError("the first layer must be Full")
            layers.append(LayerInputs("F", x.q, x.q_idx, x.w, x.swa, x.planted))
            continue
        q, q_idx, w = layer_query(rng, x.q.shape[0], cfg.Q, cfg.H, cfg.Hi)
        swa = normal_bf16(rng, (x.q.shape[0], cfg.W, D))
        planted = []
        if mode == "R":
            for b in range(x.q.shape[0]):
                nbp = (int(x.n_entries[b]) + 7) // 8
                blocks = choose_blocks(rng, nbp, cfg.K, exclude=used[b])
                plant_dominant(x.keys[b], x.n_entries[b], q_idx[b, 0], w[b, 0], blocks, rng, c=c)
                used[b] = np.concatenate([used[b], blocks])
                planted.append(blocks)
            layers.append(LayerInputs("R", q, q_idx, w, swa, planted))
        elif mode == "U":
            layers.append(LayerInputs("U", q, None, None, swa, []))
        else:
            raise ValueError(mode)
    return x, layers
