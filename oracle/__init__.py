"""CPU oracle for CSA2-style compressed sparse attention over an MXFP4 latent cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code, tables or helpers with the HIP
library; both sides read the same seeded inputs from ``synth``.

Everything here is plain NumPy in float64 (the attention and scores) or exact
integer/bit arithmetic (the MXFP4 encoding), written as the plain definition of
each step so it can be checked against the pages by eye:

* ``bf16``      -- bit-level bfloat16 <-> float64 (input decoding only).
* ``mxfp4``     -- MXFP4 (FP4 E2M1 codes + one E8M0 scale per 32 values) encode,
                   decode and the block-record byte layout of the global cache.
* ``mxfp8``     -- MXFP8 (E4M3 codes + one E8M0 scale per 32 values) encode and
                   decode of the indexer keys (the lower-precision key cache).
* ``indexer``   -- entry/block scores of the sparse indexer and the two-level
                   (hierarchical) group stage.
* ``topk``      -- top-K block selection with its tie rule and output order.
* ``attention`` -- fp64 softmax attention over the selected latent entries, the
                   sliding-window branch, and the log-sum-exp merge.
* ``modes``     -- the Full / Reindex / Reuse cross-layer compositions.

Sources (pages):
  [digest]  paper-digest.app, "DeepSeek-v4.1 Flash: Pushing the Limits of KV
            Cache Compression" -- Core Mechanics, Terminology.
  [abstract] thelatestinai.com, "DeepSeek-V4.1-Flash: Pushing the Limits of KV
            Cache Compression" -- Abstract.
  [news]    news.promptgoblins.ai, "DeepSeek Releases V4.1 Flash with 4x KV Cache
            Compression for Long-Context Agent Workflows" -- Details.
  [card]    observer.broadside.tech card, "DeepSeek-V4.1-Flash: Pushing the
            Limits of KV Cache Compression" -- Key ideas.

The pages fix the structure (one 512-d latent shared as K and V by every head,
2 positions per entry, FP4 storage, top-K blocks of 8, a hierarchical indexer,
per-layer sliding window, Full/Reindex/Reuse) but print no formula for any step;
every formula below is the plainest reading consistent with them, and each
function says which reading it takes.

Parity-pin status: every public function is pinned by tests under ``tests/``
(closed forms, brute force, special cases, invariants); none is "parity unpinned".
"""

from . import bf16, mxfp4, mxfp8, indexer, topk, attention, modes  # noqa: F401
