"""Seeded synthetic inputs for the CSA2 sparse-decode path.

This module is the only code shared by the CPU oracle and the HIP library's
tests and benchmark.  It holds none of the method's arithmetic: it draws seeded
random numbers, rounds them to bfloat16, and places "planted" relevant blocks by
copying scaled query vectors into indexer keys.  Wherever a plant needs scores
(the tight plant used by tests), the caller passes the scoring function in.

Workload shapes (the pages' structure -- 512-d shared latent, two positions per
compressed entry, blocks of 8, up to 2048 selected blocks, sliding window --
at the sizes of the five workloads below):

  tiny      B 1,  H 16, 2048 entries (256 blocks),     Hi 4, K 32,   W 128
  decode64k B 32, H 64, 32768 entries (4096 blocks),   Hi 8, K 2048, W 512
  decode1m  B 8,  H 64, 524288 entries (65536 blocks), Hi 8, K 2048, W 512,
            two-level indexer keeping 256 groups of 64 blocks
  layers128k B 64, H 64, 65536 entries, 4 layers Full/Reindex/Reuse/Reuse
  prefill   4096 query tokens after 131072 raw positions, H 64, K 2048, W 512
  specdec64k decode64k's cache with 4 query rows per sequence (1 + 3 drafts)
"""

from .gen import *  # noqa: F401,F403
from .configs import CONFIGS, Config  # noqa: F401
