"""Workload table (sizes only; no arithmetic of the method)."""

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    B: int            # sequences
    Q: int            # query rows per sequence
    H: int            # attention heads
    N: int            # compressed entries held per sequence
    Hi: int           # indexer heads
    K: int            # selected blocks per row
    W: int            # sliding window
    top_groups: int = 0      # two-level indexer: groups kept (0 = flat)
    layers: str = "F"        # cross-layer schedule, e.g. "F R I I" -> "FRII"
    prior: int = 0           # prefill: entries already in the cache before the chunk
    q_run: int = 1           # prefill: consecutive query rows that share an indexer direction
    seed: int = 0

    @property
    def nb(self):
        return self.N // 8

    @property
    def cap(self):
        # cache capacity in entries: a whole number of 512-entry groups
        return ((self.N + 511) // 512) * 512


CONFIGS = {
    "tiny": Config("tiny", B=1, Q=1, H=16, N=2048, Hi=4, K=32, W=128, seed=1000),
    "decode64k": Config("decode64k", B=32, Q=1, H=64, N=32768, Hi=8, K=2048, W=512, seed=1001),
    "decode1m": Config("decode1m", B=8, Q=1, H=64, N=524288, Hi=8, K=2048, W=512,
                       top_groups=256, seed=1002),
    "layers128k": Config("layers128k", B=64, Q=1, H=64, N=65536, Hi=8, K=2048, W=512,
                         layers="FRUU", seed=1003),
    "prefill": Config("prefill", B=1, Q=4096, H=64, N=67584, Hi=8, K=2048, W=512,
                      prior=65536, seed=1004),
    # decode with 3 draft tokens verified in the same pass: 4 query rows per sequence
    "specdec64k": Config("specdec64k", B=32, Q=4, H=64, N=32768, Hi=8, K=2048, W=512, seed=1005),
    # one GPU's share when the 64 heads are split over 4 GPUs (16 heads each;
    # the selection is the same on every GPU): the draft rows of specdec64k,
    # and a prefill chunk whose query tokens come in runs of 64 that ask for
    # the same context
    "specdec64k_h16": Config("specdec64k_h16", B=32, Q=4, H=16, N=32768, Hi=8, K=2048, W=512, seed=1005),
    "prefill_h16": Config("prefill_h16", B=1, Q=4096, H=16, N=67584, Hi=8, K=2048, W=512,
                          prior=65536, q_run=64, seed=1004),
}
