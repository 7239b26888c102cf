"""bfloat16 bit patterns -> float64 (oracle side; test infrastructure only).

Inputs of the hot path are bfloat16 (latents, queries, indexer keys, window
tokens).  They are stored as raw uint16 bit patterns; bfloat16 is the top half
of an IEEE-754 binary32, so widening is exact.
"""

import numpy as np


def to_f64(bits):
    """uint16 bfloat16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def scalar_to_f64(bits):
    """One bfloat16 bit pattern -> Python float (exact)."""
    return float(to_f64(np.array([bits], dtype=np.uint16))[0])
