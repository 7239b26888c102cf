"""CSA2-style compressed sparse attention over an MXFP4 latent cache, for MI355X (gfx950).

The compute path is libcsa2.so (hand-written HIP kernels behind the C ABI in
include/csa2.h); ``_lib`` is its ctypes binding and ``modes`` composes the
Full / Reindex / Reuse layer modes from the four calls.  Import the submodules
explicitly; importing this package loads nothing.
"""

__all__ = ["_lib", "modes", "build"]
