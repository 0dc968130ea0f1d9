"""Hierarchically tiled GEMM for MI355X (gfx950): D = act(alpha*(A@B) + beta*C + bias).

The compute path is the HIP library libhtgemm.so (include/htgemm.h, include/htlayout.h);
`htgemm` is its ctypes binding and `inputs` the seeded synthetic input generator.
"""
from . import htgemm  # noqa: F401  (loading the library is deferred to the first call)
