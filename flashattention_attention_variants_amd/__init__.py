"""Fused attention-variant forward for AMD MI355X (gfx950).

The compute lives in ``libflattn.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/flattn.h``).  ``api`` is a thin ctypes binding
with the same entry points; ``inputs`` draws seeded synthetic tensors.
Importing the package loads nothing; the first call into ``api`` loads the
library and raises if it has not been built.
"""

__all__ = ["api", "inputs", "flops"]
