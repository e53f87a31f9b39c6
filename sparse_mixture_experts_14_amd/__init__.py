"""MI355X-native sparse top-K mixture-of-experts layer (Mixtral-style: top-2 of
8 SwiGLU experts).

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI declared
in ``include/moe.h`` (``libmoe.so``).  This package is the thin Python binding:
it marshals torch device tensors to raw pointers and the current HIP stream.
"""
from . import workloads  # noqa: F401  (seeded input generators; no layer arithmetic)

__all__ = ["workloads"]
