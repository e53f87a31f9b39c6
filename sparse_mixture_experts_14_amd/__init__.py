"""MI355X-native sparse top-K mixture-of-experts layer (Mixtral-style: top-2 of
8 SwiGLU experts).

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI declared
in ``include/moe.h`` (``libmoe.so``, built by ``python -m
sparse_mixture_experts_14_amd.build``).  This package is the thin Python
binding: it marshals torch device tensors to raw pointers and the current HIP
stream; there is no CPU fallback.
"""
from . import workloads  # noqa: F401  (seeded input generators; no layer arithmetic)
from ._lib import (  # noqa: F401
    Layer, MoeError, backward, backward_workspace_bytes, block_backward, block_forward, forward,
    forward_train, load, permute, route, saved_bytes, workspace_bytes,
)

__all__ = ["Layer", "MoeError", "backward", "backward_workspace_bytes", "block_backward",
           "block_forward",
           "forward", "forward_train", "load", "permute", "route", "saved_bytes",
           "workspace_bytes", "workloads"]
