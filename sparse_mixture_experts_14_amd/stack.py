"""A chain of MoE layers run the way the benchmark runs it.

Every layer is one call of the C ABI through a single ``Layer`` call site, so
all layers share one workspace; activations alternate between two
preallocated buffers (layer l writes buffer l mod 2 and reads the other).
With ``eps`` set each call is the pre-normalised residual layer
y = x + MoE(RMSNorm(x)) (``moe_block_forward``), otherwise the plain layer
(``moe_forward``).  Plumbing only: every step of a layer runs in the library's
kernels.
"""
from __future__ import annotations

from typing import Callable, Sequence

import torch

from ._lib import Layer


class Stack:
    def __init__(self, layers: Sequence[dict], T: int, d: int, d_ff: int, n: int, K: int,
                 dtype: torch.dtype, device, eps: float | None = None):
        self.layers = list(layers)
        self.eps = eps
        self.lay = Layer(T, d, d_ff, n, K, dtype, device)
        self.bufs = [torch.empty(T, d, dtype=dtype, device=device) for _ in range(2)]

    def run(self, x0: torch.Tensor,
            before: Callable[[int], None] | None = None,
            after: Callable[[int, torch.Tensor, torch.Tensor, Layer], None] | None = None):
        """Push x0 through every layer; returns the last layer's output (one of
        the two ping-pong buffers).  ``before(l)`` runs right before layer l is
        enqueued, ``after(l, x_in, y, layer)`` right after (x_in is layer l's
        input, y its output buffer, layer.idx/gate/counts its routing)."""
        x = x0
        for i, P in enumerate(self.layers):
            y = self.bufs[i % 2]
            if before is not None:
                before(i)
            if self.eps is not None:
                self.lay.block_forward(x, P["Wg"], P["W1"], P["W3"], P["W2"], self.eps, out=y)
            else:
                self.lay.forward(x, P["Wg"], P["W1"], P["W3"], P["W2"], out=y)
            if after is not None:
                after(i, x, y, self.lay)
            x = y
        return x
