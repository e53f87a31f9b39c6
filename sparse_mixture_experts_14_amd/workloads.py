"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random tensors; it holds none of the layer's
arithmetic.  Both the GPU path and the fp64 oracle are fed from it.

Shapes follow the pages on "Mixtral of Experts" (xyznot digest, section
"Method (with core equations)": hidden size 4096, n = 8 SwiGLU experts of
intermediate size 14336, top-K = 2, 32 layers).  The pages publish no weights
and no activations, so every tensor is synthetic:

* x ~ N(0, 1); W_g ~ N(0, 1/d); W1, W3 ~ N(0, 1/d); W2 ~ N(0, 1/d_ff)
  (std 1/sqrt(fan_in)).  Draw order: x, W_g, W1, W3, W2, each as float32
  ``torch.randn`` scaled by its std, then rounded to the storage dtype (RNE).
* Storage: x[T][d], W_g[d][n], W1/W3[n][d_ff][d], W2[n][d][d_ff].
* ``skew``: routing made uneven on purpose.  A zero-mean linear router cannot
  shift the *mean* of a logit, so a shared mean direction is put into the
  tokens instead: a unit vector v (drawn right after W_g, before W1) is added
  m = 8 times to every
  token, and column j of W_g gets (mu_j / m) v with mu = (+3, 0, 0, 0, 0, 0,
  -1, -1).  Logit j then has mean mu_j: expert 0 takes roughly half of the
  assignments and experts 6 and 7 a few percent each.
* ``stack``: 32 independent layers; x is drawn from the workload seed and layer
  l's weights from seed 1000 + l.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    d_ff: int
    n: int
    K: int
    dtype: str  # "f32" or "bf16"
    seed: int = 0
    skew: bool = False
    layers: int = 1
    eps: float | None = None  # set for the pre-normalised stack layer

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the layer (tiny fp32 check, decode, prefill, skewed
# routing, 32-layer stack).
WORKLOADS = {
    "tiny": Workload("tiny", T=64, d=128, d_ff=256, n=8, K=2, dtype="f32"),
    "decode": Workload("decode", T=16, d=4096, d_ff=14336, n=8, K=2, dtype="bf16"),
    "prefill": Workload("prefill", T=4096, d=4096, d_ff=14336, n=8, K=2, dtype="bf16"),
    "skew": Workload("skew", T=16384, d=4096, d_ff=14336, n=8, K=2, dtype="bf16",
                     skew=True),
    "stack": Workload("stack", T=2048, d=4096, d_ff=14336, n=8, K=2, dtype="bf16",
                      layers=32, eps=1e-5),
}

SKEW_SHIFT = 8.0
SKEW_MU = (3.0, 0.0, 0.0, 0.0, 0.0, 0.0, -1.0, -1.0)
STACK_LAYER_SEED0 = 1000


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, std: float, dtype, g: torch.Generator, device) -> torch.Tensor:
    t = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t if dtype == torch.float32 else t.to(dtype)


def _randn_big(shape, std: float, dtype, g: torch.Generator, device) -> torch.Tensor:
    """Like _randn for [n][a][b] weights, one expert at a time so that the
    float32 staging copy stays small; the values equal those of one draw of
    the whole tensor only up to generator chunking, which is irrelevant:
    every consumer reads the tensor actually produced."""
    n = shape[0]
    out = torch.empty(*shape, dtype=dtype, device=device)
    for e in range(n):
        t = torch.randn(*shape[1:], generator=g, dtype=torch.float32, device=device)
        if std != 1.0:
            t.mul_(std)
        out[e].copy_(t)
        del t
    return out


def make_weights(w: Workload, seed: int, device="cpu") -> dict:
    """W_g, W1, W3, W2 of one layer from generator ``seed``."""
    g = _gen(seed, device)
    dt = w.torch_dtype
    Wg = _randn((w.d, w.n), 1.0 / math.sqrt(w.d), dt, g, device)
    W1 = _randn_big((w.n, w.d_ff, w.d), 1.0 / math.sqrt(w.d), dt, g, device)
    W3 = _randn_big((w.n, w.d_ff, w.d), 1.0 / math.sqrt(w.d), dt, g, device)
    W2 = _randn_big((w.n, w.d, w.d_ff), 1.0 / math.sqrt(w.d_ff), dt, g, device)
    return {"Wg": Wg, "W1": W1, "W3": W3, "W2": W2}


def make_layer(w: Workload, device="cpu", seed: int | None = None,
               experts: bool = True) -> dict:
    """x, W_g, W1, W3, W2 for a single-layer workload.  Draw order: x, W_g,
    (skew direction v), W1, W3, W2.  ``experts=False`` stops after the router
    inputs (x and W_g are the same as with experts)."""
    seed = w.seed if seed is None else seed
    g = _gen(seed, device)
    dt = w.torch_dtype
    x32 = torch.randn(w.T, w.d, generator=g, dtype=torch.float32, device=device)
    Wg32 = torch.randn(w.d, w.n, generator=g, dtype=torch.float32, device=device)
    Wg32.mul_(1.0 / math.sqrt(w.d))
    if w.skew:
        if w.n != len(SKEW_MU):
            raise ValueError("the skew construction is defined for n = 8")
        v = torch.randn(w.d, generator=g, dtype=torch.float32, device=device)
        v /= v.norm()
        x32.add_(SKEW_SHIFT * v)
        mu = torch.tensor(SKEW_MU, dtype=torch.float32, device=device)
        Wg32.add_(torch.outer(v, mu / SKEW_SHIFT))
    out = {"x": x32.to(dt), "Wg": Wg32.to(dt)}
    del x32, Wg32
    if experts:
        out["W1"] = _randn_big((w.n, w.d_ff, w.d), 1.0 / math.sqrt(w.d), dt, g, device)
        out["W3"] = _randn_big((w.n, w.d_ff, w.d), 1.0 / math.sqrt(w.d), dt, g, device)
        out["W2"] = _randn_big((w.n, w.d, w.d_ff), 1.0 / math.sqrt(w.d_ff), dt, g,
                               device)
    return out


def make_stack_input(w: Workload, device="cpu") -> torch.Tensor:
    """Layer-0 input of the stack workload."""
    g = _gen(w.seed, device)
    return torch.randn(w.T, w.d, generator=g, dtype=torch.float32,
                       device=device).to(w.torch_dtype)


def make_stack_layer(w: Workload, layer: int, device="cpu") -> dict:
    """Weights of stack layer ``layer`` (seed 1000 + layer)."""
    return make_weights(w, STACK_LAYER_SEED0 + layer, device)


def random_tokens(T: int, d: int, seed: int, dtype=torch.bfloat16, device="cpu",
                  std: float = 1.0) -> torch.Tensor:
    """Standalone N(0, std^2) tokens, e.g. a synthetic input for one layer of
    the stack tested on its own."""
    g = _gen(seed, device)
    t = torch.randn(T, d, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)
