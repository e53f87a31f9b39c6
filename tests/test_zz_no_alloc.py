"""moe_forward_noalloc (the forward with the library's static scratch instead
of a caller workspace) against moe_forward, through the C ABI: two calls in a
row on one device, the second with fewer tokens (the scratch keeps the first
call's contents), then a third on the tiled path again.  Every output --
y, idx, gate, counts -- must be bitwise equal to moe_forward's on the same
input (same kernels, deterministic), and the calls must not allocate through
torch's allocator."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_14_amd as moe
from sparse_mixture_experts_14_amd import _lib as B
from sparse_mixture_experts_14_amd import workloads as W

pytestmark = pytest.mark.gpu


def _outputs(T, n, K, x):
    dev = x.device
    return (torch.full_like(x, float("nan")), torch.full((T, K), -1, dtype=torch.int32, device=dev),
            torch.full((T, K), float("nan"), dtype=torch.float32, device=dev),
            torch.full((n,), -1, dtype=torch.int32, device=dev))


def _check(L, T, K, label):
    x = L["x"][:T].contiguous()
    n = L["Wg"].shape[1]
    print(f"[case] noalloc {label} T={T} d={x.shape[1]} d_ff={L['W1'].shape[1]} n={n} K={K}",
          flush=True)
    y, idx, gate, counts = _outputs(T, n, K, x)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    B.forward_noalloc(x, L["Wg"], L["W1"], L["W3"], L["W2"], K, y, idx, gate, counts)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    ry, ridx, rgate, rcounts = moe.forward(x, L["Wg"], L["W1"], L["W3"], L["W2"], K)
    torch.cuda.synchronize()
    assert torch.equal(idx, ridx), "idx"
    assert torch.equal(gate, rgate), "gate"
    assert torch.equal(counts, rcounts), "counts"
    assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                       ry.view(torch.int16) if ry.dtype == torch.bfloat16 else ry), "y"
    assert int(counts.sum()) == T * K
    print(f"       bitwise equal to moe_forward; counts {counts.tolist()}", flush=True)


def test_noalloc_equals_forward_on_consecutive_calls():
    w = W.WORKLOADS["decode"].with_(T=256)
    L = W.make_layer(w, device="cuda")
    # 256 tokens: the tiled GEMMs (and the largest scratch use), then 16
    # tokens: the weight stream, on a scratch still holding the first call's
    # contents, then the tiled path again on 200 tokens
    _check(L, 256, 2, "tiled")
    _check(L, 16, 2, "weight stream, smaller")
    _check(L, 200, 2, "tiled again")


def test_noalloc_fp32_and_ragged():
    Lf = W.make_layer(W.WORKLOADS["tiny"], device="cuda")
    _check(Lf, 64, 2, "fp32")
    _check(Lf, 13, 2, "fp32, smaller")
    w = W.Workload("ragged", T=97, d=264, d_ff=328, n=13, K=3, dtype="bf16", seed=3)
    Lr = W.make_layer(w, device="cuda")
    _check(Lr, 97, 3, "bf16 ragged n=13 K=3")


def test_noalloc_rejects_oversize_before_launch():
    w = W.WORKLOADS["decode"].with_(T=512)
    L = W.make_layer(w, device="cuda", experts=False)
    x = L["x"]
    dummy = torch.empty(8, w.d_ff, w.d, dtype=torch.bfloat16, device="cuda")
    dummy2 = torch.empty(8, w.d, w.d_ff, dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(x, 7.0)
    with pytest.raises(moe.MoeError) as e:
        B.forward_noalloc(x, L["Wg"], dummy, dummy, dummy2, 2, y)
    assert e.value.status == B.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a rejected call wrote its output"
