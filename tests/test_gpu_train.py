"""GPU checks of the training pair moe_forward_train / moe_backward_saved.

The forward for training must give the forward's y bit for bit, and the
backward from its saved state must give the recomputing backward's gradients
bit for bit (both run the same kernels on the same inputs); the recomputing
backward is checked against the oracle in test_gpu_backward.py.  Both GEMM
families are covered: the weight stream (few rows per expert) and the MFMA
tiles, forced and by the automatic choice."""
import pytest
import torch

import sparse_mixture_experts_14_amd as moe
from tests.gpu_common import forced_path, say, small_layer

pytestmark = pytest.mark.gpu

NAMES = ("dx", "dWg", "dW1", "dW3", "dW2")


def _dy(T, d, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(T, d, generator=g).to(torch.bfloat16).to("cuda")


@pytest.mark.parametrize("T,d,d_ff,n,K,path,seed", [
    (48, 256, 320, 8, 2, None, 1),        # few rows per expert: weight stream
    (48, 256, 320, 8, 2, "tiled", 2),
    (300, 256, 328, 8, 2, None, 3),       # tiles, ragged
    (40, 128, 192, 8, 2, "skinny", 4),
    (77, 128, 192, 4, 4, "tiled", 5),
    (600, 512, 1024, 8, 2, None, 6),
])
def test_training_pair_matches_forward_and_backward(T, d, d_ff, n, K, path, seed):
    L = small_layer(T, d, d_ff, n, K, seed=seed)
    dy = _dy(T, d, seed + 50)
    say(f"[case] training pair T={T} d={d} d_ff={d_ff} n={n} K={K} path={path}")
    with forced_path(path):
        y_ref, _, _, _ = moe.forward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], K)
        y, saved = moe.forward_train(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], K)
        g_ref = moe.backward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], dy, K)
        g = moe.backward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], dy, K, saved=saved)
        torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "forward_train y differs from forward"
    for name in NAMES:
        assert torch.equal(g[name], g_ref[name]), f"{name} from the saved state differs"
    # the saved state is read, never written: a second backward is identical
    with forced_path(path):
        g2 = moe.backward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], dy, K, saved=saved)
        torch.cuda.synchronize()
    for name in NAMES:
        assert torch.equal(g2[name], g[name]), name


def test_training_pair_no_tokens():
    L = small_layer(0, 64, 96, 4, 2, seed=7)
    y, saved = moe.forward_train(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], 2)
    dy = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    g = moe.backward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], dy, 2, saved=saved)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
    for name in ("dWg", "dW1", "dW3", "dW2"):
        assert not torch.any(g[name]), name


@pytest.mark.parametrize("T,d,d_ff,n,K,path,seed", [
    (48, 256, 320, 8, 2, None, 11),       # weight stream
    (300, 256, 328, 8, 2, None, 12),      # tiles
    (77, 128, 192, 4, 4, "tiled", 13),
])
def test_block_training_pair(T, d, d_ff, n, K, path, seed):
    # the stack layer y = x + MoE(RMSNorm(x)): forward_train's y equals
    # block_forward's, the saved-state backward equals block_backward
    eps = 1e-5
    L = small_layer(T, d, d_ff, n, K, seed=seed)
    dy = _dy(T, d, seed + 50)
    say(f"[case] block training pair T={T} d={d} d_ff={d_ff} n={n} K={K} path={path}")
    args = (L["x"], L["Wg"], L["W1"], L["W3"], L["W2"])
    with forced_path(path):
        y_ref, _, _, _ = moe.block_forward(*args, K, eps)
        y, saved = moe.forward_train(*args, K, eps=eps)
        g_ref = moe.block_backward(*args, dy, K, eps)
        g = moe.block_backward(*args, dy, K, eps, saved=saved)
        torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "block forward_train y differs from block_forward"
    for name in NAMES:
        assert torch.equal(g[name], g_ref[name]), f"{name} from the saved state differs"
