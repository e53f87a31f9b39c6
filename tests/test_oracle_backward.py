"""Pins of the oracle's backward pass (gradients of L = sum_t dy_t . y_t).

Each pin checks the fp64 gradients against something other than the
backward code itself:
* central finite differences of the oracle's own forward pass, for every
  element of every input, on tiny shapes away from routing ties;
* torch fp64 autograd of the two special cases the method reduces to -- a
  plain SwiGLU FFN (n = 1) and a dense softmax-gated mixture (K = n);
* invariants: the router-logit gradient of a token sums to zero (the gates
  are a softmax), so every row of dW_g sums to zero; reordering tokens
  reorders dx and leaves the weight gradients unchanged (up to summation
  order); a zero output gradient gives zero gradients.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _layer(rng, T, d, d_ff, n, scale_x=1.0):
    x = (scale_x * rng.standard_normal((T, d))).astype(np.float32)
    Wg = (rng.standard_normal((d, n)) / np.sqrt(d)).astype(np.float32)
    W1 = (rng.standard_normal((n, d_ff, d)) / np.sqrt(d)).astype(np.float32)
    W3 = (rng.standard_normal((n, d_ff, d)) / np.sqrt(d)).astype(np.float32)
    W2 = (rng.standard_normal((n, d, d_ff)) / np.sqrt(d_ff)).astype(np.float32)
    return x, Wg, W1, W3, W2


def _loss(x, Wg, W1, W3, W2, dy, K):
    y, idx, _, _ = oracle.forward(x, Wg, W1, W3, W2, K)
    return float(np.sum(y * dy.astype(np.float64))), idx


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(5)
    T, d, d_ff, n, K = 3, 5, 6, 4, 2
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    g = oracle.backward(x, Wg, W1, W3, W2, dy, K)
    _, idx0 = _loss(x, Wg, W1, W3, W2, dy, K)
    inputs = {"dx": x, "dWg": Wg, "dW1": W1, "dW3": W3, "dW2": W2}
    h = 2.0 ** -9
    for name, arr in inputs.items():
        flat = arr.reshape(-1)
        num = np.empty(flat.size)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = np.float32(keep + h)
            up = float(flat[i]) - float(keep)
            lp, ip = _loss(x, Wg, W1, W3, W2, dy, K)
            flat[i] = np.float32(keep - h)
            dn = float(keep) - float(flat[i])
            lm, im = _loss(x, Wg, W1, W3, W2, dy, K)
            flat[i] = keep
            assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), "routing moved"
            num[i] = (lp - lm) / (up + dn)
        ana = g[name].reshape(-1)
        np.testing.assert_allclose(ana, num, rtol=2e-5, atol=2e-6, err_msg=name)


def _t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def test_single_expert_backward_is_swiglu_autograd():
    rng = np.random.default_rng(6)
    T, d, d_ff = 7, 9, 11
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, 1)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    g = oracle.backward(x, Wg, W1, W3, W2, dy, 1)
    X = _t64(x).requires_grad_()
    A1, A3, A2 = (_t64(w[0]).requires_grad_() for w in (W1, W3, W2))
    Y = (F.silu(X @ A1.T) * (X @ A3.T)) @ A2.T
    (Y * _t64(dy)).sum().backward()
    np.testing.assert_allclose(g["dx"], X.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dW1"][0], A1.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dW3"][0], A3.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dW2"][0], A2.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dWg"], 0.0, atol=1e-12)  # one expert: gate is always 1


def test_dense_mixture_backward_when_K_equals_n():
    rng = np.random.default_rng(7)
    T, d, d_ff, n = 6, 8, 10, 4
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    g = oracle.backward(x, Wg, W1, W3, W2, dy, n)
    X = _t64(x).requires_grad_()
    G = _t64(Wg).requires_grad_()
    A1, A3, A2 = (_t64(w).requires_grad_() for w in (W1, W3, W2))
    gates = torch.softmax(X @ G, dim=1)                       # [T][n]
    h = F.silu(torch.einsum("td,efd->tef", X, A1)) * torch.einsum("td,efd->tef", X, A3)
    o = torch.einsum("tef,ecf->tec", h, A2)                    # [T][n][d]
    Y = (gates[:, :, None] * o).sum(1)
    (Y * _t64(dy)).sum().backward()
    for name, ref in (("dx", X), ("dWg", G), ("dW1", A1), ("dW3", A3), ("dW2", A2)):
        np.testing.assert_allclose(g[name], ref.grad.numpy(), rtol=1e-9, atol=1e-11,
                                   err_msg=name)


def test_router_gradient_rows_sum_to_zero():
    rng = np.random.default_rng(8)
    x, Wg, W1, W3, W2 = _layer(rng, 40, 16, 12, 8)
    dy = rng.standard_normal((40, 16)).astype(np.float32)
    g = oracle.backward(x, Wg, W1, W3, W2, dy, 2)
    np.testing.assert_allclose(g["dWg"].sum(axis=1), 0.0, atol=1e-12)
    assert np.abs(g["dWg"]).max() > 1e-3


def test_backward_token_permutation():
    rng = np.random.default_rng(9)
    T = 12
    x, Wg, W1, W3, W2 = _layer(rng, T, 10, 14, 8)
    dy = rng.standard_normal((T, 10)).astype(np.float32)
    p = rng.permutation(T)
    g = oracle.backward(x, Wg, W1, W3, W2, dy, 2)
    gp = oracle.backward(x[p], Wg, W1, W3, W2, dy[p], 2)
    assert np.array_equal(gp["dx"], g["dx"][p])  # per token: bitwise
    for name in ("dWg", "dW1", "dW3", "dW2"):
        np.testing.assert_allclose(gp[name], g[name], rtol=1e-12, atol=1e-14, err_msg=name)
    # rows= gives the same per-token dx
    rows = np.array([3, 0, 11])
    gr = oracle.backward(x, Wg, W1, W3, W2, dy, 2, rows=rows)
    assert np.array_equal(gr["dx"], g["dx"][rows])


def test_zero_output_gradient():
    rng = np.random.default_rng(10)
    x, Wg, W1, W3, W2 = _layer(rng, 5, 8, 6, 4)
    g = oracle.backward(x, Wg, W1, W3, W2, np.zeros((5, 8), np.float32), 2)
    for v in g.values():
        assert not np.any(v)


def _entries(rng, n, d, d_ff, count):
    """(name, e, row, col) samples over the three expert weight gradients."""
    out = []
    for q in range(count):
        name = ("dW1", "dW2", "dW3")[q % 3]
        rows, cols = (d, d_ff) if name == "dW2" else (d_ff, d)
        out.append((name, int(rng.integers(n)), int(rng.integers(rows)),
                    int(rng.integers(cols))))
    return out


def test_backward_entries_match_dense_autograd():
    # sampled weight-gradient entries of the K = n dense mixture against torch
    # fp64 autograd (an independent chain rule)
    rng = np.random.default_rng(11)
    T, d, d_ff, n = 9, 8, 12, 4
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    X = _t64(x)
    G = _t64(Wg)
    A1, A3, A2 = (_t64(w).requires_grad_() for w in (W1, W3, W2))
    gates = torch.softmax(X @ G, dim=1)
    h = F.silu(torch.einsum("td,efd->tef", X, A1)) * torch.einsum("td,efd->tef", X, A3)
    Y = (gates[:, :, None] * torch.einsum("tef,ecf->tec", h, A2)).sum(1)
    (Y * _t64(dy)).sum().backward()
    ref = {"dW1": A1.grad.numpy(), "dW3": A3.grad.numpy(), "dW2": A2.grad.numpy()}
    ents = _entries(rng, n, d, d_ff, 30)
    got = oracle.backward_entries(x, Wg, W1, W3, W2, dy, n, ents)
    want = np.array([ref[nm][e, i, j] for nm, e, i, j in ents])
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)


def test_backward_entries_match_full_backward():
    # routed top-2 case: the per-entry sums equal the full backward's entries
    rng = np.random.default_rng(12)
    T, d, d_ff, n = 40, 16, 24, 8
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    full = oracle.backward(x, Wg, W1, W3, W2, dy, 2)
    ents = _entries(rng, n, d, d_ff, 60)
    got = oracle.backward_entries(x, Wg, W1, W3, W2, dy, 2, ents)
    want = np.array([full[nm][e, i, j] for nm, e, i, j in ents])
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-13)
    # forced routing: the same as TopK when forced to TopK's own choice
    _, idx, _, _ = oracle.forward(x, Wg, W1, W3, W2, 2)
    got_f = oracle.backward_entries(x, Wg, W1, W3, W2, dy, 2, ents, forced=idx)
    assert np.array_equal(got_f, got)


# ---- the stack layer y = x + MoE(RMSNorm(x)) --------------------------------


def _block_loss(x, Wg, W1, W3, W2, dy, K, eps):
    y, idx, _, _ = oracle.block_forward(x, Wg, W1, W3, W2, K, eps)
    return float(np.sum(y * dy.astype(np.float64))), idx


def test_block_backward_matches_finite_differences():
    rng = np.random.default_rng(21)
    T, d, d_ff, n, K, eps = 3, 6, 5, 4, 2, 1e-2
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    g = oracle.block_backward(x, Wg, W1, W3, W2, dy, K, eps)
    _, idx0 = _block_loss(x, Wg, W1, W3, W2, dy, K, eps)
    h = 2.0 ** -9
    for name, arr in {"dx": x, "dWg": Wg, "dW1": W1, "dW3": W3, "dW2": W2}.items():
        flat = arr.reshape(-1)
        num = np.empty(flat.size)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = np.float32(keep + h)
            up = float(flat[i]) - float(keep)
            lp, ip = _block_loss(x, Wg, W1, W3, W2, dy, K, eps)
            flat[i] = np.float32(keep - h)
            dn = float(keep) - float(flat[i])
            lm, im = _block_loss(x, Wg, W1, W3, W2, dy, K, eps)
            flat[i] = keep
            assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), "routing moved"
            num[i] = (lp - lm) / (up + dn)
        np.testing.assert_allclose(g[name].reshape(-1), num, rtol=3e-5, atol=3e-6,
                                   err_msg=name)


def test_block_backward_dense_mixture_autograd():
    # K = n: x + softmax-gated mixture of every expert on rms_norm(x), torch fp64
    rng = np.random.default_rng(22)
    T, d, d_ff, n, eps = 5, 8, 10, 4, 1e-5
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    g = oracle.block_backward(x, Wg, W1, W3, W2, dy, n, eps)
    X = _t64(x).requires_grad_()
    G = _t64(Wg).requires_grad_()
    A1, A3, A2 = (_t64(w).requires_grad_() for w in (W1, W3, W2))
    U = F.rms_norm(X, (d,), eps=eps)
    gates = torch.softmax(U @ G, dim=1)
    h = F.silu(torch.einsum("td,efd->tef", U, A1)) * torch.einsum("td,efd->tef", U, A3)
    Y = X + (gates[:, :, None] * torch.einsum("tef,ecf->tec", h, A2)).sum(1)
    (Y * _t64(dy)).sum().backward()
    for name, ref in (("dx", X), ("dWg", G), ("dW1", A1), ("dW3", A3), ("dW2", A2)):
        np.testing.assert_allclose(g[name], ref.grad.numpy(), rtol=1e-9, atol=1e-11,
                                   err_msg=name)


def test_block_backward_scale_invariance():
    # eps = 0: RMSNorm(c x) = RMSNorm(x), so the weight gradients do not move,
    # dx - dy scales by 1 / c, and x . (dx - dy) = 0 per token
    rng = np.random.default_rng(23)
    x, Wg, W1, W3, W2 = _layer(rng, 10, 12, 8, 8)
    dy = rng.standard_normal((10, 12)).astype(np.float32)
    g1 = oracle.block_backward(x, Wg, W1, W3, W2, dy, 2, 0.0)
    g2 = oracle.block_backward(4.0 * x, Wg, W1, W3, W2, dy, 2, 0.0)  # exact in float32
    for name in ("dWg", "dW1", "dW3", "dW2"):
        np.testing.assert_allclose(g2[name], g1[name], rtol=1e-12, atol=1e-14, err_msg=name)
    r1 = g1["dx"] - dy
    np.testing.assert_allclose(g2["dx"] - dy, r1 / 4.0, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(np.sum(x.astype(np.float64) * r1, axis=1), 0.0, atol=1e-12)
    assert np.abs(r1).max() > 1e-3


def test_block_backward_entries_match_full_block_backward():
    rng = np.random.default_rng(24)
    T, d, d_ff, n, eps = 40, 16, 24, 8, 1e-5
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n, scale_x=3.0)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    full = oracle.block_backward(x, Wg, W1, W3, W2, dy, 2, eps)
    ents = _entries(rng, n, d, d_ff, 60)
    got = oracle.backward_entries(x, Wg, W1, W3, W2, dy, 2, ents, eps=eps)
    want = np.array([full[nm][e, i, j] for nm, e, i, j in ents])
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-13)
    # rows= gives the same per-token dx
    rows = np.array([5, 0, 39])
    gr = oracle.block_backward(x, Wg, W1, W3, W2, dy, 2, eps, rows=rows)
    assert np.array_equal(gr["dx"], full["dx"][rows])
