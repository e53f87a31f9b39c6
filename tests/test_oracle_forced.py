"""Pins of the oracle's forced-routing mode.

With ``forced`` the oracle skips TopK and takes the caller's expert set S in the
caller's slot order; the gates are then the softmax over the logits of S (the
gating equation of the xyznot digest on "Mixtral of Experts", section "Method
(with core equations)", with TopK replaced by the given set), and the output
is the gate-weighted sum of those experts (the output equation of the same
section).  The GPU parity checks use this mode for near-tie tokens and for
every backward comparison, so each entry point is checked here with sets that
TopK would NOT choose -- the 2nd and 3rd ranked experts, and TopK's own pair
in reversed slot order -- against torch fp64 evaluations (softmax, silu,
rms_norm, matmuls and autograd, all library routines).  An oracle that ignored
``forced`` fails every test below.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _layer(rng, T, d, d_ff, n):
    x = rng.standard_normal((T, d)).astype(np.float32)
    Wg = (rng.standard_normal((d, n)) / math.sqrt(d)).astype(np.float32)
    W1 = (rng.standard_normal((n, d_ff, d)) / math.sqrt(d)).astype(np.float32)
    W3 = (rng.standard_normal((n, d_ff, d)) / math.sqrt(d)).astype(np.float32)
    W2 = (rng.standard_normal((n, d, d_ff)) / math.sqrt(d_ff)).astype(np.float32)
    return x, Wg, W1, W3, W2


def _t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _forced_sets(x, Wg, K, eps=None):
    """Per token: a set TopK does not choose.  Even tokens take the experts
    ranked 2 .. K+1 in reversed rank order; odd tokens take TopK's own set in
    reversed slot order (the same experts, the smaller logit in slot 0)."""
    u = _t64(x)
    if eps is not None:
        u = F.rms_norm(u, (u.shape[1],), eps=eps)
    L = (u @ _t64(Wg)).numpy()
    T, n = L.shape
    order = np.lexsort((np.broadcast_to(np.arange(n), L.shape), -L), axis=1)
    forced = np.empty((T, K), np.int32)
    for t in range(T):
        if t % 2 == 0:
            forced[t] = order[t, 1:K + 1][::-1]
        else:
            forced[t] = order[t, :K][::-1]
    return forced, L


def _torch_layer(X, G, A1, A3, A2, forced, eps=None):
    """y of the layer with the expert set fixed per token, in torch fp64:
    gates = softmax over the forced logits in slot order."""
    U = F.rms_norm(X, (X.shape[1],), eps=eps) if eps is not None else X
    logits = U @ G
    S = torch.from_numpy(forced.astype(np.int64))
    gates = torch.softmax(torch.gather(logits, 1, S), dim=1)      # [T][K]
    rows = []
    for t in range(X.shape[0]):
        yt = X[t] if eps is not None else torch.zeros_like(X[t])
        for j in range(S.shape[1]):
            e = int(S[t, j])
            h = F.silu(A1[e] @ U[t]) * (A3[e] @ U[t])
            yt = yt + gates[t, j] * (A2[e] @ h)
        rows.append(yt)
    return torch.stack(rows), gates


@pytest.mark.parametrize("eps", [None, 1e-5])
def test_forced_forward_takes_the_given_set(eps):
    rng = np.random.default_rng(31)
    T, d, d_ff, n, K = 10, 12, 20, 6, 2
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    forced, _ = _forced_sets(x, Wg, K, eps)
    if eps is None:
        y, idx, gate, _ = oracle.forward(x, Wg, W1, W3, W2, K, forced=forced)
    else:
        y, idx, gate, _ = oracle.block_forward(x, Wg, W1, W3, W2, K, eps, forced=forced)
    ref, gref = _torch_layer(_t64(x), _t64(Wg), _t64(W1), _t64(W3), _t64(W2), forced, eps)
    assert np.array_equal(idx, forced)
    np.testing.assert_allclose(gate, gref.numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-13)
    # odd tokens hold the reversed pair: gates in slot order, the smaller first
    assert (gate[1::2, 0] <= gate[1::2, 1]).all()


def test_forced_rows_subset_and_three_slots():
    """Forced routing on a subset of tokens (rows=) with K = 3: row r of the
    forced array belongs to token rows[r]."""
    rng = np.random.default_rng(32)
    T, d, d_ff, n, K = 9, 10, 14, 7, 3
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    forced_all, _ = _forced_sets(x, Wg, K)
    rows = np.array([7, 2, 5])
    y, idx, gate, _ = oracle.forward(x, Wg, W1, W3, W2, K, rows=rows, forced=forced_all[rows])
    ref, gref = _torch_layer(_t64(x), _t64(Wg), _t64(W1), _t64(W3), _t64(W2), forced_all)
    assert np.array_equal(idx, forced_all[rows])
    np.testing.assert_allclose(gate, gref.numpy()[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(y, ref.numpy()[rows], rtol=1e-11, atol=1e-13)


def _autograd(x, Wg, W1, W3, W2, dy, forced, eps=None):
    X = _t64(x).requires_grad_()
    G = _t64(Wg).requires_grad_()
    A1, A3, A2 = (_t64(w).requires_grad_() for w in (W1, W3, W2))
    Y, _ = _torch_layer(X, G, A1, A3, A2, forced, eps)
    (Y * _t64(dy)).sum().backward()
    return {"dx": X.grad.numpy(), "dWg": G.grad.numpy(), "dW1": A1.grad.numpy(),
            "dW3": A3.grad.numpy(), "dW2": A2.grad.numpy()}


@pytest.mark.parametrize("eps", [None, 1e-5])
def test_forced_backward_matches_autograd(eps):
    rng = np.random.default_rng(33)
    T, d, d_ff, n, K = 8, 9, 13, 5, 2
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    forced, _ = _forced_sets(x, Wg, K, eps)
    if eps is None:
        g = oracle.backward(x, Wg, W1, W3, W2, dy, K, forced=forced)
    else:
        g = oracle.block_backward(x, Wg, W1, W3, W2, dy, K, eps, forced=forced)
    ref = _autograd(x, Wg, W1, W3, W2, dy, forced, eps)
    for name in ("dx", "dWg", "dW1", "dW3", "dW2"):
        np.testing.assert_allclose(g[name], ref[name], rtol=1e-9, atol=1e-11, err_msg=name)
    # dx of a token subset under its forced rows
    rows = np.array([6, 1, 3])
    if eps is None:
        gr = oracle.backward(x, Wg, W1, W3, W2, dy, K, rows=rows, forced=forced[rows])
    else:
        gr = oracle.block_backward(x, Wg, W1, W3, W2, dy, K, eps, rows=rows,
                                   forced=forced[rows])
    np.testing.assert_allclose(gr["dx"], ref["dx"][rows], rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("eps", [None, 1e-5])
def test_forced_backward_entries_match_autograd(eps):
    rng = np.random.default_rng(34)
    T, d, d_ff, n, K = 8, 9, 13, 5, 2
    x, Wg, W1, W3, W2 = _layer(rng, T, d, d_ff, n)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    forced, _ = _forced_sets(x, Wg, K, eps)
    ref = _autograd(x, Wg, W1, W3, W2, dy, forced, eps)
    used = sorted(set(forced.reshape(-1).tolist()))
    entries = []
    for e in used:
        entries += [("dW1", e, int(rng.integers(d_ff)), int(rng.integers(d))),
                    ("dW3", e, int(rng.integers(d_ff)), int(rng.integers(d))),
                    ("dW2", e, int(rng.integers(d)), int(rng.integers(d_ff)))]
    got = oracle.backward_entries(x, Wg, W1, W3, W2, dy, K, entries, forced=forced, eps=eps)
    want = np.array([ref[name][e, r, c] for (name, e, r, c) in entries])
    assert np.abs(want).max() > 1e-3
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)
