"""Comparison of the GPU layer with the fp64 oracle.

Rules (the error bars are those stated for this layer: expert indices exact
wherever the gap between the K-th and (K+1)-th logit exceeds 1e-3; bf16
storage with fp32 accumulation within 2e-2 relative L2; fp32 within 1e-5):

* Routing, on every token.  With the oracle's fp64 logits sorted,
  gap_K = l_(K) - l_(K+1).  If gap_K > TAU the GPU's expert set must equal the
  oracle's, and in the same slot order where every gap inside the top K also
  exceeds TAU.  Otherwise (a near tie) several sets are correct: the GPU's set
  must be one of them, i.e. every chosen logit is within TAU of every logit
  left out.
* Outputs, on the compared tokens.  The expected row is the oracle's output
  for the expert set the GPU chose when that set is a correct one; the
  oracle computes every correct set itself (sets come from the oracle's own
  logits, never from the GPU).  rel_L2 = ||y_gpu - y_ref|| / ||y_ref|| over
  all compared elements.
"""
from __future__ import annotations

import itertools

import numpy as np
import torch

TAU = 1e-3
TOL_BF16 = 2e-2
TOL_F32 = 1e-5
# Bound on each row's own error, |y_gpu - y_ref| over max(|y_ref|, median row
# norm): a few times the whole-output bound, far below the ~1 that a row
# computed from the wrong token or expert gives.
ROW_TOL_BF16 = 5e-2
ROW_TOL_F32 = 1e-4


def tol_for(dtype) -> float:
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def row_tol_for(dtype) -> float:
    return ROW_TOL_F32 if dtype == torch.float32 else ROW_TOL_BF16


def row_errors(y_gpu, y_ref) -> np.ndarray:
    """Per-row error |y_gpu - y_ref| / max(|y_ref|, median row norm)."""
    a = np.asarray(y_gpu, dtype=np.float64)
    b = np.asarray(y_ref, dtype=np.float64)
    rn = np.linalg.norm(b, axis=1)
    floor = max(float(np.median(rn)), 1e-300) if rn.size else 1.0
    return np.linalg.norm(a - b, axis=1) / np.maximum(rn, floor)


def valid_sets(logits_row: np.ndarray, K: int, tau: float = TAU):
    """Every K-set S with min(l_S) >= max(l_notS) - tau (all correct TopK
    choices within the tie tolerance), sorted by index."""
    n = logits_row.shape[0]
    if K == n:
        return [tuple(range(n))]
    order = np.argsort(-logits_row, kind="stable")
    kth = logits_row[order[K - 1]]
    # candidates: everything within tau of the K-th value, plus all above it
    cand = [i for i in range(n) if logits_row[i] >= kth - tau]
    out = []
    for S in itertools.combinations(sorted(cand), K):
        rest = [j for j in range(n) if j not in S]
        if min(logits_row[list(S)]) >= max(logits_row[rest]) - tau:
            out.append(tuple(S))
    return out


def routing_report(gpu_idx, gpu_gate, orc_logits, orc_idx, orc_gate, K, tau=TAU):
    """Check the GPU routing of every token against the oracle's.  Returns a
    dict; 'bad' lists tokens that break the rule."""
    gi = np.asarray(gpu_idx)
    gg = np.asarray(gpu_gate, dtype=np.float64)
    T, n = orc_logits.shape
    srt = -np.sort(-orc_logits, axis=1)
    gapK = srt[:, K - 1] - srt[:, K] if K < n else np.full(T, np.inf)
    inner = np.min(srt[:, :K - 1] - srt[:, 1:K], axis=1) if K > 1 else np.full(T, np.inf)
    bad, near = [], 0
    gate_err = 0.0
    for t in range(T):
        gset, oset = set(gi[t].tolist()), set(orc_idx[t].tolist())
        if len(gset) != K or not all(0 <= e < n for e in gset):
            bad.append(t)
            continue
        if gapK[t] > tau:
            if gset != oset:
                bad.append(t)
                continue
            if inner[t] > tau and not np.array_equal(gi[t], orc_idx[t]):
                bad.append(t)
                continue
            # gates, matched by expert
            og = dict(zip(orc_idx[t].tolist(), orc_gate[t].tolist()))
            gate_err = max(gate_err, max(abs(gg[t, j] - og[gi[t, j]]) for j in range(K)))
        else:
            near += 1
            if tuple(sorted(gset)) not in valid_sets(orc_logits[t], K, tau):
                bad.append(t)
    return {"bad": bad, "near_ties": near, "gate_max_abs_err": gate_err}


def expected_outputs(oracle_fn, rows, gpu_idx_rows, K, **kw):
    """Oracle outputs for `rows`, using for each row the correct expert set
    that matches the GPU's choice (the oracle's own choice where the GPU's is
    not a correct one, which then fails the comparison).

    oracle_fn(rows=..., forced=...) -> (y, idx, gate, logits)."""
    rows = np.asarray(rows, dtype=np.int64)
    y, idx, gate, logits = oracle_fn(rows=rows, forced=None)
    gsets = [tuple(sorted(np.asarray(r).tolist())) for r in gpu_idx_rows]
    alt_rows, alt_sets, alt_pos = [], [], []
    for p, r in enumerate(rows):
        if gsets[p] == tuple(sorted(idx[p].tolist())):
            continue
        for S in valid_sets(logits[p], K):
            if S == gsets[p]:
                alt_rows.append(r)
                alt_sets.append(S)
                alt_pos.append(p)
    if alt_rows:
        ya, _, _, _ = oracle_fn(rows=np.asarray(alt_rows), forced=np.asarray(alt_sets,
                                                                             dtype=np.int32))
        for q, p in enumerate(alt_pos):
            y[p] = ya[q]
    return y, len(alt_rows)


def rel_l2(y_gpu, y_ref) -> float:
    a = np.asarray(y_gpu, dtype=np.float64)
    b = np.asarray(y_ref, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy()
