"""Reference oracle for the sparse top-K mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  This package wraps ``liboracle.so`` (built from
``oracle.c``, plain fp64 C with OpenMP over tokens).  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it.  It shares
no code with the GPU library and the GPU library never calls it.

What it computes, and from which passages of the pages on "Mixtral of Experts":

* ``route``: logits l = x . W_g, TopK (ties to the lower expert index), softmax
  over the kept logits -- the gating equation in the xyznot digest, section
  "Method (with core equations)".
* ``forward``: y = sum_i G(x)_i SwiGLU_i(x) -- the output equation of the same
  section, with SwiGLU_i(u) = W2_i (SiLU(W1_i u) * W3_i u) (Swish plus
  elementwise product, "Key terms" of the same page).
* ``block_forward`` / ``block_route``: a layer of the stack workload,
  y = x + MoE(x / sqrt(mean(x^2) + eps)).  This pre-normalisation and residual
  are not on the pages; they define the 32-layer stack workload.

Inputs are float32 arrays (bf16 values widen exactly); all arithmetic is fp64.
Storage: x[T][d], W_g[d][n], W1/W3[n][d_ff][d], W2[n][d][d_ff].

Every function here is pinned by the CPU tests in ``tests/test_oracle_pins.py``
(closed forms, library special cases, brute force, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP).  Always recompiles."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    D = ctypes.c_double
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_route.restype = ctypes.c_int
    lib.oracle_route.argtypes = [P, P, I64, I64, I32, I32, P, P, P]
    lib.oracle_block_route.restype = ctypes.c_int
    lib.oracle_block_route.argtypes = [P, P, I64, I64, I32, I32, D, P, P, P]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [P, P, P, P, P, I64, I64, I64, I32, I32,
                                   P, I64, P, P, P, P, P]
    lib.oracle_block_forward.restype = ctypes.c_int
    lib.oracle_block_forward.argtypes = [P, P, P, P, P, I64, I64, I64, I32, I32, D,
                                         P, I64, P, P, P, P, P]
    lib.oracle_backward.restype = ctypes.c_int
    lib.oracle_backward.argtypes = [P, P, P, P, P, P, I64, I64, I64, I32, I32,
                                    P, I64, P, P, P, P, P, P]
    lib.oracle_backward_entries.restype = ctypes.c_int
    lib.oracle_backward_entries.argtypes = [P, P, P, P, P, P, I64, I64, I64, I32, I32, P,
                                            I64, P, P, P, P, P]
    lib.oracle_block_backward.restype = ctypes.c_int
    lib.oracle_block_backward.argtypes = [P, P, P, P, P, P, I64, I64, I64, I32, I32, D,
                                          P, I64, P, P, P, P, P, P]
    lib.oracle_block_backward_entries.restype = ctypes.c_int
    lib.oracle_block_backward_entries.argtypes = [P, P, P, P, P, P, I64, I64, I64, I32, I32,
                                                  D, P, I64, P, P, P, P, P]
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    """Accept a numpy array or a torch tensor (any device/dtype that widens
    exactly to float32: float32, bfloat16, float16) and return a C-contiguous
    float32 numpy array."""
    if hasattr(a, "detach"):  # torch tensor
        import torch
        t = a.detach()
        if t.dtype not in (torch.float32, torch.bfloat16, torch.float16):
            raise TypeError(f"oracle input dtype {t.dtype} does not widen exactly")
        a = t.to(device="cpu", dtype=torch.float32).contiguous().numpy()
    a = np.asarray(a)
    if a.dtype != np.float32:
        if a.dtype not in (np.float16,):
            raise TypeError(f"oracle input dtype {a.dtype} must be float32")
        a = a.astype(np.float32)
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle runs on (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())


def route(x, Wg, K: int):
    """Router of the layer on every token: (logits[T][n] f64, idx[T][K] i32,
    gate[T][K] f64).  Slot 0 is the largest logit; ties go to the lower index."""
    x = _f32(x)
    Wg = _f32(Wg)
    T, d = x.shape
    d2, n = Wg.shape
    assert d2 == d
    logits = np.empty((T, n), np.float64)
    idx = np.empty((T, K), np.int32)
    gate = np.empty((T, K), np.float64)
    rc = _load().oracle_route(_ptr(x), _ptr(Wg), T, d, n, K, _ptr(logits), _ptr(idx),
                              _ptr(gate))
    if rc != 0:
        raise ValueError(f"oracle_route rejected the sizes (rc={rc})")
    return logits, idx, gate


def block_route(x, Wg, K: int, eps: float):
    """Routing of a stack layer, i.e. of x / sqrt(mean(x^2) + eps)."""
    x = _f32(x)
    Wg = _f32(Wg)
    T, d = x.shape
    d2, n = Wg.shape
    assert d2 == d
    logits = np.empty((T, n), np.float64)
    idx = np.empty((T, K), np.int32)
    gate = np.empty((T, K), np.float64)
    rc = _load().oracle_block_route(_ptr(x), _ptr(Wg), T, d, n, K, float(eps),
                                    _ptr(logits), _ptr(idx), _ptr(gate))
    if rc != 0:
        raise ValueError(f"oracle_block_route rejected the sizes (rc={rc})")
    return logits, idx, gate


def _layer(fn_name, x, Wg, W1, W3, W2, K, rows, forced, eps=None):
    x = _f32(x)
    Wg = _f32(Wg)
    W1 = _f32(W1)
    W3 = _f32(W3)
    W2 = _f32(W2)
    T, d = x.shape
    n = Wg.shape[1]
    d_ff = W1.shape[1]
    assert Wg.shape == (d, n)
    assert W1.shape == (n, d_ff, d) and W3.shape == (n, d_ff, d)
    assert W2.shape == (n, d, d_ff)
    rows_a = None
    R = T
    if rows is not None:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R = rows_a.shape[0]
        if R and (rows_a.min() < 0 or rows_a.max() >= T):
            raise IndexError("row outside [0, T)")
    forced_a = None
    if forced is not None:
        forced_a = np.ascontiguousarray(np.asarray(forced, dtype=np.int32))
        assert forced_a.shape == (R, K)
        if forced_a.size and (forced_a.min() < 0 or forced_a.max() >= n):
            raise IndexError("forced expert outside [0, n)")
    y = np.empty((R, d), np.float64)
    idx = np.empty((R, K), np.int32)
    gate = np.empty((R, K), np.float64)
    logits = np.empty((R, n), np.float64)
    lib = _load()
    args = [_ptr(x), _ptr(Wg), _ptr(W1), _ptr(W3), _ptr(W2), T, d, d_ff, n, K]
    if eps is not None:
        args.append(float(eps))
    args += [_ptr(rows_a), R, _ptr(forced_a), _ptr(y), _ptr(idx), _ptr(gate),
             _ptr(logits)]
    rc = getattr(lib, fn_name)(*args)
    if rc != 0:
        raise ValueError(f"{fn_name} failed (rc={rc})")
    return y, idx, gate, logits


def forward(x, Wg, W1, W3, W2, K: int, rows=None, forced=None):
    """The layer on the tokens ``rows`` (all when None).  Returns
    (y[R][d], idx[R][K], gate[R][K], logits[R][n]), all fp64 / int32.
    ``forced`` ([R][K] expert ids) replaces the TopK choice."""
    return _layer("oracle_forward", x, Wg, W1, W3, W2, K, rows, forced)


def block_forward(x, Wg, W1, W3, W2, K: int, eps: float, rows=None, forced=None):
    """A stack layer y = x + MoE(RMSNorm(x)) on the tokens ``rows``."""
    return _layer("oracle_block_forward", x, Wg, W1, W3, W2, K, rows, forced, eps)


def backward(x, Wg, W1, W3, W2, dy, K: int, rows=None, forced=None, weights: bool = True):
    """Gradients of L = sum_t dy_t . y_t (fp64).  Returns a dict with dx[R][d]
    (tokens ``rows``, all when None) and -- when ``weights`` and rows is None --
    dWg[d][n], dW1[n][d_ff][d], dW3[n][d_ff][d], dW2[n][d][d_ff]."""
    return _backward(None, x, Wg, W1, W3, W2, dy, K, rows, forced, weights)


def block_backward(x, Wg, W1, W3, W2, dy, K: int, eps: float, rows=None, forced=None,
                   weights: bool = True):
    """Gradients of L = sum_t dy_t . y_t for the stack layer
    y = x + MoE(RMSNorm(x)) (fp64); same outputs as backward()."""
    return _backward(float(eps), x, Wg, W1, W3, W2, dy, K, rows, forced, weights)


def _backward(eps, x, Wg, W1, W3, W2, dy, K, rows, forced, weights):
    x = _f32(x)
    Wg = _f32(Wg)
    W1 = _f32(W1)
    W3 = _f32(W3)
    W2 = _f32(W2)
    dy = _f32(dy)
    T, d = x.shape
    n = Wg.shape[1]
    d_ff = W1.shape[1]
    assert dy.shape == (T, d)
    assert Wg.shape == (d, n)
    assert W1.shape == (n, d_ff, d) and W3.shape == (n, d_ff, d)
    assert W2.shape == (n, d, d_ff)
    rows_a = None
    R = T
    if rows is not None:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        R = rows_a.shape[0]
        weights = False
    forced_a = None
    if forced is not None:
        forced_a = np.ascontiguousarray(np.asarray(forced, dtype=np.int32))
        assert forced_a.shape == (R, K)
    out = {"dx": np.empty((R, d), np.float64)}
    if weights:
        out["dWg"] = np.empty((d, n), np.float64)
        out["dW1"] = np.empty((n, d_ff, d), np.float64)
        out["dW3"] = np.empty((n, d_ff, d), np.float64)
        out["dW2"] = np.empty((n, d, d_ff), np.float64)
    lib = _load()
    grads = (_ptr(out["dx"]), _ptr(out.get("dWg")), _ptr(out.get("dW1")),
             _ptr(out.get("dW3")), _ptr(out.get("dW2")))
    ins = (_ptr(x), _ptr(Wg), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(dy), T, d, d_ff, n, K)
    if eps is None:
        rc = lib.oracle_backward(*ins, _ptr(rows_a), R, _ptr(forced_a), *grads)
    else:
        rc = lib.oracle_block_backward(*ins, eps, _ptr(rows_a), R, _ptr(forced_a), *grads)
    if rc != 0:
        raise ValueError(f"oracle backward failed (rc={rc})")
    return out


_WHICH = {"dW1": 1, "dW2": 2, "dW3": 3}


def backward_entries(x, Wg, W1, W3, W2, dy, K: int, entries, forced=None,
                     eps: float | None = None) -> np.ndarray:
    """Selected expert weight-gradient entries (fp64), each summed over all the
    tokens routed to its expert.  ``entries``: sequence of (name, e, row, col)
    with name in dW1 / dW2 / dW3 and (row, col) indices of that matrix of
    expert e.  ``forced`` ([T][K]) replaces TopK.  ``eps``: the stack layer
    (experts and router see RMSNorm(x))."""
    x = _f32(x)
    Wg = _f32(Wg)
    W1 = _f32(W1)
    W3 = _f32(W3)
    W2 = _f32(W2)
    dy = _f32(dy)
    T, d = x.shape
    n = Wg.shape[1]
    d_ff = W1.shape[1]
    Q = len(entries)
    which = np.ascontiguousarray([_WHICH[q[0]] for q in entries], dtype=np.int32)
    ex = np.ascontiguousarray([q[1] for q in entries], dtype=np.int32)
    ri = np.ascontiguousarray([q[2] for q in entries], dtype=np.int64)
    ci = np.ascontiguousarray([q[3] for q in entries], dtype=np.int64)
    forced_a = None
    if forced is not None:
        forced_a = np.ascontiguousarray(np.asarray(forced, dtype=np.int32))
        assert forced_a.shape == (T, K)
    out = np.empty(max(Q, 1), np.float64)
    lib = _load()
    ins = (_ptr(x), _ptr(Wg), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(dy), T, d, d_ff, n, K)
    sel = (_ptr(forced_a), Q, _ptr(which), _ptr(ex), _ptr(ri), _ptr(ci), _ptr(out))
    if eps is None:
        rc = lib.oracle_backward_entries(*ins, *sel)
    else:
        rc = lib.oracle_block_backward_entries(*ins, float(eps), *sel)
    if rc != 0:
        raise ValueError(f"oracle_backward_entries failed (rc={rc})")
    return out[:Q]
