"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: torch device tensors become raw pointers, the
current torch stream becomes the hipStream_t, and every step of the layer runs
in the library's HIP kernels.  There is no fallback: if libmoe.so is missing
or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4
MOE_F32 = 0
MOE_BF16 = 1
MOE_GEMM_AUTO = 0
MOE_GEMM_TILED = 1
MOE_GEMM_STREAM = 2

EXPORTS = ("moe_abi_version", "moe_route", "moe_permute", "moe_workspace_bytes",
           "moe_forward", "moe_block_forward", "moe_set_stage_events", "moe_status_string",
           "moe_last_error", "moe_backward", "moe_backward_workspace_bytes",
           "moe_saved_bytes", "moe_forward_train", "moe_backward_saved",
           "moe_block_backward", "moe_block_forward_train", "moe_block_backward_saved",
           "moe_set_gemm_path", "moe_forward_noalloc")
STAGES = {"router": 0, "permute": 1, "gate_up": 2, "down": 3, "combine": 4,
          "bwd_recompute": 5, "bwd_dh": 6, "bwd_dx": 7, "bwd_wgrad": 8}


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {detail}")


_lib = None


def load(path: str | None = None):
    """Load libmoe.so (once).  Raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m sparse_mixture_experts_14_amd.build`")
    lib = ctypes.CDLL(p)
    V, I64, I32, SZ, F = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t,
                          ctypes.c_float)
    lib.moe_abi_version.restype = I32
    lib.moe_abi_version.argtypes = []
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route.argtypes = [V, V, I64, I64, I32, I32, ctypes.c_int, V, V, V]
    lib.moe_permute.restype = ctypes.c_int
    lib.moe_permute.argtypes = [V, I64, I32, I32, V, V, V, V]
    lib.moe_workspace_bytes.restype = SZ
    lib.moe_workspace_bytes.argtypes = [I64, I64, I64, I32, I32, ctypes.c_int]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward.argtypes = [V, V, V, V, V, I64, I64, I64, I32, I32, ctypes.c_int, V, V, SZ,
                                V, V, V, V]
    lib.moe_set_stage_events.restype = ctypes.c_int
    lib.moe_set_stage_events.argtypes = [I32, V, V]
    lib.moe_set_gemm_path.restype = ctypes.c_int
    lib.moe_set_gemm_path.argtypes = [I32]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [V, V, V, V, V, I64, I64, I64, I32, I32, ctypes.c_int,
                                        V, V, V, V, V]
    lib.moe_block_forward.restype = ctypes.c_int
    lib.moe_block_forward.argtypes = [V, V, V, V, V, I64, I64, I64, I32, I32, ctypes.c_int, F,
                                      V, V, SZ, V, V, V, V]
    lib.moe_backward_workspace_bytes.restype = SZ
    lib.moe_backward_workspace_bytes.argtypes = [I64, I64, I64, I32, I32, ctypes.c_int]
    lib.moe_backward.restype = ctypes.c_int
    lib.moe_backward.argtypes = [V, V, V, V, V, V, I64, I64, I64, I32, I32, ctypes.c_int, V, V,
                                 V, V, V, V, SZ, V]
    lib.moe_saved_bytes.restype = SZ
    lib.moe_saved_bytes.argtypes = [I64, I64, I64, I32, I32, ctypes.c_int]
    lib.moe_forward_train.restype = ctypes.c_int
    lib.moe_forward_train.argtypes = [V, V, V, V, V, I64, I64, I64, I32, I32, ctypes.c_int, V,
                                      V, SZ, V, SZ, V]
    lib.moe_backward_saved.restype = ctypes.c_int
    lib.moe_backward_saved.argtypes = [V, V, V, V, V, V, V, SZ, I64, I64, I64, I32, I32,
                                       ctypes.c_int, V, V, V, V, V, V, SZ, V]
    lib.moe_block_forward_train.restype = ctypes.c_int
    lib.moe_block_forward_train.argtypes = [V, V, V, V, V, I64, I64, I64, I32, I32,
                                            ctypes.c_int, F, V, V, SZ, V, SZ, V]
    lib.moe_block_backward_saved.restype = ctypes.c_int
    lib.moe_block_backward_saved.argtypes = [V, V, V, V, V, V, V, SZ, I64, I64, I64, I32, I32,
                                             ctypes.c_int, F, V, V, V, V, V, V, SZ, V]
    lib.moe_block_backward.restype = ctypes.c_int
    lib.moe_block_backward.argtypes = [V, V, V, V, V, V, I64, I64, I64, I32, I32, ctypes.c_int,
                                       F, V, V, V, V, V, V, SZ, V]
    if path is None:
        _lib = lib
    return lib


def _check(st: int, fn: str):
    if st != MOE_OK:
        lib = load()
        raise MoeError(st, fn, lib.moe_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def set_stage_events_raw(stage: str, start: int | None = None, end: int | None = None):
    """Record the hipEvent_t handles (start, end) around `stage` in later layer
    calls on this thread; no handles clears the hook."""
    _check(load().moe_set_stage_events(STAGES[stage], start, end), "moe_set_stage_events")


GEMM_PATHS = {None: MOE_GEMM_AUTO, "auto": MOE_GEMM_AUTO, "tiled": MOE_GEMM_TILED,
              "skinny": MOE_GEMM_STREAM, "stream": MOE_GEMM_STREAM}


def set_gemm_path(path: str | None):
    """Testing hook: later layer calls on this thread use the named bf16 GEMM
    family ("tiled", "stream"/"skinny"; None or "auto" = chosen by size)."""
    _check(load().moe_set_gemm_path(GEMM_PATHS[path]), "moe_set_gemm_path")


def workspace_bytes(T: int, d: int, d_ff: int, n: int, K: int, dtype: torch.dtype) -> int:
    code = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    return int(load().moe_workspace_bytes(T, d, d_ff, n, K, code))


def route(x: torch.Tensor, Wg: torch.Tensor, K: int):
    """(idx[T][K] int32, gate[T][K] float32) of the router on every token."""
    T, d = x.shape
    n = Wg.shape[1]
    if Wg.shape[0] != d or Wg.dtype != x.dtype:
        raise ValueError("W_g must be [d][n] with the dtype of x")
    idx = torch.empty(T, K, dtype=torch.int32, device=x.device)
    gate = torch.empty(T, K, dtype=torch.float32, device=x.device)
    st = load().moe_route(_dev(x, "x"), _dev(Wg, "W_g"), T, d, n, K, _dtype_code(x),
                          idx.data_ptr(), gate.data_ptr(), _stream(x.device))
    _check(st, "moe_route")
    return idx, gate


def permute(idx: torch.Tensor, n: int):
    """(offsets[n+1], perm[T*K], inv[T*K]) of the stable counting sort."""
    T, K = idx.shape
    if idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    offsets = torch.empty(n + 1, dtype=torch.int32, device=idx.device)
    perm = torch.empty(T * K, dtype=torch.int32, device=idx.device)
    inv = torch.empty(T * K, dtype=torch.int32, device=idx.device)
    st = load().moe_permute(_dev(idx, "idx"), T, n, K, offsets.data_ptr(), perm.data_ptr(),
                            inv.data_ptr(), _stream(idx.device))
    _check(st, "moe_permute")
    return offsets, perm, inv


class Layer:
    """A reusable call site: owns the workspace for one (T, d, d_ff, n, K,
    dtype) and the optional routing outputs."""

    def __init__(self, T, d, d_ff, n, K, dtype, device, routing_outputs=True):
        self.T, self.d, self.d_ff, self.n, self.K = T, d, d_ff, n, K
        self.dtype = dtype
        self.device = torch.device(device)
        nbytes = workspace_bytes(T, d, d_ff, n, K, dtype)
        if nbytes == 0 and T > 0:
            raise ValueError("invalid layer sizes")
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        self.ws_bytes = nbytes
        if routing_outputs:
            self.idx = torch.empty(T, K, dtype=torch.int32, device=self.device)
            self.gate = torch.empty(T, K, dtype=torch.float32, device=self.device)
            self.counts = torch.empty(n, dtype=torch.int32, device=self.device)
        else:
            self.idx = self.gate = self.counts = None

    def _args(self, x, Wg, W1, W3, W2):
        T, d, d_ff, n, K = self.T, self.d, self.d_ff, self.n, self.K
        if x.shape != (T, d) or Wg.shape != (d, n) or W1.shape != (n, d_ff, d) \
                or W3.shape != (n, d_ff, d) or W2.shape != (n, d, d_ff):
            raise ValueError("tensor shapes do not match the layer sizes")
        for t in (Wg, W1, W3, W2):
            if t.dtype != x.dtype:
                raise ValueError("all inputs must share one dtype")
        if x.dtype != self.dtype:
            raise ValueError("dtype differs from the layer's")
        return (_dev(x, "x"), _dev(Wg, "W_g"), _dev(W1, "W1"), _dev(W3, "W3"), _dev(W2, "W2"))

    def forward(self, x, Wg, W1, W3, W2, out=None):
        y = out if out is not None else torch.empty_like(x)
        px = self._args(x, Wg, W1, W3, W2)
        st = load().moe_forward(*px, self.T, self.d, self.d_ff, self.n, self.K,
                                _dtype_code(x), _dev(y, "y"), self.workspace.data_ptr(),
                                self.ws_bytes, _ptr(self.idx), _ptr(self.gate),
                                _ptr(self.counts), _stream(x.device))
        _check(st, "moe_forward")
        return y

    def block_forward(self, x, Wg, W1, W3, W2, eps, out=None):
        y = out if out is not None else torch.empty_like(x)
        px = self._args(x, Wg, W1, W3, W2)
        st = load().moe_block_forward(*px, self.T, self.d, self.d_ff, self.n, self.K,
                                      _dtype_code(x), float(eps), _dev(y, "y"),
                                      self.workspace.data_ptr(), self.ws_bytes, _ptr(self.idx),
                                      _ptr(self.gate), _ptr(self.counts), _stream(x.device))
        _check(st, "moe_block_forward")
        return y


def forward(x, Wg, W1, W3, W2, K: int):
    """y of the layer; returns (y, idx, gate, counts)."""
    n, d_ff, d = W1.shape
    L = Layer(x.shape[0], d, d_ff, n, K, x.dtype, x.device)
    y = L.forward(x, Wg, W1, W3, W2)
    return y, L.idx, L.gate, L.counts


def forward_noalloc(x, Wg, W1, W3, W2, K: int, y, idx=None, gate=None, counts=None):
    """moe_forward_noalloc: the layer into the caller's y (and the optional
    routing outputs) with the library's static scratch instead of a
    workspace; allocates nothing."""
    n, d_ff, d = W1.shape
    L = Layer.__new__(Layer)
    L.T, L.d, L.d_ff, L.n, L.K, L.dtype = x.shape[0], d, d_ff, n, K, x.dtype
    px = L._args(x, Wg, W1, W3, W2)
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("y must match x in shape and dtype")
    st = load().moe_forward_noalloc(*px, L.T, d, d_ff, n, K, _dtype_code(x), _dev(y, "y"),
                                    _ptr(idx), _ptr(gate), _ptr(counts), _stream(x.device))
    _check(st, "moe_forward_noalloc")
    return y


def block_forward(x, Wg, W1, W3, W2, K: int, eps: float):
    """y = x + MoE(RMSNorm(x)); returns (y, idx, gate, counts)."""
    n, d_ff, d = W1.shape
    L = Layer(x.shape[0], d, d_ff, n, K, x.dtype, x.device)
    y = L.block_forward(x, Wg, W1, W3, W2, eps)
    return y, L.idx, L.gate, L.counts


def backward_workspace_bytes(T: int, d: int, d_ff: int, n: int, K: int,
                             dtype: torch.dtype) -> int:
    code = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    return int(load().moe_backward_workspace_bytes(T, d, d_ff, n, K, code))


def saved_bytes(T: int, d: int, d_ff: int, n: int, K: int, dtype: torch.dtype) -> int:
    code = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    return int(load().moe_saved_bytes(T, d, d_ff, n, K, code))


def forward_train(x, Wg, W1, W3, W2, K: int, out=None, saved=None,
                  workspace: torch.Tensor | None = None, eps: float | None = None):
    """y of the layer (bf16) plus the saved state for backward(..., saved=):
    returns (y, saved) where saved is a uint8 device tensor.  ``eps``: the
    stack layer y = x + MoE(RMSNorm(x)) (then backward needs the same eps)."""
    T, d = x.shape
    n, d_ff, _ = W1.shape
    nbytes = saved_bytes(T, d, d_ff, n, K, x.dtype)
    if nbytes == 0:
        raise ValueError("invalid sizes or dtype for forward_train (bf16 only)")
    if saved is None:
        saved = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    if saved.numel() < nbytes:
        raise ValueError("saved buffer too small")
    y = out if out is not None else torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(T, d, d_ff, n, K, x.dtype), 256),
                                dtype=torch.uint8, device=x.device)
    L = Layer.__new__(Layer)
    L.T, L.d, L.d_ff, L.n, L.K, L.dtype = T, d, d_ff, n, K, x.dtype
    px = L._args(x, Wg, W1, W3, W2)
    if eps is None:
        st = load().moe_forward_train(*px, T, d, d_ff, n, K, _dtype_code(x), _dev(y, "y"),
                                      saved.data_ptr(), saved.numel(), workspace.data_ptr(),
                                      workspace.numel(), _stream(x.device))
        _check(st, "moe_forward_train")
    else:
        st = load().moe_block_forward_train(*px, T, d, d_ff, n, K, _dtype_code(x), float(eps),
                                            _dev(y, "y"), saved.data_ptr(), saved.numel(),
                                            workspace.data_ptr(), workspace.numel(),
                                            _stream(x.device))
        _check(st, "moe_block_forward_train")
    return y, saved


def block_backward(x, Wg, W1, W3, W2, dy, K: int, eps: float,
                   workspace: torch.Tensor | None = None, out: dict | None = None,
                   saved: torch.Tensor | None = None):
    """Gradients of sum(dy * y) for the stack layer y = x + MoE(RMSNorm(x))
    (bf16): the same dict as backward()."""
    return backward(x, Wg, W1, W3, W2, dy, K, workspace=workspace, out=out, saved=saved,
                    eps=eps)


def backward(x, Wg, W1, W3, W2, dy, K: int, workspace: torch.Tensor | None = None,
             out: dict | None = None, saved: torch.Tensor | None = None,
             eps: float | None = None):
    """Gradients of sum(dy * y) for bf16 inputs: a dict of dx (bf16 [T][d]) and
    dWg, dW1, dW3, dW2 (float32, in the layouts of W_g, W1, W3, W2).  ``out``
    (such a dict from an earlier call of the same sizes) is overwritten and
    returned instead of new tensors.  ``saved`` (from forward_train on the same
    inputs) replaces the recomputation of the routing and pre-activations."""
    T, d = x.shape
    n, d_ff, _ = W1.shape
    if Wg.shape != (d, n) or W1.shape != (n, d_ff, d) or W3.shape != (n, d_ff, d) \
            or W2.shape != (n, d, d_ff) or dy.shape != (T, d):
        raise ValueError("tensor shapes do not match the layer sizes")
    for t in (Wg, W1, W3, W2, dy):
        if t.dtype != x.dtype:
            raise ValueError("all inputs must share one dtype")
    nbytes = backward_workspace_bytes(T, d, d_ff, n, K, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x.device)
    if workspace.numel() < nbytes:
        raise ValueError("workspace too small")
    dev = x.device
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = {"dx": torch.empty_like(x), "dWg": torch.empty(d, n, **f32),
               "dW1": torch.empty(n, d_ff, d, **f32), "dW3": torch.empty(n, d_ff, d, **f32),
               "dW2": torch.empty(n, d, d_ff, **f32)}
    shapes = {"dx": (x.dtype, (T, d)), "dWg": (torch.float32, (d, n)),
              "dW1": (torch.float32, (n, d_ff, d)), "dW3": (torch.float32, (n, d_ff, d)),
              "dW2": (torch.float32, (n, d, d_ff))}
    for k, (dt, shp) in shapes.items():
        if out[k].dtype != dt or tuple(out[k].shape) != shp:
            raise ValueError(f"out[{k!r}] must be {dt} of shape {shp}")
    dx, dwg, dw1, dw3, dw2 = (out[k] for k in ("dx", "dWg", "dW1", "dW3", "dW2"))
    grads = (_dev(dx, "dx"), _dev(dwg, "dW_g"), _dev(dw1, "dW1"), _dev(dw3, "dW3"),
             _dev(dw2, "dW2"))
    ins = (_dev(x, "x"), _dev(Wg, "W_g"), _dev(W1, "W1"), _dev(W3, "W3"), _dev(W2, "W2"),
           _dev(dy, "dy"))
    if eps is not None and saved is not None:
        st = load().moe_block_backward_saved(*ins, _dev(saved, "saved"), saved.numel(), T, d,
                                             d_ff, n, K, _dtype_code(x), float(eps), *grads,
                                             workspace.data_ptr(), workspace.numel(),
                                             _stream(dev))
        _check(st, "moe_block_backward_saved")
    elif eps is not None:
        st = load().moe_block_backward(*ins, T, d, d_ff, n, K, _dtype_code(x), float(eps),
                                       *grads, workspace.data_ptr(), workspace.numel(),
                                       _stream(dev))
        _check(st, "moe_block_backward")
    elif saved is not None:
        st = load().moe_backward_saved(*ins, _dev(saved, "saved"), saved.numel(), T, d, d_ff,
                                       n, K, _dtype_code(x), *grads, workspace.data_ptr(),
                                       workspace.numel(), _stream(dev))
        _check(st, "moe_backward_saved")
    else:
        st = load().moe_backward(*ins, T, d, d_ff, n, K, _dtype_code(x), *grads,
                                 workspace.data_ptr(), workspace.numel(), _stream(dev))
        _check(st, "moe_backward")
    return out
