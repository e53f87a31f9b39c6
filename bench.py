#!/usr/bin/env python3
"""Throughput of the MoE layer (top-2 of 8 SwiGLU experts, d = 4096) on one
MI355X, with the roofline of its dominant kernel and the fp64 oracle's CPU
throughput beside it.

One step = one pass of the whole layer (router, permutation, gate/up GEMM,
down GEMM, combine) over the workload's synthetic batch, inputs resident in
HBM.  Default workload: the stack, 32 independent layers
y = x + MoE(RMSNorm(x)) at Mixtral shape (T = 2048 tokens, d = 4096,
d_ff = 14336, n = 8, K = 2, bf16, 90 GB of expert weights resident), the
largest configuration; one step carries the tokens through all 32 layers.
The other workloads (decode T = 16, prefill T = 4096, skewed routing
T = 16384, tiny fp32) are selected with --workload.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload stack|decode|prefill|skew|tiny]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (top-2 of 8 SwiGLU, d=4096) + % HBM / MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
F32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "sparse_mixture_experts_14_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvent:
    """A raw hipEvent_t (the library records it on the stream it launches
    on; torch.cuda.Event only knows about records made through torch)."""
    _hip = None

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._c = ctypes
        self.handle = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreate(ctypes.byref(self.handle)) != 0:
            raise RuntimeError("hipEventCreate failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = self._c.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(self._c.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if HipEvent._hip is not None and self.handle:
            HipEvent._hip.hipEventDestroy(self.handle)


def step_percentiles(marks) -> dict:
    """p10 / p50 / p90 of the per-step times between consecutive events."""
    import numpy as np
    per = np.array([a.elapsed_time(b) for a, b in zip(marks[:-1], marks[1:])])
    return {q: round(float(np.percentile(per, v)), 5)
            for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}


def kernel_source_sha(files) -> str:
    """Hash of the kernel sources with // comments and blank lines dropped
    (the sources hold no other comment form and no "//" inside a string), so
    that counters stay attached to the code they were taken on."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def dominant_kernel(w, skinny: bool):
    """The stage that moves the most bytes (decode) or does the most flops
    (the others): the gate/up grouped GEMM in every workload."""
    src = ["gemm_skinny.hip" if skinny else "gemm_bf16.hip", "common.hpp"]
    if w.dtype == "f32":
        src = ["gemm_f32.hip", "common.hpp"]
    return "gate_up", src


def algorithmic_work(w, counts):
    """Per launch of the gate/up kernel: bytes it must move (decode) and flops
    it must do.  Units: a touched expert's W1 and W3 (2 * d_ff * d elements),
    plus the gathered token rows read and the hidden rows written."""
    es = 2 if w.dtype == "bf16" else 4
    A = w.T * w.K
    touched = int(sum(1 for c in counts if c > 0))
    wbytes = touched * 2 * w.d_ff * w.d * es
    act = A * w.d * es + A * w.d_ff * es
    flops = 4.0 * A * w.d * w.d_ff
    return {"touched_experts": touched, "bytes": wbytes + act, "flops": flops}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, L, budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload's
    tokens (timing each oracle call; repeats until ~budget_s)."""
    import numpy as np

    import oracle
    H = {k: oracle._f32(v) for k, v in L.items()}
    eps = w.eps
    def run(rows):
        if eps is not None:
            return oracle.block_forward(H["x"], H["Wg"], H["W1"], H["W3"], H["W2"], w.K, eps,
                                        rows=rows)
        return oracle.forward(H["x"], H["Wg"], H["W1"], H["W3"], H["W2"], w.K, rows=rows)
    rng = np.random.default_rng(0)
    probe = np.sort(rng.choice(w.T, min(w.T, 16), replace=False))
    t0 = time.perf_counter()
    run(probe)
    per_tok = (time.perf_counter() - t0) / len(probe)
    reps, tokens, elapsed = 0, 0, 0.0
    # each call takes distinct tokens (at most all T), sized from the measured
    # per-token time to fill what is left of the budget
    while elapsed < 0.9 * budget_s or reps == 0:
        n_tok = max(1, int((budget_s - elapsed) / max(per_tok, 1e-9)))
        rows = np.sort(rng.choice(w.T, min(w.T, n_tok), replace=False))
        t0 = time.perf_counter()
        run(rows)
        dt = time.perf_counter() - t0
        elapsed += dt
        per_tok = dt / len(rows)
        tokens += len(rows)
        reps += 1
    if tokens == w.T * reps:
        sample = f"all {w.T} tokens of the workload x{reps}"
    else:
        sample = (f"{tokens} tokens in {reps} oracle call(s), each on distinct tokens drawn "
                  f"from the workload's {w.T}")
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": sample, "seconds": round(elapsed, 2),
            "cpu": cpu_model()}


def traffic_for(workload: str, src_sha: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None when there is none or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_sha") != src_sha:
        return None
    return t.get("bytes_per_launch")


# Substrings naming the gate/up kernel in a rocprofv3 counter file, and the
# plain copy kernel of the calibration run.
GATE_UP_KERNEL = {"skinny": "gemm_skinny_kernel<true", "tiled": "gemm_bf16_kernel<true"}
WGRAD_KERNEL = "gemm_wgrad_kernel"              # the backward's dominant kernel
WGRAD_SOURCES = ["gemm_bf16.hip", "common.hpp"]
COPY_KERNEL = "copy"
COPY_BYTES = 512 << 20


def copy_calibration():
    """A plain device copy of COPY_BYTES, five times: the reference kernel
    whose FETCH_SIZE / WRITE_SIZE counters scale the gate/up kernel's."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)


def _counter_mean_kib(csv_path: str, counter: str, name_part: str) -> float:
    """Mean over the matching dispatches (first one skipped when there are
    several) of a rocprofv3 derived counter, in KiB per dispatch."""
    import collections
    import csv
    per = collections.defaultdict(float)
    names = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or name_part not in r["Kernel_Name"]:
                continue
            k = int(r["Dispatch_Id"])
            per[k] += float(r["Counter_Value"])
            names[k] = r["Kernel_Name"]
    ks = sorted(per)
    if not ks:
        raise SystemExit(f"no {counter} for a kernel named *{name_part}* in {csv_path}")
    if len(ks) > 1:
        ks = ks[1:]
    return sum(per[k] for k in ks) / len(ks)


def write_traffic(workload: str, dirs, command: str, backward: bool = False):
    """profiles/traffic.json[workload] (or [workload-backward], for the
    weight-gradient product of the backward) from four rocprofv3 --pmc runs:
    the bench's FETCH_SIZE and WRITE_SIZE, then the copy calibration's."""
    from sparse_mixture_experts_14_amd import workloads as W
    w = W.WORKLOADS[workload]
    skinny = w.dtype == "bf16" and w.T * w.K <= 16 * w.n
    part = WGRAD_KERNEL if backward else GATE_UP_KERNEL["skinny" if skinny else "tiled"]
    f_k, w_k, cf_k, cw_k = (os.path.join(d, "run_counter_collection.csv") for d in dirs)
    fetch = _counter_mean_kib(f_k, "FETCH_SIZE", part) * 1024
    write = _counter_mean_kib(w_k, "WRITE_SIZE", part) * 1024
    cfetch = _counter_mean_kib(cf_k, "FETCH_SIZE", COPY_KERNEL) * 1024
    cwrite = _counter_mean_kib(cw_k, "WRITE_SIZE", COPY_KERNEL) * 1024
    fs, ws = COPY_BYTES / cfetch, COPY_BYTES / cwrite
    src = WGRAD_SOURCES if backward else dominant_kernel(w, skinny)[1]
    entry = {"source_sha": kernel_source_sha(src), "kernel": part,
             "bytes_per_launch": round(fetch * fs + write * ws),
             "fetch_bytes_raw": round(fetch), "write_bytes_raw": round(write),
             "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
             "copy_kernel_bytes": COPY_BYTES, "command": command}
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    key = workload + "-backward" if backward else workload
    data[key] = entry
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({key: entry}), flush=True)


def backward_cpu_baseline(w, L, dy, budget_s: float, train: bool = False, eps=None):
    """The fp64 oracle's backward (with train: its forward, then its backward;
    with eps: the stack layer's), as it stands, on the first tokens of the
    workload (x and dy rows; all weight gradients of that sub-batch),
    repeated until ~budget_s."""
    import oracle
    H = {k: oracle._f32(v) for k, v in L.items()}
    dyh = oracle._f32(dy)

    def run(m):
        if train and eps is not None:
            oracle.block_forward(H["x"][:m], H["Wg"], H["W1"], H["W3"], H["W2"], w.K, eps)
        elif train:
            oracle.forward(H["x"][:m], H["Wg"], H["W1"], H["W3"], H["W2"], w.K)
        if eps is not None:
            oracle.block_backward(H["x"][:m], H["Wg"], H["W1"], H["W3"], H["W2"], dyh[:m], w.K,
                                  eps)
        else:
            oracle.backward(H["x"][:m], H["Wg"], H["W1"], H["W3"], H["W2"], dyh[:m], w.K)

    t0 = time.perf_counter()
    run(1)
    per_tok = time.perf_counter() - t0
    m = int(min(w.T, max(1, budget_s / max(per_tok, 1e-9) / 2)))
    reps, tokens, elapsed = 0, 0, 0.0
    while elapsed < budget_s or reps == 0:
        t0 = time.perf_counter()
        run(m)
        elapsed += time.perf_counter() - t0
        tokens += m
        reps += 1
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{'forward and backward' if train else 'backward'} of the "
                      f"workload's first {m} tokens (x, dy rows; every gradient) x{reps}",
            "seconds": round(elapsed, 2), "cpu": cpu_model()}


def bench_backward(args, w, dev, train=False):
    """One step = one moe_backward call: routing and the forward pieces
    recomputed, dx and every weight gradient; or, with train, one training
    step: moe_forward_train (y and the saved state) then moe_backward_saved.
    The dominant kernel is the weight-gradient product (three launches per
    step, timed together)."""
    import torch

    import sparse_mixture_experts_14_amd as moe
    from sparse_mixture_experts_14_amd import workloads as W
    stack = w.name == "stack"
    if w.dtype != "bf16":
        raise SystemExit("--backward and --train run the bf16 workloads (the stack: one "
                         "layer)")
    log(f"[bench] {'training step' if train else 'backward'} workload={w.name} T={w.T} "
        f"building inputs on {dev}")
    if stack:  # the backward of layer 0 of the stack, on the stack's own input
        L = dict(W.make_stack_layer(w, 0, device=dev))
        L["x"] = W.make_stack_input(w, device=dev)
    else:
        L = W.make_layer(w, device=dev)
    eps = w.eps if stack else None
    g = torch.Generator(device=dev).manual_seed(w.seed + 7)
    dy = torch.randn(w.T, w.d, generator=g, device=dev).to(torch.bfloat16)
    ws = torch.empty(moe.backward_workspace_bytes(w.T, w.d, w.d_ff, w.n, w.K, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    grads = moe.backward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], dy, w.K, workspace=ws,
                         eps=eps)
    y = torch.empty_like(L["x"])
    saved = torch.empty(moe.saved_bytes(w.T, w.d, w.d_ff, w.n, w.K, torch.bfloat16),
                        dtype=torch.uint8, device=dev)
    fws = torch.empty(moe.workspace_bytes(w.T, w.d, w.d_ff, w.n, w.K, torch.bfloat16),
                      dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            moe._lib.set_stage_events_raw("bwd_wgrad", ev[0].handle.value, ev[1].handle.value)
        else:
            moe._lib.set_stage_events_raw("bwd_wgrad")
        if train:
            moe.forward_train(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.K, out=y,
                              saved=saved, workspace=fws, eps=eps)
            moe.backward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], dy, w.K, workspace=ws,
                         out=grads, saved=saved, eps=eps)
        else:
            moe.backward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], dy, w.K, workspace=ws,
                         out=grads, eps=eps)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")
    every = max(1, args.stage_every)
    kev = {s: (HipEvent(), HipEvent()) for s in range(args.steps) if s % every == 0}
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for s in range(args.steps):
        step(kev.get(s))
        marks[s + 1].record()
    torch.cuda.synchronize()
    moe._lib.set_stage_events_raw("bwd_wgrad")
    ms = marks[0].elapsed_time(marks[-1]) / args.steps
    k_ms = [a.elapsed_ms(b) / 3.0 for (a, b) in kev.values()]  # three launches per stage
    k_avg = sum(k_ms) / len(k_ms)
    if stack:
        _, idx, _, _ = moe.block_forward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.K, eps)
    else:
        idx, _ = moe.route(L["x"], L["Wg"], w.K)
    counts = torch.bincount(idx.view(-1).long(), minlength=w.n).cpu().tolist()
    log(f"[bench] {ms:.4f} ms/step, weight-gradient product {k_avg:.4f} ms per launch")
    A = w.T * w.K
    # per launch: one expert weight gradient [n][N1][N2] fp32 written (every
    # expert, zero or not), the two transposed activation operands read
    wbytes = w.n * w.d * w.d_ff * 4 + A * (w.d + w.d_ff) * 2
    flops = 2.0 * A * w.d * w.d_ff
    if wbytes / (HBM_PEAK_GBS * 1e9) > flops / (BF16_PEAK_TFLOPS * 1e12):
        ach = wbytes / (k_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = flops / (k_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
    sha = kernel_source_sha(WGRAD_SOURCES)
    kind = "train" if train else "backward"
    # the same kernel at the same sizes in both modes: one counter entry
    roof["traffic"] = traffic_for(w.name + "-backward", sha)
    roof["kernel"] = "weight-gradient product (MFMA tiles over each expert's rows)"
    roof["kernel_ms"] = round(k_avg, 5)
    roof["kernel_samples"] = len(k_ms)
    roof["algorithmic_bytes"] = wbytes
    roof["algorithmic_flops"] = flops
    roof["source_sha"] = sha
    out = {
        "metric": ("MoE-layer training-step tokens/s (forward keeping its routing and "
                   "pre-activations, then all gradients of sum(dy*y)" if train else
                   "MoE-layer backward tokens/s (all gradients of sum(dy*y)") +
                  ("; the stack layer x + MoE(RMSNorm(x))" if stack else "") +
                  "; top-2 of 8 SwiGLU, d=4096) + % roofline",
        "value": round(w.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) tokens and output gradients, N(0,1/fan_in) "
                "weights)",
        "config": {"workload": w.name + "-" + kind, "T": w.T, "d": w.d, "d_ff": w.d_ff,
                   "n": w.n, "K": w.K, "dtype": w.dtype,
                   **({"layers": 1, "layer": 0, "eps": eps} if stack else {})},
        "roofline": roof,
        "step_ms": step_percentiles(marks),
        # backward: gate/up recompute 4, r = W2^T dy 2, dx 4, weight gradients
        # 6; training step: forward 6 + backward without recompute 12 (x A d d_ff)
        "step_tflops": round(18.0 * A * w.d * w.d_ff / (ms * 1e-3) / 1e12 if train else
                             16.0 * A * w.d * w.d_ff / (ms * 1e-3) / 1e12, 1),
        "counts": counts,
    }
    if args.cpu_budget > 0:
        log("[bench] timing the fp64 oracle's backward on the host")
        out["cpu_baseline"] = backward_cpu_baseline(w, L, dy, args.cpu_budget, train=train,
                                                    eps=eps)
    print(json.dumps(out), flush=True)


# GEMM shapes of the layer (x[M][K] . W[N][K]^T): one expert's gate/up ([W1 ; W3], N =
# 2 d_ff) and down products at the stack layer, at prefill and under skew (expert 0), and
# the dense 8192-row products with the same flops as prefill.
BLAS_SHAPES = [("gate_up_stack_expert", 512, 4096, 28672),
               ("gate_up_prefill_expert", 1024, 4096, 28672),
               ("gate_up_skew_expert0", 15872, 4096, 28672),
               ("gate_up_dense_8192", 8192, 4096, 28672),
               ("down_stack_expert", 512, 14336, 4096),
               ("down_prefill_expert", 1024, 14336, 4096),
               ("down_skew_expert0", 15872, 14336, 4096),
               ("down_dense_8192", 8192, 14336, 4096)]


def blas_calibration(reps: int = 20):
    """hipBLASLt (torch.nn.functional.linear, bf16) on the layer's GEMM shapes with
    N(0,1) tokens and N(0,1/K) weights: a calibration of what the library GEMM
    reaches on this chip, not a part of the layer.  One JSON line per shape."""
    import torch
    import torch.nn.functional as F
    g = torch.Generator(device="cuda").manual_seed(0)
    for name, M, K, N in BLAS_SHAPES:
        x = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
        w = (torch.randn(N, K, generator=g, device="cuda") / K ** 0.5).to(torch.bfloat16)
        for _ in range(3):
            F.linear(x, w)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            F.linear(x, w)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        ms = ts[len(ts) // 2]
        print(json.dumps({"blas_shape": name, "M": M, "K": K, "N": N, "ms": round(ms, 4),
                          "tflops": round(2.0 * M * K * N / ms / 1e9, 1)}), flush=True)
        del x, w


def dense_probe(T: int, reps: int = 10):
    """The layer's own kernels on a dense problem: T positive tokens routed to
    expert 0 (K = 1), so gate/up is one [T][4096] x [28672][4096]^T product and
    down one [T][14336] x [4096][14336]^T -- the same work as the dense
    library GEMMs of blas_calibration.  Stage times from the library's own
    events.  One JSON line."""
    import statistics

    import torch

    import sparse_mixture_experts_14_amd as moe
    d, dff, n = 4096, 14336, 8
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(T, d, generator=g, device="cuda").abs().to(torch.bfloat16)
    wg = torch.zeros(d, n, device="cuda")
    wg[:, 0] = 1.0  # logit 0 = sum of |x| > 0 = every other logit
    wg = wg.to(torch.bfloat16)
    w1 = (torch.randn(n, dff, d, generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    w3 = (torch.randn(n, dff, d, generator=g, device="cuda") / d ** 0.5).to(torch.bfloat16)
    w2 = (torch.randn(n, d, dff, generator=g, device="cuda") / dff ** 0.5).to(torch.bfloat16)
    lay = moe.Layer(T, d, dff, n, 1, torch.bfloat16, "cuda")
    ev = {st: (HipEvent(), HipEvent()) for st in ("gate_up", "down")}
    res = {st: [] for st in ev}
    for it in range(reps + 2):
        for st, (a, b) in ev.items():
            moe._lib.set_stage_events_raw(st, a.handle.value, b.handle.value)
        lay.forward(x, wg, w1, w3, w2)
        torch.cuda.synchronize()
        if it >= 2:
            for st, (a, b) in ev.items():
                res[st].append(a.elapsed_ms(b))
    for st in ev:
        moe._lib.set_stage_events_raw(st)
    if int(lay.counts[0]) != T:
        raise SystemExit("dense probe: tokens did not all route to expert 0")
    gu, dn = statistics.median(res["gate_up"]), statistics.median(res["down"])
    print(json.dumps({"dense_probe_T": T, "gate_up_ms": round(gu, 4),
                      "gate_up_tflops": round(4.0 * T * d * dff / gu / 1e9, 1),
                      "down_ms": round(dn, 4),
                      "down_tflops": round(2.0 * T * d * dff / dn / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="stack",
                    choices=["tiny", "decode", "prefill", "skew", "stack"])
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for the CPU baseline (0 = skip)")
    ap.add_argument("--stage-every", type=int, default=4,
                    help="time the gate/up kernel with HIP events on every k-th timed step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the plain copy that calibrates the traffic counters")
    ap.add_argument("--traffic-from", nargs=4, metavar="DIR",
                    help="rocprofv3 --pmc output dirs (bench FETCH_SIZE, bench WRITE_SIZE, "
                         "copy FETCH_SIZE, copy WRITE_SIZE): write profiles/traffic.json "
                         "for --workload and exit")
    ap.add_argument("--traffic-command", default="",
                    help="command line recorded with --traffic-from")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_backward (all gradients of sum(dy * y)) instead of the "
                         "forward layer")
    ap.add_argument("--blas-calibration", action="store_true",
                    help="time hipBLASLt (torch F.linear) on the layer's GEMM shapes and exit")
    ap.add_argument("--dense-probe", type=int, metavar="T", default=0,
                    help="time the layer's gate/up and down kernels with T tokens all on "
                         "expert 0 (the dense problem of --blas-calibration) and exit")
    ap.add_argument("--train", action="store_true",
                    help="time a training step: moe_forward_train, then moe_backward_saved "
                         "on its saved state")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(args.workload, args.traffic_from, args.traffic_command,
                      backward=args.backward or args.train)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer is built and timed on a single MI355X; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mixture_experts_14_amd as moe
    from sparse_mixture_experts_14_amd import workloads as W
    from sparse_mixture_experts_14_amd.stack import Stack

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.load()
    if args.blas_calibration:
        blas_calibration()
        return
    if args.dense_probe:
        dense_probe(args.dense_probe)
        return
    if args.backward or args.train:
        bench_backward(args, w, dev, train=args.train)
        return
    log(f"[bench] workload={w.name} T={w.T} building inputs on {dev}")
    if w.name == "stack":
        layers = [W.make_stack_layer(w, l, device=dev) for l in range(w.layers)]
        x0 = W.make_stack_input(w, device=dev)
    else:
        L = W.make_layer(w, device=dev)
        layers = [L]
        x0 = L["x"]
    chain = Stack(layers, w.T, w.d, w.d_ff, w.n, w.K, w.torch_dtype, dev, eps=w.eps)
    lay = chain.lay

    def step(stage_ev=None):
        def before(i):
            if stage_ev is not None:
                moe._lib.set_stage_events_raw("gate_up", stage_ev[i][0].handle.value,
                                              stage_ev[i][1].handle.value)
            else:
                moe._lib.set_stage_events_raw("gate_up")
        return chain.run(x0, before=before)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")
    nl = len(layers)
    # The gate/up kernel is timed by events that the library records on its
    # stream around that stage, on every stage_every-th timed step: each
    # record is a queue marker that delays the next dispatch by a few
    # microseconds, so the other steps run without them.
    every = max(1, args.stage_every)
    timed = [s for s in range(args.steps) if s % every == 0]
    kev = {s: [(HipEvent(), HipEvent()) for _ in range(nl)] for s in timed}
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for s in range(args.steps):
        step(kev.get(s))
        marks[s + 1].record()
    torch.cuda.synchronize()
    moe._lib.set_stage_events_raw("gate_up")
    ms = marks[0].elapsed_time(marks[-1]) / args.steps
    k_ms = [a.elapsed_ms(b) for st in kev.values() for (a, b) in st]
    k_avg = sum(k_ms) / len(k_ms)
    counts = lay.counts.cpu().tolist()
    log(f"[bench] {ms:.4f} ms/step, gate/up kernel {k_avg:.4f} ms avg, counts {counts}")

    skinny = w.dtype == "bf16" and w.T * w.K <= 16 * w.n
    kname, ksrc = dominant_kernel(w, skinny)
    sha = kernel_source_sha(ksrc)
    work = algorithmic_work(w, counts)
    if w.name == "decode":
        ach = work["bytes"] / (k_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
        ach = work["flops"] / (k_avg * 1e-3) / 1e12
        roof = {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(ach, 1),
                "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    roof["traffic"] = traffic_for(w.name, sha)
    roof["kernel"] = f"{kname} ({'skinny' if skinny else 'tiled'} grouped GEMM)"
    roof["kernel_ms"] = round(k_avg, 5)
    roof["kernel_samples"] = len(k_ms)
    roof["algorithmic_bytes"] = work["bytes"]
    roof["algorithmic_flops"] = work["flops"]
    roof["touched_experts"] = work["touched_experts"]
    roof["source_sha"] = sha

    tokens = w.T  # tokens through the whole step (all layers of the stack)
    value = tokens / (ms * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "n": w.n, "K": w.K,
                   "layers": w.layers, "dtype": w.dtype},
        "roofline": roof,
        "step_ms": step_percentiles(marks),
    }
    # whole-step rate over the touched weights, for context
    if w.name in ("decode",):
        step_bytes = work["touched_experts"] * 3 * w.d_ff * w.d * 2
        out["step_hbm_gbs"] = round(step_bytes / (ms * 1e-3) / 1e9, 1)
    else:
        out["step_tflops"] = round(6.0 * w.T * w.K * w.d * w.d_ff * nl / (ms * 1e-3) / 1e12, 1)
    if args.cpu_budget > 0:
        log("[bench] timing the fp64 oracle on the host")
        Ls = dict(layers[0])
        Ls["x"] = x0
        cb = cpu_baseline(w, Ls, args.cpu_budget)
        if nl > 1:  # tokens through the whole stack: one layer's rate / layers
            cb["value"] /= nl
            cb["sample"] += f" through layer 0 only; rate divided by {nl} layers"
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
