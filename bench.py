#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one fa_forward call (one kernel launch) over the whole workload, with
inputs already resident in HBM; for the key-split workloads it is one
fa_forward_split call (the split kernel and the merge kernel, workspace
allocated beforehand); for the chain workload it is one fa_forward_chain call
(the last layer of a 4-layer Block Attention Residual block, its logits
recomputed from the Q and K of all four layers).  The default workload is B=2, H=16, S=4096,
D=64, bf16, causal.  Timing follows the CUDA-event method of the Day 26 post
(blog.ans20xx.com/posts/ai/day26): W untimed warm-up steps, then K steps with
one event recorded before each step and one after the last, on the stream the
kernels run on.  Before the warm-up steps the device is kept busy for
--settle-ms (default 60 ms) with plain bf16 matrix products, so that the timed
steps do not catch the GPU clock ramping up from idle.  Prints one JSON line.

value     = 4*B*H*S^2*D / t_step in TFLOP/s (the post's formula, not halved
            for causal), t_step = wall time of the K steps / K;
roofline  = the step's own rate against the chip's peak: useful flops
            (visible query-key pairs only) per step / mean step time where the
            workload's arithmetic intensity (useful flops per algorithmic byte)
            is above the chip's ridge point (peak flops / peak HBM bandwidth),
            else algorithmic bytes (Q, K, V, visible bias, O, LSE) / step time;
cpu_baseline = the fp64 oracle, timed on the host on a bounded sample of the
            same workload (whole heads), scaled to the same metric;
            cpu_baseline_1thread the same with one BLAS thread, on a smaller
            sample;
error_vs_oracle = max / mean |O_gpu - O_oracle| and max |LSE_gpu - LSE_oracle|
            over the heads the oracle ran, from this run's own output;
env       = GPU, runtime, torch and library versions; peak_mem_gb the peak
            device memory allocated (inputs, outputs, workspace).
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Same workload, same metric, measured on an H100-SXM by the Day 26 post
# (flash-attn v2 row of its report): context, not a target.
PAGE_FLASH_ATTN_V2_TFLOPS = 11.57
METRIC = ("attention TFLOPS (4·B·H·S²·D/t) and % MFMA bf16 peak at "
          "B2 H16 S4096 D64 causal")
# (the build script too: its compiler flags shape the generated code)
KERNEL_SOURCES = {
    p: [os.path.join(ROOT, "tiled_attention_forward_amd", "csrc", f)
        for f in (("fa_fwd.hip", "fa_device.h") if p == "forward" else ("fa_bwd.hip", "fa_device.h"))]
    + [os.path.join(ROOT, "tiled_attention_forward_amd", "build.py")]
    for p in ("forward", "backward")
}
BACKWARD_FLOP_FACTOR = 2.5  # five products against the forward's two
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU clock ramps up over the first ~30 ms of sustained load; the
    # default warm-up (300 untimed steps) covers that before timing starts.
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--pass", dest="pass_", choices=["forward", "backward"], default="forward",
                    help="time the forward (default) or the backward (dQ, dK, dV)")
    ap.add_argument("--path", choices=["fused", "split"], default=None,
                    help="entry point to time (default: the workload's own)")
    ap.add_argument("--splits", type=int, default=0,
                    help="key splits for the split path (default: the library's suggestion)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target host time for the oracle sample")
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="before the warm-up steps, keep the GPU busy this long with plain "
                         "bf16 matrix products (not the attention kernel), so that the clock "
                         "has left its idle state when the timed steps start; 0 = off")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before timing, run one plain device copy of MIB MiB (a reference "
                         "dispatch for scaling HBM byte counters); untimed")
    return ap.parse_args()


def kernel_source_hash(pass_: str = "forward") -> str:
    """sha256 over the kernels' sources of one pass (the counters in
    traffic.json were taken on the build of exactly these bytes)."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[pass_]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(workload: str, pass_: str = "forward"):
    """HBM bytes per step from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    key = workload if pass_ == "forward" else f"{workload}:{pass_}"
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha256") != kernel_source_hash(pass_):
        return None
    return rec.get("hbm_bytes_per_launch")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_baseline_backward(w, q, k, v, dout, target_s: float):
    """Time the oracle's backward on whole (batch, KV head) groups until about target_s."""
    import numpy as np

    from oracle import attention_backward

    grp = w.Hq // w.Hkv
    done, t_used = 0, 0.0
    for b in range(w.B):
        for hk in range(w.Hkv):
            hs = slice(hk * grp, (hk + 1) * grp)
            f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
            qs, gs = f(q[b:b + 1, hs]), f(dout[b:b + 1, hs])
            ks, vs = f(k[b:b + 1, hk:hk + 1]), f(v[b:b + 1, hk:hk + 1])
            t0 = time.perf_counter()
            attention_backward(qs, ks, vs, gs, None, scale=w.scale, causal=w.causal,
                               window=w.window or None)
            t_used += time.perf_counter() - t0
            done += grp
            if t_used >= target_s:
                break
        if t_used >= target_s:
            break
    per_head = BACKWARD_FLOP_FACTOR * (w.useful_flops() if w.window else w.metric_flops()) / (
        w.B * w.Hq)
    return {"value": round(per_head * done / t_used / 1e12, 6), "unit": "TFLOPS",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"backward of {done} of {w.B * w.Hq} (batch, head) slices of {w.name}, "
                      f"fp64 NumPy, {t_used:.1f} s"}


def chain_backward_factor(layers: int) -> float:
    """Products of the chain backward per visible pair against the chain
    forward's: the logits (layers), dP, dQ and dK of every layer, and dV, so
    3*layers + 2 against layers + 1."""
    return (3 * layers + 2) / (layers + 1)


def cpu_baseline_chain_backward(w, q_layers, k_layers, v, dout, target_s: float):
    """Time the oracle's chain backward on whole (batch, KV head) groups until
    about target_s."""
    import numpy as np

    from oracle import attention_chain_backward

    grp = w.Hq // w.Hkv
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    done, t_used = 0, 0.0
    for b in range(w.B):
        for hk in range(w.Hkv):
            hs = slice(hk * grp, (hk + 1) * grp)
            qs = [f(t[b:b + 1, hs]) for t in q_layers]
            ks = [f(t[b:b + 1, hk:hk + 1]) for t in k_layers]
            t0 = time.perf_counter()
            attention_chain_backward(qs, ks, f(v[b:b + 1, hk:hk + 1]), f(dout[b:b + 1, hs]),
                                     scale=w.scale, causal=w.causal)
            t_used += time.perf_counter() - t0
            done += grp
            if t_used >= target_s:
                break
        if t_used >= target_s:
            break
    per_head = chain_backward_factor(w.layers) * w.useful_flops() / (w.B * w.Hq)
    return {"value": round(per_head * done / t_used / 1e12, 6), "unit": "TFLOPS",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"chain backward of {done} of {w.B * w.Hq} (batch, head) slices of "
                      f"{w.name}, fp64 NumPy, {t_used:.1f} s"}


def cpu_baseline_chain(w, q_layers, k_layers, v, target_s: float, o_gpu=None, lse_gpu=None):
    """Time the oracle's chain on whole heads until about target_s (and the
    error of the GPU output on those heads)."""
    import numpy as np

    from oracle import attention_chain_head_rows

    grp = w.Hq // w.Hkv
    rows = np.arange(w.Nq)
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    done, t_used = 0, 0.0
    acc = _err_acc()
    for b in range(w.B):
        for h in range(w.Hq):
            hk = h // grp
            qs = [f(t[b, h]) for t in q_layers]
            ks = [f(t[b, hk]) for t in k_layers]
            vh = f(v[b, hk])
            t0 = time.perf_counter()
            o_ref, lse_ref = attention_chain_head_rows(qs, ks, vh, rows=rows, scale=w.scale,
                                                       causal=w.causal)
            t_used += time.perf_counter() - t0
            done += 1
            if o_gpu is not None:
                _err_add(acc, o_gpu[b, h], lse_gpu[b, h], o_ref, lse_ref)
            if t_used >= target_s:
                break
        if t_used >= target_s:
            break
    per_head = w.useful_flops() / (w.B * w.Hq)
    base = {"value": round(per_head * done / t_used / 1e12, 6), "unit": "TFLOPS",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {w.B * w.Hq} (batch, head) slices of {w.name}, fp64 NumPy, "
                      f"{t_used:.1f} s"}
    return base, _err_report(acc, w, f"{done} of {w.B * w.Hq} whole (batch, head) slices")


def _err_acc():
    return {"max_abs": 0.0, "sum_abs": 0.0, "n": 0, "lse_max": 0.0}


def _err_add(acc, o_gpu, lse_gpu, o_ref, lse_ref):
    import numpy as np
    d = np.abs(o_gpu.float().cpu().numpy().astype(np.float64) - o_ref)
    acc["max_abs"] = max(acc["max_abs"], float(d.max(initial=0.0)))
    acc["sum_abs"] += float(d.sum())
    acc["n"] += d.size
    dl = np.abs(lse_gpu.cpu().numpy().astype(np.float64) - lse_ref)
    acc["lse_max"] = max(acc["lse_max"], float(dl.max(initial=0.0)))


# Bars of the workloads (against the fp64 oracle): bf16/fp16 max |dO| <= 1e-2,
# mean <= 1e-3; fp32 max <= 1e-5; LSE <= 1e-3.  FP8 inputs are held to a
# derived rounding bound in the tests, not to a fixed bar.
_BARS = {"bf16": (1e-2, 1e-3), "fp16": (1e-2, 1e-3), "fp32": (1e-5, 1e-5)}


def _err_report(acc, w, what):
    if acc["n"] == 0:
        return None
    rep = {"max_abs": acc["max_abs"], "mean_abs": acc["sum_abs"] / acc["n"],
           "lse_max": acc["lse_max"], "elements": acc["n"], "compared": what}
    bars = _BARS.get(w.dtype)
    if bars is not None:
        rep["within_bars"] = bool(acc["max_abs"] <= bars[0] and rep["mean_abs"] <= bars[1]
                                  and acc["lse_max"] <= 1e-3)
    return rep


def cpu_baseline(w, q, k, v, bias, target_s: float, o_gpu=None, lse_gpu=None):
    """Time the oracle on whole heads of the same workload until about target_s;
    the same oracle results give the error of the GPU output on those heads."""
    import numpy as np

    from oracle import attention_head_rows

    grp = w.Hq // w.Hkv
    rows = np.arange(w.Nq)
    done, t_used = 0, 0.0
    acc = _err_acc()
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    for b, h in heads:
        hk = h // grp
        qh = q[b, h].cpu().float().numpy().astype(np.float64)
        kh = k[b, hk].cpu().float().numpy().astype(np.float64)
        vh = v[b, hk].cpu().float().numpy().astype(np.float64)
        bh = None if bias is None else bias[b, h].cpu().float().numpy().astype(np.float64)
        t0 = time.perf_counter()
        o_ref, lse_ref = attention_head_rows(qh, kh, vh, rows=rows, scale=w.scale,
                                             causal=w.causal, bias_rows=bh,
                                             window=w.window or None)
        t_used += time.perf_counter() - t0
        done += 1
        if o_gpu is not None:
            _err_add(acc, o_gpu[b, h], lse_gpu[b, h], o_ref, lse_ref)
        if t_used >= target_s:
            break
    per_head_flops = (w.useful_flops() if w.window else w.metric_flops()) / (w.B * w.Hq)
    base = {"value": round(per_head_flops * done / t_used / 1e12, 6), "unit": "TFLOPS",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {w.B * w.Hq} (batch, head) slices of {w.name}, fp64 NumPy, "
                      f"{t_used:.1f} s"}
    return base, _err_report(acc, w, f"{done} of {w.B * w.Hq} whole (batch, head) slices")


def cpu_baseline_one_thread(w, q, k, v, bias, target_s: float):
    """The same oracle with its BLAS held to one thread, on whole heads until
    about target_s (a smaller sample than the threaded run)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        base, _ = cpu_baseline(w, q, k, v, bias, target_s)
    base["cores"] = 1
    return base


def settle_clock(dev, ms: float) -> float:
    """Keep the device busy for about ``ms`` ms with dense bf16 products (a
    torch matmul, not the attention kernel): the GPU clock ramps up over the
    first tens of milliseconds of sustained load, and a benchmark of a few
    milliseconds would otherwise time that ramp.  Untimed; returns the
    milliseconds spent."""
    import torch
    if ms <= 0:
        return 0.0
    a = torch.full((4096, 4096), 1.0 / 4096, dtype=torch.bfloat16, device=dev)
    c = torch.empty_like(a)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(16):
            torch.mm(a, a, out=c)
        torch.cuda.synchronize(dev)
    del a, c
    return (time.perf_counter() - t0) * 1e3


def environment(lib_version: str):
    """What the numbers were measured on (the Day 26 post's report header)."""
    import platform

    import torch
    props = torch.cuda.get_device_properties(0)
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip_runtime": torch.version.hip,
            "torch": torch.__version__, "library": lib_version,
            "host_cpus": os.cpu_count(), "python": platform.python_version()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the forward has no "
              f"cross-GPU path to measure", file=sys.stderr)
        sys.exit(2)

    import torch

    from tiled_attention_forward_amd import binding, metrics
    from tiled_attention_forward_amd.workloads import (HEADLINE, WORKLOADS, make_chain_inputs,
                                                       make_inputs)

    w = WORKLOADS[args.workload or HEADLINE]
    if args.path is not None and args.path != w.path:
        w = dataclasses.replace(w, path=args.path)
    dev = torch.device("cuda:0")
    lib = binding.load_library()
    if w.layers:
        q_layers, k_layers, v = make_chain_inputs(w, w.layers, seed=args.seed, device=dev)
        q, k, bias = q_layers[-1], k_layers[-1], None
    else:
        q, k, v, bias = make_inputs(w, seed=args.seed, device=dev)
    # FP8 (E4M3) inputs give a bf16 output
    o = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "fp8" else q.dtype, device=dev)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    dtype_code = binding._dtype_code(q)
    call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(),
                 bias.data_ptr() if bias is not None else None, o.data_ptr(), lse.data_ptr(),
                 w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, float(w.scale), int(w.causal), dtype_code)
    splits = None
    backward = args.pass_ == "backward"
    if w.layers and w.path != "fused":
        print("the chain workload is timed on its fused path only", file=sys.stderr)
        sys.exit(2)
    if backward and w.layers:
        import ctypes
        g = torch.Generator(device=dev).manual_seed(args.seed + 1000)
        dout = torch.randn(q.shape, generator=g, device=dev).to(q.dtype)
        binding.forward_chain(q_layers, k_layers, v, causal=w.causal, scale=w.scale, out=o,
                              lse=lse)
        dqs = [torch.empty_like(t) for t in q_layers]
        dks = [torch.empty_like(t) for t in k_layers]
        dv = torch.empty_like(v)
        ws_bytes = binding.fa_backward_workspace_bytes(w.B, w.Hq, w.Nq)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        arr = lambda ts: (ctypes.c_void_p * w.layers)(*[t.data_ptr() for t in ts])  # noqa: E731
        entry = lib.fa_backward_chain
        call_args = (arr(q_layers), arr(k_layers), w.layers, v.data_ptr(), o.data_ptr(),
                     lse.data_ptr(), dout.data_ptr(), arr(dqs), arr(dks), dv.data_ptr(), w.B,
                     w.Hq, w.Hkv, w.Nq, w.Nk, w.D, float(w.scale), int(w.causal), dtype_code,
                     workspace.data_ptr(), ws_bytes, stream.cuda_stream)
    elif backward:
        if w.bias or w.dtype == "fp8":
            print("the backward is timed on bias-free bf16, fp16 or fp32 workloads",
                  file=sys.stderr)
            sys.exit(2)
        g = torch.Generator(device=dev).manual_seed(args.seed + 1000)
        dout = torch.randn(q.shape, generator=g, device=dev).to(q.dtype)
        binding.forward(q, k, v, None, causal=w.causal, scale=w.scale, out=o, lse=lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = binding.fa_backward_workspace_bytes(w.B, w.Hq, w.Nq)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        binding.forward(q, k, v, None, causal=w.causal, scale=w.scale, out=o, lse=lse,
                        window=w.window or None)
        entry = lib.fa_backward_window if w.window else lib.fa_backward
        call_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), None, o.data_ptr(), lse.data_ptr(),
                     dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.Hq,
                     w.Hkv, w.Nq, w.Nk, w.D, float(w.scale),
                     int(w.window) if w.window else int(w.causal), dtype_code,
                     workspace.data_ptr(), ws_bytes, stream.cuda_stream)
    elif w.path == "split":
        splits = args.splits or binding.fa_split_count(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D)
        ws_bytes = binding.fa_split_workspace_bytes(w.B, w.Hq, w.Nq, w.D, splits)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        entry = lib.fa_forward_split
        call_args = call_args + (splits, workspace.data_ptr(), ws_bytes, stream.cuda_stream)
    elif w.layers:
        import ctypes
        ptrs = ctypes.c_void_p * w.layers
        q_arr = ptrs(*[t.data_ptr() for t in q_layers])
        k_arr = ptrs(*[t.data_ptr() for t in k_layers])
        entry = lib.fa_forward_chain
        call_args = (q_arr, k_arr, w.layers, v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, float(w.scale), int(w.causal),
                     dtype_code, stream.cuda_stream)
    elif w.window:
        entry = lib.fa_forward_window
        call_args = call_args[:13] + (int(w.window), dtype_code, stream.cuda_stream)
    else:
        entry = lib.fa_forward
        call_args = call_args + (stream.cuda_stream,)

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        st = entry(*call_args)
        if st != 0:
            raise binding.FaError(st, binding.fa_status_string(st))

    settled_ms = settle_clock(dev, args.settle_ms)

    # peak device memory of the run (the Day 26 report's peak-memory column):
    # inputs, outputs and any workspace are allocated by now, so the steps
    # themselves should add nothing
    torch.cuda.synchronize()
    mem_base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # One event before each step and one after the last, all on the launch
    # stream: step i lasts from event i to event i+1 (its kernels and the
    # dispatch gap to the next step), and the K steps from event 0 to event K.
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i].record(stream)
        step()
    ev[K].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[K])
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(K))
    ms_per_step = total_ms / K
    launch_ms = statistics.fmean(per)
    mem_peak = torch.cuda.max_memory_allocated(dev)
    assert torch.isfinite(lse).all(), "non-finite LSE in the benchmark output"

    fl = (chain_backward_factor(w.layers) if w.layers else BACKWARD_FLOP_FACTOR) if backward \
        else 1.0
    # windowed attention: count the visible pairs only (the dense formula
    # would credit work the window removes)
    metric_flops = w.useful_flops() if (w.window or w.layers) else w.metric_flops()
    value = fl * metric_flops / (ms_per_step / 1e3) / 1e12
    peak = metrics.MFMA_PEAK_TFLOPS[w.dtype]
    ridge = peak * 1e12 / (metrics.HBM_PEAK_GBS * 1e9)   # flops per byte
    if not backward and w.useful_flops() / w.io_bytes() < ridge:
        achieved = w.io_bytes() / (launch_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": metrics.HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / metrics.HBM_PEAK_GBS, 4)}
    else:
        achieved = fl * w.useful_flops() / (launch_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roof["traffic"] = traffic_for(w.name, args.pass_)

    if w.layers and backward:
        metric = (f"chain attention backward TFLOPS over visible pairs "
                  f"(2·D·(3·layers+2)·pairs/t) at {w.name}")
    elif w.layers:
        metric = (f"chain attention TFLOPS over visible pairs (2·D·(layers+1)·pairs/t) at "
                  f"{w.name}")
    elif w.window:
        metric = (f"attention {'backward ' if backward else ''}TFLOPS over visible pairs "
                  f"({'2.5·' if backward else ''}4·D·pairs/t) at {w.name}")
    elif backward:
        metric = f"attention backward TFLOPS (2.5·4·B·H·Nq·Nk·D/t) at {w.name}"
    elif w.name == HEADLINE:
        metric = METRIC
    else:
        metric = f"attention TFLOPS (4·B·H·Nq·Nk·D/t) at {w.name}"
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / PAGE_FLASH_ATTN_V2_TFLOPS, 2)
                        if w.name == HEADLINE and not backward else None),
        "dtype": w.dtype,
        "data": "synthetic: i.i.d. N(0,1) inputs from a seeded generator",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq,
                   "Nk": w.Nk, "D": w.D, "causal": w.causal, "bias": w.bias,
                   "path": w.path, "splits": splits, "pass": args.pass_,
                   "window": w.window or None, "layers": w.layers or None,
                   "parallelism": "single GPU"},
        # value / bf16 dense peak: the metric's own formula counts every
        # (query, key) pair, so for causal workloads this is twice the share
        # of the matrix cores' peak that the visible pairs use
        "pct_of_bf16_peak_dense_formula": round(100.0 * value / metrics.MFMA_PEAK_TFLOPS["bf16"],
                                                2),
        "useful_tflops": round(fl * w.useful_flops() / (ms_per_step / 1e3) / 1e12, 2),
        # useful flops (visible pairs only) per step time / the dtype's peak
        "pct_of_peak_useful": round(100.0 * fl * w.useful_flops() / (ms_per_step / 1e3) / 1e12
                                    / peak, 2),
        "peak_mem_gb": round(mem_peak / 1e9, 4),
        "alloc_in_timed_steps_bytes": int(mem_peak - mem_base),
        "clock_settle_ms": round(settled_ms, 1),
        "launch_ms": {"mean": round(launch_ms, 5), "median": round(statistics.median(per), 5),
                      "p90": round(per[int(len(per) * 0.9)], 5), "min": round(per[0], 5)},
        "roofline": roof,
    }
    out["env"] = environment(binding.fa_version())
    if not args.no_cpu_baseline:
        # the oracle on the host; for the forward its results on the heads it
        # ran also give the error of this run's GPU output there
        if backward and w.layers:
            out["cpu_baseline"] = cpu_baseline_chain_backward(w, q_layers, k_layers, v, dout,
                                                              args.cpu_seconds)
        elif backward:
            out["cpu_baseline"] = cpu_baseline_backward(w, q, k, v, dout, args.cpu_seconds)
        elif w.layers:
            out["cpu_baseline"], out["error_vs_oracle"] = cpu_baseline_chain(
                w, q_layers, k_layers, v, args.cpu_seconds, o, lse)
        else:
            out["cpu_baseline"], out["error_vs_oracle"] = cpu_baseline(
                w, q, k, v, bias, args.cpu_seconds, o, lse)
            out["cpu_baseline_1thread"] = cpu_baseline_one_thread(
                w, q, k, v, bias, args.cpu_seconds / 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
