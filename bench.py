"""Benchmark: fwd+bwd throughput of the frozen-int8 + LoRA linear on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

A step is one training pass of the workload's layer stack through libqlora:
the forward of every layer (per-row activation quantization + x A, int8
MFMA product with the fused dequant + LoRA epilogue), then the backward of
every layer in reverse (dy B^T, dB, dA, and the bf16 MFMA input gradient).
For stacks of at least 4 layers (``--finish``) each layer's backward leaves
its adapter-gradient partial sums in a workspace of its own and one batched
call adds them into every layer's dA and dB after the last layer; otherwise
each layer's ``qlora_bwd`` combines its own. Both steps are timed and
reported (``batched_finish_ms_per_step``, ``layerwise_finish_ms_per_step``).
The one-time weight quantization is timed separately (``quantize_ms``).
Inputs are seeded synthetic tensors already resident in HBM. Steps are
captured once in a HIP graph and replayed; ``value`` is the workload's
algorithmic operations divided by the measured time per step.

Prints ONE JSON line (see the keys below), including the roofline of the
dominant kernel, timed live with HIP events recorded by the library around
each of its launches, and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd TFLOP/s of int8-weight+LoRA linear; % of MFMA/HBM roofline"
# MI355X published dense peaks
PEAK = {"bf16": 2.5e15, "int8": 5.0e15, "f32": 157.3e12, "hbm": 8.0e12}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", type=int, default=2, help="1..5 (default: the 32-layer MLP)")
    p.add_argument("--weights", choices=("w8", "w4g128", "w8o"), default=None,
                   help="store the workload's weights in this format instead of its own "
                        "(w8o: outlier-compensated int8, same tensors)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time budget of the oracle baseline (0: skip)")
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    p.add_argument("--finish", choices=("auto", "batched", "layerwise"), default="auto",
                   help="adapter-gradient combine of the timed step: one batched call after "
                        "the last layer, or one per layer (auto: batched for stacks of at "
                        "least 4 layers)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy (for scaling HBM counters)")
    return p.parse_args()


class Layer:
    """Device buffers and ready-made C arguments for one layer."""

    def __init__(self, w, idx, dev):
        import torch
        from quantized_frozen_weight_amd import binding as Q
        from quantized_frozen_weight_amd import workloads as WL
        self.K, self.N = w.layers[idx]
        M = w.M
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.W = torch.from_numpy(WL.weight(w, idx)).to(dev)
        x, _ = WL.as_compute_dtype(WL.activations(w, idx), w.dtype)
        dy, _ = WL.as_compute_dtype(WL.out_grad(w, idx), w.dtype)
        self.x, self.dy = x.to(dev), dy.to(dev)
        self.A = torch.from_numpy(WL.lora_A(w, idx)).to(dev)
        self.B = torch.from_numpy(WL.lora_B(w, idx)).to(dev)
        cb, sb = Q.qlora_weight_bytes(self.K, self.N, w.wfmt)
        if w.wfmt == "w8":
            self.codes = torch.empty((self.N, self.K), dtype=torch.int8, device=dev)
            self.scales = torch.empty((self.N,), dtype=torch.float32, device=dev)
        elif w.wfmt == "w8o":
            # codes, and the side buffer with the cut, the grid and the outliers
            self.codes = torch.empty((self.N, self.K), dtype=torch.int8, device=dev)
            self.scales = torch.empty((sb,), dtype=torch.uint8, device=dev)
        else:
            self.codes = torch.empty((self.N, self.K // 2), dtype=torch.uint8, device=dev)
            self.scales = torch.empty((self.N, self.K // 128), dtype=torch.float16, device=dev)
        self.y = torch.empty((M, self.N), dtype=tdt, device=dev)
        self.t = torch.empty((M, w.r), dtype=torch.float32, device=dev)
        self.dx = torch.empty((M, self.K), dtype=tdt, device=dev)
        self.dA = torch.empty((self.K, w.r), dtype=torch.float32, device=dev)
        self.dB = torch.empty((w.r, self.N), dtype=torch.float32, device=dev)
        self.lin = Q.QLinear(self.K, self.N, w.r, w.alpha, w.wfmt, self.codes,
                             self.scales, self.A, self.B)
        self.cs = self.lin.cstruct()
        self.fmt = Q._FMT[w.wfmt]
        self.dt = Q.QLORA_BF16 if w.dtype == "bf16" else Q.QLORA_F32
        self.fwd_ws = Q.qlora_fwd_workspace(self.lin, M, self.dt)
        self.bwd_ws = Q.qlora_bwd_workspace(self.lin, M, self.dt)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(data-parallel, each GPU would run the same step on its own rows and "
              "all-reduce the adapter gradients)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_frozen_weight_amd import binding as Q
    from quantized_frozen_weight_amd import workloads as WL

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = Q.lib()
    w = WL.WORKLOADS[args.workload]
    if args.weights is not None and args.weights != w.wfmt:
        w = WL.with_format(w, args.weights)
    M = w.M
    layers = [Layer(w, i, dev) for i in range(len(w.layers))]
    ws_bytes = max(max(l.fwd_ws, l.bwd_ws) for l in layers)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    wsp = ws.data_ptr()

    def check(st, what):
        if st != 0:
            raise Q.QloraError(st, what)

    # one-time weight quantization (not part of the step)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream().cuda_stream
    e0.record()
    for l in layers:
        check(lib.qlora_quantize(l.W.data_ptr(), l.K, l.N, l.fmt, l.codes.data_ptr(),
                                 l.scales.data_ptr(), stream), "quantize")
    e1.record()
    torch.cuda.synchronize()
    quantize_ms = e0.elapsed_time(e1)

    # merging the trained adapter into the int8 weight (one-time, after
    # training; not part of the step), into separate buffers
    merge_ms = None
    if w.wfmt == "w8":
        outs = [(torch.empty_like(l.codes), torch.empty_like(l.scales)) for l in layers]

        def merge_all():
            for l, (c, sc) in zip(layers, outs):
                check(lib.qlora_merge(ctypes.byref(l.cs), c.data_ptr(), sc.data_ptr(), stream),
                      "merge")
        merge_all()
        torch.cuda.synchronize()
        e0.record()
        merge_all()
        e1.record()
        torch.cuda.synchronize()
        merge_ms = e0.elapsed_time(e1)

    # 4-bit layers: the forward alone per step, with the dequantized bf16
    # product (what the step uses) and with the integer int8 x int4 product
    fwd_ms = fwd_a8w4_ms = None
    if w.wfmt == "w4g128":
        st0 = torch.cuda.current_stream().cuda_stream

        def fwd_all(fn):
            for l in layers:
                check(fn(ctypes.byref(l.cs), M, l.dt, l.x.data_ptr(), l.y.data_ptr(),
                         l.t.data_ptr(), wsp, ws_bytes, st0), "fwd")

        for fn_name in ("qlora_fwd", "qlora_fwd_a8w4"):
            fn = getattr(lib, fn_name)
            fwd_all(fn)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(20):
                fwd_all(fn)
            e1.record()
            torch.cuda.synchronize()
            if fn_name == "qlora_fwd":
                fwd_ms = e0.elapsed_time(e1) / 20
            else:
                fwd_a8w4_ms = e0.elapsed_time(e1) / 20

    # Gemma workload: its attention query projection as the multi-head layer
    # the pages list (kernel [8, 2048, 256], B [8, 4, 256]), forward + backward,
    # next to the same tensors taken as a one-head layer
    heads_leg = None
    if w.cid == 4 and w.wfmt == "w8":
        heads_leg = multi_head_leg(torch, dev, lib, check, M)

    def step(ev_b=None, repeats=1):
        st = torch.cuda.current_stream().cuda_stream
        for i, l in enumerate(layers):
            check(lib.qlora_fwd_timed(ctypes.byref(l.cs), M, l.dt, l.x.data_ptr(),
                                      l.y.data_ptr(), l.t.data_ptr(), wsp, ws_bytes, st,
                                      1, None, None), "fwd")
        for i in reversed(range(len(layers))):
            l = layers[i]
            a, b = (ev_b[i] if ev_b else (None, None))
            check(lib.qlora_bwd_timed(ctypes.byref(l.cs), M, l.dt, l.x.data_ptr(),
                                      l.dy.data_ptr(), l.t.data_ptr(), l.dx.data_ptr(),
                                      l.dA.data_ptr(), l.dB.data_ptr(), wsp, ws_bytes, st,
                                      repeats if ev_b else 1, a, b), "bwd")

    # The timed step runs each layer's backward as qlora_bwd_partial (dx and
    # the adapter-gradient partial sums, into a workspace of its own) and
    # takes every layer's dA and dB at the end with qlora_bwd_finish_batch
    # (one launch per 32 layers) instead of one combine launch per layer.
    # The workspaces are packed: the layer run k-th (the backward runs the
    # layers in reverse) starts where the partial sums of the layers run
    # before it end, so its scratch lies only over layers not yet run.
    offs, o, total = {}, 0, 256
    for i in reversed(range(len(layers))):
        offs[i] = o
        total = max(total, o + layers[i].bwd_ws)
        o += Q.qlora_bwd_partials_bytes(layers[i].lin, M, layers[i].dt)
    bpack = torch.empty((total,), dtype=torch.uint8, device=dev)
    bws_ptr = [bpack.data_ptr() + offs[i] for i in range(len(layers))]
    bws_n = [layers[i].bwd_ws for i in range(len(layers))]
    items = (Q.qlora_finish_item * len(layers))()
    for i, l in enumerate(layers):
        items[i] = Q.qlora_finish_item(ctypes.cast(ctypes.pointer(l.cs), ctypes.c_void_p), M,
                                       l.dt, l.dA.data_ptr(), l.dB.data_ptr(),
                                       bws_ptr[i], bws_n[i])

    def step_batched():
        st = torch.cuda.current_stream().cuda_stream
        for l in layers:
            check(lib.qlora_fwd(ctypes.byref(l.cs), M, l.dt, l.x.data_ptr(), l.y.data_ptr(),
                                l.t.data_ptr(), wsp, ws_bytes, st), "fwd")
        for i in reversed(range(len(layers))):
            l = layers[i]
            check(lib.qlora_bwd_partial(ctypes.byref(l.cs), M, l.dt, l.x.data_ptr(),
                                        l.dy.data_ptr(), l.t.data_ptr(), l.dx.data_ptr(),
                                        bws_ptr[i], bws_n[i], st), "bwd_partial")
        check(lib.qlora_bwd_finish_batch(items, len(layers), st), "finish_batch")

    # eager warm-up (also loads every kernel)
    for _ in range(3):
        step()
        step_batched()
    torch.cuda.synchronize()

    use_graph = not args.no_graph

    def timed(fn):
        if use_graph:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                fn()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                fn()
            torch.cuda.synchronize()
            run = g.replay
        else:
            run = fn
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps, (time.perf_counter() - t0) * 1e3 / args.steps

    batched = args.finish == "batched" or (args.finish == "auto" and len(layers) >= 4)
    # the other variant first: the first timed loop after capture runs a few
    # percent slow (measured on the one-layer 4-bit step: either variant,
    # timed first, took about 8 us more), so it also warms the GPU for the
    # step that gives ``value``
    if batched:
        ms_l, wall_l = timed(step)
        ms_b, wall_b = timed(step_batched)
    else:
        ms_b, wall_b = timed(step_batched)
        ms_l, wall_l = timed(step)
    ms, wall_ms = (ms_b, wall_b) if batched else (ms_l, wall_l)
    ops = w.total_ops()
    value = ops / (ms * 1e-3) / 1e12

    # eager time per step, for reference (host launch cost included)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        (step_batched if batched else step)()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / 10

    if args.copy_calibration:
        copy_calibration(torch, dev)
    roof = dominant_kernel_roofline(w, layers, step, torch)
    cpu = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16" if w.dtype == "bf16" else "int8+f32",
        "data": "synthetic",
        "config": {
            "workload": describe(w),
            "rows": M,
            "layers": len(w.layers),
            "rank": w.r,
            "alpha": w.alpha,
            "weights": w.wfmt,
            "ops_per_step": ops,
            "hip_graph": use_graph,
        },
        "wall_ms_per_step": round(wall_ms, 5),
        "finish": "batched" if batched else "layerwise",
        "batched_finish_ms_per_step": round(ms_b, 5),
        "layerwise_finish_ms_per_step": round(ms_l, 5),
        "eager_ms_per_step": round(eager_ms, 5),
        "quantize_ms": round(quantize_ms, 4),
        "merge_ms": None if merge_ms is None else round(merge_ms, 4),
        "fwd_ms": None if fwd_ms is None else round(fwd_ms, 4),
        "fwd_a8w4_ms": None if fwd_a8w4_ms is None else round(fwd_a8w4_ms, 4),
        "attention_query_ms": heads_leg,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def describe(w):
    shapes = {}
    for K, N in w.layers:
        shapes[(K, N)] = shapes.get((K, N), 0) + 1
    s = ", ".join(f"{c}x{K}->{N}" if c > 1 else f"{K}->{N}" for (K, N), c in shapes.items())
    return f"{w.name}: {len(w.layers)} linears, {w.M} rows, {s}, {w.wfmt} weights, " \
           f"LoRA r={w.r} alpha={w.alpha:g}, {w.dtype} activations"


# HBM traffic of the dominant kernel per launch on the benchmarked workload,
# from two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), each divided by what the same counter reads per KiB of a plain
# 256 MiB device copy in the same run. Valid only for the kernel's device
# code it was taken on: the SHA-256 of the sources that define that kernel
# and of the compiler flags; otherwise reported as null.
TRAFFIC = {
    "workload": 2,
    "sources": ["gemm_bwd.hip", "ring.hpp", "common.hpp"],
    "sha256": "8133678b98566da0d06b65a24867ea3a24a5a79fc4dd5e7d9e138a33bd066289",
    "bytes_per_launch": 14781660,
}


def kernel_sources_sha256(names):
    import hashlib
    from quantized_frozen_weight_amd import build_lib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantized_frozen_weight_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    h.update(" ".join(build_lib.HIPCC_FLAGS).encode())
    return h.hexdigest()


def copy_calibration(torch, dev):
    """A plain device-to-device copy of 256 MiB, three times (its counters
    calibrate the HBM byte counters of the kernels in the same run)."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def multi_head_leg(torch, dev, lib, check, M, K=2048, heads=8, hd=256, r=4, reps=20):
    """fwd + bwd time (ms) of a [heads, K, hd] int8 layer with B [heads, r, hd],
    and of the same tensors as a one-head layer."""
    from quantized_frozen_weight_amd import binding as Q
    N = heads * hd
    g = torch.Generator().manual_seed(4000)
    W = (torch.randn((heads, K, hd), generator=g) * 0.02).to(dev)
    A = (torch.randn((K, r), generator=g) * 0.01).to(dev)
    B = (torch.randn((heads, r, hd), generator=g) * 0.01).to(dev)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16).to(dev)
    dy = torch.randn((M, N), generator=g).to(torch.bfloat16).to(dev)
    codes, scales = Q.qlora_quantize(W, "w8")
    out = {}
    for name, h in (("heads", heads), ("plain", 1)):
        lin = Q.QLinear(K, N, r, 16.0, "w8", codes, scales, A, B, heads=h)
        ws = torch.empty((max(Q.qlora_fwd_workspace(lin, M, Q.QLORA_BF16),
                              Q.qlora_bwd_workspace(lin, M, Q.QLORA_BF16)),),
                         dtype=torch.uint8, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        t = torch.empty((M, r), dtype=torch.float32, device=dev)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dA = torch.empty((K, r), dtype=torch.float32, device=dev)
        dB = torch.empty((r * N,), dtype=torch.float32, device=dev)
        cs = lin.cstruct()
        st = torch.cuda.current_stream().cuda_stream

        def once():
            check(lib.qlora_fwd(ctypes.byref(cs), M, Q.QLORA_BF16, x.data_ptr(), y.data_ptr(),
                                t.data_ptr(), ws.data_ptr(), ws.numel(), st), "fwd")
            check(lib.qlora_bwd(ctypes.byref(cs), M, Q.QLORA_BF16, x.data_ptr(), dy.data_ptr(),
                                t.data_ptr(), dx.data_ptr(), dA.data_ptr(), dB.data_ptr(),
                                ws.data_ptr(), ws.numel(), st), "bwd")
        once()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            once()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) / reps, 4)
    return out


def dominant_kernel_roofline(w, layers, step, torch):
    """Time the backward launch (the step's largest kernel) live.

    In one eager step the library launches each layer's backward kernel 20
    times back to back (same inputs, same outputs) between two HIP events
    that it records on the stream it launches on; the average duration is
    the summed intervals over all launches. Peak: dense bf16 MFMA (float32
    vector peak for the float32 workload). Algorithmic work per launch of the fused int8
    backward: 2 M K N for dx, 2 M N r each for u and dB, 2 M K r each for dA
    and the rank-r term of dx, i.e. 2 M K N + 4 M r (N + K) flops; peak: dense
    bf16 MFMA.
    """
    n = len(layers)
    repeats = 20
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    for a, b in pairs:         # materialize the events
        a.record(); b.record()
    torch.cuda.synchronize()
    step(ev_b=[(a.cuda_event, b.cuda_event) for a, b in pairs], repeats=repeats)
    torch.cuda.synchronize()
    tot_ms = sum(a.elapsed_time(b) for a, b in pairs)
    launches = n * repeats
    avg_ms = tot_ms / launches
    if w.dtype == "bf16":   # fused backward: dx, u, dB, dA, s u A^T
        flops = sum(2.0 * w.M * l.K * l.N + 4.0 * w.M * w.r * (l.N + l.K) for l in layers) / n
        # the library's tile choice: 128 x 128 blocks over a split contraction
        # (then a fixup launch) for at most 128 such tiles and N >= 2048;
        # else 64-row producer/consumer blocks while they make at most two
        # per compute unit, else 128 x 128 blocks
        bn = 128 if w.wfmt == "w4g128" else 64

        def bwd_name(l):
            if ((w.M + 127) // 128) * ((l.K + 127) // 128) <= 128 and (l.N + 63) // 64 >= 32:
                return "bwd_wide_kernel<SPLIT> + bwd_fixup_kernel"
            if ((w.M + 63) // 64) * ((l.K + bn - 1) // bn) <= 512:
                return "bwd_pc_kernel"
            return "bwd_wide_kernel"
        names = sorted({bwd_name(l) for l in layers})
        kernel = (" + ".join(names) + " (fused backward: dx, u, dA and dB partial sums, "
                  f"bf16 MFMA, {w.wfmt} weights)")
    else:                   # float32 input gradient: dy deq(W)^T + s u A^T
        flops = sum(2.0 * w.M * l.K * l.N + 2.0 * w.M * w.r * l.K for l in layers) / n
        kernel = "dx_f32_kernel (float32 input gradient)"
    achieved = flops / (avg_ms * 1e-3) / 1e12
    peak = PEAK["bf16" if w.dtype == "bf16" else "f32"] / 1e12
    traffic = None
    if (TRAFFIC["sha256"] is not None and w.cid == TRAFFIC["workload"]
            and kernel_sources_sha256(TRAFFIC["sources"]) == TRAFFIC["sha256"]):
        traffic = TRAFFIC["bytes_per_launch"]
    return {
        "kernel": kernel,
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "avg_launch_us": round(avg_ms * 1e3, 3),
        "launches_timed": launches,
        "flops_per_launch": flops,
    }


def cpu_baseline(w, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole layers (all rows), forward + backward, until the budget is used."""
    from oracle import qlora_oracle as O
    from quantized_frozen_weight_amd import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    done_ops, spent, n = 0, 0.0, 0
    for i in range(len(w.layers)):
        W, A, B = WL.weight(w, i), WL.lora_A(w, i), WL.lora_B(w, i)
        _, x = WL.as_compute_dtype(WL.activations(w, i), w.dtype)
        _, dy = WL.as_compute_dtype(WL.out_grad(w, i), w.dtype)
        if w.wfmt == "w8":
            c, s = O.quantize_w8(W)
        elif w.wfmt == "w8o":
            q = O.quantize_w8o(W)
        else:
            c, s = O.quantize_w4(W)
        t0 = time.perf_counter()
        if w.wfmt == "w8":
            O.fwd_w8(x, c, s, A, B, w.alpha, w.dtype)
            O.bwd(x, dy, O.dequant_w8(c, s), A, B, w.alpha, w.dtype)
        elif w.wfmt == "w8o":
            O.fwd_w8o(x, q, A, B, w.alpha, w.dtype)
            O.bwd(x, dy, O.dequant_w8o(q), A, B, w.alpha, w.dtype)
        else:
            O.fwd_w4(x, c, s, A, B, w.alpha, w.dtype)
            O.bwd(x, dy, O.dequant_w4(c, s), A, B, w.alpha, w.dtype)
        spent += time.perf_counter() - t0
        done_ops += w.ops_per_layer(*w.layers[i])
        n += 1
        if spent >= budget_s:
            break
    return {
        "value": round(done_ops / spent / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} of {len(w.layers)} layers, all {w.M} rows, fwd+bwd "
                  f"(numpy float64 oracle), {spent:.1f} s",
    }


if __name__ == "__main__":
    main()
