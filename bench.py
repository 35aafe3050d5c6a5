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

Prints ONE JSON line. Besides the contract keys it carries:
  * ``step_ms``: median, p10 and p90 over the timed steps, each replay
    timed by its own pair of events (``ms_per_step`` is the total over the
    timed steps divided by their number);
  * ``cold``: the same step with a 512 MiB device write before each one
    (outside the timed interval), so no input is left in the 256 MB
    last-level cache;
  * ``launch_floor``: the step graph's kernel count and the time of a
    graph of as many empty kernels;
  * ``peaks_measured``: dense bf16 and int8 MFMA throughput and HBM copy
    and read bandwidth, re-measured on this GPU by the library's probes;
  * ``roofline``: the dominant kernel (the fused backward) timed live with
    HIP events on the stream it is launched on, against the roof its
    algorithmic flops and bytes select (MFMA or HBM), and against the
    measured peak as well;
  * ``cpu_baseline``: the CPU oracle on a bounded sample of the workload,
    median of 3 runs at the host's thread count and at one thread.
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
# MI355X published peaks: dense bf16 and int8 MFMA, float32 vector ALU, HBM
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
                   help="also run the library's copy (256 MiB) and read (1 GiB) probes, "
                        "known byte counts for scaling HBM counters")
    p.add_argument("--cold-steps", type=int, default=30,
                   help="steps timed one by one after a 512 MiB flush (0: skip)")
    p.add_argument("--no-peaks", action="store_true", help="skip re-measuring the peaks")
    p.add_argument("--pmc-summary", metavar="DIR", default=None,
                   help="no GPU work: print the per-dispatch mean of every counter, per "
                        "kernel, from the counter_collection.csv files of a rocprofv3 "
                        "--pmc run written under DIR")
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
    if args.pmc_summary is not None:
        pmc_summary(args.pmc_summary)
        return
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
    # the in-tree build, and nothing else, is what runs
    loaded = Q.loaded_path()
    assert os.path.realpath(loaded) == os.path.realpath(Q.LIB_PATH), loaded
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

    def capture(fn):
        """The step as a HIP graph (replay function, graph node count)."""
        if not use_graph:
            return fn, None
        try:
            g = torch.cuda.CUDAGraph(keep_graph=True)
        except TypeError:  # pragma: no cover - older torch
            g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        nodes = graph_nodes(g)
        if hasattr(g, "instantiate"):
            g.instantiate()
        torch.cuda.synchronize()
        return g.replay, nodes

    def timed(fn):
        run, nodes = capture(fn)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        wall = (time.perf_counter() - t0) * 1e3 / args.steps
        # the same replays one by one, each between its own pair of events
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record()
        for i in range(args.steps):
            run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
        return ms, wall, per, run, nodes

    batched = args.finish == "batched" or (args.finish == "auto" and len(layers) >= 4)
    # the other variant first: the first timed loop after capture runs a few
    # percent slow (measured on the one-layer 4-bit step: either variant,
    # timed first, took about 8 us more), so it also warms the GPU for the
    # step that gives ``value``
    if batched:
        ms_l, wall_l, _, _, _ = timed(step)
        ms_b, wall_b, per, run, nodes = timed(step_batched)
    else:
        ms_b, wall_b, _, _, _ = timed(step_batched)
        ms_l, wall_l, per, run, nodes = timed(step)
    ms, wall_ms = (ms_b, wall_b) if batched else (ms_l, wall_l)
    ops = w.total_ops()
    value = ops / (ms * 1e-3) / 1e12
    step_stats = stats(per)

    # cold: a 512 MiB write before every step (outside its events), so that
    # none of the step's inputs is left in the 256 MB last-level cache
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)
        times = []
        for i in range(args.cold_steps + 2):
            flush.fill_(i & 0xff)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            torch.cuda.synchronize()
            if i >= 2:
                times.append(a.elapsed_time(b))
        del flush
        cold = dict(stats(times), flush_bytes=512 << 20)
        cold["tflops_median"] = round(ops / (cold["median_ms"] * 1e-3) / 1e12, 3)

    floor = launch_floor(torch, lib, check, nodes) if nodes else None

    # eager time per step, for reference (host launch cost included)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        (step_batched if batched else step)()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / 10

    if args.copy_calibration:
        copy_calibration(torch, dev, lib, check)
    peaks = None if args.no_peaks else measure_peaks(torch, dev, lib, check)
    roof = dominant_kernel_roofline(w, layers, step, torch, Q, peaks)
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
        "library": os.path.relpath(loaded, ROOT),
        "step_ms": step_stats,
        "cold": cold,
        "launch_floor": floor,
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
        "peaks_measured": peaks,
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


# HBM traffic of the dominant kernel per launch on the benchmarked workload
# (the MLP's fused backward, bwd_pc_kernel), averaged over its 32 layers like
# "achieved": 31 launches at 1024 -> 1024 (14.31 MB each) and one at
# 784 -> 1024 (29.56 MB). From two rocprofv3 counter passes (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch), each divided by what the same counter
# reads per KiB for the library's read probe (1 GiB, larger than the
# last-level cache) and copy probe (256 MiB) in the same runs. Valid only for
# the kernel's device code it was taken on: the SHA-256 of the sources that
# define that kernel and of the compiler flags; otherwise reported as null.
TRAFFIC = {
    "workload": 2,
    "weights": "w8",
    "sources": ["gemm_bwd.hip", "ring.hpp", "common.hpp"],
    "sha256": "0cc5ec7215c7463eaa7b5075f2ac045f1a34989fb63deb5a902953562410e936",
    "bytes_per_launch": 14798984,
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


def stats(times_ms):
    v = sorted(times_ms)
    q = lambda f: v[min(len(v) - 1, max(0, int(round(f * (len(v) - 1)))))]  # noqa: E731
    return {"median_ms": round(q(0.5), 5), "p10_ms": round(q(0.1), 5),
            "p90_ms": round(q(0.9), 5), "samples": len(v)}


def graph_nodes(g):
    """Node count of a captured graph (kernel launches: the library records
    nothing else), from the HIP runtime the process has mapped."""
    try:
        raw = g.raw_cuda_graph()
        path = next((ln.split()[-1] for ln in open("/proc/self/maps")
                     if ln.rstrip().endswith("libamdhip64.so") or "libamdhip64.so." in ln),
                    "libamdhip64.so")
        hip = ctypes.CDLL(path)
        n = ctypes.c_size_t(0)
        if hip.hipGraphGetNodes(ctypes.c_void_p(raw), None, ctypes.byref(n)) != 0:
            return None
        return int(n.value)
    except Exception:  # pragma: no cover - API not available
        return None


def launch_floor(torch, lib, check, nodes, reps=20):
    """Time of a graph of `nodes` empty kernels (256 blocks of 256 threads):
    what the step's launches cost with no work in them."""
    st = torch.cuda.current_stream().cuda_stream
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        check(lib.qlora_probe_empty(256, 256, s.cuda_stream), "probe_empty")
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for _ in range(nodes):
            check(lib.qlora_probe_empty(256, 256, cs), "probe_empty")
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del st
    ms = e0.elapsed_time(e1) / reps
    return {"kernels_per_step": nodes, "empty_kernel_us": round(ms * 1e3 / nodes, 3),
            "floor_ms_per_step": round(ms, 5)}


def measure_peaks(torch, dev, lib, check):
    """Dense MFMA throughput (bf16, int8) and HBM copy / read bandwidth on
    this GPU, from the library's probes (best of 5 launches each)."""
    st = torch.cuda.current_stream().cuda_stream
    out = torch.empty((4096 * 256,), dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn, n=5):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(n):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e-3)
        return min(t)

    res = {}
    for kind, key in ((0, "bf16_mfma_tflops"), (1, "int8_mfma_tops")):
        ops = ctypes.c_double()
        blocks, iters = 2048, 1000
        t = best(lambda: check(lib.qlora_probe_mfma(kind, blocks, iters, out.data_ptr(), st,
                                                      ctypes.byref(ops)), "probe_mfma"))
        res[key] = round(ops.value / t / 1e12, 1)
    nbytes = 1 << 30
    src = torch.empty((nbytes,), dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    t = best(lambda: check(lib.qlora_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, 4096, st),
                           "probe_copy"))
    res["hbm_copy_gbs"] = round(2 * nbytes / t / 1e9, 1)
    del dst
    big = torch.empty((4 * nbytes,), dtype=torch.uint8, device=dev).fill_(2)
    red = torch.empty((4096 * 256 * 16,), dtype=torch.uint8, device=dev)
    t = best(lambda: check(lib.qlora_probe_read(big.data_ptr(), 4 * nbytes, 4096, red.data_ptr(), st),
                           "probe_read"))
    res["hbm_read_gbs"] = round(4 * nbytes / t / 1e9, 1)
    res["how"] = ("best of 5 launches: 2048 blocks x 4 waves x 1000 rounds of 8 independent "
                  "MFMAs; 1 GiB copy (2 GiB moved); 4 GiB read")
    return res


def copy_calibration(torch, dev, lib, check):
    """Kernels of known HBM traffic, for scaling the byte counters of a
    counter pass: the copy probe over 256 MiB (256 MiB read, 256 MiB
    written) three times, and the read probe over 1 GiB (1 GiB read, larger
    than the last-level cache) three times."""
    st = torch.cuda.current_stream().cuda_stream
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        check(lib.qlora_probe_copy(src.data_ptr(), dst.data_ptr(), n, 4096, st), "probe_copy")
    big = torch.empty(4 * n, dtype=torch.uint8, device=dev).fill_(2)
    red = torch.empty((4096 * 256 * 16,), dtype=torch.uint8, device=dev)
    for _ in range(3):
        check(lib.qlora_probe_read(big.data_ptr(), 4 * n, 4096, red.data_ptr(), st), "probe_read")
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


def dominant_kernel_roofline(w, layers, step, torch, Q, peaks):
    """Time the backward launch (the step's largest kernel) live, and place
    it on the roofline.

    In one eager step the library launches each layer's backward kernel 20
    times back to back (same inputs, same outputs) between two HIP events
    that it records on the stream it launches on; the average duration is
    the summed intervals over all launches.

    Algorithmic work per launch, averaged over the layers:
      * flops of the fused bf16 backward: 2 M K N for dx, 2 M N r each for u
        and dB, 2 M K r each for dA and the rank-r term of dx, i.e.
        2 M K N + 4 M r (N + K); of the float32 input gradient 2 M K N +
        2 M K r;
      * bytes of a backward: dy, codes, scales, x, t, A, B read, dx, dA, dB
        written, each once.
    The roof is the one these select: compute when flops / peak exceeds
    bytes / HBM bandwidth, else HBM. Compute is the dense bf16 MFMA peak for
    the bf16 backward ("mfma"); the float32 input gradient is an FMA kernel
    on the vector ALUs ("alu"), against the published float32 vector peak
    (256 CUs x 4 SIMDs x 16 lanes x 2 (packed) x 2 (FMA) x 2.4 GHz = 157.3
    TFLOP/s; code without packed float32 instructions, like this library's,
    can reach half of it). ``frac`` is the kernel's fraction of that roof,
    ``frac_measured`` the same against the peak re-measured on this GPU
    (MFMA and HBM only).
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
    avg_s = tot_ms / launches * 1e-3
    M, r = w.M, w.r
    xb = 2 if w.dtype == "bf16" else 4                 # bytes per activation
    cb = {"w8": 1.0, "w8o": 1.0, "w4g128": 0.5}[w.wfmt]
    flops = nbytes = 0.0
    for l in layers:
        K, N = l.K, l.N
        if w.dtype == "bf16":
            flops += 2.0 * M * K * N + 4.0 * M * r * (N + K)
        else:
            flops += 2.0 * M * K * N + 2.0 * M * K * r
        scale_b = 4.0 * N if w.wfmt == "w8" else (2.0 * N * K / 128 if w.wfmt == "w4g128" else 0.0)
        nbytes += (xb * M * N + cb * K * N + scale_b + xb * M * K + 4.0 * M * r + 4.0 * K * r
                   + 4.0 * r * N + xb * M * K + 4.0 * K * r + 4.0 * r * N)
    flops /= n
    nbytes /= n
    mfma_peak = PEAK["bf16" if w.dtype == "bf16" else "f32"]
    t_mfma, t_hbm = flops / mfma_peak, nbytes / PEAK["hbm"]
    compute = "mfma" if w.dtype == "bf16" else "alu"
    bound = compute if t_mfma >= t_hbm else "hbm"
    names = sorted({Q.qlora_bwd_main_kernel(l.lin, M, l.dt) for l in layers})
    kernel = " + ".join(names) + (f" ({w.wfmt} weights, {w.dtype})")
    if bound != "hbm":
        achieved, peak, unit = flops / avg_s / 1e12, mfma_peak / 1e12, "TFLOP/s"
        mpeak = peaks.get("bf16_mfma_tflops") if (peaks and w.dtype == "bf16") else None
    else:
        achieved, peak, unit = nbytes / avg_s / 1e9, PEAK["hbm"] / 1e9, "GB/s"
        mpeak = peaks.get("hbm_read_gbs") if peaks else None
    traffic = None
    if (TRAFFIC["sha256"] is not None and w.cid == TRAFFIC["workload"]
            and w.wfmt == TRAFFIC["weights"]
            and kernel_sources_sha256(TRAFFIC["sources"]) == TRAFFIC["sha256"]):
        traffic = TRAFFIC["bytes_per_launch"]
    return {
        "kernel": kernel,
        "bound": bound,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "avg_launch_us": round(avg_s * 1e6, 3),
        "launches_timed": launches,
        "flops_per_launch": flops,
        "bytes_per_launch": nbytes,
        "mfma_frac": round(flops / avg_s / mfma_peak, 4),
        "hbm_frac": round(nbytes / avg_s / PEAK["hbm"], 4),
        "roofline_us": round(max(t_mfma, t_hbm) * 1e6, 3),
        "frac_measured": None if not mpeak else round(achieved / mpeak, 4),
        "measured_peak": mpeak,
    }


def cpu_baseline(w, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same
    workload: whole layers (all rows), forward + backward. The sample is
    the first layers whose one run fits about budget_s / 6; it runs three
    times at the host's thread count and (its first layer) three times at
    one thread; medians are reported."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import qlora_oracle as O
    from quantized_frozen_weight_amd import workloads as WL
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])

    prepared = []

    def layer_inputs(i):
        W, A, B = WL.weight(w, i), WL.lora_A(w, i), WL.lora_B(w, i)
        _, x = WL.as_compute_dtype(WL.activations(w, i), w.dtype)
        _, dy = WL.as_compute_dtype(WL.out_grad(w, i), w.dtype)
        if w.wfmt == "w8":
            q = O.quantize_w8(W)
        elif w.wfmt == "w8o":
            q = O.quantize_w8o(W)
        else:
            q = O.quantize_w4(W)
        return x, dy, q, A, B

    def run_layer(x, dy, q, A, B):
        if w.wfmt == "w8":
            O.fwd_w8(x, q[0], q[1], A, B, w.alpha, w.dtype)
            O.bwd(x, dy, O.dequant_w8(*q), A, B, w.alpha, w.dtype)
        elif w.wfmt == "w8o":
            O.fwd_w8o(x, q, A, B, w.alpha, w.dtype)
            O.bwd(x, dy, O.dequant_w8o(q), A, B, w.alpha, w.dtype)
        else:
            O.fwd_w4(x, q[0], q[1], A, B, w.alpha, w.dtype)
            O.bwd(x, dy, O.dequant_w4(*q), A, B, w.alpha, w.dtype)

    def run(sample):
        t0 = time.perf_counter()
        for args in sample:
            run_layer(*args)
        return time.perf_counter() - t0

    # the sample: layers until one pass takes about budget / 6
    spent = 0.0
    for i in range(len(w.layers)):
        prepared.append(layer_inputs(i))
        spent += run([prepared[-1]])
        if spent >= budget_s / 6:
            break
    ops = sum(w.ops_per_layer(*w.layers[i]) for i in range(len(prepared)))
    full = sorted(run(prepared) for _ in range(3))[1]
    with threadpool_limits(limits=1):
        one = sorted(run(prepared[:1]) for _ in range(3))[1]
    ops1 = w.ops_per_layer(*w.layers[0])
    return {
        "value": round(ops / full / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(prepared)} of {len(w.layers)} layers, all {w.M} rows, fwd+bwd "
                  f"(numpy float64 oracle), median of 3 runs of {full:.2f} s",
        "value_1thread": round(ops1 / one / 1e12, 5),
        "sample_1thread": f"layer 0, median of 3 runs of {one:.2f} s",
    }


def pmc_summary(d):
    """Per-kernel table of a rocprofv3 --pmc run: for each kernel (name, grid,
    workgroup) the number of dispatches and, per counter, the mean and the
    median over dispatches of the counter's value summed over its instances
    (shader engines, channels) within a dispatch."""
    import collections
    import csv
    import glob
    import re
    rows = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = re.sub(r"\(.*", "", row.get("Kernel_Name", "")
                              .replace("(anonymous namespace)::", "").replace("qlora::", ""))
                key = (name, row.get("Grid_Size"), row.get("Workgroup_Size"))
                rows[key][row["Counter_Name"]][row.get("Dispatch_Id")] += float(row["Counter_Value"])
    print("| kernel | grid | wg | dispatches | counter | mean | median |")
    print("|---|---|---|---|---|---|---|")
    order = sorted(rows.items(), key=lambda kv: -max(len(v) for v in kv[1].values()))
    for (name, grid, wg), counters in order:
        for c, per in sorted(counters.items()):
            v = sorted(per.values())
            print(f"| {name} | {grid} | {wg} | {len(v)} | {c} | {sum(v) / len(v):.6g} "
                  f"| {v[len(v) // 2]:.6g} |")


if __name__ == "__main__":
    main()
