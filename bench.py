#!/usr/bin/env python3
"""Benchmark of the N:M bitmask sparse GEMV on one MI355X.

Workload: the seven linear projections of one Llama-3.1-8B-shaped decoder
layer (q, o 4096x4096; k, v 1024x4096; gate, up 14336x4096; down 4096x14336),
each a seeded synthetic 2:4 fp16 matrix (weights N(0, 0.02), the 2 largest
|w| of every 4 kept), x ~ N(0, 1) with 0.1% outlier channels x20, batch 1.
A step is one pass of the hot path over the layer: the seven nm_spmv calls.

Measurement:
* every projection has its own rotation of packed copies totalling >= 1 GiB,
  so no call finds its weights in the 256 MiB Infinity Cache or in L2;
* the steps' launches are captured in HIP graphs of several consecutive
  steps each (the kernels are a few microseconds long, shorter than a Python
  launch, and a graph replay costs about 10 us of its own), as a decode loop
  captures a token's layers; the value is the strictly serial chain of the
  seven launches; a graph that follows the layer's data flow (q, k, v as
  parallel branches, then o, then gate and up in parallel, then down) and
  the serial chain at one graph per step are timed beside it;
* the K timed steps are bracketed by torch.cuda.synchronize() and HIP events;
* per-kernel duration: a graph of at least 128 back-to-back launches of one
  projection cycling over its rotation, HIP events around each replay,
  divided by the launches;
* value = algorithmic bytes of the layer (packed values + mask words + x + y,
  each moved once) / step time.
The dense comparison runs the same protocol with nm_dense_gemv and with
torch.nn.functional.linear on dense copies.  The CPU baseline times the oracle
(fp64 dense-masked product) on the same layer on the host cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_gemv_memory_amd import native, synth, workloads  # noqa: E402

METRIC = "µs/call and achieved HBM GB/s (% of peak) for 2:4 sparse GEMV, batch 1"
PEAK_GBS = 8000.0  # MI355X HBM3E, published
ROTATE_BYTES = 1 << 30
DEV = torch.device("cuda:0")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def t16(a, dtype="f16"):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(DEV)


def pow2_copies(nbytes):
    return max(2, 1 << math.ceil(math.log2(max(1.0, ROTATE_BYTES / nbytes))))


class Proj:
    """One projection: host inputs, packed rotation copies, dense copies."""

    def __init__(self, mt, batches, want_dense):
        self.mt = mt
        self.name = mt.name
        t0 = time.time()
        self.W = synth.weights(mt.rows, mt.cols, seed=mt.seed, dtype=mt.dtype)
        self.keep = synth.topn_mask(self.W, mt.n, mt.m)
        self.X = {b: synth.activations(b, mt.cols, seed=mt.seed, dtype=mt.dtype, outliers=mt.outliers)
                  for b in batches}
        Wd = t16(self.W, mt.dtype)
        values, bits = native.nm_pack(Wd, torch.from_numpy(self.keep).to(DEV), mt.n, mt.m)
        self.sbytes = {b: workloads.sparse_bytes(mt.rows, mt.cols, mt.n, mt.m, b, 4) for b in batches}
        self.dbytes = {b: workloads.dense_bytes(mt.rows, mt.cols, b, 4) for b in batches}
        packed = values.numel() * 2 + bits.numel() * 4
        self.nc = pow2_copies(packed)
        self.vals = [values] + [native.clone_packed(values) for _ in range(self.nc - 1)]
        self.bits = [bits] + [bits.clone() for _ in range(self.nc - 1)]
        self.ndc = pow2_copies(Wd.numel() * 2) if want_dense else 0
        self.dense = ([Wd] + [Wd.clone() for _ in range(self.ndc - 1)]) if want_dense else []
        if not want_dense:
            del Wd
        self.Xd = {b: t16(self.X[b], mt.dtype) for b in batches}
        self.Y = {b: torch.empty((b, mt.rows), dtype=torch.float32, device=DEV) for b in batches}
        self.args = {}
        log(f"  {self.name:5s} {mt.rows}x{mt.cols}: {self.nc} packed copies "
            f"({self.nc * packed / 2**30:.2f} GiB), {self.ndc} dense copies, {time.time() - t0:.1f}s")

    def sparse_call(self, b, c):
        """Launch the sparse product on copy c at batch b (raw C call)."""
        L = native.lib()
        mt = self.mt
        dt = native.NM_BF16 if mt.dtype == "bf16" else native.NM_F16
        st = L.nm_spmm_small(self.vals[c].data_ptr(), self.bits[c].data_ptr(), self.Xd[b].data_ptr(),
                             self.Y[b].data_ptr(), b, mt.rows, mt.cols, mt.n, mt.m, dt,
                             native.NM_F32, torch.cuda.current_stream().cuda_stream) if b > 1 else \
            L.nm_spmv(self.vals[c].data_ptr(), self.bits[c].data_ptr(), self.Xd[b].data_ptr(),
                      self.Y[b].data_ptr(), mt.rows, mt.cols, mt.n, mt.m, dt,
                      native.NM_F32, torch.cuda.current_stream().cuda_stream)
        if st != native.NM_OK:
            raise native.NMError(st, f"{self.name} sparse b={b}")

    def dense_call(self, b, c):
        L = native.lib()
        mt = self.mt
        dt = native.NM_BF16 if mt.dtype == "bf16" else native.NM_F16
        st = L.nm_dense_gemv(self.dense[c].data_ptr(), self.Xd[b].data_ptr(), self.Y[b].data_ptr(), b,
                             mt.rows, mt.cols, dt, native.NM_F32,
                             torch.cuda.current_stream().cuda_stream)
        if st != native.NM_OK:
            raise native.NMError(st, f"{self.name} dense b={b}")

    def torch_call(self, b, c):
        torch.nn.functional.linear(self.Xd[b], self.dense[c])


def capture(fn):
    """Capture fn() (a few kernel launches) into a HIP graph."""
    fn()  # eager run first: initialises everything outside capture
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def time_steps(graphs, steps, warmup, per_graph=1):
    """Replay graphs (each holding per_graph consecutive steps) in turn for
    warmup + steps steps; return ms per timed step."""
    n = len(graphs)
    nw, nt = warmup // per_graph, steps // per_graph
    for i in range(nw):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(nt):
        graphs[(nw + i) % n].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (nt * per_graph)


def steps_per_graph(steps, warmup, cap=16):
    """The largest count <= cap that divides both the timed and the warm-up
    step counts, so both are whole graphs."""
    g = math.gcd(steps, warmup)
    return max(d for d in range(1, cap + 1) if g % d == 0)


# The layer's data flow: q, k, v read the same x and are independent; o
# follows them; gate and up read the same x; down follows them.
LAYER_STAGES = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
_side = []


def chain_graphs(projs, call, b, nsteps, copies_attr, parallel=True, per_graph=1):
    """Graphs of per_graph consecutive steps each (step s on rotation copy s).
    parallel: the independent projections of a stage run on side streams
    (default priority) as parallel graph branches; otherwise the seven
    launches of a step form one serial chain."""
    by_name = {p.name: p for p in projs}
    while len(_side) < 2:
        _side.append(torch.cuda.Stream())

    def one_step(s):
        if not parallel:
            for p in projs:
                call(p, b, s % getattr(p, copies_attr))
            return
        main = torch.cuda.current_stream()
        for stage in LAYER_STAGES:
            side = _side[:len(stage) - 1]
            for st in side:
                st.wait_stream(main)
            call(by_name[stage[0]], b, s % getattr(by_name[stage[0]], copies_attr))
            for name, st in zip(stage[1:], side):
                with torch.cuda.stream(st):
                    call(by_name[name], b, s % getattr(by_name[name], copies_attr))
            for st in side:
                main.wait_stream(st)

    graphs = []
    for g0 in range(0, nsteps, per_graph):
        graphs.append(capture(lambda g0=g0: [one_step(s) for s in range(g0, g0 + per_graph)]))
    return graphs


# A replay of a graph costs about 10 us beyond its kernels (launch and the
# end-of-graph release); 128 back-to-back launches make that < 0.1 us each.
MIN_LAUNCHES_PER_REPLAY = 128


def per_kernel_stats(p, call, b, ncopies, reps):
    """Duration of one launch: a graph of back-to-back launches cycling over
    the projection's rotation (at least MIN_LAUNCHES_PER_REPLAY launches, so
    the graph's own launch cost spreads thin), HIP events around each replay,
    divided by the launch count.  Returns the median over the replays and their 10th and
    90th percentiles (µs per launch); per-dispatch percentiles come from the
    profiler's kernel trace (--summarize-trace)."""
    launches = ncopies * max(1, -(-MIN_LAUNCHES_PER_REPLAY // ncopies))
    g = capture(lambda: [call(p, b, c % ncopies) for c in range(launches)])
    g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, z in evs:
        a.record()
        g.replay()
        z.record()
    torch.cuda.synchronize()
    us = 1e3 * np.array([a.elapsed_time(z) for a, z in evs]) / launches
    return {"us": float(np.median(us)), "p10": float(np.percentile(us, 10)),
            "p90": float(np.percentile(us, 90))}


def per_kernel_us(p, call, b, ncopies, reps):
    """Median duration of one launch (see per_kernel_stats)."""
    return per_kernel_stats(p, call, b, ncopies, reps)["us"]


def cpu_baseline(projs, gpu_y, min_cpu_seconds=10.0):
    """The oracle on the whole layer at batch 1, on the host cores; projs are
    (name, W, keep, X, sbytes) of the layer's projections."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = max(1, min(threads, os.cpu_count() or 1))
    total_bytes = sum(sb[1] for _, _, _, _, sb in projs)
    reps, wall = 0, 0.0
    errs = {}
    while True:
        t0 = time.perf_counter()
        for name, W, keep, X, _ in projs:
            y = oracle.masked_gemv(W, keep, X[1], False, threads=threads)
            if reps == 0:
                got = gpu_y[name].astype(np.float64)
                errs[name] = float(np.linalg.norm(got - y[0]) / np.linalg.norm(y[0]))
        wall += time.perf_counter() - t0
        reps += 1
        if wall * threads >= min_cpu_seconds or reps >= 20:
            break
    sec_per_layer = wall / reps
    # one core: the same layer pass once more with a single thread (the
    # per-row summation order is the same, so the result is identical)
    t0 = time.perf_counter()
    for _, W, keep, X, _ in projs:
        oracle.masked_gemv(W, keep, X[1], False, threads=1)
    sec_1 = time.perf_counter() - t0
    return {
        "value": total_bytes / sec_per_layer / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"the whole workload: all 7 projections of the layer at batch 1, {reps} passes "
                   f"on {threads} threads and 1 pass on one thread (fp64 dense-masked product, "
                   f"C + OpenMP over rows); {1e6 * sec_per_layer:.0f} us per layer pass"),
        "us_per_step": 1e6 * sec_per_layer,
        "single_core": {"value": total_bytes / sec_1 / 1e9, "unit": "GB/s", "cores": 1,
                        "us_per_step": 1e6 * sec_1},
        "gpu_vs_oracle_rel_l2": errs,
        "host": platform.processor() or platform.machine(),
        "host_cpus": os.cpu_count(),
    }


# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of
# `bench.py --counters`, each scaled by the same counter's reading for a plain
# 64 MiB copy (fetch x 2.0, write x 1.0), keyed by the SHA-256 of the kernel
# source they were taken on.  Any change to the source makes the figure stale,
# and it is then reported as null.
MEASURED_TRAFFIC = {
    # (rows, cols): (kernel_digest() when measured, bytes per launch) at batch
    # 1; see profiles/nm_spmv_2of4_hbm_counters.md
    (14336, 4096): ("5ddfbc6d4d2838a4f4a6857beb7bb3b319bd12e7a16d221176aa3ddb675658c0",
                    66268478),
    (8192, 8192): ("5ddfbc6d4d2838a4f4a6857beb7bb3b319bd12e7a16d221176aa3ddb675658c0",
                   75736120),
}


def code_digest(text: str) -> str:
    """SHA-256 of C/C++ source with comments removed and whitespace collapsed,
    so that an edit of comments alone keeps the digest of the measured code."""
    import hashlib
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def kernel_digest():
    """code_digest of the product kernels' source: nm_sparse.hip and the
    device helpers it includes."""
    csrc = os.path.join(ROOT, "sparse_gemv_memory_amd", "csrc")
    return code_digest("".join(open(os.path.join(csrc, f)).read()
                               for f in ("nm_sparse.hip", "nm_device.h")))


def measured_traffic(rows, cols):
    digest = kernel_digest()
    entry = MEASURED_TRAFFIC.get((rows, cols))
    if entry and entry[0] == digest:
        return entry[1]
    return None


def counters_run():
    """Eager launches with known byte counts, for hardware-counter passes:
    the 14336x4096 layer at batch 1 (VALU row kernel) and 8 (matrix cores),
    the 8192x8192 layer at batch 1, then plain copies of known size."""
    mt = [m for m, _ in workloads.config_matrices(2) if m.name == "gate"][0]
    p = Proj(mt, (1, 8), False)
    torch.cuda.synchronize()
    for b in (1, 8):  # batch 1: the VALU row kernel; batch 8: the matrix-core kernel
        for c in range(5):
            p.sparse_call(b, c)
        torch.cuda.synchronize()
    mq = [m for m, _ in workloads.config_matrices(4) if m.name == "70b.q"][0]
    q = GpuProj(mq, False)
    torch.cuda.synchronize()
    for c in range(5):
        q.sparse_call(1, c)
    torch.cuda.synchronize()
    n = 64 << 20
    src = torch.empty(n, dtype=torch.uint8, device=DEV).fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"q8192_bytes_per_launch": q.sbytes[1],
                      "q8192_write_bytes": mq.rows * 4,
                      "sparse_kernel_bytes_per_launch": p.sbytes[1],
                      "sparse_kernel_read_bytes": p.sbytes[1] - mt.rows * 4,
                      "sparse_kernel_write_bytes": mt.rows * 4,
                      "batch8_bytes_per_launch": p.sbytes[8],
                      "batch8_write_bytes": 8 * mt.rows * 4,
                      "copy_bytes_each_way": n}), flush=True)


def shapes_run(cfg_id, args, mats=None):
    """Workloads 1, 3 and 4 (and the other densities): per-matrix µs/call and
    GB/s (cache-cold rotation), sparse and dense, at every batch the workload
    lists."""
    want_dense = not args.no_dense
    rows_out = []
    for mt, batches in (mats if mats is not None else workloads.config_matrices(cfg_id)):
        p = Proj(mt, batches, want_dense)
        for b in batches:
            us = per_kernel_us(p, Proj.sparse_call, b, p.nc, args.reps)
            row = {"matrix": mt.name, "rows": mt.rows, "cols": mt.cols, "pattern": f"{mt.n}:{mt.m}",
                   "dtype": mt.dtype, "batch": b, "us": round(us, 3),
                   "GB/s": round(p.sbytes[b] / us / 1e3, 1),
                   "frac_of_peak": round(p.sbytes[b] / us / 1e3 / PEAK_GBS, 4)}
            if want_dense:
                dus = per_kernel_us(p, Proj.dense_call, b, p.ndc, args.reps)
                tus = per_kernel_us(p, Proj.torch_call, b, p.ndc, args.reps)
                row.update({"dense_us": round(dus, 3), "torch_linear_us": round(tus, 3),
                            "speedup_vs_best_dense": round(min(dus, tus) / us, 3)})
            rows_out.append(row)
            log(f"  {mt.name:14s} {mt.rows:5d}x{mt.cols:5d} {mt.n}:{mt.m} {mt.dtype} b={b}: {us:8.2f} us "
                f"{row['GB/s']:7.1f} GB/s ({100 * row['frac_of_peak']:.1f}%)"
                + (f"  dense {row['dense_us']:.2f} torch {row['torch_linear_us']:.2f}" if want_dense else ""))
        del p
        torch.cuda.empty_cache()
    return rows_out


def bitmask_run(args):
    """Unstructured 50% bitmasks (per-row largest half) on the 8B gate and down
    shapes, batch 1 and 8: µs/call and GB/s, cache-cold rotation, against the
    2:4 kernel's bytes and the dense products."""
    out = []
    for i, (name, rows, cols) in enumerate(workloads.LLAMA8B_LAYER):
        if name not in ("gate", "down"):
            continue
        seed = synth.layer_seed(7, 0, i)
        W = synth.weights(rows, cols, seed=seed)
        keep = synth.topk_row_mask(W, 0.5)
        Wd = t16(W)
        values, bits, offs = native.nm_pack_bitmask(Wd, torch.from_numpy(keep).to(DEV))
        nbytes_w = values.numel() * 2 + bits.numel() * 4 + offs.numel() * 8
        nc = pow2_copies(nbytes_w)
        vals = [values] + [native.clone_packed(values) for _ in range(nc - 1)]
        bts = [bits] + [bits.clone() for _ in range(nc - 1)]
        ndc = pow2_copies(Wd.numel() * 2)
        dense = [Wd] + [Wd.clone() for _ in range(ndc - 1)]
        for b in (1, 8):
            X = t16(synth.activations(b, cols, seed=seed))
            Y = torch.empty((b, rows), dtype=torch.float32, device=DEV)
            L = native.lib()

            def call(c, X=X, Y=Y, b=b):
                st = L.nm_spmm_bitmask(vals[c].data_ptr(), bts[c].data_ptr(), offs.data_ptr(),
                                       X.data_ptr(), Y.data_ptr(), b, rows, cols, native.NM_F16,
                                       native.NM_F32, torch.cuda.current_stream().cuda_stream)
                if st != native.NM_OK:
                    raise native.NMError(st, "nm_spmm_bitmask")

            def dcall(c, X=X, Y=Y, b=b):
                st = L.nm_dense_gemv(dense[c].data_ptr(), X.data_ptr(), Y.data_ptr(), b, rows, cols,
                                     native.NM_F16, native.NM_F32, torch.cuda.current_stream().cuda_stream)
                if st != native.NM_OK:
                    raise native.NMError(st, "nm_dense_gemv")

            g = capture(lambda: [call(c) for c in range(nc)])
            gd = capture(lambda: [dcall(c) for c in range(ndc)])
            gt = capture(lambda: [torch.nn.functional.linear(X, dense[c]) for c in range(ndc)])
            res = {}
            for key, graph, n in (("us", g, nc), ("dense_us", gd, ndc), ("torch_linear_us", gt, ndc)):
                graph.replay()
                torch.cuda.synchronize()
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(args.reps)]
                for a, z in evs:
                    a.record()
                    graph.replay()
                    z.record()
                torch.cuda.synchronize()
                res[key] = round(1e3 * float(np.median([a.elapsed_time(z) for a, z in evs])) / n, 3)
            nbytes = nbytes_w + b * cols * 2 + b * rows * 4
            row = {"matrix": f"{name} 50% unstructured", "rows": rows, "cols": cols, "batch": b,
                   "bytes": nbytes, **res, "GB/s": round(nbytes / res["us"] / 1e3, 1),
                   "frac_of_peak": round(nbytes / res["us"] / 1e3 / PEAK_GBS, 4)}
            out.append(row)
            log(f"  {name:5s} {rows}x{cols} 50% unstructured b={b}: {res['us']:8.2f} us "
                f"{row['GB/s']:7.1f} GB/s ({100 * row['frac_of_peak']:.1f}%)  dense {res['dense_us']:.2f} "
                f"torch {res['torch_linear_us']:.2f}")
        del vals, bts, dense
        torch.cuda.empty_cache()
    return out


def pack_gpu(W, n, m):
    """nm_pack of a GPU fp16 matrix under the top-n |w| of every m mask
    (ties to the lower column), the mask drawn on the GPU."""
    rows, cols = W.shape
    mag = W.abs().view(rows, cols // m, m).float()
    pos = torch.arange(m, device=DEV, dtype=torch.float32) * 1e-9
    idx = (mag - pos).topk(n, dim=-1).indices
    keep = torch.zeros((rows, cols // m, m), dtype=torch.uint8, device=DEV)
    keep.scatter_(-1, idx, 1)
    return native.nm_pack(W, keep.view(rows, cols), n, m)


def gpu_layer(rows, cols, n, m, seed, want_dense, dtype="f16"):
    """A seeded synthetic matrix drawn on the GPU (timing only: the kernels'
    time does not depend on the values): W = fp16 or bf16 of 0.02 z, the n
    largest |w| of every m kept (ties to the lower column), packed by
    nm_pack."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    W = (torch.randn((rows, cols), device=DEV, generator=g) * 0.02).to(
        torch.bfloat16 if dtype == "bf16" else torch.float16)
    values, bits = pack_gpu(W, n, m)
    return values, bits, (W if want_dense else None)


# The 2:4 layers of 14336x4096 weights and more besides the 8B layer's own:
# the Llama-3.3-70B and Qwen3-32B projections of workload 4 with at least
# 58.7 M weights, timed at batch 1 in the default run.
LARGE_LAYERS = ("70b.q", "70b.gate", "70b.down", "qwen32b.gate", "qwen32b.down")


class GpuProj(Proj):
    """A 2:4 fp16 projection drawn and packed on the GPU (gpu_layer; the
    kernels' time does not depend on the values), x drawn as in Proj, with
    Proj's rotation of packed and dense copies and its launch calls."""

    def __init__(self, mt, want_dense):
        self.mt, self.name = mt, mt.name
        t0 = time.time()
        values, bits, W = gpu_layer(mt.rows, mt.cols, mt.n, mt.m, mt.seed, want_dense, mt.dtype)
        packed = values.numel() * 2 + bits.numel() * 4
        self.nc = pow2_copies(packed)
        self.vals = [values] + [native.clone_packed(values) for _ in range(self.nc - 1)]
        self.bits = [bits] + [bits.clone() for _ in range(self.nc - 1)]
        self.ndc = pow2_copies(W.numel() * 2) if want_dense else 0
        self.dense = ([W] + [W.clone() for _ in range(self.ndc - 1)]) if want_dense else []
        self.X = {1: synth.activations(1, mt.cols, seed=mt.seed, dtype=mt.dtype, outliers=True)}
        self.Xd = {1: t16(self.X[1], mt.dtype)}
        self.Y = {1: torch.empty((1, mt.rows), dtype=torch.float32, device=DEV)}
        self.sbytes = {1: workloads.sparse_bytes(mt.rows, mt.cols, mt.n, mt.m, 1, 4)}
        log(f"  {self.name:12s} {mt.rows}x{mt.cols}: {self.nc} packed copies "
            f"({self.nc * packed / 2**30:.2f} GiB), {self.ndc} dense copies, {time.time() - t0:.1f}s")


def large_layers_run(args, want_dense):
    """Batch-1 µs/call (median, p10, p90 over replays), GB/s and fraction of
    the 8 TB/s peak of the LARGE_LAYERS shapes, cache-cold, beside the dense
    GEMV and torch linear; one shape resident at a time."""
    out = {}
    for mt, _ in workloads.config_matrices(4):
        if mt.name not in LARGE_LAYERS:
            continue
        p = GpuProj(mt, want_dense)
        st = per_kernel_stats(p, Proj.sparse_call, 1, p.nc, args.reps)
        gbs = p.sbytes[1] / st["us"] / 1e3
        d = {"us": round(st["us"], 3), "us_p10": round(st["p10"], 3), "us_p90": round(st["p90"], 3),
             "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_GBS, 4),
             "bytes_per_launch": p.sbytes[1], "traffic": measured_traffic(mt.rows, mt.cols)}
        if want_dense:
            dus = per_kernel_us(p, Proj.dense_call, 1, p.ndc, args.reps)
            tus = per_kernel_us(p, Proj.torch_call, 1, p.ndc, args.reps)
            d.update({"dense_us": round(dus, 3), "torch_linear_us": round(tus, 3),
                      "speedup_vs_best_dense": round(min(dus, tus) / st["us"], 3)})
        out[f"{mt.name} {mt.rows}x{mt.cols}"] = d
        log(f"  {mt.name:12s} {mt.rows:5d}x{mt.cols:5d}: {st['us']:7.2f} us  {gbs:7.1f} GB/s "
            f"({100 * gbs / PEAK_GBS:.1f}% of 8 TB/s)"
            + (f"  dense {d['dense_us']:.2f} us, torch {d['torch_linear_us']:.2f} us" if want_dense else ""))
        del p
        torch.cuda.empty_cache()
    return out


def fused_layer_run(args):
    """The decode-layer step with the gate/up activation: one Llama-3.1-8B
    layer's products, 2:4 fp16, three ways, each step one HIP graph over one
    of five resident layers (1.2 GB packed, beyond the 256 MB Infinity Cache):
      - sparse fused (4 launches): q|k|v row-concatenated into one 6144x4096
        product, o, gate/up interleaved into one 28672x4096 product with the
        SwiGLU epilogue (nm_spmm_swiglu, 16-bit h), down on h;
      - sparse unfused (7 launches + torch silu * mul): the projections one by
        one, as in the headline step;
      - dense (torch linear, hipBLASLt): q|k|v and gate|up concatenated, torch
        silu * mul, down."""
    L = native.lib()
    NL = 5
    hid, inter = 4096, 14336
    mats = []
    t0 = time.time()
    for layer in range(NL):
        g = torch.Generator(device=DEV)
        g.manual_seed(7000 + layer)
        W = {name: (torch.randn((r, c), device=DEV, generator=g) * 0.02).half()
             for name, r, c in workloads.LLAMA8B_LAYER}
        qkv = torch.cat([W["q"], W["k"], W["v"]])
        gu = torch.empty((2 * inter, hid), dtype=torch.float16, device=DEV)
        gu[0::2] = W["gate"]
        gu[1::2] = W["up"]
        d = {"qkv": pack_gpu(qkv, 2, 4), "gu": pack_gpu(gu, 2, 4)}
        for name in W:
            d[name] = pack_gpu(W[name], 2, 4)
        if not args.no_dense:
            d["dense_qkv"] = qkv
            d["dense_o"] = W["o"]
            d["dense_gu"] = torch.cat([W["gate"], W["up"]])
            d["dense_down"] = W["down"]
        del W, gu
        mats.append(d)
    torch.cuda.synchronize()
    log(f"  {NL} layers resident ({time.time() - t0:.1f}s)")
    F16, F32 = native.NM_F16, native.NM_F32

    def spmm(v, bt, X, Y, B, rows, cols, out_dt=F32):
        st = L.nm_spmm_small(v.data_ptr(), bt.data_ptr(), X.data_ptr(), Y.data_ptr(), B, rows, cols,
                             2, 4, F16, out_dt, torch.cuda.current_stream().cuda_stream)
        assert st == 0, st

    out = {}
    for B in (1, 4, 8):
        x = torch.randn((B, hid), device=DEV).half()
        xa = torch.randn((B, hid), device=DEV).half()
        h16 = torch.empty((B, inter), dtype=torch.float16, device=DEV)
        y_qkv = torch.empty((B, 6144), device=DEV)
        y = {r: torch.empty((B, r), device=DEV) for r in (1024, 4096, 14336)}
        yg = torch.empty((B, inter), device=DEV)
        yu = torch.empty((B, inter), device=DEV)

        def fused(d):
            spmm(*d["qkv"], x, y_qkv, B, 6144, hid)
            spmm(*d["o"], xa, y[4096], B, hid, hid)
            st = L.nm_spmm_swiglu(d["gu"][0].data_ptr(), d["gu"][1].data_ptr(), x.data_ptr(),
                                  h16.data_ptr(), B, inter, hid, 2, 4, F16, F16,
                                  torch.cuda.current_stream().cuda_stream)
            assert st == 0, st
            spmm(*d["down"], h16, y[4096], B, hid, inter)

        def unfused(d):
            for name, r in (("q", 4096), ("k", 1024), ("v", 1024)):
                spmm(*d[name], x, y[r], B, r, hid)
            spmm(*d["o"], xa, y[4096], B, hid, hid)
            spmm(*d["gate"], x, yg, B, inter, hid)
            spmm(*d["up"], x, yu, B, inter, hid)
            h16.copy_(torch.nn.functional.silu(yg) * yu)
            spmm(*d["down"], h16, y[4096], B, hid, inter)

        def dense(d):
            F = torch.nn.functional
            F.linear(x, d["dense_qkv"])
            F.linear(xa, d["dense_o"])
            gu = F.linear(x, d["dense_gu"])
            h = F.silu(gu[:, :inter]) * gu[:, inter:]
            F.linear(h, d["dense_down"])

        res = {}
        for kind, fn in (("sparse_fused", fused), ("sparse_unfused", unfused), ("torch_dense", dense)):
            if kind == "torch_dense" and args.no_dense:
                continue
            graphs = [capture(lambda d=d, fn=fn: fn(d)) for d in mats]
            ms = time_steps(graphs, args.steps, args.warmup)
            res[kind] = {"ms_per_step": round(ms, 5), "launches": {"sparse_fused": 4,
                         "sparse_unfused": 8, "torch_dense": 5}[kind]}
            del graphs
        sb = sum(workloads.sparse_bytes(r, c, 2, 4, B, 4) for _, r, c in workloads.LLAMA8B_LAYER)
        res["sparse_bytes_per_step"] = sb
        res["fused_GB/s"] = round(sb / (res["sparse_fused"]["ms_per_step"] * 1e-3) / 1e9, 1)
        res["fused_vs_unfused"] = round(res["sparse_unfused"]["ms_per_step"]
                                        / res["sparse_fused"]["ms_per_step"], 3)
        if "torch_dense" in res:
            res["fused_vs_torch_dense"] = round(res["torch_dense"]["ms_per_step"]
                                                / res["sparse_fused"]["ms_per_step"], 3)
        out[f"batch{B}"] = res
        log(f"  batch {B}: " + ", ".join(f"{k} {v['ms_per_step'] * 1e3:.1f} us" for k, v in res.items()
                                         if isinstance(v, dict))
            + f"; fused {res['fused_GB/s']} GB/s, {res['fused_vs_unfused']}x unfused"
            + (f", {res['fused_vs_torch_dense']}x torch dense" if "torch_dense" in res else ""))
    return out


def hessian_run(args):
    """Calibration side: H += 2 X X^T for one layer input width (Llama-3.1-8B:
    4096 for q/k/v/gate/up, 14336 for down) over batches of decode-step
    activations.  Per call: the kernel time, the HBM rate of its H traffic
    (read + write 8 d^2 bytes plus X) and the contraction's flop rate, beside
    torch (hipBLASLt) doing the same update in fp32 (addmm on fp32 copies of
    X) and with fp16 inputs (mm, then an fp32 add).  Then the 2:4 mask
    selection of the layer that reads each width, scored with H's diagonal,
    beside torch's topk over groups of 4 and a scatter."""
    out = {}
    for d in (4096, 14336):
        H = torch.zeros((d, d), device=DEV)
        for ntok in (16, 64, 256, 1024):
            X = torch.randn((d, ntok), device=DEV).half()
            Xf = X.float()
            L = native.lib()
            def ours():
                st = L.nm_hessian_accumulate(H.data_ptr(), X.data_ptr(), d, ntok, ntok, native.NM_F16,
                                             2.0, torch.cuda.current_stream().cuda_stream)
                assert st == 0, st
            def torch32():
                torch.addmm(H, Xf, Xf.t(), alpha=2.0, out=H)
            def torch16():
                H.add_(torch.mm(X, X.t()), alpha=2.0)
            res = {}
            for kind, fn in (("nm_hessian", ours), ("torch_addmm_fp32", torch32),
                             ("torch_mm_fp16_then_add", torch16)):
                g = capture(fn)
                ms = time_steps([g], max(10, args.steps // 5), 3)
                res[kind] = round(ms * 1e3, 2)
                del g
            nbytes = 8 * d * d + 2 * d * ntok
            us = res["nm_hessian"]
            res.update({"GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_GBS, 3),
                        "TFLOP/s": round(2.0 * d * d * ntok / (us * 1e-6) / 1e12, 1)})
            out[f"d{d}_ntok{ntok}"] = res
            log(f"  d={d} ntok={ntok}: " + ", ".join(f"{k} {v}" for k, v in res.items()))
            del X, Xf
        # the 2:4 selection of the layer that reads this width, scored with
        # H's diagonal (|w| * ||x_c|| order), against torch's group topk
        rows = 14336 if d == 4096 else 4096
        W = (torch.randn((rows, d), device=DEV) * 0.02).half()
        keep = torch.empty((rows, d), dtype=torch.uint8, device=DEV)
        hd = H.diagonal()
        def sel_ours():
            st = L.nm_select_nm(W.data_ptr(), H.data_ptr(), d + 1, rows, d, 2, 4, native.NM_F16,
                                keep.data_ptr(), torch.cuda.current_stream().cuda_stream)
            assert st == 0, st
        def sel_torch():
            sc = (W.float().square() * hd).view(rows, d // 4, 4)
            idx = sc.topk(2, dim=-1).indices
            keep.view(rows, d // 4, 4).zero_().scatter_(-1, idx, 1)
        res = {}
        for kind, fn in (("nm_select_nm", sel_ours), ("torch_topk_scatter", sel_torch)):
            g = capture(fn)
            ms = time_steps([g], max(10, args.steps // 5), 3)
            res[kind] = round(ms * 1e3, 2)
            del g
        nbytes = 3 * rows * d + 4 * d
        res.update({"GB/s": round(nbytes / (res["nm_select_nm"] * 1e-6) / 1e9, 1)})
        out[f"select_2of4_{rows}x{d}"] = res
        log(f"  select 2:4 {rows}x{d}: " + ", ".join(f"{k} {v}" for k, v in res.items()))
        del H, W, keep
        torch.cuda.empty_cache()
    return out


def prefill_run(args):
    """Prefill-side contrast: the 8B gate (14336x4096) and down (4096x14336)
    shapes, 2:4 fp16, as the batch of tokens grows, against the dense GEMM.
    Per batch: nm_spmm_prefill (sparse matrix cores, GEMM tiling), the decode
    entry point nm_spmm_small (batch <= 8), nm_dense_gemv (batch <= 8) and
    torch linear (hipBLASLt) on the dense weights; four resident copies of
    each (cache-cold at small batch), us per call and dense-equivalent
    TFLOP/s (2 R K B / time).  The prefill product and torch linear both
    write fp16 output; the decode entry points write fp32.  Prefill and torch
    linear are timed as eager back-to-back launches (HIP events over 16 calls,
    best of 5), the way a prefill runs, and also as graph replays (the
    `_graph` keys): a split-K prefill captured in a graph allocates its
    workspace per replay (a memory node), where eager calls keep one per
    stream."""
    out = {}
    L = native.lib()
    for name, R, K in (("gate", 14336, 4096), ("down", 4096, 14336)):
        mats = [gpu_layer(R, K, 2, 4, 1000 + i, True) for i in range(4)]
        res = {}
        for B in (1, 8, 16, 64, 128, 256, 512, 1024, 2048, 4096):
            X = torch.randn((B, K), device=DEV).half()
            Y = torch.empty((B, R), device=DEV)
            Yh = torch.empty((B, R), dtype=torch.float16, device=DEV)
            def run(fn):
                g = capture(lambda: [fn(i) for i in range(8)])
                ms = time_steps([g], max(5, args.steps // 10), 2) / 8
                del g
                return ms * 1e3

            def eager(fn, n=16, reps=5):
                for i in range(4):
                    fn(i)
                torch.cuda.synchronize()
                best = float("inf")
                for _ in range(reps):
                    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    for i in range(n):
                        fn(i)
                    z.record()
                    torch.cuda.synchronize()
                    best = min(best, a.elapsed_time(z) / n * 1e3)
                return best
            def pre(i):
                v, b, _ = mats[i % 4]
                st = L.nm_spmm_prefill(v.data_ptr(), b.data_ptr(), X.data_ptr(), Yh.data_ptr(), B, R,
                                       K, 2, 4, native.NM_F16, native.NM_F16,
                                       torch.cuda.current_stream().cuda_stream)
                assert st == 0, st
            def dense(i):
                torch.nn.functional.linear(X, mats[i % 4][2], out=Yh)
            row = {"nm_spmm_prefill": round(eager(pre), 2), "torch_linear": round(eager(dense), 2),
                   "nm_spmm_prefill_graph": round(run(pre), 2), "torch_linear_graph": round(run(dense), 2)}
            if B <= 8:
                def small(i):
                    v, b, _ = mats[i % 4]
                    st = L.nm_spmm_small_cfg(v.data_ptr(), b.data_ptr(), X.data_ptr(), Y.data_ptr(), B,
                                             R, K, 2, 4, native.NM_F16, native.NM_F32, None,
                                             torch.cuda.current_stream().cuda_stream)
                    assert st == 0, st
                def dgemv(i):
                    st = L.nm_dense_gemv_cfg(mats[i % 4][2].data_ptr(), X.data_ptr(), Y.data_ptr(), B,
                                             R, K, native.NM_F16, native.NM_F32, None,
                                             torch.cuda.current_stream().cuda_stream)
                    assert st == 0, st
                row["nm_spmm_small"] = round(run(small), 2)
                row["nm_dense_gemv"] = round(run(dgemv), 2)
            best_sparse = min(v for k, v in row.items() if k.startswith("nm_spmm") and not k.endswith("_graph"))
            best_dense = min(v for k, v in row.items() if k in ("torch_linear", "nm_dense_gemv"))
            row["prefill_TFLOP/s"] = round(2.0 * R * K * B / (row["nm_spmm_prefill"] * 1e-6) / 1e12, 1)
            row["dense_TFLOP/s"] = round(2.0 * R * K * B / (row["torch_linear"] * 1e-6) / 1e12, 1)
            row["speedup_best_sparse_vs_best_dense"] = round(best_dense / best_sparse, 3)
            res[B] = row
            log(f"  {name} {R}x{K} B={B}: " + ", ".join(f"{k} {v}" for k, v in row.items()))
            del X, Y, Yh
        out[f"{name} {R}x{K}"] = res
        del mats
        torch.cuda.empty_cache()
    return out


def decode_run(args):
    """Workload 5: 32 stacked Llama-3.1-8B-shaped layers (224 matrices, 2:4
    fp16, a different seed per matrix), all resident; one token = the 224
    products chained in one HIP graph, at batch 1, 2, 4 and 8, against the
    dense fp16 chain (nm_dense_gemv and torch linear).  Beside it, the same
    weights as 32 fused layer steps (q|k|v concatenated, gate/up with the
    SwiGLU epilogue, 128 launches per token)."""
    want_dense = not args.no_dense
    mats = [mt for mt, _ in workloads.config_matrices(5)]
    t0 = time.time()
    store = []
    for mt in mats:
        v, bt, W = gpu_layer(mt.rows, mt.cols, mt.n, mt.m, mt.seed, want_dense)
        store.append((mt, v, bt, W))
    torch.cuda.synchronize()
    log(f"  224 matrices resident ({time.time() - t0:.1f}s): "
        f"{sum(v.numel() * 2 + b.numel() * 4 for _, v, b, _ in store) / 1e9:.2f} GB packed")
    # the same weights fused per layer: q|k|v row-concatenated, gate/up
    # row-interleaved for the SwiGLU epilogue (redrawn from the same seeds)
    fused = []
    for layer in range(32):
        lm = {mt.name: mt for mt in mats[7 * layer:7 * layer + 7]}
        def redraw(mt):
            g = torch.Generator(device=DEV)
            g.manual_seed(mt.seed)
            return (torch.randn((mt.rows, mt.cols), device=DEV, generator=g) * 0.02).half()
        qkv = torch.cat([redraw(lm["q"]), redraw(lm["k"]), redraw(lm["v"])])
        gu = torch.empty((2 * 14336, 4096), dtype=torch.float16, device=DEV)
        gu[0::2] = redraw(lm["gate"])
        gu[1::2] = redraw(lm["up"])
        fused.append({"qkv": pack_gpu(qkv, 2, 4), "gu": pack_gpu(gu, 2, 4),
                      "o": [(v, bt) for mt, v, bt, _ in store if mt is lm["o"]][0],
                      "down": [(v, bt) for mt, v, bt, _ in store if mt is lm["down"]][0]})
        del qkv, gu
    torch.cuda.synchronize()
    L = native.lib()
    out = {}
    for B in (1, 2, 4, 8):
        X = {k: torch.randn((B, k), device=DEV).half() for k in (4096, 14336)}
        Y = {r: torch.empty((B, r), device=DEV) for r in (1024, 4096, 14336)}
        def sparse_token():
            st_ = torch.cuda.current_stream().cuda_stream
            for mt, v, bt, _ in store:
                st = L.nm_spmm_small(v.data_ptr(), bt.data_ptr(), X[mt.cols].data_ptr(),
                                     Y[mt.rows].data_ptr(), B, mt.rows, mt.cols, mt.n, mt.m,
                                     native.NM_F16, native.NM_F32, st_)
                assert st == 0, st
        def dense_token():
            st_ = torch.cuda.current_stream().cuda_stream
            for mt, _, _, W in store:
                st = L.nm_dense_gemv(W.data_ptr(), X[mt.cols].data_ptr(), Y[mt.rows].data_ptr(), B,
                                     mt.rows, mt.cols, native.NM_F16, native.NM_F32, st_)
                assert st == 0, st
        def torch_token():
            for mt, _, _, W in store:
                torch.nn.functional.linear(X[mt.cols], W)
        Yqkv = torch.empty((B, 6144), device=DEV)
        H16 = torch.empty((B, 14336), dtype=torch.float16, device=DEV)
        def fused_token():
            st_ = torch.cuda.current_stream().cuda_stream
            for d in fused:
                for (v, bt), Xin, Yout, rows, cols in ((d["qkv"], X[4096], Yqkv, 6144, 4096),
                                                       (d["o"], X[4096], Y[4096], 4096, 4096)):
                    st = L.nm_spmm_small(v.data_ptr(), bt.data_ptr(), Xin.data_ptr(), Yout.data_ptr(),
                                         B, rows, cols, 2, 4, native.NM_F16, native.NM_F32, st_)
                    assert st == 0, st
                st = L.nm_spmm_swiglu(d["gu"][0].data_ptr(), d["gu"][1].data_ptr(), X[4096].data_ptr(),
                                      H16.data_ptr(), B, 14336, 4096, 2, 4, native.NM_F16,
                                      native.NM_F16, st_)
                assert st == 0, st
                v, bt = d["down"]
                st = L.nm_spmm_small(v.data_ptr(), bt.data_ptr(), H16.data_ptr(), Y[4096].data_ptr(),
                                     B, 4096, 14336, 2, 4, native.NM_F16, native.NM_F32, st_)
                assert st == 0, st
        sbytes = sum(workloads.sparse_bytes(mt.rows, mt.cols, mt.n, mt.m, B, 4) for mt, *_ in store)
        dbytes = sum(workloads.dense_bytes(mt.rows, mt.cols, B, 4) for mt, *_ in store)
        res = {}
        for kind, fn, nbytes in (("sparse", sparse_token, sbytes), ("sparse_fused", fused_token, sbytes),
                                 ("dense", dense_token, dbytes), ("torch_linear", torch_token, dbytes)):
            if kind in ("dense", "torch_linear") and not want_dense:
                continue
            g = capture(fn)
            ms = time_steps([g], args.steps, args.warmup)
            res[kind] = {"ms_per_token": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
            del g
        if want_dense:
            res["speedup_vs_best_dense"] = round(
                min(res["dense"]["ms_per_token"], res["torch_linear"]["ms_per_token"])
                / res["sparse"]["ms_per_token"], 3)
        out[f"batch{B}"] = res
        log(f"  batch {B}: " + ", ".join(f"{k} {v['ms_per_token']} ms/token ({v['GB/s']} GB/s)"
                                         for k, v in res.items() if isinstance(v, dict)))
    return out


def summarize_trace(path, min_run=16):
    """Per-dispatch statistics of a rocprofv3 kernel-trace CSV, by contiguous
    run: consecutive dispatches of one kernel, grid and workgroup size form a
    run (each per-kernel timing of this benchmark is one run: back-to-back
    replays of one projection's rotation), and runs of at least min_run
    dispatches are listed in dispatch order with the count and the mean,
    p10, p50, p90, min and max of End - Start in µs."""
    import csv
    with open(path, newline="") as f:
        recs = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    runs = []
    for r in recs:
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if runs and runs[-1][0] == key:
            runs[-1][1].append(us)
        else:
            runs.append((key, [us]))
    print("| run | kernel | grid threads | WG | dispatches | mean us | p10 | p50 | p90 | min | max |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    i = 0
    for (name, grid, wg), us in runs:
        if len(us) < min_run:
            continue
        i += 1
        a = np.array(us)
        # drop the return type, namespace and parameter list; keep template arguments
        short = name.replace("void (anonymous namespace)::", "").split("(")[0] or name
        short = short if len(short) <= 90 else short[:87] + "..."
        print(f"| {i} | `{short}` | {grid} | {wg} | {len(a)} | {a.mean():.3f} | {np.percentile(a, 10):.3f} | "
              f"{np.percentile(a, 50):.3f} | {np.percentile(a, 90):.3f} | {a.min():.3f} | {a.max():.3f} |")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=20, help="replays per per-kernel timing")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense comparison")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batch4", action="store_true")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the 70B / Qwen3-32B layers of >= 58.7 M weights at batch 1")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print per-kernel dispatch statistics (count, mean, p10, p50, p90) of a "
                         "rocprofv3 kernel-trace CSV and exit (no GPU needed)")
    ap.add_argument("--workload", default="llama8b-layer",
                    choices=["llama8b-layer", "single", "patterns", "70b-qwen", "decode-32-layers",
                             "llama8b-layer-fused", "calibration-hessian", "prefill-contrast",
                             "densities", "unstructured"],
                    help="llama8b-layer (default, the headline line): one Llama-3.1-8B layer; "
                         "single: the 4096x4096 matrix; patterns: 4:8/8:16/16:32 bf16 on the 8B "
                         "shapes; 70b-qwen: Llama-3.3-70B and Qwen3-32B shapes; "
                         "decode-32-layers: 32 stacked 8B layers timed per token; "
                         "llama8b-layer-fused: the 8B layer step with q|k|v and gate/up fused "
                         "(SwiGLU epilogue) against the unfused and dense steps; "
                         "calibration-hessian: H += 2 X X^T at the 8B input widths; "
                         "prefill-contrast: 2:4 gate/down shapes as the batch grows to 4096 "
                         "tokens, sparse matrix cores against the dense GEMM; densities: "
                         "1:4, 3:4, 1:8, 3:8 fp16 on the 8B gate and down shapes (generic "
                         "window kernel) against the dense GEMV; unstructured: 50% per-row "
                         "bitmasks on the same shapes")
    ap.add_argument("--counters", action="store_true",
                    help="short eager run for rocprofv3 --pmc: the 14336x4096 sparse kernel on "
                         "5 cache-cold copies, then 5 plain copies of 64 MiB (the known-size "
                         "reference for FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the N:M SpMV path is built and timed on a single "
              "MI355X (row or K sharding across GPUs is a design note, not implemented)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    native.lib()  # fail loudly if the HIP library is missing

    if args.counters:
        counters_run()
        return
    if args.workload == "llama8b-layer-fused":
        log("workload llama8b-layer-fused")
        body = {"per_step": fused_layer_run(args)}
        print(json.dumps({"metric": "decode-layer step time, fused vs unfused sparse and dense",
                          "workload": args.workload, "n_gpus": 1, "data": "synthetic",
                          "unit": "ms/step", **body}), flush=True)
        return
    if args.workload == "prefill-contrast":
        log("workload prefill-contrast")
        body = {"per_call_us": prefill_run(args)}
        print(json.dumps({"metric": "2:4 product us per call as the batch grows, sparse vs dense",
                          "workload": args.workload, "n_gpus": 1, "data": "synthetic",
                          "dtype": "f16 inputs, fp32 sparse output, f16 torch output", **body}),
              flush=True)
        return
    if args.workload == "calibration-hessian":
        log("workload calibration-hessian")
        body = {"per_call_us": hessian_run(args)}
        print(json.dumps({"metric": "Hessian accumulation H += 2 X X^T, us per call",
                          "workload": args.workload, "n_gpus": 1, "data": "synthetic",
                          "dtype": "f16 inputs, fp32 H", **body}), flush=True)
        return
    if args.workload == "unstructured":
        log("workload unstructured (50% per-row bitmasks on the 8B gate and down shapes)")
        body = {"per_matrix": bitmask_run(args)}
        print(json.dumps({"metric": METRIC.replace("2:4", "50% unstructured bitmask"),
                          "workload": args.workload, "n_gpus": 1, "data": "synthetic",
                          "peak_GB/s": PEAK_GBS, **body}), flush=True)
        return
    if args.workload == "densities":
        log("workload densities (1:4, 3:4, 1:8, 3:8 on the 8B gate and down shapes)")
        body = {"per_matrix": shapes_run(0, args, mats=workloads.density_matrices())}
        print(json.dumps({"metric": METRIC.replace("2:4", "N:M at densities other than 50%"),
                          "workload": args.workload, "n_gpus": 1, "data": "synthetic",
                          "peak_GB/s": PEAK_GBS, **body}), flush=True)
        return
    if args.workload != "llama8b-layer":
        cfg_id = {"single": 1, "patterns": 3, "70b-qwen": 4, "decode-32-layers": 5}[args.workload]
        log(f"workload {args.workload} ({cfg_id})")
        if cfg_id == 5:
            body = {"per_token": decode_run(args)}
        else:
            body = {"per_matrix": shapes_run(cfg_id, args)}
        print(json.dumps({"metric": METRIC, "workload": args.workload, "n_gpus": 1,
                          "data": "synthetic", "peak_GB/s": PEAK_GBS, **body}), flush=True)
        return
    batches = (1,) if args.no_batch4 else (1, 4)
    want_dense = not args.no_dense
    log(f"building the Llama-3.1-8B layer workload (2:4 fp16), batches {batches}")
    projs = [Proj(mt, batches, want_dense) for mt, _ in workloads.config_matrices(2)]
    layer_bytes = {b: sum(p.sbytes[b] for p in projs) for b in batches}
    nsteps = min(args.steps + args.warmup, 256)
    spg = steps_per_graph(args.steps, args.warmup)

    timings = {}
    kinds = [("sparse", Proj.sparse_call, "nc")]
    if want_dense:
        kinds += [("dense", Proj.dense_call, "ndc"), ("torch", Proj.torch_call, "ndc")]
    for b in batches:
        for kind, call, attr in kinds:
            for par in (True, False):
                g = chain_graphs(projs, call, b, nsteps, attr, parallel=par, per_graph=spg)
                torch.cuda.synchronize()
                timings[(kind, b, par)] = time_steps(g, args.steps, args.warmup, spg)
                del g
        # the same serial chain with one graph per step (each step pays the
        # graph's own launch cost)
        g = chain_graphs(projs, Proj.sparse_call, b, nsteps, "nc", parallel=False)
        torch.cuda.synchronize()
        timings[("sparse-1", b, False)] = time_steps(g, args.steps, args.warmup)
        del g
        for k, v in timings.items():
            if k[1] == b:
                log(f"  {k[0]:8s} b={b} {'layer graph' if k[2] else 'serial chain'}: "
                    f"{1e3 * v:8.1f} us/step")

    # per-kernel durations (batch 1) and the roofline of the dominant kernel
    per = {}
    for p in projs:
        st = per_kernel_stats(p, Proj.sparse_call, 1, p.nc, args.reps)
        us = st["us"]
        d = {"us": round(us, 3), "us_p10": round(st["p10"], 3), "us_p90": round(st["p90"], 3),
             "GB/s": round(p.sbytes[1] / us / 1e3, 1),
             "frac_of_peak": round(p.sbytes[1] / us / 1e3 / PEAK_GBS, 4)}
        if want_dense:
            dus = per_kernel_us(p, Proj.dense_call, 1, p.ndc, args.reps)
            tus = per_kernel_us(p, Proj.torch_call, 1, p.ndc, args.reps)
            d.update({"dense_us": round(dus, 3), "torch_linear_us": round(tus, 3),
                      "speedup_vs_best_dense": round(min(dus, tus) / us, 3)})
        per[f"{p.name} {p.mt.rows}x{p.mt.cols}"] = d
        log(f"  {p.name:5s} {p.mt.rows:5d}x{p.mt.cols:5d}: {us:7.2f} us  "
            f"{d['GB/s']:7.1f} GB/s ({100 * d['frac_of_peak']:.1f}% of 8 TB/s)"
            + (f"  dense {d['dense_us']:.2f} us, torch {d['torch_linear_us']:.2f} us" if want_dense else ""))
    # batch 2 (the VALU row kernel) and batch 8 (the sparse matrix cores) on
    # the 8B layer's shapes, beside torch linear on the dense weights
    small = {2: {}, 8: {}}
    if not args.no_batch4:
        for b, names in ((2, ("q", "k", "gate", "down")), (8, ("q", "gate", "down"))):
            for p in projs:
                if p.name not in names:
                    continue
                mt = p.mt
                p.X[b] = synth.activations(b, mt.cols, seed=mt.seed, dtype=mt.dtype, outliers=mt.outliers)
                p.Xd[b] = t16(p.X[b], mt.dtype)
                p.Y[b] = torch.empty((b, mt.rows), dtype=torch.float32, device=DEV)
                p.sbytes[b] = workloads.sparse_bytes(mt.rows, mt.cols, mt.n, mt.m, b, 4)
                st = per_kernel_stats(p, Proj.sparse_call, b, p.nc, args.reps)
                d = {"us": round(st["us"], 3), "us_p10": round(st["p10"], 3), "us_p90": round(st["p90"], 3),
                     "GB/s": round(p.sbytes[b] / st["us"] / 1e3, 1),
                     "frac_of_peak": round(p.sbytes[b] / st["us"] / 1e3 / PEAK_GBS, 4)}
                if want_dense:
                    d["torch_linear_us"] = round(per_kernel_us(p, Proj.torch_call, b, p.ndc, args.reps), 3)
                small[b][f"{p.name} {mt.rows}x{mt.cols}"] = d
                log(f"  {p.name:5s} {mt.rows:5d}x{mt.cols:5d} batch {b}: {d['us']:7.2f} us  "
                    f"{d['GB/s']:7.1f} GB/s ({100 * d['frac_of_peak']:.1f}% of 8 TB/s)"
                    + (f"  torch {d['torch_linear_us']:.2f} us" if want_dense else ""))
                del p.X[b], p.Xd[b], p.Y[b]
    batch8 = small[8]
    # the dominant kernel: the launch shape with the most time per step (the
    # 14336x4096 shape runs twice per layer, as gate and up)
    shape_time = {}
    for p in projs:
        key = (p.mt.rows, p.mt.cols)
        shape_time.setdefault(key, [0.0, []])
        shape_time[key][0] += per[f"{p.name} {p.mt.rows}x{p.mt.cols}"]["us"]
        shape_time[key][1].append(p)
    (drows, dcols), (_, dps) = max(shape_time.items(), key=lambda kv: kv[1][0])
    dus = float(np.mean([per[f"{p.name} {drows}x{dcols}"]["us"] for p in dps]))
    dbytes = dps[0].sbytes[1]
    roofline = {"bound": "hbm", "achieved": round(dbytes / dus / 1e3, 1), "peak": PEAK_GBS,
                "unit": "GB/s", "frac": round(dbytes / dus / 1e3 / PEAK_GBS, 4),
                "traffic": measured_traffic(drows, dcols),
                "kernel": f"nm_spmv_rows_kernel {drows}x{dcols} 2:4 fp16 batch 1",
                "bytes_per_launch": dbytes, "us_per_launch": round(dus, 3),
                "launches_per_step": len(dps)}

    # the larger 2:4 layers of workload 4 at batch 1 (the 8B layer's
    # projections are freed first)
    gpu_y = {}
    if not args.no_cpu_baseline:
        for p in projs:
            p.sparse_call(1, 0)
        torch.cuda.synchronize()
        for p in projs:
            gpu_y[p.name] = p.Y[1][0].cpu().numpy()
    host = [(p.name, p.W, p.keep, p.X, p.sbytes) for p in projs]
    del projs, shape_time, dps, p
    torch.cuda.empty_cache()
    large = {} if args.no_large else large_layers_run(args, want_dense)
    # which of the named 2:4 layers of >= 58.7 M weights reach 70% of peak at batch 1
    target = {k: v["frac_of_peak"] for k, v in list(per.items()) + list(large.items())
              if int(k.split()[-1].split("x")[0]) * int(k.split("x")[-1]) >= 14336 * 4096}

    ms = timings[("sparse", 1, False)]
    res = {
        "metric": METRIC,
        "value": round(layer_bytes[1] / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped decoder layer, 7 projections "
                               "(q,o 4096x4096; k,v 1024x4096; gate,up 14336x4096; down 4096x14336), "
                               "2:4 fp16, x N(0,1) + 0.1% outlier channels x20",
                   "batch": 1, "pattern": "2:4", "bytes_per_step": layer_bytes[1],
                   "launches_per_step": len(host),
                   "timing": f"the 7 launches of a step in series, {spg} consecutive steps per HIP "
                             "graph (each step on its own rotation copy), >=1 GiB rotation per "
                             "projection (cache-cold); per-call figures from graphs of >= "
                             f"{MIN_LAUNCHES_PER_REPLAY} back-to-back launches"},
        "frac_of_peak": round(layer_bytes[1] / (ms * 1e-3) / 1e9 / PEAK_GBS, 4),
        "us_per_call": per,
        "roofline": roofline,
        "large_layers_batch1": large,
        "layers_at_or_above_70pct": {"frac_of_peak": target,
                                     "met": sum(1 for v in target.values() if v >= 0.70),
                                     "of": len(target)},
    }
    res["ms_per_step_parallel_branches"] = round(timings[("sparse", 1, True)], 5)
    res["ms_per_step_one_graph_per_step"] = round(timings[("sparse-1", 1, False)], 5)

    def best_dense(b):
        return min(timings[(k, b, par)] for k in ("dense", "torch") for par in (False, True))

    if want_dense:
        res["dense_ms_per_step"] = {f"{k} {'parallel branches' if par else 'serial'}":
                                    round(timings[(k, 1, par)], 5)
                                    for k in ("dense", "torch") for par in (False, True)}
        res["speedup_vs_best_dense"] = round(best_dense(1) / ms, 3)
    if 4 in batches:
        ms4 = timings[("sparse", 4, False)]
        b4 = {"ms_per_step": round(ms4, 5), "GB/s": round(layer_bytes[4] / (ms4 * 1e-3) / 1e9, 1),
              "frac_of_peak": round(layer_bytes[4] / (ms4 * 1e-3) / 1e9 / PEAK_GBS, 4),
              "ms_per_step_parallel_branches": round(timings[("sparse", 4, True)], 5),
              "ms_per_step_one_graph_per_step": round(timings[("sparse-1", 4, False)], 5)}
        if want_dense:
            b4["speedup_vs_best_dense"] = round(best_dense(4) / ms4, 3)
        res["batch4"] = b4
    if small[2]:
        res["batch2_per_call"] = small[2]
    if batch8:
        res["batch8_per_call"] = batch8
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(host, gpu_y)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
