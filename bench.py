#!/usr/bin/env python3
"""Benchmark: SGMV LoRA add-on (lora_apply) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Workload: Llama-2-7B decode projection, H1 = H2 = 4096, r = 16, 64 rows in
64 one-row segments (a distinct adapter per row), fp16 with fp32
accumulation, scale 2.  One step = one lora_apply over the batch (segment
lookup, shrink, expand, fused scale + accumulate into y).  Inputs are
seeded synthetic arrays resident in HBM before timing starts.

So that timed calls read HBM rather than the 256 MB Infinity Cache, the
step rotates through enough copies of the inputs (same values, different
addresses) to exceed 1 GiB.  The K timed steps are captured in one HIP graph
(so host launch cost does not pace the GPU) and timed with HIP events on the
stream they run on.

Prints one JSON line: rows/s, ms per step, achieved algorithmic HBM GB/s
and its fraction of the 8 TB/s peak (``roofline``), and the CPU oracle's
rows/s on a bounded sample of the same workload (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16/bf16, published
MALL_BYTES = 256 << 20
ROTATE_BYTES = 1 << 30          # >= 4x the Infinity Cache


def algorithmic_bytes(w) -> int:
    """What one call must move: each segment's A and B once, x once, y read
    and written once (covered rows only)."""
    e = w.elem_bytes
    lens = w.seg_lengths
    segs = int((lens > 0).sum())
    rows = int(lens.sum())
    weights = segs * (w.H1 * w.r + w.r * w.H2) * e
    return weights + rows * w.H1 * e + 2 * rows * w.H2 * e


def entry_bytes(w, entry: str) -> int:
    """Algorithmic bytes of one call of an entry point: lora_apply as above;
    sgmv_shrink reads each segment's A once and x once and writes v (float32);
    sgmv_expand reads each segment's B once and v, and reads and writes y."""
    if entry == "apply":
        return algorithmic_bytes(w)
    e = w.elem_bytes
    lens = w.seg_lengths
    segs = int((lens > 0).sum())
    rows = int(lens.sum())
    if entry == "shrink":
        return segs * w.H1 * w.r * e + rows * w.H1 * e + rows * w.r * 4
    return segs * w.r * w.H2 * e + rows * w.r * 4 + 2 * rows * w.H2 * e


def algorithmic_flops(w) -> int:
    rows = int(w.seg_lengths.sum())
    return 2 * rows * w.r * (w.H1 + w.H2)


class BenchState:
    """Device copies of a workload, rotated over `nsets` buffer sets."""

    def __init__(self, w, nsets: int, device="cuda:0", row_ids=None, projections=1,
                 entry="apply"):
        import torch
        import segmented_gather_gemv_sgmv_amd as sg
        self.entry = entry
        self.w = w
        self.sg = sg
        dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        self.dtype = dt
        dev = torch.device(device)
        to = lambda a: torch.from_numpy(a).to(dev).to(dt)
        base = dict(x=to(w.x), A=to(w.A), B=to(w.B), y0=to(w.y0))
        self.seg = torch.from_numpy(w.seg_indptr).to(dev)
        self.ids = torch.from_numpy(w.adapter_ids).to(dev)
        self.sets = []
        self.projections = projections
        for i in range(nsets):
            if projections == 1:
                s = {k: (v if i == 0 else v.clone()) for k, v in base.items() if k != "y0"}
                s["y"] = base["y0"].clone()
                if entry != "apply":  # float32 v [R, r] of the separate entry points
                    s["v"] = torch.randn(w.num_rows, w.r, device=dev) * 0.5
            else:  # one copy of the shape per projection
                s = {k: [v.clone() for _ in range(projections)] for k, v in base.items()
                     if k != "y0"}
                s["y"] = [base["y0"].clone() for _ in range(projections)]
            self.sets.append(s)
        self.y0 = base["y0"]
        nbytes = sg.lora_apply_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.H2, w.r, dt)
        nbytes = max(nbytes, sg.shrink_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.r, dt))
        if projections > 1:
            nbytes = max(nbytes, sg.lora_apply_multi_workspace_bytes(
                [(w.H1, w.H2)] * projections, w.num_rows, w.num_segments, w.r, dt))
        self.device = dev
        self.row_ids_mode = row_ids
        if row_ids:
            # Per-row adapter ids (the rows of the workload are already grouped,
            # so both builders return the workload's own segments).
            R, N = w.num_rows, w.num_adapters
            per_row = np.full(R, -1, dtype=np.int32)
            for k in range(w.num_segments):
                per_row[w.seg_indptr[k]:w.seg_indptr[k + 1]] = w.adapter_ids[k]
            self.row_ids = torch.from_numpy(per_row).to(dev)
            M = R if row_ids == "runs" else min(R, N)
            self.built = [torch.empty(n, dtype=torch.int32, device=dev)
                          for n in ((R + 1, R, 1) if row_ids == "runs" else (R, M + 1, M, 1))]
            nbytes = max(nbytes, sg.lora_apply_workspace_bytes(R, M, w.H1, w.H2, w.r, dt))
        self.workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def step(self, i: int):
        s = self.sets[i % len(self.sets)]
        seg, ids = self.seg, self.ids
        if self.row_ids_mode == "runs":
            seg, ids, _ = self.sg.build_segments(self.row_ids, self.w.num_adapters, out=self.built)
        elif self.row_ids_mode == "grouped":
            _, seg, ids, _ = self.sg.group_rows(self.row_ids, self.w.num_adapters, out=self.built)
        if self.projections > 1:
            self.sg.lora_apply_multi(
                [(s["y"][p], s["x"][p], s["A"][p], s["B"][p], self.w.scale)
                 for p in range(self.projections)], seg, ids, workspace=self.workspace)
            return
        if self.entry == "shrink":
            self.sg.sgmv_shrink(s["v"], s["x"], s["A"], seg, ids, workspace=self.workspace)
            return
        if self.entry == "expand":
            self.sg.sgmv_expand(s["y"], s["v"], s["B"], seg, ids, self.w.scale)
            return
        self.sg.lora_apply(s["y"], s["x"], s["A"], s["B"], seg, ids, self.w.scale,
                           workspace=self.workspace)

    def reset_outputs(self):
        for s in self.sets:
            for y in (s["y"] if isinstance(s["y"], list) else [s["y"]]):
                y.copy_(self.y0)

    def capture(self, nsteps: int, first: int = 0):
        """A HIP graph of `nsteps` consecutive steps starting at set `first`."""
        import torch
        side = torch.cuda.Stream(self.device)
        side.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(side):
            self.step(first)  # settle lazy initialisation off the capture
        torch.cuda.current_stream(self.device).wait_stream(side)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(nsteps):
                self.step(first + k)
        return g


# Byte offset of the sticky flag in the workspace: the last int of the
# 256 KiB counter region (include/sgmv.h, "Workspace").
FLAG_OFFSET = 65536 * 4 - 4


def read_flag(ws) -> int:
    import torch
    return int(ws[FLAG_OFFSET:FLAG_OFFSET + 4].view(torch.int32).item())


def clear_flag(ws) -> None:
    ws[FLAG_OFFSET:FLAG_OFFSET + 4].zero_()


def run_gpu(w, steps: int, warmup: int, device="cuda:0", row_ids=None, projections=1,
            warm=False, entry="apply", replays=5):
    """Times `steps` consecutive steps captured in one HIP graph, replayed
    `replays` times, each replay bracketed by HIP events on the replay
    stream; the per-step time is the median over the replays, so that it
    does not move with the graph length.  Also reads the fused kernels'
    sticky flag (an expand workgroup stopped waiting for its shrink
    workgroups and recomputed its input) over the timed replays."""
    import torch
    per_set = (w.x.size + w.A.size + w.B.size + w.y0.size) * w.elem_bytes * projections
    nsets = 1 if warm else max(1, min(512, math.ceil(ROTATE_BYTES / max(per_set, 1))))
    st = BenchState(w, nsets, device, row_ids, projections, entry)
    for i in range(warmup):
        st.step(i)
    torch.cuda.synchronize(device)
    graph = st.capture(steps, first=warmup)
    torch.cuda.synchronize(device)
    clear_flag(st.workspace)
    torch.cuda.synchronize(device)
    stream = torch.cuda.current_stream(device)
    t0 = time.perf_counter()
    per_replay_ms = []
    for _ in range(max(1, replays)):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize(device)
        per_replay_ms.append(start.elapsed_time(end))
    wall = time.perf_counter() - t0
    flag = read_flag(st.workspace)
    gpu_ms = float(np.median(per_replay_ms))
    # Spread: a graph of `chunk` steps (every buffer set at least once)
    # replayed `reps` times, each replay timed on its own; the per-call means
    # of the replays give p10 / p50 / p90.
    chunk = max(100, nsets)
    reps = 20
    g2 = st.capture(chunk, first=warmup)
    torch.cuda.synchronize(device)
    samples = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g2.replay()
        b.record(stream)
        torch.cuda.synchronize(device)
        samples.append(a.elapsed_time(b) * 1e3 / chunk)
    pct = np.percentile(np.asarray(samples), [10, 50, 90]).tolist()
    return dict(gpu_ms=gpu_ms, wall_s=wall, nsets=nsets, per_set_bytes=per_set,
                us_p10_p50_p90=pct, spread_steps=chunk, spread_replays=reps,
                replays=len(per_replay_ms),
                us_per_step_each_replay=[m * 1e3 / steps for m in per_replay_ms],
                fallback_flag=flag)


KERNEL_SOURCES = ("segmented_gather_gemv_sgmv_amd/csrc/sgmv_api.hip",
                  "segmented_gather_gemv_sgmv_amd/csrc/sgmv_mixed.hpp",
                  "segmented_gather_gemv_sgmv_amd/csrc/sgmv_mfma.hpp",
                  "segmented_gather_gemv_sgmv_amd/csrc/sgmv_fused.hpp",
                  "segmented_gather_gemv_sgmv_amd/csrc/sgmv_gemv.hpp",
                  "segmented_gather_gemv_sgmv_amd/csrc/sgmv_device.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_lora_mixed_kernel_llama7b_decode.json")


def kernel_source_hash() -> str:
    """SHA-256 over the HIP sources the measured kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload_name: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE and
    WRITE_SIZE counts (scaled by the copy-kernel calibration), or None when
    they were taken on other kernel sources or another workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash() or t.get("workload") != workload_name:
        return None
    return t.get("traffic_bytes_per_launch")


def run_linear(w, mode: str, steps: int, warmup: int, device="cuda:0"):
    """Times the adapted linear layer y = x W^T + bias + s (x A_a) B_a over the
    workload's batch: ``fused`` is one lora_linear call, ``unfused`` is
    torch's addmm for the base product followed by lora_apply.  W [H2, H1]
    and bias are seeded N(0, 1/H1) and N(0, 1) draws in the workload's dtype;
    buffers rotate over >= 1 GiB as in run_gpu and the timed steps run as one
    HIP graph."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    dev = torch.device(device)
    rng = np.random.default_rng(1)
    W0 = torch.from_numpy(rng.standard_normal((w.H2, w.H1), dtype=np.float32)
                          / np.float32(math.sqrt(w.H1))).to(dev).to(dt)
    b0 = torch.from_numpy(rng.standard_normal(w.H2, dtype=np.float32)).to(dev).to(dt)
    to = lambda a: torch.from_numpy(a).to(dev).to(dt)
    x0, A0, B0 = to(w.x), to(w.A), to(w.B)
    seg = torch.from_numpy(w.seg_indptr).to(dev)
    ids = torch.from_numpy(w.adapter_ids).to(dev)
    e = w.elem_bytes
    per_set = (W0.numel() + x0.numel() + A0.numel() + B0.numel() + w.num_rows * w.H2) * e
    nsets = max(1, min(256, math.ceil(ROTATE_BYTES / per_set)))
    sets = [dict(W=W0 if i == 0 else W0.clone(), b=b0 if i == 0 else b0.clone(),
                 x=x0 if i == 0 else x0.clone(), A=A0 if i == 0 else A0.clone(),
                 B=B0 if i == 0 else B0.clone(),
                 y=torch.empty((w.num_rows, w.H2), dtype=dt, device=dev)) for i in range(nsets)]
    nbytes = max(sg.lora_linear_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.H2, w.r, dt),
                 sg.lora_apply_workspace_bytes(w.num_rows, w.num_segments, w.H1, w.H2, w.r, dt))
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % nsets]
        if mode == "fused":
            sg.lora_linear(s["x"], s["W"], s["A"], s["B"], seg, ids, w.scale, bias=s["b"],
                           out=s["y"], workspace=ws)
        elif mode == "base":
            torch.addmm(s["b"], s["x"], s["W"].t(), out=s["y"])
        else:
            torch.addmm(s["b"], s["x"], s["W"].t(), out=s["y"])
            sg.lora_apply(s["y"], s["x"], s["A"], s["B"], seg, ids, w.scale, workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize(dev)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step(warmup)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(steps):
            step(warmup + k)
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize(dev)
    us = start.elapsed_time(end) * 1e3 / steps
    # What the fused layer must move: W, bias, x, y written once, each
    # segment's adapter.
    segs = int((w.seg_lengths > 0).sum())
    abytes = (w.H1 * w.H2 + w.H2 + w.num_rows * (w.H1 + w.H2) + segs * w.r * (w.H1 + w.H2)) * e
    return {"mode": mode, "workload": w.name, "us_per_call": us, "buffer_sets_rotated": nsets,
            "algorithmic_bytes": abytes, "achieved_hbm_GBps": abytes / us / 1e3,
            "hbm_peak_frac": abytes / us / 1e3 / HBM_PEAK_GBPS,
            "base_flops_TFLOPs": 2.0 * w.num_rows * w.H1 * w.H2 / us / 1e6}


SWEEP_ROWS = (1, 2, 4, 8, 16, 32, 64, 128, 256)


def rows_sweep(steps: int, warmup: int, rows=SWEEP_ROWS):
    """Latency against batch size at the Llama-2-7B decode shape (4096 ->
    4096, r = 16, fp16), the pages' microbenchmark: for each number of rows,
    lora_apply with every row on its own adapter and with all rows on one
    adapter, the base layer's own GEMM (torch's addmm, W [4096, 4096]), and
    the base GEMM followed by the distinct-adapter add-on.  All cold (inputs
    rotated over >= 1 GiB), each a HIP graph of `steps` steps timed with HIP
    events.  Yields one dict per row count."""
    import workloads as wl
    for R in rows:
        out = {"rows": R}
        for tag, distinct in (("distinct", True), ("same", False)):
            w = wl.decode_batch(R, distinct=distinct)
            res = run_gpu(w, steps, warmup, replays=3)
            us = res["gpu_ms"] * 1e3 / steps
            out[f"sgmv_{tag}_us"] = us
            out[f"sgmv_{tag}_GBps"] = algorithmic_bytes(w) / us / 1e3
            out[f"sgmv_{tag}_fallback_flag"] = res["fallback_flag"]
        w = wl.decode_batch(R, distinct=True)
        out["base_gemm_us"] = run_linear(w, "base", steps, warmup)["us_per_call"]
        out["base_plus_sgmv_us"] = run_linear(w, "unfused", steps, warmup)["us_per_call"]
        yield out


def ranks_sweep(steps: int, warmup: int):
    """lora_apply across ranks, cold, against its algorithmic bytes: the
    prefill shape (4096 rows, 4096 -> 4096, the same 16 segments and
    adapters) at ranks 16..128 in fp16 and bf16 (the ranks the matrix cores
    serve), and the decode shape (64 rows, each its own adapter) at ranks
    8..128 in fp16, bf16 and fp32.  Yields one dict per (shape, dtype, rank)."""
    import numpy as np
    import workloads as wl
    lengths = [int(n) for n in np.diff(wl.prefill(seed=0).seg_indptr)]
    cases = [("prefill", d, r) for d in ("f16", "bf16") for r in (16, 32, 64, 128)]
    cases += [("decode", d, r) for d in ("f16", "bf16", "f32") for r in (8, 16, 32, 64, 128)]
    for shape, dtype, r in cases:
        if shape == "prefill":
            w = wl.make_workload(f"prefill_4096_r{r}_{dtype}", dtype, 4096, 4096, r, 16, lengths,
                                 list(range(16)), 2.0, seed=1)
        else:
            w = wl.decode_batch(64, distinct=True, r=r, dtype=dtype, num_adapters=64)
        res = run_gpu(w, steps, warmup, replays=3)
        us = res["gpu_ms"] * 1e3 / steps
        gbps = algorithmic_bytes(w) / us / 1e3
        yield {"shape": shape, "dtype": dtype, "r": r, "us": us,
               "algorithmic_bytes": algorithmic_bytes(w), "achieved_hbm_GBps": gbps,
               "frac_of_8TBps": gbps / 8000.0, "fallback_flag": res["fallback_flag"]}


def copy_floor(w, steps: int, warmup: int, device="cuda:0", nbytes=None):
    """What a plain device-to-device copy moving the workload's algorithmic
    bytes per call (half read, half written) costs under the same method:
    buffers rotated over >= 1 GiB so that every copy reads HBM, the timed
    copies captured in one HIP graph, HIP events on the replay stream.  A
    reference for how fast any single launch can move that many bytes cold
    on this device; not a figure of the SGMV kernels."""
    import torch
    dev = torch.device(device)
    half = max((algorithmic_bytes(w) if nbytes is None else nbytes) // 2 // 16 * 16, 16)
    nsets = max(2, min(512, math.ceil(ROTATE_BYTES / (2 * half))))
    src = [torch.empty(half, dtype=torch.uint8, device=dev).fill_(1) for _ in range(nsets)]
    dst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(nsets)]
    for i in range(warmup):
        dst[i % nsets].copy_(src[i % nsets])
    torch.cuda.synchronize(dev)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        dst[0].copy_(src[0])
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(steps):
            dst[(warmup + k) % nsets].copy_(src[(warmup + k) % nsets])
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize(dev)
    us = start.elapsed_time(end) * 1e3 / steps
    moved = 2 * half
    return {"mode": "copy floor", "workload": w.name, "bytes_moved_per_copy": moved,
            "us_per_copy": us, "GBps": moved / us / 1e3, "hbm_peak_frac": moved / us / 1e3 / HBM_PEAK_GBPS,
            "buffer_sets_rotated": nsets}


def copy_calibration(nbytes: int, reps: int = 20):
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters (run it under rocprofv3 --pmc)."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def _host_threads() -> int:
    """Threads the host offers this process: its CPU affinity, capped by
    OMP_NUM_THREADS when that is set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def _row_groups(w, groups: int):
    """The batch cut into `groups` contiguous row ranges of about equal size,
    each with the segment table clipped to its rows (a segment split at a
    cut becomes two segments with the same adapter: the rows are
    independent).  Each range is an independent sub-batch for one thread."""
    R = w.num_rows
    bounds = [round(R * g / groups) for g in range(groups + 1)]
    out = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        if hi <= lo:
            continue
        s_lo = w.seg_indptr[:-1]
        s_hi = w.seg_indptr[1:]
        keep = (s_hi > lo) & (s_lo < hi)
        a = np.clip(s_lo[keep], lo, hi) - lo
        b = np.clip(s_hi[keep], lo, hi) - lo
        seg = np.concatenate([a[:1], b]).astype(np.int32) if keep.any() else np.zeros(1, np.int32)
        out.append((lo, hi, seg, w.adapter_ids[keep].astype(np.int32)))
    return out


def cpu_baseline(w, budget_s: float = 10.0):
    """The CPU oracle (plain fp64 loops, as it stands) on the same batch: one
    thread on the whole batch, then every host thread at once, each running
    the oracle on its own contiguous range of rows (the oracle's ctypes
    call releases the GIL, so the threads run in parallel).  Each leg runs
    for about ``budget_s`` / 2 seconds."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    orc = oracle.get()
    rows_per_batch = int(w.seg_lengths.sum())

    calls = 0
    t0 = time.perf_counter()
    while True:
        orc.lora_apply(w.y0, w.x, w.A, w.B, w.seg_indptr, w.adapter_ids, w.scale)
        calls += 1
        el1 = time.perf_counter() - t0
        if el1 >= budget_s / 2:
            break
    single = rows_per_batch * calls / el1

    nthreads = _host_threads()
    groups = _row_groups(w, nthreads)

    def one(g):
        lo, hi, seg, ids = g
        orc.lora_apply(w.y0[lo:hi], w.x[lo:hi], w.A, w.B, seg, ids, w.scale)

    batches = 0
    with ThreadPoolExecutor(max_workers=len(groups)) as pool:
        t0 = time.perf_counter()
        while True:
            list(pool.map(one, groups))
            batches += 1
            el2 = time.perf_counter() - t0
            if el2 >= budget_s / 2:
                break
    multi = rows_per_batch * batches / el2
    return dict(value=multi, unit="rows/s", cores=len(groups), kind="oracle",
                sample=f"{batches} full {w.num_rows}-row batches of the same workload over "
                       f"{len(groups)} threads, each thread a contiguous range of rows "
                       f"({el2:.1f} s); single thread: {calls} batches ({el1:.1f} s)",
                single_thread={"value": single, "unit": "rows/s", "cores": 1},
                nproc=os.cpu_count(), affinity=(len(os.sched_getaffinity(0))
                                                if hasattr(os, "sched_getaffinity") else None),
                OMP_NUM_THREADS=os.environ.get("OMP_NUM_THREADS"))


def adapter_load(w, reps: int = 20, device="cuda:0"):
    """On-demand loading: the workload's whole adapter stack copied from
    pinned host memory (the cold start of one layer's stack) in one call and
    with one call per adapter, and one adapter alone; HIP events around
    `reps` repetitions each."""
    import torch
    import segmented_gather_gemv_sgmv_amd as sg
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    dev = torch.device(device)
    hA = torch.empty(w.A.shape, dtype=dt, pin_memory=True)
    hB = torch.empty(w.B.shape, dtype=dt, pin_memory=True)
    hA.copy_(torch.from_numpy(w.A).to(dt))
    hB.copy_(torch.from_numpy(w.B).to(dt))
    A_dev = torch.empty(w.A.shape, dtype=dt, device=dev)
    B_dev = torch.empty(w.B.shape, dtype=dt, device=dev)
    N = w.num_adapters

    def load(slots):
        if slots == "all":  # the whole stack in one call: two copies
            sg.load_adapter(A_dev, B_dev, 0, hA, hB)
            return
        for k in slots:
            sg.load_adapter(A_dev, B_dev, k, hA[k], hB[k])

    def timed(slots):
        load(slots)
        torch.cuda.synchronize(dev)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            load(slots)
        b.record()
        torch.cuda.synchronize(dev)
        return a.elapsed_time(b) / 1e3 / reps

    per_adapter = (w.H1 * w.r + w.r * w.H2) * w.elem_bytes
    t_all = timed("all")
    t_each = timed(range(N))
    t_one = timed([0])
    ok = torch.equal(A_dev.cpu(), hA) and torch.equal(B_dev.cpu(), hB)
    return {
        "metric": "on-demand adapter load, host (pinned) to device stack",
        "value": N * per_adapter / t_all / 1e9, "unit": "GB/s", "higher_is_better": True,
        "n_gpus": 1, "data": "synthetic (seeded)",
        "config": {"workload": w.name, "adapters": N, "bytes_per_adapter": per_adapter,
                   "repetitions": reps},
        "us_whole_stack": t_all * 1e6, "us_whole_stack_one_call_per_adapter": t_each * 1e6,
        "us_one_adapter": t_one * 1e6, "copied_correctly": ok,
    }


# Timed workloads by name: the decode projection the metric is quoted on, and
# the other seeded configurations (each a lora_apply call of its own shape).
WORKLOADS = {
    "llama7b_decode": lambda wl: wl.llama7b_decode(seed=0),
    "skewed_decode": lambda wl: wl.skewed_decode(seed=0),
    "skewed_decode_control": lambda wl: wl.skewed_decode(seed=0, control=True),
    "prefill": lambda wl: wl.prefill(seed=0),
    "mlp_up_decode": lambda wl: wl.mlp_up_decode(seed=0),
    "tiny": lambda wl: wl.tiny(seed=0),
    "mixed": lambda wl: wl.mixed_batch(seed=0),
}
WORKLOAD_SHAPES = {
    "llama7b_decode": "Llama-2-7B decode shapes",
    "skewed_decode": "Llama-2-7B shapes, Zipf segment lengths",
    "skewed_decode_control": "Llama-2-7B shapes, one segment",
    "prefill": "Llama-2-7B prefill shapes",
    "mlp_up_decode": "Llama-13B up-projection decode shapes",
    "tiny": "tiny shapes",
    "mixed": "Llama-2-7B shapes, two 512-row prefill segments and 128 one-row decode segments",
}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain BYTES-sized device copy (counter calibration)")
    ap.add_argument("--row-ids", choices=("runs", "grouped"), default=None,
                    help="start every step from per-row adapter ids: build the segment "
                         "table on the device (run table or grouped table), then lora_apply")
    ap.add_argument("--adapter-load", action="store_true",
                    help="instead: time on-demand loading of the workload's adapters from "
                         "pinned host memory into the device stacks (sgmv_load_adapter)")
    ap.add_argument("--warm", action="store_true",
                    help="no buffer rotation: the same inputs every step, resident in the "
                         "256 MB Infinity Cache (a warm figure, not the HBM one)")
    ap.add_argument("--projections", type=int, default=1, choices=range(1, 9), metavar="P",
                    help="P add-ons of the workload's shape over the same batch in one "
                         "lora_apply_multi call (e.g. a layer's q/k/v/o projections)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead: latency against rows per call (1..256) at the decode shape, "
                         "distinct and identical adapters, beside the base layer's GEMM")
    ap.add_argument("--ranks", action="store_true",
                    help="instead: the prefill shape at ranks 16..128 (fp16, bf16) and the decode "
                         "shape at ranks 8..128 (fp16, bf16, fp32)")
    ap.add_argument("--linear", choices=("fused", "unfused", "base"), default=None,
                    help="instead: time the adapted linear layer over the workload's batch, "
                         "base product fused in (lora_linear) or not (addmm + lora_apply)")
    ap.add_argument("--entry", choices=("apply", "shrink", "expand"), default="apply",
                    help="entry point timed: lora_apply (default), or sgmv_shrink / sgmv_expand "
                         "alone, each against its own algorithmic bytes")
    ap.add_argument("--floor", action="store_true",
                    help="instead: time a plain device copy moving the workload's algorithmic "
                         "bytes per call, cold, as a reference floor for one launch")
    ap.add_argument("--workload", default="llama7b_decode", choices=sorted(WORKLOADS),
                    help="workload to time (default: the Llama-2-7B decode projection); the "
                         "others are the remaining seeded configurations")
    args = ap.parse_args(argv)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "SGMV shards by segments with no exchange, so per-GPU throughput is the "
              "figure of interest.", file=sys.stderr)
        return 2

    import torch
    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1

    w = WORKLOADS[args.workload](wl)
    if args.adapter_load:
        print(json.dumps(adapter_load(w)), flush=True)
        return 0
    if args.floor:
        print(json.dumps(copy_floor(w, args.steps, args.warmup)), flush=True)
        return 0
    if args.linear:
        print(json.dumps(run_linear(w, args.linear, args.steps, args.warmup)), flush=True)
        return 0
    if args.sweep:
        for point in rows_sweep(min(args.steps, 400), min(args.warmup, 40)):
            print(json.dumps(point), flush=True)
        return 0
    if args.ranks:
        for point in ranks_sweep(min(args.steps, 200), min(args.warmup, 20)):
            print(json.dumps(point), flush=True)
        return 0
    P = args.projections
    entry = args.entry
    if entry != "apply" and (P != 1 or args.row_ids):
        print("bench.py: --entry shrink|expand times one add-on with a given segment table",
              file=sys.stderr)
        return 2
    res = run_gpu(w, args.steps, args.warmup, row_ids=args.row_ids, projections=P, warm=args.warm,
                  entry=entry)
    step_s = res["gpu_ms"] / 1e3 / args.steps
    rows = int(w.seg_lengths.sum()) * P  # a row through one add-on is one SGMV row
    abytes = entry_bytes(w, entry) * P
    flops = algorithmic_flops(w) * P
    if entry == "shrink":
        flops = 2 * rows * w.r * w.H1
    elif entry == "expand":
        flops = 2 * rows * w.r * w.H2
    achieved = abytes / step_s / 1e9
    line = {
        "metric": "SGMV rows/s and achieved HBM GB/s (% of peak) per layer call, H=4096 r=16",
        "value": rows / step_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; " + WORKLOAD_SHAPES[args.workload] + ", no weights)",
        "config": {
            "workload": w.name, "H1": w.H1, "H2": w.H2, "r": w.r, "rows": rows,
            "segments": w.num_segments, "adapters_in_stack": w.num_adapters, "scale": w.scale,
            "buffer_sets_rotated": res["nsets"], "launch": "hip graph of all timed steps",
            "projections": P,
            "cache": "warm (inputs reused every step)" if args.warm else "cold (rotated buffers)",
            "segment_table": ("given" if args.row_ids is None
                              else f"built on the device from per-row ids ({args.row_ids})"),
            "entry_point": {"apply": "lora_apply", "shrink": "sgmv_shrink",
                            "expand": "sgmv_expand"}[entry],
        },
        "us_per_call": step_s * 1e6,
        "timing": f"median over {res['replays']} replays of the {args.steps}-step graph, "
                  "HIP events on the replay stream",
        "us_per_call_each_replay": res["us_per_step_each_replay"],
        "fallback_flag": res["fallback_flag"],
        "us_per_call_p10_p50_p90": res["us_p10_p50_p90"],
        "spread": f"per-call means of {res['spread_replays']} separately timed replays "
                  f"of a {res['spread_steps']}-step graph",
        "achieved_hbm_GBps": achieved,
        "hbm_peak_frac": achieved / HBM_PEAK_GBPS,
        "roofline": {
            "bound": "hbm",
            "kernel": ("lora_mixed_kernel (one launch per step)"
                       if args.workload == "llama7b_decode" and args.row_ids is None and P == 1
                       and entry == "apply" else "every launch of one step"),
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": (measured_traffic(w.name)
                        if args.row_ids is None and P == 1 and not args.warm and entry == "apply"
                        else None),
            "algorithmic_bytes_per_launch": abytes,
            "tflops": flops / step_s / 1e12,
        },
        "wall_s_timed": res["wall_s"],
    }
    if not args.warm:
        # A plain copy moving the same bytes per launch, cold, same method.
        fl = copy_floor(w, args.steps, args.warmup, nbytes=abytes)
        line["roofline"]["copy_floor"] = {"us": fl["us_per_copy"], "GBps": fl["GBps"],
                                          "frac_of_peak": fl["hbm_peak_frac"],
                                          "kernel_vs_floor": step_s * 1e6 / fl["us_per_copy"]}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
