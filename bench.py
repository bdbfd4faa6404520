#!/usr/bin/env python3
"""Benchmark of the fused MQA attention step on one MI355X.

A step is one pass of the whole hot path over one batch of resident inputs:
pad (in place) -> block map -> fused Q.K^T / online softmax / P.V.  The default
workload is decode on a raw sliding-window layer: 64 sequences x 1 token x 64
query heads x head dim 512 over a 128-row float16 ring each.  The headline value
is K/V bytes per second over whole steps; the prefill chunks (2048 tokens) are
reported beside it in TFLOP/s.

Protocol:
* inputs: seeded synthetic workloads, uploaded once per input set before timing;
  ``--sets`` copies rotate so consecutive steps never find their data in the
  256 MB last-level cache (20 x 29.4 MB for the decode batch);
* timed region: K steps, replayed from HIP graphs (one graph per rotation of the
  input sets), bracketed by torch.cuda.synchronize() and wall-clock time;
* kernel time: HIP events on the launch stream around each attention launch,
  queued behind a GPU spin so that the events bracket back-to-back kernels and
  not host enqueue gaps; the average feeds the roofline object;
* cpu_baseline: the float64 NumPy oracle on the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn decode KV GB/s (%HBM peak) + 2048-tok prefill TFLOP/s (%MFMA peak), d=512"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix throughput, published
DECODE_KERNEL_SRC = os.path.join(ROOT, "query_flashattention_amd", "csrc", "attn_staged.hip")

DESCRIPTIONS = {
    "decode_swa": "decode, raw sliding-window layer: 64 sequences x 1 token x 64 q-heads x d512, "
                  "1 KV head, full 128-row fp16 ring (seeded write pointer), fp32 out",
    "decode_r128": "decode, ratio-128 layer at 32K context: 1 sequence x 1 token x 64 q-heads x d512, "
                   "128 ring rows + 256 compressed slots (last block partly valid)",
    "decode_r128_b64": "decode, ratio-128 layer at 32K context, 64 sequences",
    "decode_r4": "decode, ratio-4 indexed layer at 8K context: 64 sequences x 1 token x 64 q-heads x d512, "
                 "128 ring rows + top-512 of 2048 compressed rows per sequence",
    "prefill_swa": "prefill chunk, raw layer: 2048 tokens x 64 q-heads x d512, causal + 128 window",
    "prefill_r4": "prefill chunk, ratio-4 layer at position 30720: 2048 tokens x 64 q-heads x d512, "
                  "2175 raw rows (causal + 128 window) + top-512 of 7680 compressed rows per token",
    "decode_swa_fp8": "decode_swa with FP8 K/V rows (E4M3 codes + one float32 scale per row)",
    "decode_r128_fp8": "decode_r128_b64 with FP8 K/V rows",
    "decode_r4_fp8": "decode_r4 with FP8 K/V rows",
    "prefill_r4_fp8": "prefill_r4 with FP8 K/V rows",
}


# --------------------------------------------------------------------------- algorithmic counts

def counts(w):
    """Algorithmic FLOPs and compulsory HBM bytes of one attention launch.

    FLOPs: 4*H*D per visible (token, row) pair (Q.K^T and P.V, 2 flops per MAC).
    Bytes: every K/V row some token sees, once per sequence, Q read once and O
    written once; rows gathered through an index list are also counted once per
    (token, entry) as gather traffic (mostly served by the caches).
    Visible rows per token come from the window interval and the validity
    bytes of the workload (interval arithmetic on the inputs, no attention)."""
    import numpy as np
    import torch

    b, t, h, d = w.q.shape
    es = w.q.element_size()
    # a K or V row: d elements, or d E4M3 codes plus its float32 scale
    row_bytes = d + 4 if w.r0.k.dtype == torch.uint8 else d * es
    n0 = w.r0.n_rows
    toks = np.arange(t, dtype=np.int64)
    pairs = 0
    kv_rows = 0        # distinct K/V rows read from HBM
    gathered = 0       # rows fetched per (token, index entry)
    for bi in range(b):
        v0 = np.ones(n0, bool) if w.r0.valid is None else (w.r0.valid[bi, :n0].numpy() != 0)
        if w.window > 0:
            hi = np.minimum(n0 - 1, w.q_pos0 + toks - w.k_pos0)
            lo = np.maximum(0, w.q_pos0 + toks - w.k_pos0 - w.window + 1)
        else:
            hi = np.full(t, n0 - 1)
            lo = np.zeros(t, dtype=np.int64)
        cover = np.zeros(n0 + 1, dtype=np.int64)
        csum = np.concatenate([[0], np.cumsum(v0)])
        for a, z in zip(lo, hi):
            if z >= a:
                pairs += int(csum[z + 1] - csum[a])
                cover[a] += 1
                cover[z + 1] -= 1
        kv_rows += int(((np.cumsum(cover)[:n0] > 0) & v0).sum())
        if w.r1 is not None and w.r1.n_rows > 0:
            n1 = w.r1.n_rows
            v1 = np.ones(n1, bool) if w.r1.valid is None else (w.r1.valid[bi, :n1].numpy() != 0)
            if w.r1_index is None:
                pairs += t * int(v1.sum())
                kv_rows += int(v1.sum())
            else:
                idx = w.r1_index[bi].numpy().astype(np.int64)
                ok = (idx >= 0) & (idx < n1)
                ok[ok] = v1[idx[ok]]
                pairs += int(ok.sum())
                gathered += int(ok.sum())
                kv_rows += int(np.unique(idx[ok]).size)
    flops = 4.0 * h * d * pairs
    kv_bytes = 2.0 * row_bytes * kv_rows
    q_bytes = float(b * t * h * d * es)
    o_bytes = float(b * t * h * d * 4)
    return {"flops": flops, "kv_bytes": kv_bytes, "q_bytes": q_bytes, "o_bytes": o_bytes,
            "pairs": pairs, "gather_bytes": 2.0 * row_bytes * gathered}


# --------------------------------------------------------------------------- GPU timing

class Runner:
    """Resident input sets, graphs of whole steps and timing helpers for one workload."""

    def __init__(self, name, n_sets, device="cuda:0", splits=None):
        import torch
        from query_flashattention_amd import ds4attn as da, pipeline, workloads

        self.torch, self.da, self.pipeline = torch, da, pipeline
        self.name = name
        self.w = workloads.named(name)
        self.kind = "decode" if name.startswith("decode") else "prefill"
        self.bq = 1 if self.kind == "decode" else da.ds4attn_prefill_bq()
        self.sets = [pipeline.to_device(self.w, device) for _ in range(n_sets)]
        self.blks = []
        for dp in self.sets:
            nt, nb = da.ds4attn_blockmap_dims(dp.args(), self.bq)
            self.blks.append(torch.empty((dp.q.shape[0], nt, nb), dtype=torch.uint8, device=device))
        # the workspace of the library's own split plan (splits=None: ds4attn_decode
        # picks it) or of a chosen split (ds4attn_decode_split); None when unsplit
        self.splits = splits

        def ws_bytes(a):
            if splits is None:
                return da.ds4attn_workspace_bytes(a, self.kind == "prefill")
            return da.ds4attn_decode_workspace_bytes(a, splits)

        self.ws = []
        for dp in self.sets:
            n = ws_bytes(dp.args())
            self.ws.append(torch.empty(n, dtype=torch.uint8, device=device) if n else None)
        # parts per token: the workspace holds one record set per part
        self.parts = 1
        if self.kind == "decode":
            a = self.sets[0].args()
            per_part = da.ds4attn_decode_workspace_bytes(a, 2) // 2
            self.parts = max(1, ws_bytes(a) // per_part) if per_part else 1
        torch.cuda.synchronize()

    def step(self, i):
        self.pipeline.step(self.sets[i], self.kind, self.bq, self.blks[i], splits=self.splits,
                           workspace=self.ws[i])

    def attention_only(self, i):
        dp = self.sets[i]
        blk = self.blks[i]
        if self.splits is not None and self.splits > 1:
            self.da.ds4attn_decode_split(dp.args(), dp.q, blk if blk.numel() else None, self.bq, dp.o,
                                         self.splits, self.ws[i])
            return
        fn = self.da.ds4attn_decode if self.kind == "decode" else self.da.ds4attn_prefill
        fn(dp.args(), dp.q, blk if blk.numel() else None, self.bq, dp.o, self.ws[i])

    def capture(self):
        """One graph per full rotation of the input sets and one per single set."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(len(self.sets)):
                self.step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g_all):
            for i in range(len(self.sets)):
                self.step(i)
        self.g_one = []
        for i in range(len(self.sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(i)
            self.g_one.append(g)
        torch.cuda.synchronize()

    def timed_steps(self, k):
        """Wall-clock seconds for exactly k steps (graph replays), synchronised on both sides."""
        torch = self.torch
        r = len(self.sets)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(k // r):
            self.g_all.replay()
        for i in range(k % r):
            self.g_one[i].replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def spin_ms(self, ms):
        """Queue a GPU busy-wait of about `ms` milliseconds (calibrated once)."""
        torch = self.torch
        if not hasattr(self, "_cycles_per_ms"):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 10_000_000
            e0.record()
            torch.cuda._sleep(n)
            e1.record()
            torch.cuda.synchronize()
            self._cycles_per_ms = n / max(e0.elapsed_time(e1), 1e-3)
        torch.cuda._sleep(int(self._cycles_per_ms * ms))

    def kernel_ms(self, launches):
        """Average duration (ms) of the attention kernel: HIP events on the launch
        stream around graph replays that hold only attention launches (the input sets
        in turn, at least 20 launches per graph; maps and padding prepared
        beforehand), so the figure is the kernel's
        own time plus the short gap between back-to-back dispatches.  Also the
        latency of single launches (one event pair each) for context."""
        torch = self.torch
        r = len(self.sets)
        for i in range(r):
            dp = self.sets[i]
            dp.r0.pad_in_place()
            if dp.r1 is not None:
                dp.r1.pad_in_place()
            self.da.ds4attn_blockmap(dp.args(), self.bq, self.blks[i] if self.blks[i].numel() else None)
        torch.cuda.synchronize()
        # (at least 20 launches per graph, the sets in turn: with few large input sets
        # a graph of one round would time its own launch overhead with every replay)
        rounds = max(1, 20 // r)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(rounds):
                for i in range(r):
                    self.attention_only(i)
        g.replay()
        torch.cuda.synchronize()
        per_graph = rounds * r
        reps = max(1, launches // per_graph)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        self.spin_ms(20.0)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        mean = e0.elapsed_time(e1) / (reps * per_graph)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(launches)]
        self.spin_ms(20.0)
        for k in range(launches):
            evs[k][0].record()
            self.attention_only(k % r)
            evs[k][1].record()
        torch.cuda.synchronize()
        d = sorted(a.elapsed_time(b) for a, b in evs)
        return {"mean": mean, "launches": reps * per_graph, "single_launch_median": d[len(d) // 2],
                "single_launch_p10": d[len(d) // 10], "single_launch_p90": d[(9 * len(d)) // 10]}


# --------------------------------------------------------------------------- CPU baseline

def _oracle_rate(p, seconds):
    from oracle import reference as ref
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref.attention(p)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return reps, el


def host_cpu():
    """The host the CPU baseline ran on: the cores in the process's affinity mask
    and the CPU model (from /proc/cpuinfo)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline(w, kv_bytes_per_step, seconds):
    """The float64 oracle on the host, over whole batches of the same workload,
    repeated until `seconds` of CPU work; K/V GB/s on the same algorithmic bytes.
    Run with the BLAS threads the process has, and again with one thread."""
    from oracle import reference as ref
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads, threadpool_limits = 1, None
    p = ref.from_workload(w)
    reps, el = _oracle_rate(p, seconds)
    out = {"value": round(kv_bytes_per_step * reps / el / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"float64 NumPy oracle over the whole batch ({w.q.shape[0]} sequences), "
                     f"{reps} repetitions in {el:.1f} s",
           **host_cpu()}
    if threadpool_limits is not None:
        with threadpool_limits(1):
            reps1, el1 = _oracle_rate(p, seconds / 2)
        out["single_thread"] = {"value": round(kv_bytes_per_step * reps1 / el1 / 1e9, 3), "unit": "GB/s",
                                "cores": 1, "sample": f"{reps1} repetitions in {el1:.1f} s"}
    return out


# --------------------------------------------------------------------------- measured peaks

def measured_peaks(torch):
    """Achievable HBM read bandwidth and float16 MFMA throughput of this device,
    from the probe library (libds4probes.so): a streaming read of 4 GiB, and a loop
    of independent MFMA chains on 2 waves per SIMD.  Also the shader clock during
    the MFMA loop (cycles over 100 MHz reference ticks)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "query_flashattention_amd", "libds4probes.so"))
    lib.ds4probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_void_p]
    lib.ds4probe_mfma_loop.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p]
    lib.ds4probe_mfma_loop_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.ds4probe_mfma_loop_flops.restype = ctypes.c_int64
    stream = torch.cuda.current_stream().cuda_stream
    nbytes, grid, reps = 4 << 30, 4096, 5
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    assert lib.ds4probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        assert lib.ds4probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, stream) == 0
    e1.record()
    torch.cuda.synchronize()
    hbm = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sink
    mgrid, iters = 512, 4000
    out = torch.empty(mgrid * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * mgrid * 4, dtype=torch.int64, device="cuda")
    assert lib.ds4probe_mfma_loop(iters, out.data_ptr(), clocks.data_ptr(), mgrid, stream) == 0
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        assert lib.ds4probe_mfma_loop(iters, out.data_ptr(), clocks.data_ptr(), mgrid, stream) == 0
    e1.record()
    torch.cuda.synchronize()
    tflops = lib.ds4probe_mfma_loop_flops(iters, mgrid) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    ck = clocks.view(-1, 2).cpu().double()
    mhz = float((ck[:, 0] / (ck[:, 1] * 10e-9)).median()) / 1e6
    return {"hbm_read_GBps": round(hbm, 1), "mfma_f16_TFLOPs": round(tflops, 1),
            "shader_clock_MHz_in_mfma_loop": round(mhz, 1),
            "method": "libds4probes.so: 5 streaming reads of 4 GiB (4096 x 256 threads, 16-byte loads); "
                      f"{mgrid} workgroups x 4 waves x {iters} x 8 independent v_mfma_f32_16x16x32_f16"}


def decode_kernel_label(w, parts=1):
    """The decode kernel the library picks for a workload split into `parts` (the
    same rule as its dispatch: the KEYS split when each part's share of the longest
    possible block list holds at least 40 blocks, 8 for FP8 rows)."""
    nb0 = -(-w.r0.n_rows // 32)
    if w.window > 0:
        nb0 = min(nb0, w.window // 32 + 2)
    nb1 = 0
    if w.r1 is not None and w.r1.n_rows > 0:
        nb1 = -(-w.r1_index.shape[-1] // 32) if w.r1_index is not None else -(-w.r1.n_rows // 32)
    least = 8 if w.r0.k_scale is not None else 40
    if (nb0 + nb1) // max(1, parts) >= least:
        return 2
    groups = w.q.shape[0] * w.q.shape[1] * (w.q.shape[2] // 16)
    wide = parts == 1 and w.r1_index is None and w.q.shape[2] % 32 == 0 and groups > 256
    return 3 if wide else 1


def prefill_cpu_tflops(w, n_tokens, seconds):
    """Oracle TFLOP/s on a sample of tokens of a prefill chunk (for context lines)."""
    import numpy as np
    from oracle import reference as ref
    p = ref.from_workload(w)
    rng = np.random.default_rng(0)
    toks = sorted(rng.choice(w.q.shape[1], n_tokens, replace=False).tolist())
    pairs = sum(len(a) + len(b) for a, b in (ref.visible_rows(p, 0, t) for t in toks))
    t0 = time.perf_counter()
    reps = 0
    while True:
        ref.attention(p, tokens=[(0, t) for t in toks])
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return 4.0 * w.q.shape[2] * w.q.shape[3] * pairs * reps / el / 1e12


# --------------------------------------------------------------------------- main

def traffic_from_profiles(kernel_src):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken on the
    current kernel source (the summary records the source's SHA-256)."""
    path = os.path.join(ROOT, "profiles", "decode_swa_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(kernel_src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if rec.get("kernel_source_sha256") != sha:
            return None
        return rec.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None


def topk_timing(rows, n, k, n_sets=4, reps=25):
    """Mean duration of one ds4attn_topk launch over [rows, n] float32 scores (HIP
    events around graph replays, input sets rotated), with its algorithmic bytes
    (scores read once, indices written once)."""
    import torch
    from query_flashattention_amd import ds4attn as da, workloads

    sets = [workloads.indexer_scores(300 + i, rows, n).to("cuda") for i in range(n_sets)]
    outs = [torch.empty((rows, k), dtype=torch.int32, device="cuda") for _ in range(n_sets)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s, o in zip(sets, outs):
            da.ds4attn_topk(s, k, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s, o in zip(sets, outs):
            da.ds4attn_topk(s, k, o)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n_sets)
    nbytes = 4.0 * rows * n + 4.0 * rows * k
    return {"rows": rows, "n": n, "k": k, "kernel_us_mean": round(ms * 1e3, 2),
            "algorithmic_bytes": nbytes, "gbs_kernel": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "rows_per_s": round(rows / (ms * 1e-3), 1)}


def compress_timing(b, ratio, n_state, n_new, d=512, n_sets=4, reps=25):
    """Mean duration of one ds4attn_compress call (pooling, plus the state update when
    rows remain) over seeded inputs, with its algorithmic bytes: every stream row's
    values (float16) and scores (float32) read once, the compressed rows and the new
    state written once."""
    import torch
    from query_flashattention_amd import ds4attn as da, workloads

    ins = [workloads.compress_inputs(500 + i, b, ratio, n_state, n_new, d) for i in range(n_sets)]
    dev = [(ci.state_kv.cuda(), ci.state_score.cuda(), ci.kv_new.cuda(), ci.score_new.cuda()) for ci in ins]
    n_out = (n_state + n_new) // ratio
    outs = [torch.empty(b, max(n_out, 1), d, dtype=torch.float16, device="cuda") for _ in range(n_sets)]

    def calls():
        for (skv, ssc, kv, sc), o in zip(dev, outs):
            da.ds4attn_compress(skv, ssc, n_state, kv, sc, ratio, o)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        calls()
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n_sets)
    n_next = (n_state + n_new) % ratio
    nbytes = b * ((n_state + n_new) * 6.0 * d + n_out * 2.0 * d + n_next * 6.0 * d)
    return {"batch": b, "ratio": ratio, "n_state": n_state, "n_new": n_new, "head_dim": d,
            "compressed_rows_per_seq": n_out, "kernel_us_mean": round(ms * 1e3, 2),
            "algorithmic_bytes": nbytes, "gbs_kernel": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def quantize_timing(b, n, d=512, n_sets=4, reps=25):
    """Mean duration of one ds4attn_quantize_fp8 launch over [b, n, d] float16 rows,
    with its algorithmic bytes (rows read once; codes and scales written once)."""
    import torch
    from query_flashattention_amd import ds4attn as da

    g = torch.Generator().manual_seed(401)
    xs = [torch.randn(b, n, d, generator=g).half().to("cuda") for _ in range(n_sets)]
    outs = [(torch.empty(b, n, d, dtype=torch.uint8, device="cuda"),
             torch.empty(b, n, dtype=torch.float32, device="cuda")) for _ in range(n_sets)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for x, (c, sc) in zip(xs, outs):
            da.ds4attn_quantize_fp8(x, c, sc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for x, (c, sc) in zip(xs, outs):
            da.ds4attn_quantize_fp8(x, c, sc)
    gr.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n_sets)
    nbytes = b * n * (2.0 * d + d + 4)
    return {"rows": b * n, "head_dim": d, "kernel_us_mean": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
            "gbs_kernel": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def run_workload(name, steps, warmup, n_sets, launches, splits=None):
    r = Runner(name, n_sets, splits=splits)
    for k in range(warmup):
        r.step(k % n_sets)
    r.capture()
    for _ in range(2):
        r.g_all.replay()
    secs = r.timed_steps(steps)
    kern = r.kernel_ms(launches)
    return r, secs, kern


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_swa", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--sets", type=int, default=20, help="input sets rotated to keep caches cold")
    ap.add_argument("--launches", type=int, default=100, help="attention launches timed by events")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-extra", action="store_true", help="skip the prefill / ratio-128 lines")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak probes")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention step of one sequence batch does not span GPUs here)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    from query_flashattention_amd import ds4attn as da
    da.lib()

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "copies": 5}))
        return

    name = args.workload
    n_sets = args.sets if name.startswith("decode") else 2
    runner, secs, kern = run_workload(name, args.steps, args.warmup, n_sets, args.launches)
    c = counts(runner.w)
    ms_step = secs * 1e3 / args.steps
    b, t, h, d = runner.w.q.shape
    compulsory = c["kv_bytes"] + c["q_bytes"] + c["o_bytes"]
    kern_s = kern["mean"] * 1e-3
    if runner.kind == "decode":
        value = c["kv_bytes"] / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = compulsory / kern_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profiles(DECODE_KERNEL_SRC) if name == "decode_swa" else None,
                "kernel": "attn_staged_kernel<%d,%s,%s,false> (ds4attn_decode)" % (
                    decode_kernel_label(runner.w), str(runner.w.r1_index is not None).lower(),
                    str(name.endswith("_fp8")).lower()),
                "bytes_per_launch": compulsory, "kernel_ms_mean": round(kern["mean"], 5),
                "kernel_launches_timed": kern["launches"],
                "single_launch_ms_median": round(kern["single_launch_median"], 5),
                "single_launch_ms_p10": round(kern["single_launch_p10"], 5),
                "single_launch_ms_p90": round(kern["single_launch_p90"], 5)}
    else:
        value = c["flops"] / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = c["flops"] / kern_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "attn_staged_kernel<0,%s,%s,false> (ds4attn_prefill)" % (
                    str(runner.w.r1_index is not None).lower(), str(name.endswith("_fp8")).lower()),
                "flops_per_launch": c["flops"],
                "kernel_ms_mean": round(kern["mean"], 5), "kernel_launches_timed": kern["launches"],
                "single_launch_ms_median": round(kern["single_launch_median"], 5),
                "single_launch_ms_p10": round(kern["single_launch_p10"], 5),
                "single_launch_ms_p90": round(kern["single_launch_p90"], 5)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[name], "name": name, "batch": b, "tokens": t, "heads": h,
                   "head_dim": d, "input_sets_rotated": n_sets, "step": "pad + blockmap + attention"},
        "roofline": roof,
    }
    if not args.no_peaks:
        pk = measured_peaks(torch)
        out["measured_peaks"] = pk
        meas = pk["hbm_read_GBps"] if roof["unit"] == "GB/s" else pk["mfma_f16_TFLOPs"]
        roof["peak_measured"] = meas
        roof["frac_of_measured"] = round(roof["achieved"] / meas, 4)
    if runner.kind == "decode":
        out["kv_bytes_per_step"] = c["kv_bytes"]
        out["pct_hbm_peak_kv"] = round(100 * value / HBM_PEAK_GBS, 2)
        out["kernel_kv_gbs"] = round(c["kv_bytes"] / kern_s / 1e9, 1)
    del runner
    torch.cuda.empty_cache()

    if not args.no_extra and name == "decode_swa":
        extra = {}
        for other in ("prefill_swa", "prefill_r4", "decode_r128", "decode_r128_b64", "decode_r4",
                      "decode_swa_fp8", "decode_r128_fp8", "decode_r4_fp8", "prefill_r4_fp8"):
            sets = 2 if other.startswith("prefill") else (64 if other == "decode_r128" else 20)
            steps = 20 if other.startswith("prefill") else 200
            r, s, k = run_workload(other, steps, 3, sets, 20 if other.startswith("prefill") else 100)
            cc = counts(r.w)
            ms = s * 1e3 / steps
            entry = {"ms_per_step": round(ms, 5), "kernel_ms_mean": round(k["mean"], 5),
                     "single_launch_ms_median": round(k["single_launch_median"], 5),
                     "single_launch_ms_p10": round(k["single_launch_p10"], 5),
                     "single_launch_ms_p90": round(k["single_launch_p90"], 5)}
            if not other.startswith("prefill"):
                entry["kernel_split"] = {1: "DIMS", 2: "KEYS", 3: "WIDE"}[decode_kernel_label(r.w, r.parts)]
                entry["split_parts"] = r.parts
            if other.startswith("prefill"):
                entry["tflops_step"] = round(cc["flops"] / (ms * 1e-3) / 1e12, 2)
                entry["tflops_kernel"] = round(cc["flops"] / (k["mean"] * 1e-3) / 1e12, 2)
                entry["pct_mfma_peak_kernel"] = round(100 * entry["tflops_kernel"] / MFMA_F16_PEAK_TFLOPS, 2)
                entry["algorithmic_gflop"] = round(cc["flops"] / 1e9, 3)
                hbm = cc["q_bytes"] + cc["o_bytes"] + cc["kv_bytes"]
                entry["compulsory_hbm_gbs_kernel"] = round(hbm / (k["mean"] * 1e-3) / 1e9, 1)
            else:
                entry["kv_gbs_kernel"] = round(cc["kv_bytes"] / (k["mean"] * 1e-3) / 1e9, 1)
                entry["kernel_us_mean"] = round(k["mean"] * 1e3, 2)
            extra[other] = entry
            del r
            torch.cuda.empty_cache()
        # one sequence of the ratio-128 layer (12 key blocks) without the split that
        # ds4attn_decode picks for it (the decode_r128 line above: the planned parts
        # per head group plus the combine pass)
        r, s_, k = run_workload("decode_r128", 200, 3, 64, 100, splits=1)
        extra["decode_r128_unsplit"] = {"ms_per_step": round(s_ * 1e3 / 200, 5),
                                         "kernel_ms_mean": round(k["mean"], 5),
                                         "single_launch_ms_median": round(k["single_launch_median"], 5),
                                         "kernel_us_mean": round(k["mean"] * 1e3, 2),
                                         "note": "one workgroup per 16 heads walks all 12 blocks"}
        del r
        torch.cuda.empty_cache()
        # top-k index selection feeding the ratio-4 layers: the prefill chunk's 2048
        # tokens over 7680 compressed rows, and the decode batch's 64 over 2048
        extra["topk_prefill_r4"] = topk_timing(2048, 7680, 512)
        extra["topk_decode_r4"] = topk_timing(64, 2048, 512)
        # the FP8 quantize step over a 64-sequence x 2048-row cache of float16 rows
        extra["quantize_fp8_64x2048"] = quantize_timing(64, 2048)
        extra["compress_prefill_r4"] = compress_timing(1, 4, 0, 2048)
        extra["compress_prefill_r128"] = compress_timing(1, 128, 0, 2048)
        extra["compress_decode_r128_b64"] = compress_timing(64, 128, 127, 1)
        out["extra"] = extra

    if args.cpu_seconds > 0:
        w = __import__("query_flashattention_amd.workloads", fromlist=["named"]).named(name)
        if name.startswith("decode"):
            out["cpu_baseline"] = cpu_baseline(w, c["kv_bytes"], args.cpu_seconds)
        else:
            tf = prefill_cpu_tflops(w, 64, args.cpu_seconds)
            out["cpu_baseline"] = {"value": round(tf, 4), "unit": "TFLOP/s", "kind": "oracle",
                                   "sample": "64 sampled tokens of the chunk", **host_cpu()}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
