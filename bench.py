"""Benchmark of the layerwise QK-Norm hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload gqa_prefill|rank_slice|small_dense|decode_t1|...]

A step is one pass of the whole path over one batch: for the default
workload (GQA prefill: T = 8192 tokens, Q 5120 + K 1024 columns normalized,
V 1024 passed through, bf16 packed [8192, 7168], S = 1) that is one
qknorm_fused call, out of place into a separate packed buffer. Inputs are
resident in HBM before timing starts, and the buffer sets rotate over more
than 1 GiB so that each step streams from HBM rather than from the 256 MB
Infinity Cache.

Prints one JSON line: tokens/s for the whole job, the roofline of the kernel
(algorithmic bytes per launch / mean launch time measured with HIP events on
the launch stream, against the 8 TB/s HBM peak) and the CPU oracle timed on
the host as a baseline.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
ROTATE_MIN_BYTES = 1 << 30      # > 256 MB Infinity Cache + 8 x 4 MB L2
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["layerwise_qk_norm_qknorm_amd/csrc/qknorm_kernels.hip",
                  "layerwise_qk_norm_qknorm_amd/csrc/qknorm_internal.hpp",
                  "layerwise_qk_norm_qknorm_amd/csrc/qknorm_api.cpp"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def to_device(a, dev):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    if a.dtype == np.uint8:
        return torch.from_numpy(a.copy()).view(torch.float8_e4m3fn).to(dev)
    return torch.from_numpy(a.copy()).to(dev)


# ----------------------------------------------------------------------------- ceiling kernels
class CeilingLib:
    """ctypes handle of libstreamceil.so: the plain streaming copy and read
    kernels (16-byte loads, ordinary or non-temporal, and non-temporal 16-byte
    stores) that give the practical HBM ceiling for the bytes a QK-Norm call
    moves."""

    def __init__(self, path=None):
        import ctypes
        from layerwise_qk_norm_qknorm_amd import build_lib
        path = path or build_lib.CEIL_LIB
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.qkceil_stream.argtypes = [vp, i64, vp, i64, i64, i64, ci, ci, ci, ci, vp, vp]
        lib.qkceil_stream.restype = ci
        lib.qkceil_last_error.restype = ctypes.c_char_p
        lib.qkceil_last_error.argtypes = []
        self.lib = lib

    def stream(self, x, ldx, y, ldy, rows, row_bytes, per, block, xk, ntl, sink, stream):
        rc = self.lib.qkceil_stream(x, ldx, y, ldy, rows, row_bytes, per, block, xk, ntl, sink, stream)
        if rc:
            raise RuntimeError(f"qkceil_stream: {self.lib.qkceil_last_error().decode()}")


# (chunks per thread, threads per block, blocks per XCD per run (0: blocks in
# order), non-temporal loads) tried for the ceiling of each call: 12 launch
# shapes, each with ordinary and with non-temporal loads
_CEIL_SHAPES = ((1, 256, 0), (2, 256, 0), (3, 256, 0), (4, 256, 0), (1, 512, 0), (2, 512, 0), (1, 1024, 0),
                (2, 1024, 0), (1, 256, 16), (1, 512, 8), (1, 512, 16), (1, 1024, 16))
CEIL_CONFIGS = tuple(c + (0,) for c in _CEIL_SHAPES) + tuple(c + (1,) for c in _CEIL_SHAPES)
SHAPES_CEIL_CONFIGS = ((1, 256, 0, 0), (1, 512, 0, 0), (2, 512, 0, 0), (1, 512, 16, 0),
                       (1, 256, 0, 1), (1, 512, 0, 1), (1, 512, 16, 1), (1, 1024, 16, 1))


def _current_stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


# ----------------------------------------------------------------------------- steps
class Step:
    """A timed unit: one library call over buffer set i % n_sets. Subclasses
    fill `sets`, `bytes` (algorithmic bytes per call), `name`, and `spans(i)`:
    the (x, ldx, y, ldy, rows, row_bytes) byte spans of Q/K columns that the
    call reads (and writes) in set i, for the streaming ceiling."""

    copy = True   # the call writes what it reads (False: read only)
    launches = 1

    def _rotate(self, per_set):
        return max(1, -(-ROTATE_MIN_BYTES // per_set))


def _packed_span(w, x, y):
    esz = x.element_size()
    return (x.data_ptr(), w.ld * esz, y.data_ptr() if y is not None else None, w.ld * esz, w.T,
            (w.hq + w.hk) * esz)


class FusedStep(Step):
    """One qknorm_fused (or qknorm_headwise) call over a buffer set: packed
    QKV rows, or separate Q and K arrays for the workloads laid out that way."""

    def __init__(self, w, inp, dev, shards):
        import torch
        import layerwise_qk_norm_qknorm_amd as qk
        self.qk, self.w, self.shards = qk, w, shards
        if w.packed:
            x0 = to_device(inp.qkv, dev)
            srcs = [x0]
        else:
            srcs = [to_device(inp.q, dev), to_device(inp.k, dev)]
            x0 = srcs[0]
        per_set = 2 * sum(t.numel() * t.element_size() for t in srcs)
        self.n_sets = self._rotate(per_set)
        self.sets = []
        for i in range(self.n_sets):
            xs = srcs if i == 0 else [t.clone() for t in srcs]
            self.sets.append((xs, [torch.zeros_like(t) for t in srcs]))
        esz = x0.element_size()
        gsz = inp.gamma_q.dtype.itemsize   # bf16 gamma for FP8 rows
        if w.head_dim:   # headwise: one shared [head_dim] gamma per tensor
            self.gq = to_device(inp.gamma_q[:w.head_dim], dev)
            self.gk = to_device(inp.gamma_k[:w.head_dim], dev)
            self.bytes = 2 * w.T * (w.hq + w.hk) * esz + 2 * w.head_dim * gsz
            self.name = "qknorm_headwise"
        else:
            self.gq = to_device(inp.gamma_q, dev)
            self.gk = to_device(inp.gamma_k, dev)
            self.bytes = 2 * w.T * (w.hq + w.hk) * esz + (w.hq + w.hk) * gsz
            self.name = "qknorm_fused"
        self.stream_bytes = 2 * w.T * (w.hq + w.hk) * esz
        self.footprint = self.n_sets * per_set

    def spans(self, i):
        xs, ys = self.sets[i % self.n_sets]
        if self.w.packed:
            return [_packed_span(self.w, xs[0], ys[0])]
        return [(x.data_ptr(), x.shape[1] * x.element_size(), y.data_ptr(), y.shape[1] * y.element_size(),
                 x.shape[0], x.shape[1] * x.element_size()) for x, y in zip(xs, ys)]

    def __call__(self, i):
        xs, ys = self.sets[i % self.n_sets]
        hq, hk = self.w.hq, self.w.hk
        if self.w.packed:
            x, y = xs[0], ys[0]
            q, k, oq, ok = x[:, :hq], x[:, hq:hq + hk], y[:, :hq], y[:, hq:hq + hk]
        else:
            (q, k), (oq, ok) = xs, ys
        if self.w.head_dim:
            self.qk.qknorm_headwise(q, k, self.gq, self.gk, self.w.eps, self.w.head_dim, 0, oq, ok)
        else:
            self.qk.qknorm_fused(q, k, self.gq, self.gk, self.w.eps, self.shards, oq, ok)


class PartialStep(Step):
    """qknorm_partial_stats on one rank's slice (Phase A: the local sums of
    squares, one plane of 2 x T float32), each call on its own buffer set."""

    copy = False

    def __init__(self, w, inp, dev):
        import torch
        import layerwise_qk_norm_qknorm_amd as qk
        self.qk, self.w = qk, w
        x0 = to_device(inp.qkv, dev)
        per_set = x0.numel() * x0.element_size() + 8 * w.T
        self.n_sets = self._rotate(per_set)
        self.sets = [(x0 if i == 0 else x0.clone(), torch.empty((1, 2, w.T), dtype=torch.float32, device=dev))
                     for i in range(self.n_sets)]
        esz = x0.element_size()
        self.bytes = w.T * (w.hq + w.hk) * esz + 8 * w.T
        self.stream_bytes = w.T * (w.hq + w.hk) * esz
        self.footprint = self.n_sets * per_set
        self.name = "qknorm_partial_stats"

    def spans(self, i):
        return [_packed_span(self.w, self.sets[i % self.n_sets][0], None)]

    def __call__(self, i):
        x, planes = self.sets[i % self.n_sets]
        hq, hk = self.w.hq, self.w.hk
        self.qk.qknorm_partial_stats(x[:, :hq], x[:, hq:hq + hk], 1, planes)


class ApplyStep(Step):
    """qknorm_apply_with_stats on one rank's slice: the local plane plus the
    peers' planes (computed once before timing, as if received), added in
    rank order, full widths as divisors (Phase B and the final scaling), each
    call on its own buffer set."""

    def __init__(self, w, inp, dev):
        import torch
        import layerwise_qk_norm_qknorm_amd as qk
        self.qk, self.w = qk, w
        x0 = to_device(inp.qkv, dev)
        P = inp.peer_q.shape[0]
        planes0 = torch.empty((1 + P, 2, w.T), dtype=torch.float32, device=dev)
        qk.qknorm_partial_stats(x0[:, :w.hq], x0[:, w.hq:w.hq + w.hk], 1, planes0[0:1])
        for p in range(P):
            pq, pk = to_device(inp.peer_q[p], dev), to_device(inp.peer_k[p], dev)
            qk.qknorm_partial_stats(pq, pk, 1, planes0[1 + p:2 + p])
        per_set = 2 * x0.numel() * x0.element_size() + planes0.numel() * 4
        self.n_sets = self._rotate(per_set)
        self.sets = [(x0 if i == 0 else x0.clone(), torch.zeros_like(x0), planes0.clone())
                     for i in range(self.n_sets)]
        self.gq = to_device(inp.gamma_q, dev)
        self.gk = to_device(inp.gamma_k, dev)
        esz = x0.element_size()
        gsz = inp.gamma_q.dtype.itemsize
        h = w.hq + w.hk
        self.bytes = 2 * w.T * h * esz + 8 * (1 + P) * w.T + h * gsz
        self.stream_bytes = 2 * w.T * h * esz
        self.footprint = self.n_sets * per_set
        self.name = "qknorm_apply_with_stats"

    def spans(self, i):
        x, y, _ = self.sets[i % self.n_sets]
        return [_packed_span(self.w, x, y)]

    def __call__(self, i):
        x, y, planes = self.sets[i % self.n_sets]
        hq, hk = self.w.hq, self.w.hk
        self.qk.qknorm_apply_with_stats(x[:, :hq], x[:, hq:hq + hk], self.gq, self.gk, self.w.eps, planes,
                                        self.w.hq_full, self.w.hk_full, y[:, :hq], y[:, hq:hq + hk])


class CeilingStep(Step):
    """The streaming ceiling of a call: a plain copy (or read) of exactly the
    Q/K column bytes that `step` moves, over the same rotating buffer sets,
    with `per` chunks per thread and `block` threads per block, runs of `xk`
    blocks per XCD (0: blocks in order), non-temporal loads if `ntl`."""

    def __init__(self, step, lib, per, block, xk, ntl, sink):
        self.step, self.lib, self.per, self.block, self.xk, self.sink = step, lib, per, block, xk, sink
        self.ntl = ntl
        self.n_sets = step.n_sets
        self.copy = step.copy
        self.bytes = step.stream_bytes
        self.launches = len(step.spans(0))
        self.name = f"stream_{'copy' if step.copy else 'read'}(per={per}, block={block}" + \
            (f", xcd_run={xk}" if xk else "") + (", nt loads)" if ntl else ")")

    def __call__(self, i):
        st = _current_stream()
        for x, ldx, y, ldy, rows, row_bytes in self.step.spans(i):
            self.lib.stream(x, ldx, y if self.copy else None, ldy, rows, row_bytes, self.per, self.block,
                            self.xk, self.ntl, self.sink, st)


class ContiguousCopy(Step):
    """Buffers of `nbytes` copied (or read) whole: the plain device copy of a
    known byte count, for the counter calibration and the ceiling table."""

    def __init__(self, nbytes, dev, copy=True):
        import torch
        n = nbytes // 16 * 16
        self.copy = copy
        per_set = 2 * n if copy else n
        self.n_sets = self._rotate(per_set)
        self.sets = [(torch.ones(n // 2, dtype=torch.bfloat16, device=dev),
                      torch.empty(n // 2, dtype=torch.bfloat16, device=dev) if copy else None)
                     for _ in range(self.n_sets)]
        self.stream_bytes = self.bytes = (2 if copy else 1) * n
        self.n = n
        self.footprint = self.n_sets * per_set
        self.name = "contiguous " + ("copy" if copy else "read")

    def spans(self, i):
        a, b = self.sets[i % self.n_sets]
        return [(a.data_ptr(), self.n, b.data_ptr() if b is not None else None, self.n, 1, self.n)]


# ----------------------------------------------------------------------------- timing
def time_steps(step, steps, warmup, graph=True):
    """Runs `warmup` untimed calls, then times exactly `steps` calls: wall
    clock and HIP events on the launch stream (the current stream, which the
    binding launches on), with a device synchronization on both sides.

    graph=True: the `steps` calls are captured once in a HIP graph, which is
    replayed once untimed (its first launch uploads it) and then once timed,
    so the events see the kernels back to back, not the host's pace (a call
    through the Python binding costs about 8 us of host time, more than some
    of these kernels take). graph=False: eager calls from Python."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(steps):
                    step(warmup + i)
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del g
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            step(warmup + i)
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ev_ms = start.elapsed_time(end)
    return wall, ev_ms / 1000.0


def ceiling_sweep(step, dev, steps=200, warmup=100, configs=CEIL_CONFIGS, verbose=True, graph=True):
    """Times the streaming copy (or read) of the bytes `step` moves for each
    (per, block) in `configs`; returns the rows and the fastest."""
    import torch
    lib = CeilingLib()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    rows = []
    for per, block, xk, ntl in configs:
        cs = CeilingStep(step, lib, per, block, xk, ntl, sink.data_ptr())
        _, ev = time_steps(cs, steps, warmup, graph=graph)
        us = ev / steps * 1e6
        row = {"kernel": cs.name, "per": per, "block": block, "xcd_run": xk, "nt_loads": ntl, "bytes": cs.bytes,
               "us": us,
               "GBps": cs.bytes / (us * 1e-6) / 1e9}
        row["frac_of_peak"] = row["GBps"] / HBM_PEAK_GBPS
        rows.append(row)
        if verbose:
            log(f"[ceiling] {cs.name}: {us:.2f} us, {row['GBps']:.0f} GB/s ({row['frac_of_peak']:.3f} of peak)")
    best = max(rows, key=lambda r: r["GBps"])
    return rows, best


def cpu_baseline(w, inp, min_seconds=10.0, max_seconds=30.0):
    """The float64 oracle on the host: whole passes over the workload's tokens,
    chunked over a thread pool, until at least `min_seconds` have passed."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    # The GPU machine's CPU share for one GPU is 16 threads, whatever the
    # affinity mask shows; both counts are recorded.
    affinity = len(os.sched_getaffinity(0))
    cores = min(affinity, 16)
    chunk = 256
    spans = [(a, min(a + chunk, w.T)) for a in range(0, w.T, chunk)]

    peer_planes = None
    if w.peers:  # received planes: prepared before timing, as on the GPU side
        import numpy as np
        peer_planes = np.stack([oracle.qknorm_partial_stats(inp.peer_q[p], inp.peer_k[p], w.dtype, 1)[0]
                                for p in range(inp.peer_q.shape[0])]).astype(np.float32)

    def work(span):
        a, b = span
        if w.peers:
            import numpy as np
            local = oracle.qknorm_partial_stats(inp.q[a:b], inp.k[a:b], w.dtype, 1).astype(np.float32)
            st = np.concatenate([local, peer_planes[:, :, a:b]])
            oracle.qknorm_apply_with_stats(inp.q[a:b], inp.k[a:b], inp.gamma_q, inp.gamma_k, w.dtype, w.eps, st,
                                           w.hq_full, w.hk_full)
        elif w.head_dim:
            oracle.qknorm_headwise(inp.q[a:b], inp.k[a:b], inp.gamma_q[:w.head_dim], inp.gamma_k[:w.head_dim],
                                   w.dtype, w.eps, w.head_dim, 0)
        else:
            oracle.qknorm_fused(inp.q[a:b], inp.k[a:b], inp.gamma_q, inp.gamma_k, w.dtype, w.eps, w.shards[0])
        return b - a

    tokens = 0
    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as ex:
        while True:
            tokens += sum(ex.map(work, spans))
            passes += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or el >= max_seconds:
                break
    el = time.perf_counter() - t0
    # the same work on one thread, over as many chunks as fit in about 2 s
    t1, tokens1, i = time.perf_counter(), 0, 0
    while time.perf_counter() - t1 < 2.0 and i < 4 * len(spans):
        tokens1 += work(spans[i % len(spans)])
        i += 1
    el1 = time.perf_counter() - t1
    return {
        "value": tokens / el,
        "unit": "tokens/s",
        "cores": cores,
        "affinity_cores": affinity,
        "kind": "oracle",
        "value_1_thread": tokens1 / el1,
        "sample": f"{w.key}: all {w.T} tokens x {passes} passes ({tokens} tokens, {el:.1f} s), "
                  f"float64 NumPy oracle incl. {w.dtype} decode and rounding, {chunk}-token chunks on {cores} "
                  f"threads; value_1_thread: {tokens1} tokens on one thread ({el1:.1f} s)",
    }


# rocprofv3 --pmc counters of the requests the L2 (TCC) sends to the memory
# fabric (EA), summed over the L2 channels; two runs, one per direction (at
# most 4 TCC counters per run).
READ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_DRAM_sum")
WRITE_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_DRAM_sum")


def load_traffic(workload, call, kernel_hash):
    """HBM bytes per launch of `call` from the committed counter summary, if
    it was taken on the current kernel sources (else None)."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_hash:
        log(f"[bench] {path} was taken on kernel sources {d.get('kernel_source_hash')}, now {kernel_hash}: "
            "traffic reported as null")
        return None
    k = d.get("kernels", {}).get(call)
    return k.get("traffic_bytes_per_launch") if k else None


def _call_of(kernel_name):
    """The library call (or ceiling kernel) a dispatched kernel belongs to."""
    n = kernel_name
    if "stream_rows<" in n:
        return "stream_copy" if n.split("stream_rows<")[1].split(">")[0].split(",")[1].strip() == "true" \
            else "stream_read"
    if "qknorm_heads" in n:
        return "qknorm_headwise"
    if "qknorm_stats_slot_waves<" in n:
        return "qknorm_partial_stats"
    if "qknorm_rows<" in n:
        mode = n.split("qknorm_rows<")[1].split(">")[0].split(",")[2].strip()
        return {"0": "qknorm_fused", "1": "qknorm_partial_stats", "2": "qknorm_apply_with_stats"}.get(mode)
    return None


def _counter_medians(dirs):
    """{call: {counter: median over its dispatches}} from rocprofv3 counter CSVs."""
    import csv
    import glob
    vals = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as f:
                for r in csv.DictReader(f):
                    call = _call_of(r.get("Kernel_Name", ""))
                    if call:
                        vals.setdefault(call, {}).setdefault(r["Counter_Name"], []).append(
                            float(r["Counter_Value"]))
    return {c: {k: sorted(v)[len(v) // 2] for k, v in cs.items()} for c, cs in vals.items()}, \
        {c: {k: len(v) for k, v in cs.items()} for c, cs in vals.items()}


def request_bytes(m):
    """Bytes the L2 requested from the fabric, from the request counters.
    Reads: 128 bytes per TCC_EA0_RDREQ that is not a 32-byte one
    (TCC_EA0_RDREQ_32B). On MI355X with ROCm 7 these requests are whole
    128-byte lines, but TCC_BUBBLE (the counter of 128-byte read requests,
    which rocprofv3's FETCH_SIZE expression relies on) reads 0, so FETCH_SIZE
    counts them as 64 bytes, half the bytes moved. Writes: 64 bytes per
    TCC_EA0_WRREQ_64B and 32 per other TCC_EA0_WRREQ (the WRITE_SIZE
    expression). record_traffic checks both against the streaming copy or
    read of a known byte count profiled in the same runs."""
    out = {}
    if "TCC_EA0_RDREQ_sum" in m:
        rd, r32 = m["TCC_EA0_RDREQ_sum"], m.get("TCC_EA0_RDREQ_32B_sum", 0.0)
        out["read_bytes"] = 128.0 * (rd - r32) + 32.0 * r32
    if "TCC_EA0_WRREQ_sum" in m:
        wr, w64 = m["TCC_EA0_WRREQ_sum"], m.get("TCC_EA0_WRREQ_64B_sum", 0.0)
        out["write_bytes"] = 64.0 * w64 + 32.0 * (wr - w64)
    return out


def record_traffic(workload, dirs, commands):
    """Turns rocprofv3 --pmc runs of `bench.py --workload <workload>` (read
    counters in one run, write counters in another) into HBM bytes per launch
    for each call of the workload, checked against the streaming copy or read
    of the same bytes in the same runs, whose byte count is known exactly."""
    from layerwise_qk_norm_qknorm_amd import inputs as I
    med, counts = _counter_medians(dirs)
    w = I.WORKLOADS[workload]
    esz = {"bf16": 2, "f32": 4, "fp8": 1}[w.dtype]
    gsz = 4 if w.dtype == "f32" else 2
    h = w.hq + w.hk
    span = w.T * h * esz
    algo = {
        "qknorm_fused": 2 * span + h * gsz,
        "qknorm_headwise": 2 * span + 2 * w.head_dim * gsz,
        "qknorm_partial_stats": span + 8 * w.T,
        "qknorm_apply_with_stats": 2 * span + 8 * (1 + w.peers) * w.T + h * gsz,
        "stream_copy": 2 * span,
        "stream_read": span,
    }
    kernels = {}
    for call, m in sorted(med.items()):
        b = request_bytes(m)
        rec = {"dispatches": counts[call], "counters_median": m, **b}
        if "read_bytes" in b and "write_bytes" in b:
            rec["traffic_bytes_per_launch"] = b["read_bytes"] + b["write_bytes"]
            rec["algorithmic_bytes_per_launch"] = algo.get(call)
            if algo.get(call):
                rec["traffic_over_algorithmic"] = rec["traffic_bytes_per_launch"] / algo[call]
        kernels[call] = rec
        log(f"[traffic] {call}: {json.dumps(rec)}")
    # The streaming kernels move a known byte count: the formula must give it.
    for call, known_read, known_write in (("stream_copy", span, span), ("stream_read", span, 0)):
        k = kernels.get(call)
        if k and "read_bytes" in k and "write_bytes" in k:
            for got, want in ((k["read_bytes"], known_read), (k["write_bytes"], known_write)):
                if abs(got - want) > 0.005 * max(want, 1):
                    raise SystemExit(f"[traffic] {call}: counters give {got} bytes, {want} known: formula does not hold")
            k["check"] = "read and write bytes within 0.5% of the known bytes"
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(), "kernels": kernels,
           "formula": " ".join(request_bytes.__doc__.split()), "commands": commands}
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def latency_table(dev, reps=200):
    """Per-call times of the small, launch- and latency-bound workloads:
    median of single calls bracketed by HIP events, the mean over
    back-to-back calls from Python through the plain binding and through a
    PreparedCall (arguments checked and marshalled once), the host time per
    call of each, and the mean over 100 calls replayed from a HIP graph (GPU
    time per call; buffers stay cache resident at these sizes)."""
    import torch
    import layerwise_qk_norm_qknorm_amd as qk
    from layerwise_qk_norm_qknorm_amd import inputs as I

    rows = []
    cases = [(I.TINY, s) for s in I.TINY.shards] + [(I.SMALL_DENSE, s) for s in I.SMALL_DENSE.shards]
    cases += [(w, s) for w in I.DECODE for s in w.shards]
    cases += [(w, "headwise") for w in I.DECODE]   # 128-wide heads, one shared gamma per tensor
    for w, shards in cases:
        headwise = shards == "headwise"
        inp = I.make_inputs(w)
        if w.packed:
            x = to_device(inp.qkv, dev)
            y = torch.zeros_like(x)
            args = (x[:, :w.hq], x[:, w.hq:w.hq + w.hk])
            outs = (y[:, :w.hq], y[:, w.hq:w.hq + w.hk])
        else:
            args = (to_device(inp.q, dev), to_device(inp.k, dev))
            outs = (torch.zeros_like(args[0]), torch.zeros_like(args[1]))
        if headwise:
            gq, gk = to_device(inp.gamma_q[:128], dev), to_device(inp.gamma_k[:128], dev)

            def call():
                qk.qknorm_headwise(*args, gq, gk, w.eps, 128, 0, *outs)
        else:
            gq, gk = to_device(inp.gamma_q, dev), to_device(inp.gamma_k, dev)

            def call():
                qk.qknorm_fused(*args, gq, gk, w.eps, shards, *outs)

        for _ in range(20):
            call()
        torch.cuda.synchronize()
        # host time per call: the binding's checks and marshalling, the
        # library's validation and planning, and the launch
        t0 = time.perf_counter()
        for _ in range(reps):
            call()
        host_us = (time.perf_counter() - t0) * 1e6 / reps
        torch.cuda.synchronize()
        # the same call marshalled once (PreparedCall): the library and the launch only
        if headwise:
            prepared = qk.prepare_headwise(*args, gq, gk, w.eps, 128, 0, *outs)
        else:
            prepared = qk.prepare_fused(*args, gq, gk, w.eps, shards, *outs)
        for _ in range(20):
            prepared()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            prepared()
        host_prepared_us = (time.perf_counter() - t0) * 1e6 / reps
        torch.cuda.synchronize()
        single = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            b.synchronize()
            single.append(a.elapsed_time(b) * 1e3)
        single.sort()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        b.synchronize()
        b2b_us = a.elapsed_time(b) * 1e3 / reps
        a.record()
        for _ in range(reps):
            prepared()
        b.record()
        b.synchronize()
        b2b_prepared_us = a.elapsed_time(b) * 1e3 / reps
        # The same calls captured in a HIP graph: GPU time per call without
        # the host-side cost of the Python binding.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(100):
                call()
        graph.replay()
        torch.cuda.synchronize()
        graph_us = []
        for _ in range(5):
            a.record()
            graph.replay()
            b.record()
            b.synchronize()
            graph_us.append(a.elapsed_time(b) * 1e3 / 100)
        esz = 2 if w.dtype == "bf16" else 4
        ld = w.ld if w.packed else w.hq
        if headwise:
            nbytes = 2 * w.T * (w.hq + w.hk) * esz + 2 * 128 * esz
            plan = qk.describe_headwise_plan(w.hq, w.hk, w.T, 128, w.dtype, 0, ld=ld)
        else:
            nbytes = 2 * w.T * (w.hq + w.hk) * esz + (w.hq + w.hk) * esz
            plan = qk.describe_plan(0, w.hq, w.hk, w.T, w.dtype, shards, ld=ld)
        row = {"workload": w.key, "call": "qknorm_headwise" if headwise else "qknorm_fused", "tokens": w.T,
               "shards": 1 if headwise else shards, "plan": plan,
               "single_call_us_p10": single[reps // 10], "single_call_us_median": single[reps // 2],
               "single_call_us_p90": single[(9 * reps) // 10],
               "back_to_back_us": b2b_us, "host_us_per_call": host_us, "graph_replay_us": min(graph_us),
               "bytes": nbytes}
        row["back_to_back_prepared_us"] = b2b_prepared_us
        row["host_us_per_call_prepared"] = host_prepared_us
        row["GBps_graph_replay"] = nbytes / (row["graph_replay_us"] * 1e-6) / 1e9
        rows.append(row)
        print(json.dumps(row), flush=True)
    return rows


def shapes_table(dev, T=8192, steps=100):
    """The fused call, then the headwise call (128-wide heads, one shared
    gamma), over the prefill row widths of `inputs.PREFILL_WIDTHS` in bf16,
    FP8 and fp32 rows, with the planner's launch for each; one JSON line per
    shape.
    `us` is GPU time per call: `steps` calls over the rotating buffer sets
    replayed from a HIP graph, best of three replays (at the narrow widths a
    call from Python costs more host time than the kernel takes, so
    back-to-back launches, `us_back_to_back`, do not keep the GPU busy).
    `ceiling_us` is the streaming ceiling of the same bytes (the copy kernel
    of libstreamceil.so over the same buffers, best of the launch shapes in
    SHAPES_CEIL_CONFIGS)."""
    import torch
    import layerwise_qk_norm_qknorm_amd as qk
    from layerwise_qk_norm_qknorm_amd import inputs as I

    from dataclasses import replace

    rows = []
    for head_dim, dtype in [(0, d) for d in ("bf16", "fp8", "f32")] + [(128, d) for d in ("bf16", "fp8", "f32")]:
        for hq, hk, hv in I.PREFILL_WIDTHS:
            w = replace(I.prefill_width(dtype, hq, hk, hv, T), head_dim=head_dim)
            step = FusedStep(w, I.make_inputs(w), dev, 1)
            time_steps(step, 10, 300, graph=False)
            b2b = min(time_steps(step, steps, 20, graph=False)[1] for _ in range(3)) / steps
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step(0)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(steps):
                    step(i)
            graph.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            best = None
            for _ in range(3):
                a.record()
                graph.replay()
                b.record()
                b.synchronize()
                t = a.elapsed_time(b) * 1e-3 / steps
                best = t if best is None else min(best, t)
            plan = (qk.describe_headwise_plan(hq, hk, T, head_dim, dtype, 0, ld=w.ld) if head_dim
                    else qk.describe_plan(0, hq, hk, T, dtype, 1, ld=w.ld))
            del graph
            _, ceil = ceiling_sweep(step, dev, steps, 50, SHAPES_CEIL_CONFIGS, verbose=False)
            row = {"workload": w.key, "call": step.name, "head_dim": head_dim, "dtype": dtype, "tokens": T,
                   "hq": hq, "hk": hk, "hv": hv, "plan": plan, "us": best * 1e6,
                   "us_back_to_back": b2b * 1e6, "bytes": step.bytes, "GBps": step.bytes / best / 1e9,
                   "frac_of_peak": step.bytes / best / 1e9 / HBM_PEAK_GBPS,
                   "ceiling_us": ceil["us"], "ceiling_launch": f"{ceil['per']}x{ceil['block']}",
                   "frac_of_ceiling": ceil["us"] / (best * 1e6)}
            rows.append(row)
            print(json.dumps(row), flush=True)
            del step
            torch.cuda.empty_cache()
    return rows


TIMELINE_CALLS = (("gqa_prefill", "fused"), ("gqa_prefill_fp8", "fused"), ("rank_slice", "partial"),
                  ("rank_slice", "apply"), ("rank_slice_fp8", "partial"), ("rank_slice_fp8", "apply"))


def timeline_summary(rec):
    """Launch-shape figures from one launch's block records [grid, 3] (start
    and end on the 100 MHz real-time counter, XCC id << 32 | hardware id):
    all in microseconds from the first block's start."""
    import numpy as np
    if not (rec[:, 1] > 0).all():
        raise RuntimeError(f"{int((rec[:, 1] == 0).sum())} of {len(rec)} blocks left no record")
    start = rec[:, 0].astype(np.int64)
    end = rec[:, 1].astype(np.int64)
    t0 = start.min()
    s, e = (start - t0) / 100.0, (end - t0) / 100.0
    first_end = e.min()
    first_gen = s < first_end          # blocks already running when the first one ends
    xcc = (rec[:, 2] >> 32).astype(np.int64)
    xcd_end = np.array([e[xcc == x].max() for x in np.unique(xcc)])
    return {"blocks": int(len(s)), "span_us": float(e.max()), "first_generation_blocks": int(first_gen.sum()),
            "first_generation_start_spread_us": float(s[first_gen].max()), "first_block_end_us": float(first_end),
            "median_block_us": float(np.median(e - s)), "last_block_start_us": float(s.max()),
            "last_start_to_end_us": float(e.max() - s.max()), "xcds": int(len(xcd_end)),
            "last_xcd_after_median_xcd_us": float(xcd_end.max() - np.median(xcd_end))}


def timeline(dev, reps=5):
    """Per-block start and end clocks of single launches inside a stream of
    launches, from the timing-only builds (libqknorm_clocks.so in place of
    libqknorm.so, libstreamceil_clocks.so for the ceiling at 1 chunk x 512
    threads): one JSON line per call and kernel, the median of `reps`
    launches of each figure of timeline_summary."""
    import ctypes
    import numpy as np
    import torch
    from layerwise_qk_norm_qknorm_amd import binding, build_lib
    from layerwise_qk_norm_qknorm_amd import inputs as I
    if binding._lib is not None:
        raise RuntimeError("--timeline must load libqknorm_clocks.so before any other library call")
    if os.environ.get("QKNORM_MAX_GRID"):
        raise RuntimeError("--timeline takes one block per token group (QKNORM_MAX_GRID must be unset)")
    for path in (build_lib.CLOCKS_LIB, build_lib.CEIL_CLOCKS_LIB):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
    binding._LIB_PATH = build_lib.CLOCKS_LIB
    qk = binding.load_library()
    qk.qknorm_set_block_clocks.argtypes = [ctypes.c_void_p]
    ceil = CeilingLib(build_lib.CEIL_CLOCKS_LIB)
    ceil.lib.qkceil_set_block_clocks.argtypes = [ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    rows = []
    for wl, call in TIMELINE_CALLS:
        w = I.WORKLOADS[wl]
        inp = I.make_inputs(w)
        step = {"fused": FusedStep, "partial": PartialStep, "apply": ApplyStep}[call]
        step = step(w, inp, dev, 1) if call == "fused" else step(w, inp, dev)
        plan = _plan_text(binding, w, step.name, 1)
        tpb = int(re.search(r"tokens/block=(\d+)", plan).group(1))
        gl = re.search(r"groups/block=(\d+)", plan)   # blocks that loop over several token groups
        grid_k = -(-(-(-w.T // tpb)) // (int(gl.group(1)) if gl else 1))
        cs = CeilingStep(step, ceil, 1, 512, 0, 1, sink.data_ptr())
        if cs.launches != 1:
            raise RuntimeError(f"{wl}: the ceiling takes {cs.launches} launches; one is timed")
        chunks = step.stream_bytes // (2 if step.copy else 1) // 16
        for kind, st, grid, setter in (("kernel", step, grid_k, qk.qknorm_set_block_clocks),
                                       ("ceiling", cs, -(-chunks // 512), ceil.lib.qkceil_set_block_clocks)):
            _, ev = time_steps(st, 200, 300, graph=False)   # warm-up, and the eager rate of this build
            runs = []
            for rep in range(reps):
                buf = torch.zeros(grid * 3, dtype=torch.int64, device=dev)
                for i in range(30):
                    st(i)
                setter(buf.data_ptr())
                st(30)
                setter(None)
                for i in range(31, 40):
                    st(i)
                torch.cuda.synchronize()
                runs.append(timeline_summary(buf.cpu().numpy().reshape(grid, 3)))
            med = {k: float(np.median([r[k] for r in runs])) for k in runs[0]}
            row = {"workload": wl, "call": step.name, "kernel": kind, "grid": grid,
                   "plan": plan if kind == "kernel" else cs.name, "eager_us_per_launch": ev / 200 * 1e6, **med}
            rows.append(row)
            print(json.dumps(row), flush=True)
        del step, cs
        torch.cuda.empty_cache()
    return rows


def _plan_text(qk, w, call, shards):
    if call == "qknorm_headwise":
        return qk.describe_headwise_plan(w.hq, w.hk, w.T, w.head_dim, w.dtype, 0, ld=w.ld)
    op = {"qknorm_fused": 0, "qknorm_partial_stats": 1, "qknorm_apply_with_stats": 2}[call]
    return qk.describe_plan(op, w.hq, w.hk, w.T, w.dtype, shards if op == 0 else 1,
                            ld=w.ld if w.packed else w.hq)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="gqa_prefill")
    ap.add_argument("--shards", type=int, default=None, help="S for the fused workloads (default: first listed)")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's token count T (a size sweep; the default is the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-ceiling sweep")
    ap.add_argument("--ceiling-configs", default="",
                    help="ceiling launches to sweep, as PERxBLOCK[xXCDRUN[xNTLOADS]],... (default: all of CEIL_CONFIGS)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager calls from Python instead of one HIP-graph replay of the timed calls")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="time the streaming copy and read kernels on contiguous buffers of this many bytes")
    ap.add_argument("--record-traffic", nargs="+", metavar="PMC_DIR",
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc output directories "
                         "(no GPU needed)")
    ap.add_argument("--timeline", action="store_true",
                    help="per-block start/end clocks of single launches of the headline calls and their ceilings, "
                         "from the timing-only builds (one JSON line per call and kernel)")
    ap.add_argument("--latency", action="store_true",
                    help="per-call times of the tiny, small-dense and decode workloads (one JSON line each)")
    ap.add_argument("--shapes", action="store_true",
                    help="the fused and headwise calls over a range of prefill row widths (one JSON line each)")
    ap.add_argument("--traffic-commands", default="", help="the rocprofv3 commands, recorded with the result")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.workload, args.record_traffic, [c for c in args.traffic_commands.split(";;") if c])
        return

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by exchanging 2 float32 sums per token per rank, not implemented here)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import layerwise_qk_norm_qknorm_amd as qk
    from layerwise_qk_norm_qknorm_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    if args.timeline:   # loads the timing-only library in place of libqknorm.so
        log(f"[bench] device {torch.cuda.get_device_name(0)}; block clocks from the timing-only builds")
        timeline(dev)
        return
    qk.load_library()
    log(f"[bench] device {torch.cuda.get_device_name(0)}; library {qk.library_path()}")

    if args.latency:
        latency_table(dev)
        return

    if args.shapes:
        shapes_table(dev)
        return

    if args.copy_bytes:
        for copy in (True, False):
            step = ContiguousCopy(args.copy_bytes, dev, copy)
            rows, best = ceiling_sweep(step, dev, args.steps, args.warmup, graph=not args.eager)
            print(json.dumps({"metric": f"streaming {'copy' if copy else 'read'} of a contiguous buffer",
                              "buffer_bytes": step.n, "bytes_per_launch": step.bytes, "steps": args.steps,
                              "rotating_sets": step.n_sets, "best": best, "sweep": rows}), flush=True)
        return

    w = I.WORKLOADS[args.workload]
    t_own = w.T
    title = w.title
    if args.tokens and args.tokens != w.T:
        w = w.with_T(args.tokens)
        title = f"{w.title}; T overridden to {w.T}"
    shards = args.shards or w.shards[0]
    log(f"[bench] workload {w.key}: {title}")
    t0 = time.perf_counter()
    inp = I.make_inputs(w)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")
    # One rank's slice runs the split path: Phase A, then Phase B with the
    # received planes. Each call is timed alone over its own rotating sets.
    steps = [PartialStep(w, inp, dev), ApplyStep(w, inp, dev)] if w.peers else [FusedStep(w, inp, dev, shards)]
    torch.cuda.synchronize()
    plans = [_plan_text(qk, w, s.name, shards) for s in steps]
    for s, plan in zip(steps, plans):
        log(f"[bench] {s.name}: {plan}; {s.n_sets} rotating buffer sets, {s.footprint / 2**20:.0f} MiB")

    # The streaming ceilings of the same bytes, on the same buffers (before
    # the timed calls: this also brings clocks and buffers to steady state).
    ceilings = [None] * len(steps)
    if not args.no_ceiling:
        for n, s in enumerate(steps):
            ceilings[n] = ceiling_sweep(s, dev, steps=max(args.steps, 100), warmup=100, graph=not args.eager,
                                        configs=CEIL_CONFIGS if not args.ceiling_configs else
                                        [tuple((int(v) for v in (c + "x0x0").split("x")[:4]))
                                         for c in args.ceiling_configs.split(",")])

    khash = kernel_source_hash()
    kernels, wall_total = [], 0.0
    for s, plan, ceil in zip(steps, plans, ceilings):
        wall, ev = time_steps(s, args.steps, args.warmup, graph=not args.eager)
        wall_total += wall
        mean = ev / args.steps
        achieved = s.bytes / mean / 1e9
        log(f"[bench] {s.name}: {args.steps} calls, wall {wall * 1e3:.2f} ms, events {ev * 1e3:.2f} ms, "
            f"{mean * 1e6:.2f} us per call, {achieved:.0f} GB/s")
        k = {
            "kernel": s.name,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": load_traffic(w.key, s.name, khash) if w.T == t_own else None,
            "algorithmic_bytes_per_launch": s.bytes,
            "mean_launch_us": mean * 1e6,
            "plan": plan,
        }
        if ceil is not None:
            best = ceil[1]
            # the ceiling moves the Q/K bytes only; compare rates of those bytes
            rate = s.stream_bytes / mean / 1e9
            k["ceiling"] = {"kernel": best["kernel"], "achieved": best["GBps"], "us": best["us"],
                            "bytes": best["bytes"], "frac": best["frac_of_peak"]}
            k["frac_of_ceiling"] = rate / best["GBps"]
        k["kernel_source_hash"] = khash
        kernels.append(k)
    dominant = max(kernels, key=lambda k: k["mean_launch_us"])
    out = {
        "metric": "QK-Norm tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU",
        "value": w.T * args.steps / wall_total,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_total / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; inputs resident in HBM, rotating buffer sets > 1 GiB)",
        "config": {
            "workload": title,
            "key": w.key,
            "tokens": w.T,
            "hq": w.hq, "hk": w.hk, "hv": w.hv,
            "layout": f"packed [{w.T}, {w.ld}]" if w.packed else "separate Q/K arrays",
            "shards": shards,
            "calls_per_step": " + ".join(s.name for s in steps),
            "out_of_place": True,
            "rotating_sets": [s.n_sets for s in steps],
            "timing": "eager calls" if args.eager else "one HIP-graph replay of the timed calls",
        },
        "roofline": dominant,
        "cpu_baseline": None,
    }
    if len(kernels) > 1:
        out["roofline_kernels"] = kernels
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(w, inp)
        log(f"[bench] oracle: {out['cpu_baseline']['value']:.0f} tokens/s on {out['cpu_baseline']['cores']} threads")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
