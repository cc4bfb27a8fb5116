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


# ----------------------------------------------------------------------------- steps
class FusedStep:
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
        self.n_sets = max(1, -(-ROTATE_MIN_BYTES // per_set))
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
        self.footprint = self.n_sets * per_set
        self.launches = 1

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


class SplitStep:
    """One rank's share of the split path: qknorm_partial_stats on the local
    slice, then qknorm_apply_with_stats with the local plane and the peer
    planes (computed once before timing, as if received)."""

    def __init__(self, w, inp, dev):
        import torch
        import layerwise_qk_norm_qknorm_amd as qk
        self.qk, self.w = qk, w
        x0 = to_device(inp.qkv, dev)
        per_set = 2 * x0.numel() * x0.element_size()
        self.n_sets = max(1, -(-ROTATE_MIN_BYTES // per_set))
        P = inp.peer_q.shape[0]
        self.sets = []
        for i in range(self.n_sets):
            x = x0 if i == 0 else x0.clone()
            y = torch.zeros_like(x0)
            planes = torch.empty((1 + P, 2, w.T), dtype=torch.float32, device=dev)
            self.sets.append((x, y, planes))
        for p in range(P):
            pq, pk = to_device(inp.peer_q[p], dev), to_device(inp.peer_k[p], dev)
            part = qk.qknorm_partial_stats(pq, pk, 1)
            for s in self.sets:
                s[2][1 + p].copy_(part[0])
        self.gq = to_device(inp.gamma_q, dev)
        self.gk = to_device(inp.gamma_k, dev)
        esz = x0.element_size()
        gsz = inp.gamma_q.dtype.itemsize
        h = w.hq + w.hk
        self.bytes_partial = w.T * h * esz + 8 * w.T
        self.bytes_apply = 2 * w.T * h * esz + 8 * (1 + P) * w.T + h * gsz
        self.bytes = self.bytes_partial + self.bytes_apply
        self.footprint = self.n_sets * per_set
        self.launches = 2
        self.name = "qknorm_partial_stats+qknorm_apply_with_stats"

    def __call__(self, i):
        x, y, planes = self.sets[i % self.n_sets]
        hq, hk = self.w.hq, self.w.hk
        self.qk.qknorm_partial_stats(x[:, :hq], x[:, hq:hq + hk], 1, planes[0:1])
        self.qk.qknorm_apply_with_stats(x[:, :hq], x[:, hq:hq + hk], self.gq, self.gk, self.w.eps, planes,
                                        self.w.hq_full, self.w.hk_full, y[:, :hq], y[:, hq:hq + hk])


class CopyStep:
    """A plain device copy of a known byte count (calibration for the
    hardware counters and the practical bandwidth ceiling)."""

    def __init__(self, nbytes, dev):
        import torch
        n = nbytes // 2
        self.sets = [(torch.ones(n, dtype=torch.bfloat16, device=dev), torch.empty(n, dtype=torch.bfloat16,
                                                                                   device=dev))
                     for _ in range(max(1, -(-ROTATE_MIN_BYTES // (2 * nbytes))))]
        self.n_sets = len(self.sets)
        self.bytes = 2 * n * 2
        self.footprint = self.n_sets * 2 * nbytes
        self.launches = 1
        self.name = "copy"

    def __call__(self, i):
        a, b = self.sets[i % self.n_sets]
        b.copy_(a)


# ----------------------------------------------------------------------------- timing
def time_steps(step, steps, warmup):
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
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


def cpu_baseline(w, inp, min_seconds=10.0, max_seconds=30.0):
    """The float64 oracle on the host: whole passes over the workload's tokens,
    chunked over a thread pool, until at least `min_seconds` have passed."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    cores = min(len(os.sched_getaffinity(0)), 16)
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
        "kind": "oracle",
        "value_1_thread": tokens1 / el1,
        "sample": f"{w.key}: all {w.T} tokens x {passes} passes ({tokens} tokens, {el:.1f} s), "
                  f"float64 NumPy oracle incl. {w.dtype} decode and rounding, {chunk}-token chunks on {cores} "
                  f"threads; value_1_thread: {tokens1} tokens on one thread ({el1:.1f} s)",
    }


def load_traffic(workload, kernel_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
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
    return d.get("traffic_bytes_per_launch")


def _counter_rows(directory, counter):
    """(kernel name, value) for every dispatch in the counter CSVs under `directory`."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r.get("Kernel_Name", ""), float(r["Counter_Value"])))
    return rows


def _median(v):
    v = sorted(v)
    return v[len(v) // 2] if v else None


def record_traffic(workload, d_fetch, d_write, d_copy_fetch, d_copy_write, copy_bytes, commands):
    """Turns four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, for the
    kernel and for a plain copy of `copy_bytes`) into HBM bytes per launch,
    stored with the hash of the kernel sources they were taken on."""
    from layerwise_qk_norm_qknorm_amd import inputs as I
    med = {}
    for key, d, ctr, pat in (("fetch", d_fetch, "FETCH_SIZE", "qknorm_rows"),
                             ("write", d_write, "WRITE_SIZE", "qknorm_rows"),
                             ("copy_fetch", d_copy_fetch, "FETCH_SIZE", "copy"),
                             ("copy_write", d_copy_write, "WRITE_SIZE", "copy")):
        vals = [v for n, v in _counter_rows(d, ctr) if pat in n]
        if key.startswith("copy"):  # the timed copies, not set-up traffic
            top = max(vals)
            vals = [v for v in vals if v > 0.5 * top]
        med[key] = _median(vals)
        log(f"[traffic] {key}: {len(vals)} dispatches, median {med[key]} KiB")
    f_scale = copy_bytes / (med["copy_fetch"] * 1024.0)
    w_scale = copy_bytes / (med["copy_write"] * 1024.0)
    w = I.WORKLOADS[workload]
    esz = {"bf16": 2, "f32": 4, "fp8": 1}[w.dtype]
    gsz = 4 if w.dtype == "f32" else 2
    algo = 2 * w.T * (w.hq + w.hk) * esz + ((2 * w.head_dim) if w.head_dim else (w.hq + w.hk)) * gsz
    traffic = med["fetch"] * 1024.0 * f_scale + med["write"] * 1024.0 * w_scale
    out = {
        "workload": workload,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_kib_per_dispatch": med["fetch"],
        "write_kib_per_dispatch": med["write"],
        "copy_known_bytes": copy_bytes,
        "copy_fetch_kib": med["copy_fetch"],
        "copy_write_kib": med["copy_write"],
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "traffic_bytes_per_launch": traffic,
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": traffic / algo,
        "commands": commands,
    }
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def latency_table(dev, reps=200):
    """Per-call times of the small, launch- and latency-bound workloads:
    median of single calls bracketed by HIP events, the mean over
    back-to-back calls from Python, and the mean over 100 calls replayed from
    a HIP graph (GPU time per call; buffers stay cache resident at these sizes)."""
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
               "back_to_back_us": b2b_us, "graph_replay_us": min(graph_us), "bytes": nbytes}
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
    back-to-back launches, `us_back_to_back`, do not keep the GPU busy)."""
    import torch
    import layerwise_qk_norm_qknorm_amd as qk
    from layerwise_qk_norm_qknorm_amd import inputs as I

    from dataclasses import replace

    rows = []
    for head_dim, dtype in [(0, d) for d in ("bf16", "fp8", "f32")] + [(128, d) for d in ("bf16", "fp8", "f32")]:
        for hq, hk, hv in I.PREFILL_WIDTHS:
            w = replace(I.prefill_width(dtype, hq, hk, hv, T), head_dim=head_dim)
            step = FusedStep(w, I.make_inputs(w), dev, 1)
            time_steps(step, 10, 300)
            b2b = min(time_steps(step, steps, 20)[1] for _ in range(3)) / steps
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
            row = {"workload": w.key, "call": step.name, "head_dim": head_dim, "dtype": dtype, "tokens": T,
                   "hq": hq, "hk": hk, "hv": hv, "plan": plan, "us": best * 1e6,
                   "us_back_to_back": b2b * 1e6, "bytes": step.bytes, "GBps": step.bytes / best / 1e9,
                   "frac_of_peak": step.bytes / best / 1e9 / HBM_PEAK_GBPS}
            rows.append(row)
            print(json.dumps(row), flush=True)
            del graph, step
            torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # Warm-up long enough (tens of ms at the prefill shapes) for clocks and
    # the rotating buffers' first touches to settle before timing.
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="gqa_prefill")
    ap.add_argument("--shards", type=int, default=None, help="S for the fused workloads (default: first listed)")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's token count T (a size sweep; the default is the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="time a plain copy of this many bytes instead (calibration)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc output (no GPU needed)")
    ap.add_argument("--traffic-copy-bytes", type=int, default=100663296)
    ap.add_argument("--latency", action="store_true",
                    help="per-call times of the tiny, small-dense and decode workloads (one JSON line each)")
    ap.add_argument("--shapes", action="store_true",
                    help="the fused and headwise calls over a range of prefill row widths (one JSON line each)")
    ap.add_argument("--traffic-commands", default="", help="the rocprofv3 commands, recorded with the result")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic, args.traffic_copy_bytes,
                       [c for c in args.traffic_commands.split(";;") if c])
        return

    if args.gpus != 1:
        print(f"bench.py: the kernels run on one GPU; --gpus {args.gpus} is not supported "
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
    qk.load_library()
    log(f"[bench] device {torch.cuda.get_device_name(0)}; library {qk.library_path()}")

    if args.latency:
        latency_table(dev)
        return

    if args.shapes:
        shapes_table(dev)
        return

    if args.copy_bytes:
        step = CopyStep(args.copy_bytes, dev)
        wall, ev = time_steps(step, args.steps, args.warmup)
        gbps = step.bytes / (ev / args.steps) / 1e9
        print(json.dumps({"metric": "plain device copy", "bytes_per_launch": step.bytes,
                          "ms_per_launch": ev / args.steps * 1e3, "GBps": gbps,
                          "frac_of_peak": gbps / HBM_PEAK_GBPS, "steps": args.steps}), flush=True)
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
    if w.peers:
        step = SplitStep(w, inp, dev)
        plan = "; ".join(qk.describe_plan(op, w.hq, w.hk, w.T, w.dtype, 1, ld=w.ld) for op in (1, 2))
    else:
        step = FusedStep(w, inp, dev, shards)
        if w.head_dim:
            plan = qk.describe_headwise_plan(w.hq, w.hk, w.T, w.head_dim, w.dtype, 0, ld=w.ld)
        else:
            plan = qk.describe_plan(0, w.hq, w.hk, w.T, w.dtype, shards, ld=w.ld if w.packed else w.hq)
    torch.cuda.synchronize()
    log(f"[bench] plan: {plan}; {step.n_sets} rotating buffer sets, {step.footprint / 2**20:.0f} MiB")

    wall, ev = time_steps(step, args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    mean_launch_s = ev / args.steps
    achieved = step.bytes / mean_launch_s / 1e9
    log(f"[bench] {args.steps} steps: wall {wall * 1e3:.2f} ms, events {ev * 1e3:.2f} ms, "
        f"{mean_launch_s * 1e6:.2f} us per step, {achieved:.0f} GB/s")

    khash = kernel_source_hash()
    traffic = load_traffic(w.key, khash) if w.T == t_own else None  # counters were taken at the workload's T
    out = {
        "metric": "QK-Norm tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU",
        "value": w.T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
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
            "calls_per_step": step.name,
            "out_of_place": True,
            "rotating_sets": step.n_sets,
            "plan": plan,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_step": step.bytes,
            "mean_step_us": mean_launch_s * 1e6,
            "kernel_source_hash": khash,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        out["cpu_baseline"] = cpu_baseline(w, inp)
        log(f"[bench] oracle: {out['cpu_baseline']['value']:.0f} tokens/s on {out['cpu_baseline']['cores']} threads")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
