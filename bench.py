#!/usr/bin/env python3
"""Throughput of the INT4 weight-quantized linear layer on one MI355X.

Headline (one JSON line on stdout): W4A8 decode GEMV, Gemma3-1B-like MLP
up-projection, x [1, 1152] fp32 ~ N(0,1), W [1152, 6912] ~ N(0, 0.02)
quantized to symmetric per-channel int4.  One step = one ``w4a8_linear``
call = the whole forward of the layer (per-row int8 activation quantization,
int4 unpack, int8 x int8 -> int32 product, dequantization), launched from a
captured HIP graph.  ``value`` = algorithmic bytes per step (packed weights +
scales + x + y) x steps / wall time.  The packed weights rotate over enough
copies (> 512 MB) that every step reads them from HBM, not from the 256 MB
Infinity Cache.  Weights are quantized once, before timing (post-training
quantization is a one-shot offline step).

Also reported in the same line:
  roofline      the dominant kernel's achieved GB/s (algorithmic bytes per
                launch / average launch duration, from HIP events recorded on
                the kernel's stream around the timed graph replay, which holds
                only that kernel) against the 8 TB/s HBM peak; the duration
                from events attached to single dispatches is reported beside it;
  parts         the other workloads (Gemma M=8, 7B-class M=1/16/64, the
                4096^3 prefill in int8 TOPS, the same layers with int8
                weights (W8A8), 7B-class decode with AWQ-style channel
                scaling, the 70B-class W4A16 layer, and the offline weight
                transforms: dequantization, LoRA merge, AWQ fold) and the
                weight quantizers, each with per-kernel durations;
  cpu_baseline  the CPU oracle on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-parts]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # dense int8 MFMA
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA
ROTATE_BYTES = 640 << 20     # > 2 x the 256 MB Infinity Cache
METRIC = "W4A8 linear: GB/s (M=1 GEMV) and int8 TOPS (M=4096), % of roofline"
PLAIN_WRITES = {"write67m": 67108864}  # the 4096 x 4096 prefill's fp32 output


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------- HIP events
class Hip:
    """Raw hipEvent_t handles from the HIP runtime already loaded by torch."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        maps = open("/proc/self/maps").read()
        libs = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
        assert len(libs) == 1, f"more than one HIP runtime mapped: {libs}"

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.h.hipEventCreate(ctypes.byref(ev))
        assert rc == 0, rc
        return ev.value

    def record(self, ev, stream):
        rc = self.h.hipEventRecord(ev, stream)
        assert rc == 0, rc

    def elapsed_ms(self, a, b):
        assert self.h.hipEventSynchronize(b) == 0
        f = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(f), a, b)
        assert rc == 0, rc
        return float(f.value)

    def destroy(self, ev):
        self.h.hipEventDestroy(ev)


# ------------------------------------------------------------- workloads
def w4a8_bytes(M, K, N):
    """Algorithmic bytes of one W4A8 forward: packed int4 weights, fp32 channel
    scales, fp32 activations in, fp32 outputs out."""
    return N * ((K + 1) // 2) + 4 * N + 4 * M * K + 4 * M * N


def w8a8_bytes(M, K, N):
    """Algorithmic bytes of one W8A8 forward: int8 weights, fp32 channel
    scales, fp32 activations in, fp32 outputs out."""
    return N * K + 4 * N + 4 * M * K + 4 * M * N


def w4a16_bytes(M, K, N, g):
    """Packed int4 weights, fp32 scale + zero point per group, bf16 x, fp32 y."""
    return N * ((K + 1) // 2) + 8 * N * (K // g) + 2 * M * K + 4 * M * N


class W4A8Case:
    """One W4A8 layer (or, with w8=True, the same layer as W8A8)."""

    def __init__(self, w4, torch, name, shape_name, M, rotate=True, copies=None, w8=False,
                 pp=False):
        import workloads
        d = workloads.generate(shape_name, M=M)
        self.name, self.M, self.K, self.N = name, M if M else d["M"], d["K"], d["N"]
        self.torch, self.w4, self.w8 = torch, w4, w8
        dev = torch.device("cuda")
        self.x = torch.from_numpy(d["x"]).to(dev)
        W = torch.from_numpy(d["W"]).to(dev)
        t0 = time.perf_counter()
        if w8:
            p, s = w4.w8_quantize_weight(W)
        else:
            p, s, _ = w4.w4_quantize_weight(W, "sym")
        self.pp = pp
        if pp:  # one-time conversion to the shuffled tile layout
            p = w4.w4_prepack_weights(p)
        torch.cuda.synchronize()
        self.quant_s = time.perf_counter() - t0
        del W
        wbytes = p.numel() + 4 * s.numel()
        self.copies = max(1, math.ceil(ROTATE_BYTES / wbytes)) if rotate else 2
        if copies:
            self.copies = copies
        self.P = [p] + [p.clone() for _ in range(self.copies - 1)]
        self.S = [s] + [s.clone() for _ in range(self.copies - 1)]
        self.y = torch.empty((self.M, self.N), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(1, w4.w4a8_workspace_bytes(self.M, self.K, self.N)),
                              dtype=torch.uint8, device=dev)
        self.bytes = (w8a8_bytes if w8 else w4a8_bytes)(self.M, self.K, self.N)
        self.ops = 2 * self.M * self.N * self.K
        self.host_x, self.host_W = d["x"], d["W"]

    def step(self, i):
        c = i % self.copies
        if self.pp:
            self.w4.w4a8_linear_prepacked(self.x, self.P[c], self.S[c], Y=self.y,
                                          workspace=self.ws)
            return
        f = self.w4.w8a8_linear if self.w8 else self.w4.w4a8_linear
        f(self.x, self.P[c], self.S[c], Y=self.y, workspace=self.ws)


class AwqCase(W4A8Case):
    """A W4A8 layer with AWQ-style channel scaling: scales from the layer's
    own input rows (alpha 1/4), weights quantized from W diag(s), the
    division by s fused into the activation quantization."""

    def __init__(self, w4, torch, name, shape_name, M):
        import workloads
        super().__init__(w4, torch, name, shape_name, M)
        dev = torch.device("cuda")
        self.s = w4.awq_channel_scales(self.x, (1, 4))
        W = torch.from_numpy(workloads.generate(shape_name, M=M)["W"]).to(dev)
        p, sw, _ = w4.w4_quantize_weight(w4.awq_fold_weight(W, self.s), "sym")
        del W
        self.P = [p] + [p.clone() for _ in range(self.copies - 1)]
        self.S = [sw] + [sw.clone() for _ in range(self.copies - 1)]
        self.bytes += 4 * self.K  # the channel scales

    def step(self, i):
        c = i % self.copies
        self.w4.w4a8_linear_awq(self.x, self.P[c], self.S[c], self.s, Y=self.y, workspace=self.ws)


def offline_parts(w4, torch, hip):
    """Offline weight transforms on the 7B-class layer [4096, 11008], timed with
    events: dequantization, the LoRA merge (dequantize + add delta + requantize)
    and the AWQ fold; each reads / writes the fp32 weights once or twice."""
    import workloads
    dev = torch.device("cuda")
    d = workloads.generate("mlp7b", M=1)
    W = torch.from_numpy(d["W"]).to(dev)
    K, N = W.shape
    p, s, _ = w4.w4_quantize_weight(W, "sym")
    delta = torch.randn(K, 16, device=dev) @ torch.randn(16, N, device=dev) * 1e-3
    work = torch.empty_like(W)
    Wd = torch.empty_like(W)
    po, so = torch.empty_like(p), torch.empty_like(s)
    sc = torch.ones(K, device=dev)

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        a, b = hip.event(), hip.event()
        st = torch.cuda.current_stream().cuda_stream
        hip.record(a, st)
        for _ in range(reps):
            fn()
        hip.record(b, st)
        ms = hip.elapsed_ms(a, b) / reps
        hip.destroy(a)
        hip.destroy(b)
        return ms

    fp32 = 4 * K * N
    res = []
    ms = timed(lambda: w4.w4_dequantize_weight(p, s, None, K, "sym", W=Wd))
    res.append({"workload": "dequant_weight_7b", "ms": round(ms, 4),
                "GBps": round((fp32 + p.numel() + 4 * N) / ms / 1e6, 1)})
    ms = timed(lambda: w4.w4_merge_delta(p, s, None, delta, "sym", work=work))
    res.append({"workload": "lora_merge_7b", "ms": round(ms, 4),
                "note": "dequantize + add delta (one kernel), then absmax, codes, scales"})
    ms = timed(lambda: w4.awq_fold_weight(W, sc, W_out=Wd))
    res.append({"workload": "awq_fold_7b", "ms": round(ms, 4), "GBps": round(2 * fp32 / ms / 1e6, 1)})
    return res


class W4A16Case:
    """The 70B-class W4A16 layer; with prepacked=True the weights and tables
    are converted once (offline) to the GPU-shuffled layout."""

    def __init__(self, w4, torch, copies=None, prepacked=False):
        import numpy as np
        import workloads
        d = workloads.w4a16_inputs()
        self.name = "w4a16_70b_m16"
        self.M, self.K, self.N, self.g = d["M"], d["K"], d["N"], d["group"]
        self.torch, self.w4 = torch, w4
        dev = torch.device("cuda")
        self.x = torch.from_numpy(d["x_bf16"].view(np.int16)).to(dev)
        W = torch.from_numpy(d["W"]).to(dev)
        t0 = time.perf_counter()
        p, s, z = w4.w4_quantize_weight(W, "asym", self.g)
        torch.cuda.synchronize()
        self.quant_s = time.perf_counter() - t0
        del W
        wbytes = p.numel() + 8 * s.numel()
        self.copies = copies or max(1, math.ceil(ROTATE_BYTES / wbytes))
        self.prepacked = prepacked
        if prepacked:
            self.name = "w4a16_70b_m16_prepacked"
            p, s = w4.w4a16_prepack(p, s, z)
            z = None
            torch.cuda.synchronize()
        self.P = [p] + [p.clone() for _ in range(self.copies - 1)]
        self.Sc = [s] + [s.clone() for _ in range(self.copies - 1)]
        self.Z = [z] * self.copies if z is None else [z] + [z.clone() for _ in range(self.copies - 1)]
        self.y = torch.empty((self.M, self.N), dtype=torch.float32, device=dev)
        self.bytes = w4a16_bytes(self.M, self.K, self.N, self.g)
        self.ops = 2 * self.M * self.N * self.K

    def step(self, i):
        c = i % self.copies
        if self.prepacked:
            self.w4.w4a16_linear_prepacked(self.x, self.P[c], self.Sc[c], self.N, Y=self.y)
        else:
            self.w4.w4a16_linear(self.x, self.P[c], self.Sc[c], self.Z[c], self.g, Y=self.y)


def graph_step_time(torch, case, steps, warmup, hip=None):
    """Wall time per step of `steps` steps replayed from one captured graph.
    With `hip`, also the GPU time per step from HIP events recorded on the
    replay stream around the same replay: returns (wall, events)."""
    for i in range(warmup):
        case.step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                case.step(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()                      # untimed replay
    torch.cuda.synchronize()
    if hip is not None:
        ea, eb = hip.event(), hip.event()
        stream = torch.cuda.current_stream().cuda_stream
        hip.record(ea, stream)
    t0 = time.perf_counter()
    g.replay()
    if hip is not None:
        hip.record(eb, stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    del g
    if hip is None:
        return dt / steps
    ev = hip.elapsed_ms(ea, eb) / 1e3
    hip.destroy(ea)
    hip.destroy(eb)
    return dt / steps, ev / steps


def region_time(torch, hip, step, est_s, min_launches, min_region_s=2e-3):
    """Average duration (s) of one launch from HIP events recorded on the
    replay stream around one replay of a graph of L back-to-back launches,
    L >= min_launches and L * est_s >= min_region_s (so the graph's own launch
    latency is spread over at least about 2 ms).  est_s sizes the first
    graph; when the replay runs faster than that estimate (a replayed graph
    launches faster than timed steps) and the region falls short of
    min_region_s, the graph is captured again, sized by the measured rate.
    Returns (seconds, L)."""
    L = max(int(min_launches), int(math.ceil(min_region_s / max(est_s, 1e-7))))
    sec = region_replay(torch, hip, step, L)
    if sec * L < min_region_s:
        L = max(int(min_launches), int(math.ceil(1.05 * min_region_s / max(sec, 1e-7))))
        sec = region_replay(torch, hip, step, L)
    return sec, L


def region_replay(torch, hip, step, L):
    """Seconds per launch over one timed replay of a graph of L launches."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(L):
                step(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()                      # untimed replay
    torch.cuda.synchronize()
    ea, eb = hip.event(), hip.event()
    stream = torch.cuda.current_stream().cuda_stream
    hip.record(ea, stream)
    g.replay()
    hip.record(eb, stream)
    torch.cuda.synchronize()
    sec = hip.elapsed_ms(ea, eb) / 1e3 / L
    hip.destroy(ea)
    hip.destroy(eb)
    del g
    return sec


def demangle(name):
    """Readable form of a kernel symbol (c++filt if present, else as is)."""
    import shutil
    import subprocess
    if name.startswith("_Z") and shutil.which("c++filt"):
        r = subprocess.run(["c++filt", name], capture_output=True, text=True)
        if r.returncode == 0 and r.stdout.strip():
            return r.stdout.strip()
    return name


def platform_probes(torch, hip, w4, head_grid):
    """The platform references: an empty launch (1 workgroup and the headline
    kernel's grid) and plain streaming reads of the headline's, the 7B-class
    layer's and the 70B-class W4A16 layer's algorithmic bytes, each over
    buffers rotating through more than the Infinity Cache, timed over >= 2 ms
    of back-to-back graph launches."""
    out = {}
    for blocks in (1, head_grid):
        sec, L = region_time(torch, hip, lambda i: w4.w4_probe_empty(blocks), 2e-6, 200)
        out[f"empty_launch_{blocks}wg_us"] = round(sec * 1e6, 3)
    out["empty_launch_launches"] = L
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    reads = []
    for label, nbytes in (("headline", 4041216), ("mlp7b_m1", 22648832),
                          ("w4a16_70b", 134217728)):
        copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
        est = nbytes / 5e12 + 2e-6
        sec, L = region_time(torch, hip, lambda i: w4.w4_probe_read(bufs[i % copies], sink),
                             est, 20)
        reads.append({"bytes": nbytes, "as": label, "us": round(sec * 1e6, 3),
                      "GBps": round(nbytes / sec / 1e9, 1), "launches": L,
                      "rotating_copies": copies})
        del bufs
        torch.cuda.empty_cache()
    out["plain_read"] = reads
    # a plain write of the prefill product's fp32 output (4 M N bytes) into one
    # buffer, as the product writes its output
    nbytes = PLAIN_WRITES["write67m"]
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sec, L = region_time(torch, hip, lambda i: w4.w4_probe_write(dst, i), nbytes / 5e12 + 2e-6, 20)
    out["plain_write"] = [{"bytes": nbytes, "as": "prefill_output", "us": round(sec * 1e6, 3),
                           "GBps": round(nbytes / sec / 1e9, 1), "launches": L}]
    del dst
    torch.cuda.empty_cache()
    # the matrix units' clock under load (shader-clock / 100 MHz counters of
    # each workgroup) and their int8 rate, on constant operands and on random
    # bytes (the switching activity of a real product lowers the clock)
    import statistics
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    times = torch.zeros((cus, 4), dtype=torch.int64, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(20251014)
    rnd = torch.randint(-2 ** 31, 2 ** 31 - 1, (cus * 512 * 32,), dtype=torch.int32, device="cuda",
                        generator=g)
    iters = 9000

    def mfma_leg(ops):
        w4.w4_probe_mfma(cus, 100, times, sink, ops)
        torch.cuda.synchronize()
        a, b = hip.event(), hip.event()
        st = torch.cuda.current_stream().cuda_stream
        hip.record(a, st)
        w4.w4_probe_mfma(cus, iters, times, sink, ops)
        hip.record(b, st)
        sec = hip.elapsed_ms(a, b) / 1e3
        hip.destroy(a)
        hip.destroy(b)
        t = times.cpu().numpy().astype("float64")
        clocks = (t[:, 1] - t[:, 0]) / ((t[:, 3] - t[:, 2]) / 1e8)
        return {"clock_GHz": round(statistics.median(clocks.tolist()) / 1e9, 4),
                "clock_GHz_min": round(float(clocks.min()) / 1e9, 4),
                "int8_TOPS": round(cus * 8 * 16 * iters * 32768 / sec / 1e12, 1),
                "ms": round(sec * 1e3, 3)}

    const = mfma_leg(None)
    out["mfma_probe"] = {"clock_GHz": const["clock_GHz"], "clock_GHz_min": const["clock_GHz_min"],
                         "int8_TOPS_constant_operands": const["int8_TOPS"], "ms": const["ms"],
                         "random_operands": mfma_leg(rnd)}
    del rnd
    p = torch.cuda.get_device_properties(0)
    out["device"] = {"name": p.name, "arch": p.gcnArchName, "cus": p.multi_processor_count,
                     "pci": f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}",
                     "uuid": str(p.uuid), "hbm_bytes": p.total_memory}
    return out


def kernel_time(torch, hip, w4, case, launches):
    """Average duration (s) of the product kernel, from start/stop events
    attached to each dispatch, over `launches` rotating launches."""
    evs = [(hip.event(), hip.event()) for _ in range(launches)]
    for i in range(min(10, launches)):
        case.step(i)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        w4.w4_time_next_kernel(a, b)
        case.step(i)
    torch.cuda.synchronize()
    ms = [hip.elapsed_ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    ms.sort()
    return sum(ms) / len(ms) / 1e3, ms[len(ms) // 2] / 1e3


def src_digest():
    h = hashlib.sha256()
    for f in ("gemv.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "int4_weight_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "gemv_dot4_gemma_m1_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("src_digest") != kernel_digest:
        return None
    return t.get("traffic_bytes_per_launch")


def _host_cores():
    """Threads for the all-cores legs: the CPUs this process may run on, at
    most 16 (the host share of one GPU on the benchmark boxes)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _run_threads(fns, seconds):
    """Call fns[i]() repeatedly on thread i until `seconds` have passed (each
    thread finishes its current call).  The oracle's ctypes calls release the
    GIL, so the threads run on separate cores.  Returns (calls, wall seconds)."""
    import threading
    counts = [0] * len(fns)
    stop = time.perf_counter() + seconds

    def run(i):
        while True:
            fns[i]()
            counts[i] += 1
            if time.perf_counter() >= stop:
                break

    ths = [threading.Thread(target=run, args=(i,)) for i in range(len(fns))]
    t0 = time.perf_counter()
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    return counts, time.perf_counter() - t0


def _slices(n, parts):
    edges = [n * i // parts for i in range(parts + 1)]
    return [(edges[i], edges[i + 1]) for i in range(parts) if edges[i + 1] > edges[i]]


def cpu_baseline(case, seconds=5.0):
    """The CPU oracle, as it is, on the machine's host cores: the headline layer on
    one thread and on all cores (threads split the output channels, each
    calling the oracle's whole forward on its slice), then bounded samples of
    the 4096^3 prefill (64 of its 4096 rows) and of the 70B-class W4A16 layer
    (its first 2048 of 28672 output channels) on all cores."""
    import numpy as np
    import oracle
    import workloads
    cores = _host_cores()
    res = {}
    # headline, one thread
    pref, sref = oracle.quantize_weight_sym(case.host_W)
    counts, dt = _run_threads([lambda: oracle.w4a8_linear(case.host_x, pref, sref)], seconds)
    per = dt / counts[0]
    single = {"value": round(case.bytes / per / 1e9, 4), "unit": "GB/s", "cores": 1,
              "sample": f"{counts[0]} calls of the oracle's w4a8_linear on the whole headline "
                        f"layer ({case.M}x{case.K}x{case.N}), {dt:.1f} s, {per * 1e3:.2f} ms "
                        f"per call"}
    # headline, all cores: thread i runs the forward of channels n0..n1
    sl = _slices(case.N, cores)
    fns = [(lambda a, b: (lambda: oracle.w4a8_linear(
        case.host_x, np.ascontiguousarray(pref[a:b]), np.ascontiguousarray(sref[a:b]))))(a, b)
        for a, b in sl]
    counts, dt = _run_threads(fns, seconds)
    layers = sum(c * (b - a) for c, (a, b) in zip(counts, sl)) / case.N
    res.update({"value": round(case.bytes * layers / dt / 1e9, 4), "unit": "GB/s",
                "cores": len(sl), "kind": "oracle",
                "sample": f"the headline layer ({case.M}x{case.K}x{case.N}) with its output "
                          f"channels split over {len(sl)} threads, each calling the oracle's "
                          f"w4a8_linear on its slice: {layers:.0f} whole layers in {dt:.1f} s",
                "single_core": single})
    # prefill sample, all cores
    d = workloads.generate("prefill")
    xs = np.ascontiguousarray(d["x"][:64])
    pp, ps = oracle.quantize_weight_sym(d["W"])
    K, N = d["K"], d["N"]
    sl = _slices(N, cores)
    fns = [(lambda a, b: (lambda: oracle.w4a8_linear(
        xs, np.ascontiguousarray(pp[a:b]), np.ascontiguousarray(ps[a:b]))))(a, b) for a, b in sl]
    counts, dt = _run_threads(fns, seconds)
    ops = sum(c * 2 * xs.shape[0] * K * (b - a) for c, (a, b) in zip(counts, sl))
    res["prefill"] = {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": len(sl),
                      "sample": f"64 of the 4096 rows of the 4096x4096x4096 prefill, output "
                                f"channels split over {len(sl)} threads (oracle w4a8_linear), "
                                f"{ops / 1e9:.1f} G int ops in {dt:.1f} s"}
    del d, pp
    # W4A16 sample, all cores
    w = workloads.w4a16_inputs(N=2048)
    g, M, K = w["group"], w["M"], w["K"]
    qp, qs, qz = oracle.quantize_weight_asym(w["W"], g)
    sl = _slices(2048, cores)
    fns = [(lambda a, b: (lambda: oracle.w4a16_linear(
        w["x_bf16"], np.ascontiguousarray(qp[a:b]), np.ascontiguousarray(qs[a:b]),
        np.ascontiguousarray(qz[a:b]), g)))(a, b) for a, b in sl]
    counts, dt = _run_threads(fns, seconds)
    cols = sum(c * (b - a) for c, (a, b) in zip(counts, sl))
    full_n = workloads.SHAPES["w4a16"].N
    layer_bytes = w4a16_bytes(M, K, full_n, g)
    res["w4a16"] = {"value": round(layer_bytes * cols / full_n / dt / 1e9, 4), "unit": "GB/s",
                    "cores": len(sl),
                    "sample": f"the first 2048 of the 28672 output channels of the 16x8192x28672 "
                              f"group-128 layer, split over {len(sl)} threads (oracle "
                              f"w4a16_linear, fp64 sums), {cols} channel-rows in {dt:.1f} s; "
                              f"value = the layer's bytes x channels done / {full_n} / time"}
    res["host"] = {"cpu_model": _cpu_model(), "logical_cpus": os.cpu_count(),
                   "threads_used": cores}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-parts", action="store_true", help="headline workload only")
    ap.add_argument("--only", default=None,
                    help="run one workload's product kernel (for profilers): gemma_m1, gemma_m8, "
                         "mlp7b_m1, mlp7b_m16, mlp7b_m64, prefill, w4a16, w4a16_prepacked, "
                         "w8a8_gemma_m1, "
                         "w8a8_mlp7b_m1, w8a8_prefill, pp_<W4A8 workload> (shuffled tiles); "
                         "copy (a 64 MiB device copy, for counter calibration); "
                         "write67m (a plain streaming write of the 4096^3 prefill's fp32 "
                         "output bytes); "
                         "empty (an empty kernel of the headline's grid); read4m, read22m, "
                         "read134m (plain streaming reads of the headline's, the 7B-class and "
                         "the 70B-class W4A16 layer's bytes)")
    ap.add_argument("--launches", type=int, default=200)
    ap.add_argument("--copies", type=int, default=0,
                    help="with --only: number of rotating weight copies (0 = enough to exceed "
                         "the Infinity Cache)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards over output channels with no exchange, so each GPU runs a "
              "smaller-N layer of the same kind).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_weight_quantized_amd as w4
    w4.lib()  # fails loudly when the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    hip = Hip()

    if args.only in PLAIN_WRITES:
        # a plain write of the prefill product's output bytes into one buffer
        dst = torch.empty(PLAIN_WRITES[args.only], dtype=torch.uint8, device="cuda")
        for i in range(args.warmup + args.steps):
            w4.w4_probe_write(dst, i)
        torch.cuda.synchronize()
        log(f"{args.only}: {args.warmup + args.steps} launches done")
        return
    if args.only == "empty" or (args.only or "").startswith("read"):
        # platform references for the profilers: an empty launch of the
        # headline kernel's grid, or plain reads of 4 / 22.6 / 134 MB
        # (the headline's, the 7B-class layer's and the W4A16 layer's bytes)
        # over rotating buffers
        if args.only == "empty":
            for _ in range(args.warmup + args.steps):
                w4.w4_probe_empty(432)
        else:
            nbytes = {"read4m": 4041216, "read22m": 22648832, "read134m": 134217728}[args.only]
            copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
            bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
            sink = torch.zeros(64, dtype=torch.int32, device="cuda")
            for i in range(args.warmup + args.steps):
                w4.w4_probe_read(bufs[i % copies], sink)
        torch.cuda.synchronize()
        log(f"{args.only}: {args.warmup + args.steps} launches done")
        return
    if args.only == "copy":
        # a plain device copy of known size (calibrates the HBM byte counters)
        src = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy: {args.warmup + args.steps} copies of {src.numel()} bytes done")
        return
    if args.only:
        specs = {"gemma_m1": ("gemma", 1), "gemma_m8": ("gemma", 8), "mlp7b_m1": ("mlp7b", 1),
                 "mlp7b_m16": ("mlp7b", 16), "mlp7b_m64": ("mlp7b", 64),
                 "prefill": ("prefill", None)}
        w8 = args.only.startswith("w8a8_")
        pp = args.only.startswith("pp_")
        key = args.only[5:] if w8 else args.only[3:] if pp else args.only
        if args.only.startswith("w4a16"):
            case = W4A16Case(w4, torch, copies=args.copies,
                             prepacked=args.only == "w4a16_prepacked")
        else:
            case = W4A8Case(w4, torch, args.only, *specs[key], copies=args.copies, w8=w8,
                            pp=pp)
        for i in range(args.warmup + args.steps):
            case.step(i)
        torch.cuda.synchronize()
        log(f"{args.only}: {args.warmup + args.steps} launches done ({w4.w4_last_path()})")
        return

    log("headline: gemma3-1b up-projection, W4A8, M=1")
    head = W4A8Case(w4, torch, "gemma_m1", "gemma", 1)
    step_s, steps_region_s = graph_step_time(torch, head, args.steps, args.warmup, hip)
    path = w4.w4_last_path()
    kernel = demangle(w4.w4_last_kernel())
    # each step is this one kernel launch: its average launch duration is the
    # event time of a region of back-to-back launches / launches, over a
    # region of >= 2 ms so that the graph's own launch latency is amortized
    region_s, region_launches = region_time(torch, hip, head.step, step_s, args.steps)
    k_avg, k_med = kernel_time(torch, hip, w4, head, args.launches)
    value = head.bytes / step_s / 1e9
    achieved = head.bytes / region_s / 1e9
    digest = src_digest()
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "Gemma3-1B-like MLP up-projection, W4A8 decode GEMV",
                   "M": 1, "K": head.K, "N": head.N, "weights": "int4 symmetric per-channel",
                   "activations": "int8 per-row dynamic", "launch": "hipGraph of all steps",
                   "rotating_weight_copies": head.copies, "product_kernel": path},
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(digest),
                     "algorithmic_bytes_per_launch": head.bytes,
                     "kernel_us_avg": round(region_s * 1e6, 3),
                     "timing": "HIP events on the replay stream around one replay of a graph "
                               "of back-to-back launches of this kernel, divided by its launches",
                     "region_launches": region_launches,
                     "region_ms": round(region_s * region_launches * 1e3, 3),
                     "kernel_us_timed_steps_region": round(steps_region_s * 1e6, 3),
                     "kernel_us_dispatch_events_avg": round(k_avg * 1e6, 3),
                     "kernel_us_dispatch_events_median": round(k_med * 1e6, 3),
                     "src_digest": digest},
    }
    log(f"headline: step {step_s * 1e6:.2f} us ({args.steps} steps), kernel "
        f"{region_s * 1e6:.3f} us (region of {region_launches} launches), "
        f"{k_avg * 1e6:.2f} us (per-dispatch events), {value:.0f} GB/s")

    if not args.no_parts:
        log("platform: empty launches and plain reads")
        out["platform"] = platform_probes(torch, hip, w4, (head.N + 15) // 16)
    parts = []
    if not args.no_parts:
        def w4a8_part(name, shape, M, bound, rotate=True, w8=False, pp=False):
            log(f"part: {name}")
            c = W4A8Case(w4, torch, name, shape, M, rotate=rotate, w8=w8, pp=pp)
            st = graph_step_time(torch, c, 200, 10)
            p = w4.w4_last_path()
            # one launch when the activation quantization runs inside the
            # product kernel, else a quantizer launch before it
            fused = p.startswith(("gemv_dot4", "w8_gemv_dot4")) or "mfma_fused" in p
            launches = 1 if fused else 2
            stl, L = region_time(torch, hip, c.step, st, 200)
            kd, km = kernel_time(torch, hip, w4, c, min(args.launches, 100))
            # the product kernel's time: with one launch per step, the region's
            # time per launch (as for the headline); else its dispatch events,
            # which also hold that launch's own dispatch latency
            ka = stl if launches == 1 else kd
            r = {"workload": name, "M": c.M, "K": c.K, "N": c.N, "product_kernel": p,
                 "launches_per_step": launches,
                 "step_us": round(stl * 1e6, 3), "step_region_launches": L,
                 "kernel_us_avg": round(ka * 1e6, 3),
                 "kernel_timing": "graph region" if launches == 1 else "dispatch events",
                 "kernel_us_dispatch_events": round(kd * 1e6, 3),
                 "algorithmic_bytes": c.bytes, "int_ops": c.ops,
                 "rotating_weight_copies": c.copies,
                 "weight_quantize_ms": round(c.quant_s * 1e3, 3)}
            if bound == "hbm":
                # the step's rate (every launch of the step, fp32 activations
                # in) is the figure; the product kernel's own rate counts what
                # that kernel reads: fp32 activations when fused, else the
                # int8 codes and row scales the quantizer wrote
                kb = c.bytes if fused else c.bytes - 4 * c.M * c.K + c.M * c.K + 4 * c.M
                r["GBps_step"] = round(c.bytes / stl / 1e9, 1)
                r["frac_hbm_step"] = round(c.bytes / stl / 1e9 / HBM_PEAK_GBS, 4)
                r["product_kernel_bytes"] = kb
                r["GBps_kernel"] = round(kb / ka / 1e9, 1)
                r["frac_hbm_kernel"] = round(kb / ka / 1e9 / HBM_PEAK_GBS, 4)
            else:
                r["TOPS_kernel"] = round(c.ops / ka / 1e12, 1)
                r["TOPS_step"] = round(c.ops / stl / 1e12, 1)
                r["frac_int8_mfma_kernel"] = round(c.ops / ka / 1e12 / INT8_PEAK_TOPS, 4)
                r["frac_int8_mfma_step"] = round(c.ops / stl / 1e12 / INT8_PEAK_TOPS, 4)
            parts.append(r)
            del c
            torch.cuda.empty_cache()

        w4a8_part("gemma_m8", "gemma", 8, "hbm")
        w4a8_part("mlp7b_m1", "mlp7b", 1, "hbm")
        w4a8_part("mlp7b_m16", "mlp7b", 16, "hbm")
        w4a8_part("mlp7b_m64", "mlp7b", 64, "hbm")
        w4a8_part("prefill_4096", "prefill", None, "mfma", rotate=False)
        w4a8_part("pp_gemma_m1", "gemma", 1, "hbm", pp=True)
        w4a8_part("pp_gemma_m8", "gemma", 8, "hbm", pp=True)
        w4a8_part("pp_mlp7b_m1", "mlp7b", 1, "hbm", pp=True)
        w4a8_part("pp_mlp7b_m16", "mlp7b", 16, "hbm", pp=True)
        w4a8_part("pp_mlp7b_m64", "mlp7b", 64, "hbm", pp=True)
        w4a8_part("pp_prefill_4096", "prefill", None, "mfma", rotate=False, pp=True)
        w4a8_part("w8a8_gemma_m1", "gemma", 1, "hbm", w8=True)
        w4a8_part("w8a8_mlp7b_m1", "mlp7b", 1, "hbm", w8=True)
        w4a8_part("w8a8_mlp7b_m16", "mlp7b", 16, "hbm", w8=True)
        w4a8_part("w8a8_prefill_4096", "prefill", None, "mfma", rotate=False, w8=True)
        for name, M in (("awq_mlp7b_m1", 1), ("awq_mlp7b_m16", 16)):
            log(f"part: {name}")
            c = AwqCase(w4, torch, name, "mlp7b", M)
            st = graph_step_time(torch, c, 200, 10)
            p = w4.w4_last_path()
            st, L = region_time(torch, hip, c.step, st, 200)
            kd, km = kernel_time(torch, hip, w4, c, 100)
            one = p.startswith("gemv_dot4")
            parts.append({"workload": name, "M": c.M, "K": c.K, "N": c.N, "product_kernel": p,
                          "launches_per_step": 1 if one else 2,
                          "step_us": round(st * 1e6, 3), "step_region_launches": L,
                          "kernel_us_avg": round((st if one else kd) * 1e6, 3),
                          "kernel_timing": "graph region" if one else "dispatch events",
                          "kernel_us_dispatch_events": round(kd * 1e6, 3),
                          "algorithmic_bytes": c.bytes,
                          "GBps_step": round(c.bytes / st / 1e9, 1),
                          "frac_hbm_step": round(c.bytes / st / 1e9 / HBM_PEAK_GBS, 4),
                          "rotating_weight_copies": c.copies})
            del c
            torch.cuda.empty_cache()
        log("part: offline weight transforms")
        parts.extend(offline_parts(w4, torch, hip))
        for pp in (False, True):
            log(f"part: w4a16_70b_m16{' prepacked' if pp else ''}")
            c = W4A16Case(w4, torch, prepacked=pp)
            st = graph_step_time(torch, c, 50, 5)
            p = w4.w4_last_path()
            st, L = region_time(torch, hip, c.step, st, 50)
            kd, km = kernel_time(torch, hip, w4, c, 50)
            ka = st  # one launch per step: the region's time per launch
            parts.append({"workload": c.name, "M": c.M, "K": c.K, "N": c.N, "group": c.g,
                          "product_kernel": p, "launches_per_step": 1,
                          "step_us": round(st * 1e6, 3), "step_region_launches": L,
                          "kernel_us_avg": round(ka * 1e6, 3), "kernel_timing": "graph region",
                          "kernel_us_dispatch_events": round(kd * 1e6, 3),
                          "algorithmic_bytes": c.bytes,
                          "GBps_kernel": round(c.bytes / ka / 1e9, 1),
                          "GBps_step": round(c.bytes / st / 1e9, 1),
                          "frac_hbm_kernel": round(c.bytes / ka / 1e9 / HBM_PEAK_GBS, 4),
                          "TFLOPS_kernel": round(c.ops / ka / 1e12, 2),
                          "rotating_weight_copies": c.copies,
                          "weight_quantize_ms": round(c.quant_s * 1e3, 3)})
            del c
            torch.cuda.empty_cache()
        pre = [p for p in parts if p["workload"] == "prefill_4096"][0]
        pps = [p for p in parts if p["workload"] == "pp_prefill_4096"]
        out["prefill_int8"] = {"metric": "int8 TOPS (M=4096 prefill GEMM)",
                               "TOPS_kernel": pre["TOPS_kernel"], "TOPS_step": pre["TOPS_step"],
                               "peak": INT8_PEAK_TOPS,
                               "frac_kernel": pre["frac_int8_mfma_kernel"]}
        if pps:  # the same product on the shuffled weight tiles
            out["prefill_int8"]["shuffled_tiles"] = {
                "TOPS_kernel": pps[0]["TOPS_kernel"], "TOPS_step": pps[0]["TOPS_step"],
                "frac_kernel": pps[0]["frac_int8_mfma_kernel"]}
    out["parts"] = parts
    out["headline_weight_quantize_ms"] = round(head.quant_s * 1e3, 3)
    if not args.no_cpu:
        log("cpu baseline: oracle")
        out["cpu_baseline"] = cpu_baseline(head)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
