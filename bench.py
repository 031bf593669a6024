#!/usr/bin/env python3
"""Throughput of the quantization hot path on one MI355X.

A step is one pass of the whole path over the streaming workload (BF16
65536 x 16384 = 2 GiB, N(0,1) with 0.5 % outlier channels x200): quantize
with the fused dequantization and error statistics to each of the seven
format / granularity pairs (INT8 and E4M3 per tensor, E4M3 and E5M2 per
row, MXFP4, NVFP4, INT4 g128), each call absmax -> scale -> saturating RNE
cast -> pack -> x^ in registers -> statistics.  `value` is the algorithmic
bytes of the step (x read once and codes + scales written once, per format)
divided by the timed wall time, inputs resident in HBM.  The per-tensor
formats and NVFP4's global scale re-read x for their absmax pre-pass; that
re-read is moved traffic, not algorithmic bytes.

Also reported:
  ceiling     streaming kernels (read-only, write-only, copy, read:write 2:1
              and 4:1) at 4 / 8 / 16 words of 16 B in flight per lane over a
              grid sweep: the practical HBM ceilings of this chip;
  per_format  every workload (c1-c5 and the stream), each format with
              statistics on and off: median, p10 and p90 over repeated
              graph replays (after about 40 ms of untimed replays, so that
              the clocks have settled under load), GB/s, fractions of 8 TB/s, of the copy ceiling
              and of the matching read:write ceiling; moved-bytes GB/s for
              the calls with an absmax pre-pass; the dequantize call;
  roofline    the dominant kernel of the step against the HBM peak;
  cpu_baseline the CPU oracle on a bounded sample of the stream workload,
              multi-threaded and on one thread, with the host CPU named;
  zp_gemm / mx_gemm / mxw_gemm  the dequantize-GEMM consumers.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0                # dense BF16 matrix-core peak
MFMA_FP4_PEAK_TFS = 10100.0                # dense FP4 matrix-core peak
GEMM_TOKENS = (1, 16, 64, 256, 2048)
MX_GEMM_TOKENS = (16, 128, 256, 2048, 8192)
T0 = time.perf_counter()


def progress(msg):
    """One line per finished part of the run, on stderr."""
    print(f"[bench {time.perf_counter() - T0:7.1f} s] {msg}", file=sys.stderr, flush=True)


METRIC = "quantize GB/s (bytes in+out) and % of MI355X HBM peak, per format"
NSETS = 4                                  # input / output sets rotated by the small workloads
STREAM_FORMATS = (("int8", "tensor"), ("e4m3", "tensor"), ("e4m3", "row"), ("e5m2", "row"),
                  ("mxfp4", "block"), ("nvfp4", "block"), ("int4", "block"))
# the kernel the roofline object describes: the per-row E4M3 cast of the stream
ROOFLINE_CALL = ("e4m3", "row")
CEILING_KINDS = {0: "read", 1: "write", 2: "copy", 3: "read2_write1", 4: "read4_write1"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-format workloads and the GEMMs")
    ap.add_argument("--no-gemm", action="store_true", help="skip the dequantize-GEMM consumers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="profiling aid: run one call type in a loop (e.g. stream:e4m3:row, c2:e4m3:row, "
                         "c4:nvfp4:block:static, c5:int4:block:nostats, ceiling, copy, zp_gemm:16, mx_gemm:2048)")
    ap.add_argument("--reps", type=int, default=30, help="timed graph replays per breakdown entry")
    return ap.parse_args()


def to_device(x_np):
    """numpy float32 / uint16 (BF16 bits) -> device tensor."""
    import numpy as np
    import torch
    if x_np.dtype == np.uint16:
        return torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(x_np).to("cuda:0")


def algo_bytes(fmt, gran, rows, cols, in_elem):
    """Bytes the method itself must move: x once, codes + scales once.
    Returns (quantize bytes, codes + scales bytes)."""
    n = rows * cols
    codes = n // 2 if fmt in ("mxfp4", "nvfp4", "int4", "int4zp") else n
    if fmt in ("int8", "e4m3", "e5m2"):
        scales = 4 if gran == "tensor" else 4 * rows
    elif fmt == "mxfp4":
        scales = n // 32
    elif fmt == "nvfp4":
        scales = n // 16 + 4
    elif fmt == "int4zp":
        scales = 4 * (n // 128) + n // 256      # FP32 scale and a 4-bit shift per group
    else:
        scales = 2 * (n // 128)
    return n * in_elem + codes + scales, codes + scales


def has_prepass(fmt, gran, var=""):
    """Calls whose scale needs the tensor absmax first (x is read twice)."""
    return var != "static" and (gran == "tensor" or fmt == "nvfp4")


def mix_kind(fmt, in_elem):
    """The read:write ceiling matching a format's byte ratio."""
    if fmt in ("int8", "e4m3", "e5m2"):
        return 3 if in_elem == 2 else 4      # BF16 -> 1 B: 2:1; FP32 -> 1 B: 4:1
    return 4                                 # BF16 -> 4 bits: 4:1


def backlog():
    """Queue a short spin on the stream so that the events and graph
    launches recorded next queue behind it: the GPU then runs them back to
    back and the events time device work only, not host launch latency."""
    import torch
    torch.cuda._sleep(2_000_000)


def time_graph(body, reps, warm_ms=40.0):
    """Capture body() in a graph, replay it `reps` times with HIP events on
    the current stream around each replay; returns per-replay milliseconds.
    Untimed replays worth about warm_ms of device time run first: after an
    idle gap the first tens of milliseconds of heavy load run slower than
    the steady state (the clocks settle under the power limit), and the
    timings are of the steady state."""
    import torch
    s = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    g.replay()
    b.record(s)
    torch.cuda.synchronize()
    nwarm = min(1000, max(1, math.ceil(warm_ms / max(a.elapsed_time(b), 1e-3))))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    backlog()
    for _ in range(nwarm):
        g.replay()
    for a, b in evs:
        a.record(s)
        g.replay()
        b.record(s)
    torch.cuda.synchronize()
    del g
    return [a.elapsed_time(b) for a, b in evs]


def summarize(ms_list, n_calls, nbytes):
    ms = sorted(m / n_calls for m in ms_list)
    k = len(ms)
    med, p10, p90 = ms[k // 2], ms[k // 10], ms[(9 * k) // 10]
    mean = sum(ms) / k
    return {"us": round(1e3 * med, 2), "p10_us": round(1e3 * p10, 2), "p90_us": round(1e3 * p90, 2),
            "mean_us": round(1e3 * mean, 2), "GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


# Call variants: rule flags, or static scaling with an absmax computed once
# beforehand (the calibrated mode).
VARIANTS = {"": {}, "mx-nearest": {"flags": 1}, "mx-up": {"flags": 2}, "nv-rne": {"flags": 4}, "static": None}


class Workload:
    """nsets device copies of one synthetic input plus outputs per format
    (entries (fmt, gran) or (fmt, gran, variant)), with and without
    statistics."""

    def __init__(self, name, formats, nsets=NSETS):
        import torch

        from synth import synth
        import int_quantization_amd as iq
        self.iq = iq
        self.name = name
        x_np = synth.make(name)
        x0 = to_device(x_np)
        del x_np
        self.nsets = nsets
        self.xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
        self.rows, self.cols = x0.shape
        self.in_elem = x0.element_size()
        self.formats = formats
        self.ws = [iq.workspace_for(iq.desc_for(x0, *formats[0][:2]), x0.device) for _ in range(nsets)]
        self.amax = [iq.amax(x) for x in self.xs] if any(len(f) > 2 and f[2] == "static" for f in formats) else None
        self.q = {}
        for spec in formats:
            fmt, gran, var = (*spec, "")[:3]
            self.q[(fmt, gran, var)] = [iq.quantize(x, fmt, gran, stats=True, workspace=w, **self._kw(var, i))
                                        for i, (x, w) in enumerate(zip(self.xs, self.ws))]
        self.out = None
        torch.cuda.synchronize()

    def _kw(self, var, i):
        return {"static_amax": self.amax[i]} if var == "static" else dict(VARIANTS[var])

    def quant(self, fmt, gran, i, var="", stats=True):
        q = self.q[(fmt, gran, var)][i]
        out = q if stats else self.iq.Quantized(q.codes, q.scales, q.global_scale, None, None, q.fmt, q.gran,
                                                q.rows, q.cols, q.shifts)
        self.iq.quantize(self.xs[i], fmt, gran, workspace=self.ws[i], out=out, **self._kw(var, i))

    def dequant(self, fmt, gran, i, var=""):
        import torch
        if self.out is None:
            dt = torch.bfloat16 if self.in_elem == 2 else torch.float32
            self.out = [torch.empty((self.rows, self.cols), dtype=dt, device="cuda:0")
                        for _ in range(min(2, self.nsets))]
        self.iq.dequantize(self.q[(fmt, gran, var)][i], out=self.out[i % len(self.out)])

    def bytes(self, fmt, gran):
        qb, code_b = algo_bytes(fmt, gran, self.rows, self.cols, self.in_elem)
        return qb, code_b + self.rows * self.cols * self.in_elem

    def release(self):
        import torch
        self.xs = self.ws = self.q = self.out = self.amax = None
        torch.cuda.empty_cache()


# ---- practical ceilings ------------------------------------------------------------
def ceiling(reps=10, grids=(1024, 2048, 4096, 8192, 16384)):
    """Best GB/s (bytes read + written) per streaming kernel kind over the
    depths, cache policies and grids swept; 1 GiB on the heavier side."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "int_quantization_amd", "libiq_bench.so"))
    lib.iqb_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
    n = 1 << 30
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda:0").normal_()
    dst = torch.empty(n // 4, dtype=torch.float32, device="cuda:0")
    res, sweep = {}, []
    for kind, name in CEILING_KINDS.items():
        wr = {0: 0, 1: n, 2: n, 3: n // 2, 4: n // 4}[kind]
        rd = 0 if kind == 1 else n
        best = None
        for depth in (4, 8, 16):
            for nt in (1, 0):
                for grid in grids:
                    def body():
                        cs = torch.cuda.current_stream().cuda_stream   # the capturing stream
                        for _ in range(2):
                            rc = lib.iqb_stream(kind, depth, nt, src.data_ptr(), dst.data_ptr(), n, grid, cs)
                            assert rc == 0, rc
                    t = summarize(time_graph(body, reps), 2, rd + wr)
                    sweep.append((name, depth, nt, grid, t["GBps"]))
                    if best is None or t["GBps"] > best["GBps"]:
                        best = {"GBps": t["GBps"], "frac_hbm": t["frac_hbm"], "depth": depth, "nontemporal": nt,
                                "grid": grid, "us": t["us"], "bytes": rd + wr}
        res[name] = best
        progress(f"ceiling {name}: {best['GBps']} GB/s")
    del src, dst
    torch.cuda.empty_cache()
    return res, sweep


# ---- the step: every format over the 2 GiB stream ------------------------------------
def headline(args, W):
    import torch
    step_bytes = sum(W.bytes(f, g)[0] for f, g in STREAM_FORMATS)

    def step():
        for f, g in STREAM_FORMATS:
            W.quant(f, g, 0)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    del graph
    return step_bytes, elapsed


def measure_workload(W, fmts, reps, ceil):
    """stats on / off quantize and dequantize timings of each format."""
    res = {}
    n = 2 * W.nsets if W.nsets > 1 else 2
    copy_gbs = ceil["copy"]["GBps"] if ceil else None
    for spec in fmts:
        fmt, gran, var = (*spec, "")[:3]
        qb, dq = W.bytes(fmt, gran)
        entry = {"bytes": qb}
        mix = ceil[CEILING_KINDS[mix_kind(fmt, W.in_elem)]]["GBps"] if ceil else None
        for stats in (True, False):
            def q():
                for k in range(n):
                    W.quant(fmt, gran, k % W.nsets, var, stats=stats)
            t = summarize(time_graph(q, reps), n, qb)
            if copy_gbs:
                t["frac_copy"] = round(t["GBps"] / copy_gbs, 4)
                t["frac_mix"] = round(t["GBps"] / mix, 4)
            if has_prepass(fmt, gran, var):
                moved = qb + W.rows * W.cols * W.in_elem
                t["moved_bytes"] = moved
                t["moved_GBps"] = round(moved / (t["us"] * 1e-6) / 1e9, 1)
                t["moved_frac_hbm"] = round(t["moved_GBps"] / HBM_PEAK_GBS, 4)
            entry["stats_on" if stats else "stats_off"] = t
        entry["stats_cost"] = round(entry["stats_on"]["us"] / entry["stats_off"]["us"] - 1, 4)

        def d():
            for k in range(n):
                W.dequant(fmt, gran, k % W.nsets, var)
        td = summarize(time_graph(d, max(5, reps // 3)), n, dq)
        entry["dequantize"] = {"us": td["us"], "GBps": td["GBps"], "bytes": dq}
        res[f"{W.name}:{fmt}/{gran}" + (f"/{var}" if var else "")] = entry
    return res


def breakdown(args, ceil):
    res = {}
    plan = [("c1", [("int8", "tensor"), ("e4m3", "tensor"), ("int8", "tensor", "static"),
                    ("e4m3", "tensor", "static")]),
            ("c2", [("e4m3", "row"), ("e5m2", "row")]),
            ("c3", [("mxfp4", "block"), ("mxfp4", "block", "mx-nearest"), ("mxfp4", "block", "mx-up")]),
            ("c4", [("nvfp4", "block"), ("nvfp4", "block", "nv-rne"), ("nvfp4", "block", "static")]),
            ("c5", [("int4", "block"), ("int4zp", "block")])]
    for name, fmts in plan:
        W = Workload(name, fmts)
        res.update(measure_workload(W, fmts, args.reps, ceil))
        W.release()
        progress(f"per-format {name} done")
    return res


# ---- counter summaries ---------------------------------------------------------------
def source_hash():
    h = hashlib.sha256()
    for p in ("int_quantization_amd/csrc/iq_kernels.hip", "int_quantization_amd/csrc/iq_launch.h"):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ---- CPU oracle baseline ---------------------------------------------------------------
def host_cpu():
    model, cores = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None and core is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    return {"model": model, "physical_cores": len(cores) or None, "logical_cpus": os.cpu_count(),
            "allowed_cpus": allowed}


def cpu_baseline(rows=512, min_seconds=10.0, min_seconds_1t=5.0):
    """The oracle (unchanged) on the first `rows` rows of the stream workload:
    the step's seven quantize calls (absmax, scale, cast, pack, x^ and
    statistics), repeated until `min_seconds` of CPU work have been timed,
    on the host share of one GPU (at most 16 threads), then on one thread."""
    from oracle import oracle as O
    from synth import synth
    info = host_cpu()
    threads = max(1, min(info["allowed_cpus"], 16))
    x = synth.make("stream", nrows=rows)
    step_bytes = sum(algo_bytes(f, g, rows, x.shape[1], 2)[0] for f, g in STREAM_FORMATS)

    def run(nthreads, min_s):
        reps = 0
        t0 = time.perf_counter()
        while True:
            for f, g in STREAM_FORMATS:
                O.quantize(x, f, g, want_xhat=False, threads=nthreads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                return reps, dt

    reps, dt = run(threads, min_seconds)
    reps1, dt1 = run(1, min_seconds_1t)
    return {"value": round(step_bytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "value_1thread": round(step_bytes * reps1 / dt1 / 1e9, 4),
            "host": info,
            "sample": f"{reps} x the whole step on rows 0-{rows - 1} of the stream workload (BF16 {rows}x16384, "
                      f"{rows * 16384 * 2 / 2**20:.0f} MiB): quantize with x^ and statistics to INT8 and E4M3 per "
                      f"tensor, E4M3 and E5M2 per row, MXFP4, NVFP4 and INT4 g128; rows split over {threads} "
                      f"threads; {dt:.1f} s.  One thread: {reps1} steps in {dt1:.1f} s"}


# ---- the dequantize-GEMM consumers ------------------------------------------------------
class GemmWorkload:
    """Puzzle 12's consumer on the c5 weights (28672 x 8192 as asymmetric
    INT4, quantized on the GPU) over NSETS copies, so that consecutive calls
    read weights the memory-side cache does not hold."""

    def __init__(self):
        import int_quantization_amd as iq
        from synth import synth
        w = to_device(synth.make("c5"))
        q = iq.quantize(w, "int4zp", "block", stats=False)
        del w
        self.q = [q] + [iq.Quantized(q.codes.clone(), q.scales.clone(), None, None, None, q.fmt, q.gran, q.rows,
                                     q.cols, q.shifts.clone()) for _ in range(NSETS - 1)]
        self.n0, self.K = q.rows, q.cols

    def inputs(self, n1):
        import torch
        from synth import synth
        x = to_device(synth.make("c2", nrows=n1))
        xs = [x] + [x.clone() for _ in range(NSETS - 1)]
        outs = [torch.empty((self.n0, n1), dtype=torch.float32, device="cuda") for _ in range(NSETS)]
        return xs, outs

    def call(self, i, xs, outs):
        import int_quantization_amd as iq
        iq.zp_gemm(self.q[i % NSETS], xs[i % NSETS], out=outs[i % NSETS])

    def bytes_flops(self, n1):
        n0, K = self.n0, self.K
        b = n0 * K // 2 + n0 * (K // 128) * 4 + n0 * (K // 256) + n1 * K * 2 + n0 * n1 * 4
        return b, 2.0 * n0 * K * n1


def gemm_entry(us, b, fl, peak_tfs, kernel):
    t_hbm = b / (HBM_PEAK_GBS * 1e3)            # microseconds at the HBM peak
    t_mfma = fl / (peak_tfs * 1e6)              # microseconds at the matrix-core peak
    return {"avg_us": round(us, 2), "GB/s": round(b / us / 1e3, 1), "TFLOP/s": round(fl / us / 1e6, 1),
            "bound": "hbm" if t_hbm >= t_mfma else "mfma", "frac": round(max(t_hbm, t_mfma) / us, 4),
            "bytes": b, "flops": fl, "kernel": kernel}


def gemm_breakdown(args):
    """iq_zp_gemm per token count against both bounds (HBM bytes, BF16 MFMA
    flops) and the fraction of the larger one reached."""
    import torch
    G = GemmWorkload()
    res = {"weights": f"c5 {G.n0}x{G.K} asymmetric INT4 (group 128), {NSETS} copies", "x": "BF16 [n1, K]"}
    n = 2 * NSETS
    for n1 in GEMM_TOKENS:
        xs, outs = G.inputs(n1)

        def body():
            for k in range(n):
                G.call(k, xs, outs)

        us = summarize(time_graph(body, args.reps), n, 1)["mean_us"]
        b, fl = G.bytes_flops(n1)
        res[f"n1={n1}"] = gemm_entry(us, b, fl, MFMA_BF16_PEAK_TFS, "k_zp_gemv" if n1 <= 32 else "k_zp_gemm")
        del xs, outs
    del G
    torch.cuda.empty_cache()
    return res


class MxGemmWorkload:
    """The c3 weights (14336 x 4096) as MXFP4 over NSETS copies."""

    def __init__(self):
        import int_quantization_amd as iq
        from synth import synth
        w = to_device(synth.make("c3"))
        q = iq.quantize(w, "mxfp4", "block", stats=False)
        del w
        self.q = [q] + [iq.Quantized(q.codes.clone(), q.scales.clone(), None, None, None, q.fmt, q.gran, q.rows,
                                     q.cols) for _ in range(NSETS - 1)]
        self.n0, self.K = q.rows, q.cols


def mx_gemm_breakdown(args):
    """iq_mx_gemm (MXFP4 x MXFP4) and iq_mxw_gemm (MXFP4 x BF16) per token
    count against both bounds."""
    import torch
    import int_quantization_amd as iq
    from synth import synth
    G = MxGemmWorkload()
    mx = {"weights": f"c3 {G.n0}x{G.K} MXFP4, {NSETS} copies", "activations": "a3 BF16 [n1, 4096] -> MXFP4"}
    mxw = {"weights": f"c3 {G.n0}x{G.K} MXFP4, {NSETS} copies", "activations": "a3 BF16 [n1, 4096]"}
    n = 2 * NSETS
    for n1 in MX_GEMM_TOKENS:
        x = to_device(synth.make("a3", nrows=n1))
        qa = iq.quantize(x, "mxfp4", "block", stats=False)
        outs = [torch.empty((G.n0, n1), dtype=torch.float32, device="cuda") for _ in range(NSETS)]

        def body():
            for k in range(n):
                iq.mx_gemm(G.q[k % NSETS], qa, out=outs[k % NSETS])

        def bodyw():
            for k in range(n):
                iq.mxw_gemm(G.q[k % NSETS], x, out=outs[k % NSETS])

        us = summarize(time_graph(body, args.reps), n, 1)["mean_us"]
        b = (G.n0 + n1) * (G.K // 2 + G.K // 32) + G.n0 * n1 * 4
        fl = 2.0 * G.n0 * G.K * n1
        # LDS-DMA 256 x 256 tiles from 1024 tokens (the c3 weights give 224 or more)
        kname = "k_mx_gemv" if n1 <= 64 else "k_mx_gemm_dma" if n1 >= 1024 else "k_mx_gemm"
        mx[f"n1={n1}"] = gemm_entry(us, b, fl, MFMA_FP4_PEAK_TFS, kname)
        us = summarize(time_graph(bodyw, args.reps), n, 1)["mean_us"]
        b = G.n0 * (G.K // 2 + G.K // 32) + n1 * G.K * 2 + G.n0 * n1 * 4
        # 256 x 256 tiles once the c3 weights' 112 rows of 128 x 256 tiles need
        # more than one round of the 256 CUs' resident workgroups (n1 > 512)
        kname = "k_mxw_gemv" if n1 <= 64 else "k_mxw_gemm_wide" if n1 > 512 else "k_mxw_gemm"
        mxw[f"n1={n1}"] = gemm_entry(us, b, fl, MFMA_BF16_PEAK_TFS, kname)
        del x, qa, outs
    del G
    torch.cuda.empty_cache()
    return mx, mxw


# ---- profiling aid ------------------------------------------------------------------------
def only(args):
    """Loop one call type (for rocprofv3 runs)."""
    import torch
    if args.only == "ceiling":
        res, _ = ceiling(reps=3)
        print(json.dumps({"ceiling": res}), flush=True)
        return
    if args.only == "copy":
        # the calibration kernel of the HBM counters: a 1 GiB copy (reads 1 GiB, writes 1 GiB)
        lib = ctypes.CDLL(os.path.join(ROOT, "int_quantization_amd", "libiq_bench.so"))
        lib.iqb_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
        n = 1 << 30
        src = torch.empty(n // 4, dtype=torch.float32, device="cuda:0").normal_()
        dst = torch.empty(n // 4, dtype=torch.float32, device="cuda:0")
        cs = torch.cuda.current_stream().cuda_stream
        for _ in range(args.warmup + args.steps):
            assert lib.iqb_stream(2, 4, 1, src.data_ptr(), dst.data_ptr(), n, 4096, cs) == 0
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read": n, "bytes_written": n, "calls": args.warmup + args.steps}),
              flush=True)
        return
    if args.only.startswith(("zp_gemm:", "mx_gemm:", "mxw_gemm:")):
        import int_quantization_amd as iq
        from synth import synth
        kind, n1 = args.only.split(":")
        n1 = int(n1)
        if kind == "zp_gemm":
            G = GemmWorkload()
            xs, outs = G.inputs(n1)
            for s in range(args.warmup + args.steps):
                G.call(s, xs, outs)
        else:
            G = MxGemmWorkload()
            x = to_device(synth.make("a3", nrows=n1))
            qa = iq.quantize(x, "mxfp4", "block", stats=False)
            outs = [torch.empty((G.n0, n1), dtype=torch.float32, device="cuda") for _ in range(NSETS)]
            for s in range(args.warmup + args.steps):
                if kind == "mx_gemm":
                    iq.mx_gemm(G.q[s % NSETS], qa, out=outs[s % NSETS])
                else:
                    iq.mxw_gemm(G.q[s % NSETS], x, out=outs[s % NSETS])
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "calls": args.warmup + args.steps}), flush=True)
        return
    name, fmt, gran, *rest = args.only.split(":")
    stats = "nostats" not in rest
    rest = [r for r in rest if r != "nostats"]
    var = rest[0] if rest else ""
    W = Workload(name, [(fmt, gran, var)], nsets=1 if name == "stream" else NSETS)
    # the calls are replayed from a graph, as the per-format timings replay them
    n = 2 * W.nsets if W.nsets > 1 else 2

    def q():
        for k in range(n):
            W.quant(fmt, gran, k % W.nsets, var, stats=stats)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q()
    for _ in range(args.warmup + args.steps):
        g.replay()
    torch.cuda.synchronize()
    print(json.dumps({"only": args.only, "calls": n * (args.warmup + args.steps)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (one MI355X per run)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    import int_quantization_amd as iq
    iq.load_library()
    if args.only:
        return only(args)

    ceil = None
    if not args.no_breakdown:
        ceil, _ = ceiling()

    # ---- the step ---------------------------------------------------------------------
    W = Workload("stream", STREAM_FORMATS, nsets=1)
    progress("stream workload on the device")
    step_bytes, elapsed = headline(args, W)
    value = step_bytes * args.steps / elapsed / 1e9
    progress(f"step: {value:.1f} GB/s, {elapsed / args.steps * 1e3:.3f} ms")
    per_format = measure_workload(W, STREAM_FORMATS, max(5, args.reps // 3), ceil)
    W.release()
    progress("per-format stream done")

    rk = f"stream:{ROOFLINE_CALL[0]}/{ROOFLINE_CALL[1]}"
    r = per_format[rk]["stats_on"]
    roofline = {"bound": "hbm", "achieved": r["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(r["GBps"] / HBM_PEAK_GBS, 4), "traffic": read_traffic("stream_e4m3_row"),
                "kernel": "iq_quantize E4M3 per row with statistics on the stream: one launch of "
                          "k_quant_row<BF16, E4M3, 4 chunks per lane, 512 threads, full rows, statistics> "
                          "(the statistics fold runs inside it)",
                "bytes_per_launch": per_format[rk]["bytes"], "avg_launch_us": r["us"],
                "timing": "HIP events on the launch stream around replays of a graph of 2 calls, after "
                          "about 40 ms of untimed replays; median"}

    extra = {}
    if ceil:
        extra["ceiling"] = ceil
    if not args.no_breakdown:
        per_format.update(breakdown(args, ceil))
        if not args.no_gemm:
            extra["zp_gemm"] = gemm_breakdown(args)
            extra["mx_gemm"], extra["mxw_gemm"] = mx_gemm_breakdown(args)
            progress("GEMMs done")
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    progress("cpu baseline done")

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "stream: BF16 65536x16384 (2 GiB), N(0,1) with 0.5% outlier channels x200, seed 6; "
                               "quantize (+ fused dequant + error statistics) to INT8 and E4M3 per tensor, E4M3 "
                               "and E5M2 per row, MXFP4, NVFP4 and INT4 g128",
                   "rows": 65536, "cols": 16384, "input": "bf16",
                   "formats": [f"{f}/{g}" for f, g in STREAM_FORMATS], "step_bytes": step_bytes,
                   "launch": "hip graph per step"},
        "frac_hbm": round(value / HBM_PEAK_GBS, 4),
        "roofline": roofline, "cpu_baseline": cpu, **extra, "per_format": per_format,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
