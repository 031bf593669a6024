#!/usr/bin/env python3
"""Throughput of the quantization hot path on one MI355X.

A step is one pass of the whole path over the activation workload
(BF16 8192 x 8192, N(0,1) with 0.5 % outlier channels x200): per-row
E4M3 quantize (absmax, scale, saturating RNE cast, pack, fused dequant and
error statistics), the standalone dequantize of those codes to BF16, and
the same two calls for E5M2.  `value` is the algorithmic bytes of the step
(every input read once plus every output written once) divided by the
timed wall time, inputs already resident in HBM.

Buffers rotate over 4 sets so that no call reads data the previous calls
touched within the last ~400 MB of traffic (the 256 MB memory-side cache
cannot serve the timed reads).

Also reported: the dominant kernel's HBM roofline, a per-format breakdown
over the other workloads, Puzzle 12's dequantize-then-dot consumer over
asymmetric INT4 weights at several token counts (against both the HBM and
the BF16 matrix-core bound), the FP4 GEMM over two MXFP4 operands on the
block-scaled matrix cores, MXFP4 weights against BF16 activations, a
hand-written 16-byte copy kernel as the
practical ceiling, and the CPU oracle timed on the host on a bounded sample.
"""
import argparse
import ctypes
import hashlib
import json
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
METRIC = "quantize GB/s (bytes in+out) and % of MI355X HBM peak, per format"
NSETS = 4


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-format workloads")
    ap.add_argument("--stream", action="store_true", help="add the 2 GiB streaming pass to the breakdown")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="profiling aid: run one call type in a loop (e.g. c2:e4m3:row, c5:int4:block, "
                         "c4:nvfp4:block:static, copy, zp_gemm:16, mx_gemm:2048, mxw_gemm:2048)")
    ap.add_argument("--reps", type=int, default=20, help="timed repetitions per breakdown entry")
    ap.add_argument("--eager", action="store_true", help="launch every call from Python instead of graphs")
    return ap.parse_args()


def to_device(x_np):
    """numpy float32 / uint16 (BF16 bits) -> device tensor."""
    import numpy as np
    import torch
    if x_np.dtype == np.uint16:
        return torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(x_np).to("cuda:0")


def algo_bytes(fmt, gran, rows, cols, in_elem):
    """Bytes the method itself must move: x once, codes + scales once."""
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


def timed(fn, reps, stream):
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return {"median_us": 1e3 * ms[len(ms) // 2], "p10_us": 1e3 * ms[len(ms) // 10],
            "p90_us": 1e3 * ms[(9 * len(ms)) // 10], "mean_us": 1e3 * sum(ms) / len(ms)}


# Call variants of the breakdown: rule flags, or static scaling with an
# absmax computed once beforehand (the calibrated mode).
VARIANTS = {"": {}, "mx-nearest": {"flags": 1}, "mx-up": {"flags": 2}, "nv-rne": {"flags": 4}, "static": None}


class Workload:
    """NSETS device copies of one synthetic input plus outputs per format
    (entries (fmt, gran) or (fmt, gran, variant))."""

    def __init__(self, name, formats, x_np=None):
        import torch

        from synth import synth
        self.name = name
        self.w = synth.WORKLOADS[name]
        x_np = synth.make(name) if x_np is None else x_np
        x0 = to_device(x_np)
        self.xs = [x0] + [x0.clone() for _ in range(NSETS - 1)]
        self.rows, self.cols = x_np.shape
        self.in_elem = 2 if x_np.dtype.itemsize == 2 else 4
        self.formats = formats
        import int_quantization_amd as iq
        self.iq = iq
        self.ws = [iq.workspace_for(iq.desc_for(x0, *formats[0][:2]), x0.device) for _ in range(NSETS)]
        self.amax = [iq.amax(x) for x in self.xs] if any(len(f) > 2 and f[2] == "static" for f in formats) else None
        self.q = {}
        for spec in formats:
            fmt, gran, var = (*spec, "")[:3]
            self.q[(fmt, gran, var)] = [iq.quantize(x, fmt, gran, stats=True, workspace=w, **self._kw(var, i))
                                        for i, (x, w) in enumerate(zip(self.xs, self.ws))]
        out_dt = torch.bfloat16 if self.in_elem == 2 else torch.float32
        self.out = [torch.empty((self.rows, self.cols), dtype=out_dt, device=x0.device) for _ in range(NSETS)]
        torch.cuda.synchronize()

    def _kw(self, var, i):
        return {"static_amax": self.amax[i]} if var == "static" else dict(VARIANTS[var])

    def quant(self, fmt, gran, i, var=""):
        self.iq.quantize(self.xs[i], fmt, gran, workspace=self.ws[i], out=self.q[(fmt, gran, var)][i],
                         **self._kw(var, i))

    def dequant(self, fmt, gran, i, j, var=""):
        self.iq.dequantize(self.q[(fmt, gran, var)][j], out=self.out[i])

    def bytes(self, fmt, gran):
        qb, code_b = algo_bytes(fmt, gran, self.rows, self.cols, self.in_elem)
        dq = code_b + self.rows * self.cols * self.in_elem
        return qb, dq


def copy_ceiling(reps=20):
    """GB/s (read + write) of the 16-byte copy kernel over 1 GiB."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "int_quantization_amd", "libiq_bench.so"))
    lib.iqb_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
    n = 1 << 30
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = [torch.empty(n // 4, dtype=torch.float32, device="cuda:0") for _ in range(2)]
    s = torch.cuda.current_stream()
    best = None
    for grid in (1024, 2048, 4096, 8192):
        k = [0]

        def run():
            rc = lib.iqb_copy(src.data_ptr(), dst[k[0] & 1].data_ptr(), n, grid, s.cuda_stream)
            k[0] += 1
            assert rc == 0

        run()
        t = timed(run, reps, s)
        gbs = 2 * n / (t["median_us"] * 1e-6) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "grid": grid, "median_us": round(t["median_us"], 2)}
    return best


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


def cpu_baseline(rows=8192, min_seconds=10.0):
    """The oracle (unchanged) on the activation workload: the same two
    formats' quantize + dequantize as one GPU step, repeated until at least
    `min_seconds` of CPU work have been timed."""
    import numpy as np

    from oracle import oracle as O
    from synth import synth
    threads = max(1, min(os.cpu_count() or 1, 16))   # the host share of one GPU
    x = synth.make("c2", nrows=rows)
    total, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        for fmt in ("e4m3", "e5m2"):
            r = O.quantize(x, fmt, "row", threads=threads)
            O.dequantize(r["codes"], r["scales"], fmt, "row", rows, x.shape[1], None, O.BF16)
            qb, code_b = algo_bytes(fmt, "row", rows, x.shape[1], 2)
            total += qb + code_b + x.size * 2
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(total / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x the whole activation step ({rows} of 8192 rows, BF16 {rows}x8192): per-row E4M3 "
                      f"and E5M2 quantize with x^ and statistics, then dequantize to BF16; quantize rows split "
                      f"over {threads} threads, dequantize serial; {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build runs on one MI355X)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    import int_quantization_amd as iq
    iq.load_library()
    stream = torch.cuda.current_stream()

    if args.only:
        return only(args)

    # ---- the step: activation workload, E4M3 and E5M2 per row ---------------------
    fmts = [("e4m3", "row"), ("e5m2", "row")]
    W = Workload("c2", fmts)
    step_bytes = 0
    for f in fmts:
        qb, dq = W.bytes(*f)
        step_bytes += qb + dq

    def step(i):
        j = (i - 1) % NSETS
        for f in fmts:
            W.quant(*f, i)
            W.dequant(*f, i, j)

    for s in range(NSETS):   # eager warm-up: also fills the launch caches before capture
        step(s)
    torch.cuda.synchronize()
    graphs = None
    if not args.eager:
        # One graph per buffer set (4 library calls, 6 kernels each); replaying
        # them removes host launch overhead from the timed region.
        graphs = []
        for i in range(NSETS):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        torch.cuda.synchronize()

    def run_step(k):
        if graphs is None:
            step(k % NSETS)
        else:
            graphs[k % NSETS].replay()

    for k in range(args.warmup):
        run_step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.warmup, args.warmup + args.steps):
        run_step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    value = step_bytes * args.steps / elapsed / 1e9

    # ---- per-call durations: graphs of 2*NSETS consecutive calls of one kind -------
    calls = {}
    per_call_graph = 2 * NSETS
    for a, b in fmts:
        for kind in ("quantize", "dequantize"):
            def body():
                for n in range(per_call_graph):
                    if kind == "quantize":
                        W.quant(a, b, n % NSETS)
                    else:
                        W.dequant(a, b, n % NSETS, (n + 1) % NSETS)
            if graphs is None:
                t = timed(body, 10, stream)
            else:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    body()
                g.replay()
                t = timed(g.replay, 10, stream)
            us = t["mean_us"] / per_call_graph
            q, d = W.bytes(a, b)
            calls[f"{a}/{b}/{kind}"] = {"avg_us": round(us, 2),
                                        "GB/s": round((q if kind == "quantize" else d) / (us * 1e-6) / 1e9, 1)}
    qb, _ = W.bytes("e4m3", "row")
    dom_us = calls["e4m3/row/quantize"]["avg_us"]
    achieved = qb / (dom_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic("c2_e4m3_row"),
                "kernel": "iq_quantize E4M3 per-row (k_quant_row + k_stats_finalize)",
                "bytes_per_launch": qb, "avg_launch_us": dom_us,
                "timing": "HIP events around a replayed graph of %d consecutive calls" % per_call_graph}
    del graphs, W
    torch.cuda.empty_cache()

    extra = {"calls": calls}
    if not args.no_breakdown:
        extra["copy_ceiling"] = copy_ceiling()
        extra["per_format"] = breakdown(args)
        extra["zp_gemm"] = gemm_breakdown(args)
        extra["mx_gemm"] = mx_gemm_breakdown(args)
        extra["mxw_gemm"] = mxw_gemm_breakdown(args)
    cpu = None if args.no_cpu_baseline else cpu_baseline()

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "activations BF16 8192x8192, N(0,1) with 0.5% outlier channels x200, seed 2; "
                               "per-row E4M3 and E5M2: quantize (+fused dequant + error stats) and dequantize "
                               "to BF16", "rows": 8192, "cols": 8192, "input": "bf16",
                   "formats": ["e4m3/row", "e5m2/row"], "step_bytes": step_bytes, "buffer_sets": NSETS,
                   "launch": "eager" if args.eager else "hip graph per step"},
        "roofline": roofline, "cpu_baseline": cpu, **extra,
    }
    print(json.dumps(line), flush=True)


def time_calls(body, n_calls, use_graph, reps, stream):
    """Mean microseconds per call of `body` (which issues n_calls calls),
    from HIP events around graph replays (or eager calls)."""
    import torch
    if not use_graph:
        t = timed(body, reps, stream)
        return t["mean_us"] / n_calls, t
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    t = timed(g.replay, reps, stream)
    del g
    return t["mean_us"] / n_calls, t


def breakdown(args):
    import torch
    res = {}
    plan = [("c1", [("int8", "tensor"), ("e4m3", "tensor"), ("int8", "tensor", "static"),
                    ("e4m3", "tensor", "static")]),
            ("c2", [("e4m3", "row"), ("e5m2", "row")]),
            ("c3", [("mxfp4", "block"), ("mxfp4", "block", "mx-nearest"), ("mxfp4", "block", "mx-up")]),
            ("c4", [("nvfp4", "block"), ("nvfp4", "block", "nv-rne"), ("nvfp4", "block", "static")]),
            ("c5", [("int4", "block"), ("int4zp", "block")])]
    if args.stream:
        from synth import synth
        plan.append(("stream", list(synth.WORKLOADS["stream"].formats)))
    stream = torch.cuda.current_stream()
    n = 2 * NSETS
    for name, fmts in plan:
        W = Workload(name, fmts)
        for spec in fmts:
            fmt, gran, var = (*spec, "")[:3]

            def q():
                for k in range(n):
                    W.quant(fmt, gran, k % NSETS, var)

            def d():
                for k in range(n):
                    W.dequant(fmt, gran, k % NSETS, (k + 1) % NSETS, var)

            q()
            torch.cuda.synchronize()
            uq, _ = time_calls(q, n, not args.eager, args.reps, stream)
            ud, _ = time_calls(d, n, not args.eager, args.reps, stream)
            qb, dq = W.bytes(fmt, gran)
            gq = qb / (uq * 1e-6) / 1e9
            gd = dq / (ud * 1e-6) / 1e9
            res[f"{name}:{fmt}/{gran}" + (f"/{var}" if var else "")] = {
                "quantize_GBps": round(gq, 1), "quantize_frac_hbm": round(gq / HBM_PEAK_GBS, 4),
                "quantize_us": round(uq, 2), "dequantize_GBps": round(gd, 1), "dequantize_us": round(ud, 2),
                "quantize_bytes": qb, "dequantize_bytes": dq}
        del W
        torch.cuda.empty_cache()
    return res


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


def gemm_breakdown(args):
    """Time iq_zp_gemm per token count; each entry gives both bounds (HBM
    bytes, BF16 MFMA flops) and the fraction of the larger one reached."""
    import torch
    stream = torch.cuda.current_stream()
    G = GemmWorkload()
    res = {"weights": f"c5 {G.n0}x{G.K} asymmetric INT4 (group 128), {NSETS} copies", "x": "BF16 [n1, K]"}
    n = 2 * NSETS
    for n1 in GEMM_TOKENS:
        xs, outs = G.inputs(n1)

        def body():
            for k in range(n):
                G.call(k, xs, outs)

        body()
        torch.cuda.synchronize()
        us, _ = time_calls(body, n, not args.eager, args.reps, stream)
        b, fl = G.bytes_flops(n1)
        t_hbm = b / (HBM_PEAK_GBS * 1e3)            # microseconds at the HBM peak
        t_mfma = fl / (MFMA_BF16_PEAK_TFS * 1e6)     # microseconds at the MFMA peak
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
        res[f"n1={n1}"] = {"avg_us": round(us, 2), "GB/s": round(b / us / 1e3, 1),
                           "TFLOP/s": round(fl / us / 1e6, 1), "bound": bound,
                           "frac": round(max(t_hbm, t_mfma) / us, 4), "bytes": b, "flops": fl,
                           "kernel": "k_zp_gemv" if n1 <= 32 else "k_zp_gemm"}
        del xs, outs
    del G
    torch.cuda.empty_cache()
    return res


class MxGemmWorkload:
    """FP4 GEMM over two MXFP4 operands: the c3 weights (14336 x 4096,
    quantized on the GPU) over NSETS copies, and the a3 activations quantized
    on the GPU."""

    def __init__(self):
        import int_quantization_amd as iq
        from synth import synth
        w = to_device(synth.make("c3"))
        q = iq.quantize(w, "mxfp4", "block", stats=False)
        del w
        self.q = [q] + [iq.Quantized(q.codes.clone(), q.scales.clone(), None, None, None, q.fmt, q.gran, q.rows,
                                     q.cols) for _ in range(NSETS - 1)]
        self.n0, self.K = q.rows, q.cols

    def inputs(self, n1):
        import torch
        import int_quantization_amd as iq
        from synth import synth
        x = to_device(synth.make("a3", nrows=n1))
        qa = iq.quantize(x, "mxfp4", "block", stats=False)
        outs = [torch.empty((self.n0, n1), dtype=torch.float32, device="cuda") for _ in range(NSETS)]
        return x, qa, outs

    def call(self, i, qa, outs):
        import int_quantization_amd as iq
        iq.mx_gemm(self.q[i % NSETS], qa, out=outs[i % NSETS])

    def bytes_flops(self, n1):
        n0, K = self.n0, self.K
        b = (n0 + n1) * (K // 2 + K // 32) + n0 * n1 * 4
        return b, 2.0 * n0 * K * n1


def mx_gemm_breakdown(args):
    """Time iq_mx_gemm per token count against both bounds (HBM bytes, FP4
    matrix-core flops), and the MXFP4 quantize of those activations."""
    import torch
    import int_quantization_amd as iq
    stream = torch.cuda.current_stream()
    G = MxGemmWorkload()
    res = {"weights": f"c3 {G.n0}x{G.K} MXFP4, {NSETS} copies", "activations": "a3 BF16 [n1, 4096] -> MXFP4"}
    n = 2 * NSETS
    for n1 in MX_GEMM_TOKENS:
        x, qa, outs = G.inputs(n1)

        def body():
            for k in range(n):
                G.call(k, qa, outs)

        def quant():
            for k in range(n):
                iq.quantize(x, "mxfp4", "block", stats=False, out=qa)

        body()
        torch.cuda.synchronize()
        us, _ = time_calls(body, n, not args.eager, args.reps, stream)
        uq, _ = time_calls(quant, n, not args.eager, args.reps, stream)
        b, fl = G.bytes_flops(n1)
        t_hbm = b / (HBM_PEAK_GBS * 1e3)
        t_mfma = fl / (MFMA_FP4_PEAK_TFS * 1e6)
        res[f"n1={n1}"] = {"avg_us": round(us, 2), "GB/s": round(b / us / 1e3, 1),
                           "TFLOP/s": round(fl / us / 1e6, 1), "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                           "frac": round(max(t_hbm, t_mfma) / us, 4), "bytes": b, "flops": fl,
                           "activation_quantize_us": round(uq, 2),
                           "kernel": "k_mx_gemv" if n1 <= 64 else "k_mx_gemm"}
        del x, qa, outs
    del G
    torch.cuda.empty_cache()
    return res


def mxw_gemm_breakdown(args):
    """Time iq_mxw_gemm (the c3 weights as MXFP4 over NSETS copies against a3
    activations kept in BF16) per token count against both bounds (HBM
    bytes, BF16 matrix-core flops)."""
    import torch
    import int_quantization_amd as iq
    from synth import synth
    stream = torch.cuda.current_stream()
    G = MxGemmWorkload()
    res = {"weights": f"c3 {G.n0}x{G.K} MXFP4, {NSETS} copies", "activations": "a3 BF16 [n1, 4096]"}
    n = 2 * NSETS
    for n1 in MX_GEMM_TOKENS:
        x = to_device(synth.make("a3", nrows=n1))
        outs = [torch.empty((G.n0, n1), dtype=torch.float32, device="cuda") for _ in range(NSETS)]

        def body():
            for k in range(n):
                iq.mxw_gemm(G.q[k % NSETS], x, out=outs[k % NSETS])

        body()
        torch.cuda.synchronize()
        us, _ = time_calls(body, n, not args.eager, args.reps, stream)
        b = G.n0 * (G.K // 2 + G.K // 32) + n1 * G.K * 2 + G.n0 * n1 * 4
        fl = 2.0 * G.n0 * G.K * n1
        t_hbm = b / (HBM_PEAK_GBS * 1e3)
        t_mfma = fl / (MFMA_BF16_PEAK_TFS * 1e6)
        res[f"n1={n1}"] = {"avg_us": round(us, 2), "GB/s": round(b / us / 1e3, 1),
                           "TFLOP/s": round(fl / us / 1e6, 1), "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                           "frac": round(max(t_hbm, t_mfma) / us, 4), "bytes": b, "flops": fl,
                           "kernel": "k_mxw_gemv" if n1 <= 64 else "k_mxw_gemm"}
        del x, outs
    del G
    torch.cuda.empty_cache()
    return res


def only(args):
    """Loop one call type (for rocprofv3 runs)."""
    import torch
    stream = torch.cuda.current_stream()
    if args.only == "copy":
        print(json.dumps({"copy_ceiling": copy_ceiling(args.reps)}), flush=True)
        return
    if args.only.startswith("mxw_gemm:"):
        import int_quantization_amd as iq
        from synth import synth
        n1 = int(args.only.split(":")[1])
        G = MxGemmWorkload()
        x = to_device(synth.make("a3", nrows=n1))
        outs = [torch.empty((G.n0, n1), dtype=torch.float32, device="cuda") for _ in range(NSETS)]
        for s in range(args.warmup + args.steps):
            iq.mxw_gemm(G.q[s % NSETS], x, out=outs[s % NSETS])
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "calls": args.warmup + args.steps}), flush=True)
        return
    if args.only.startswith("mx_gemm:"):
        n1 = int(args.only.split(":")[1])
        G = MxGemmWorkload()
        _, qa, outs = G.inputs(n1)
        for s in range(args.warmup + args.steps):
            G.call(s, qa, outs)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "calls": args.warmup + args.steps}), flush=True)
        return
    if args.only.startswith("zp_gemm:"):
        n1 = int(args.only.split(":")[1])
        G = GemmWorkload()
        xs, outs = G.inputs(n1)
        for s in range(args.warmup + args.steps):
            G.call(s, xs, outs)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "calls": args.warmup + args.steps}), flush=True)
        return
    name, fmt, gran, *rest = args.only.split(":")
    var = rest[0] if rest else ""
    W = Workload(name, [(fmt, gran, var)])
    for s in range(args.warmup + args.steps):
        W.quant(fmt, gran, s % NSETS, var)
    for s in range(args.steps):
        W.dequant(fmt, gran, s % NSETS, (s + 1) % NSETS, var)
    torch.cuda.synchronize()
    print(json.dumps({"only": args.only, "calls": args.warmup + args.steps}), flush=True)


if __name__ == "__main__":
    main()
