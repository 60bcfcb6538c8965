#!/usr/bin/env python3
"""Benchmark of the block-quantized matmul hot path on one MI355X.

One step runs every hot-path call once, each on synthetic Llama-shaped layer
inputs already resident in HBM:
  * Q4_0 decode GEMV, 1024 x 1024, batch 1 (the small configuration);
  * Q4_0 decode GEMV, K = 4096, N = 4096 / 11008 / 12288 (7B layer shapes,
    12288 = fused QKV), batch 1 and 4;
  * Q4_K decode GEMV, K = 8192, N = 28672 (70B FFN), batch 1 and 8;
  * Q8_0 x fp16 prefill GEMM, M = 512 tokens, N = 14336, K = 4096;
  * dense fp32 GEMM, M = N = K = 2048.
Weights rotate over enough device copies (>= 512 MiB per weight set, twice the
256 MB Infinity Cache) that every launch reads them from HBM, not from cache.

Reported (one JSON line on stdout):
  value          quantized-GEMV effective HBM bandwidth: algorithmic bytes of
                 the step's GEMV launches / the GEMV share of the timed steps
                 (GB/s); every share is timed with HIP events on the launch
                 stream around HIP-graph segments of the step;
  roofline       the dominant GEMV kernel (the GEMV case with the longest
                 launch) against the 8 TB/s HBM peak, timed the same way
                 inside the steps; traffic from the committed rocprofv3
                 counter summary;
  rooflines      the same figures for every case (GEMVs against HBM, GEMMs
                 against their matrix-core peaks);
  prefill_gemm   Q8_0 x fp16 GEMM TFLOP/s against the 2.5 PFLOP/s f16 peak;
  fp32_gemm      fp32 GEMM TFLOP/s against the 157.3 TFLOP/s fp32 peak;
  cases          every call timed alone: kernel time, GB/s or TFLOP/s;
  context        measured after the timed steps, for reading the figures
                 above: a plain streaming-read kernel over the Q4_K weight
                 copies (the HBM rate a simple kernel reaches here), every
                 GEMV on one weight copy back to back (cache-resident, not
                 HBM), the host wall time per call of the smallest GEMVs
                 called one by one (launch overhead included), and the
                 vendor library's GEMMs at the same shapes (torch.matmul on
                 hipBLASLt: fp16 with dense fp16 weights, and fp32);
  cpu_baseline   the fp64 CPU oracle on the same GEMV inputs (host cores),
                 with a shorter one-thread sample and the host CPU model.

Algorithmic bytes count the packed weights, the activations and the outputs,
each moved once; flops are 2*M*N*K.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
F16_PEAK_TFLOPS = 2500.0       # dense fp16 MFMA
F32_PEAK_TFLOPS = 157.3        # fp32 matrix
ROTATE_BYTES = 512 * 2**20     # per weight set: 2x the MALL
METRIC = "quantized GEMV effective HBM GB/s (% of peak); prefill GEMM TFLOP/s (% MFMA)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_cases.json")
CSRC = os.path.join(ROOT, "block_quantized_matmul_amd", "csrc")
PROBE_LIB = os.path.join(ROOT, "block_quantized_matmul_amd", "liblqmm_probe.so")


def kernel_source_sha256():
    """Hash over every library source file: a counter summary taken on other
    sources no longer describes the kernels."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")) and name != "probe.hip":
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # The GPU raises its clocks over the first tens of milliseconds of
    # sustained work; 100 untimed steps (about 40 ms) reach the steady state
    # that a serving loop runs in.
    p.add_argument("--warmup", type=int, default=100)
    # Before the warmup steps, the steps are replayed untimed for at least
    # this long, so that short warmups (a few steps, well under a
    # millisecond) also start the timed steps at steady clocks.
    p.add_argument("--settle-ms", type=float, default=300.0)
    p.add_argument("--no-context", action="store_true",
                   help="skip the context figures (counter runs)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    p.add_argument("--cases", default="", help="comma-separated subset of case names")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="wall time of the CPU-oracle baseline sample (whole passes)")
    p.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "BENCH_LOG", "OUT_MD", "COMMAND"),
                   help="host only: write a markdown summary of a rocprofv3 kernel trace of "
                        "this benchmark (timed launches per case apart from the others)")
    p.add_argument("--summarize-series", nargs=4,
                   metavar=("TRACE_DIR", "BENCH_LOG", "OUT_MD", "COMMAND"),
                   help="write a markdown summary of the timed launches' durations in order")
    p.add_argument("--summarize-traffic", nargs=3, metavar=("PMC_DIR", "CALIB_MIB", "COMMAND"),
                   help="host only: write the GEMV cases' HBM traffic summary from rocprofv3 "
                        "--pmc runs under PMC_DIR/<case>.fetch and PMC_DIR/<case>.write")
    p.add_argument("--summarize-counters", nargs=3, metavar=("PMC_DIR", "OUT_MD", "COMMAND"),
                   help="host only: write a markdown summary of rocprofv3 --kernel-trace --pmc "
                        "passes over the GEMM cases (PMC_DIR/pass<n>/)")
    p.add_argument("--eager", action="store_true",
                   help="launch from Python one call at a time instead of replaying HIP graphs")
    return p.parse_args()


class Rot:
    """Device copies of one weight set, handed out round robin so that two
    consecutive launches never read the same copy (even when two cases share
    the set)."""

    def __init__(self, copies):
        self.copies, self.i = copies, 0

    def next(self):
        t = self.copies[self.i % len(self.copies)]
        self.i += 1
        return t


class Case:
    def __init__(self, name, kind, bytes_, flops, launch, nrot, make_out, launch_warm=None,
                 section="step"):
        self.name, self.kind = name, kind
        self.section = section  # "step": the hot path; "next": further format x phase pairs
        self.bytes, self.flops = bytes_, flops
        self.launch = launch          # launch(): one call on the next weight copy
        self.launch_warm = launch_warm  # one call on the same weight copy every time
        self.nrot = nrot
        self.make_out = make_out      # host array of the last output
        self.avg_ms = None


def build_cases(torch, only):
    import numpy as np

    import block_quantized_matmul_amd as bq
    import synth

    dev = torch.device("cuda:0")
    cases = []
    inputs = {}  # for the CPU-baseline / parity leg
    stream_sets = {}  # weight copies the streaming-read probe reads

    def rot(nbytes):
        return max(2, math.ceil(ROTATE_BYTES / nbytes))

    def copies(arr, n):
        t = torch.from_numpy(np.ascontiguousarray(arr).reshape(-1)).to(dev)
        return [t] + [t.clone() for _ in range(n - 1)]

    def rotset(arr, n):
        return Rot(copies(arr, n))

    want = lambda n: not only or n in only

    # Q4_0 decode GEMV, the small configuration (1024 x 1024, batch 1)
    name = "q4_0_gemv_1024x1024_b1"
    if want(name):
        c0 = synth.make("q4_0_gemv_1024")
        wbytes = c0.W.nbytes
        R = rot(wbytes)
        Ws = rotset(c0.W, R)
        x = torch.from_numpy(c0.x.copy()).to(dev)
        y = torch.empty((1, c0.N), dtype=torch.float32, device=dev)
        alg = wbytes + c0.K * 4 + c0.N * 4

        def launch(Ws=Ws, x=x, y=y, N=c0.N):
            bq.lqmm_gemv_q4_0(Ws.next(), x, N, out=y)

        def launch_warm(W0=Ws.copies[0], x=x, y=y, N=c0.N):
            bq.lqmm_gemv_q4_0(W0, x, N, out=y)

        cases.append(Case(name, "gemv", alg, 2 * c0.N * c0.K, launch, R,
                          lambda y=y: y.cpu().numpy(), launch_warm))
        inputs[name] = ("q4_0", c0.W, c0.x.copy(), c0.N, c0.K)

    # Q4_0 decode GEMVs: one weight set per N, shared by batch 1 and 4
    for N in (4096, 11008, 12288):
        names = [f"q4_0_gemv_{N}x4096_b{b}" for b in (1, 4)]
        if not any(want(n) for n in names):
            continue
        c4 = synth.make(names[1])        # batch-4 case; its W is the shared one
        wbytes = c4.W.nbytes
        R = rot(wbytes)
        Ws = rotset(c4.W, R)
        for b, name in zip((1, 4), names):
            if not want(name):
                continue
            x = torch.from_numpy(c4.x[:b].copy()).to(dev)
            y = torch.empty((b, N), dtype=torch.float32, device=dev)
            alg = wbytes + b * 4096 * 4 + b * N * 4

            def launch(Ws=Ws, x=x, y=y, N=N):
                bq.lqmm_gemv_q4_0(Ws.next(), x, N, out=y)

            def launch_warm(W0=Ws.copies[0], x=x, y=y, N=N):
                bq.lqmm_gemv_q4_0(W0, x, N, out=y)

            cases.append(Case(name, "gemv", alg, 2 * b * N * 4096, launch, R,
                              lambda y=y: y.cpu().numpy(), launch_warm))
            inputs[name] = ("q4_0", c4.W, c4.x[:b].copy(), N, 4096)

    # Q4_K decode GEMV at the 70B FFN shape, batch 1 and 8
    names = ["q4_k_gemv_28672x8192_b1", "q4_k_gemv_28672x8192_b8"]
    if any(want(n) for n in names):
        ck = synth.make(names[1])
        wbytes = ck.W.nbytes
        R = rot(wbytes)
        Ws = rotset(ck.W, R)
        for b, name in zip((1, 8), names):
            if not want(name):
                continue
            x = torch.from_numpy(ck.x[:b].copy()).to(dev)
            y = torch.empty((b, ck.N), dtype=torch.float32, device=dev)
            alg = wbytes + b * ck.K * 4 + b * ck.N * 4

            def launch(Ws=Ws, x=x, y=y, N=ck.N):
                bq.lqmm_gemv_q4_k(Ws.next(), x, N, out=y)

            def launch_warm(W0=Ws.copies[0], x=x, y=y, N=ck.N):
                bq.lqmm_gemv_q4_k(W0, x, N, out=y)

            cases.append(Case(name, "gemv", alg, 2 * b * ck.N * ck.K, launch, R,
                              lambda y=y: y.cpu().numpy(), launch_warm))
            inputs[name] = ("q4_k", ck.W, ck.x[:b].copy(), ck.N, ck.K)
        stream_sets["q4_k_28672x8192"] = Ws

    # Q8_0 x fp16 prefill GEMM
    name = "q8_0_gemm_512x14336x4096"
    if want(name):
        cg = synth.make(name)
        wbytes = cg.W.nbytes
        R = rot(wbytes)
        Ws = rotset(cg.W, R)
        X = torch.from_numpy(cg.X).to(dev)
        Y = torch.empty((cg.M, cg.N), dtype=torch.float16, device=dev)
        alg = wbytes + cg.M * cg.K * 2 + cg.M * cg.N * 2

        def launch(Ws=Ws, X=X, Y=Y, N=cg.N):
            bq.lqmm_gemm_q8_0_f16(Ws.next(), X, N, out=Y)

        cases.append(Case(name, "gemm_f16", alg, 2 * cg.M * cg.N * cg.K, launch, R,
                          lambda Y=Y: Y.cpu().numpy()))
        inputs[name] = ("q8_0", cg.W, cg.X, cg.N, cg.K)

    # fp32 GEMM
    name = "sgemm_2048"
    if want(name):
        s = synth.make(name)
        R = rot(s.A.nbytes + s.B.nbytes)
        AB = Rot(list(zip([t.view(s.M, s.K) for t in copies(s.A, R)],
                          [t.view(s.K, s.N) for t in copies(s.B, R)])))
        C = torch.empty((s.M, s.N), dtype=torch.float32, device=dev)
        alg = (s.M * s.K + s.K * s.N + s.M * s.N) * 4

        def launch(AB=AB, C=C):
            A, B = AB.next()
            bq.lqmm_sgemm(A, B, out=C)

        cases.append(Case(name, "gemm_f32", alg, 2 * s.M * s.N * s.K, launch, R,
                          lambda C=C: C.cpu().numpy()))
        inputs[name] = ("sgemm", s.A, s.B, s.N, s.K)

    # The other format x phase pairs and the further formats, at the same
    # layer shapes (reported apart from the step: "next_formats").
    next_gemv = {"q8_0": (bq.lqmm_gemv_q8_0, ["q8_0_gemv_4096x4096_b1", "q8_0_gemv_11008x4096_b1",
                                              "q8_0_gemv_12288x4096_b4"]),
                 "q6_k": (bq.lqmm_gemv_q6_k, ["q6_k_gemv_11008x4096_b1"]),
                 "q2_k": (bq.lqmm_gemv_q2_k, ["q2_k_gemv_11008x4096_b1"]),
                 "q1_0": (bq.lqmm_gemv_q1_0, ["q1_0_gemv_11008x4096_b1"])}
    for fmt, (fn, names) in next_gemv.items():
        for name in names:
            if not want(name):
                continue
            c = synth.make(name)
            wbytes = c.W.nbytes
            R = rot(wbytes)
            Ws = rotset(c.W, R)
            x = torch.from_numpy(c.x.copy()).to(dev)
            y = torch.empty((c.batch, c.N), dtype=torch.float32, device=dev)

            def launch(Ws=Ws, x=x, y=y, N=c.N, fn=fn):
                fn(Ws.next(), x, N, out=y)

            cases.append(Case(name, "gemv", wbytes + c.batch * c.K * 4 + c.batch * c.N * 4,
                              2 * c.batch * c.N * c.K, launch, R, lambda y=y: y.cpu().numpy(),
                              section="next"))
    name = "i4g32_gemv_11008x4096_b1"
    if want(name):
        c = synth.make(name)
        wbytes = c.Wq.nbytes + c.scales.nbytes + c.zeros.nbytes
        R = rot(wbytes)
        Wq, sc, z = copies(c.Wq.view(np.int32), R), copies(c.scales, R), copies(c.zeros, R)
        trio = Rot([(Wq[i], sc[i].view(c.N, -1), z[i].view(c.N, -1)) for i in range(R)])
        x = torch.from_numpy(c.x.copy()).to(dev)
        y = torch.empty((c.batch, c.N), dtype=torch.float32, device=dev)

        def launch(trio=trio, x=x, y=y, N=c.N):
            a, b, d = trio.next()
            bq.lqmm_gemv_i4g32(a, b, d, x, N, out=y)

        cases.append(Case(name, "gemv", wbytes + c.batch * c.K * 4 + c.batch * c.N * 4,
                          2 * c.batch * c.N * c.K, launch, R, lambda y=y: y.cpu().numpy(),
                          section="next"))
    for fmt, fn in (("q4_0", bq.lqmm_gemm_q4_0_f16), ("q4_k", bq.lqmm_gemm_q4_k_f16)):
        name = f"{fmt}_gemm_512x14336x4096"
        if not want(name):
            continue
        cg = synth.make(name)
        wbytes = cg.W.nbytes
        R = rot(wbytes)
        Ws = rotset(cg.W, R)
        X = torch.from_numpy(cg.X).to(dev)
        Y = torch.empty((cg.M, cg.N), dtype=torch.float16, device=dev)

        def launch(Ws=Ws, X=X, Y=Y, N=cg.N, fn=fn):
            fn(Ws.next(), X, N, out=Y)

        cases.append(Case(name, "gemm_f16", wbytes + cg.M * cg.K * 2 + cg.M * cg.N * 2,
                          2 * cg.M * cg.N * cg.K, launch, R, lambda Y=Y: Y.cpu().numpy(),
                          section="next"))
    return cases, inputs, stream_sets


_capture_stream = None


def capture_stream(torch):
    """The one stream every graph is captured on. The binding keys its
    default split-K workspaces by stream: calls made eagerly on this stream
    before capture allocate them, so that no allocation (and no zero fill)
    is recorded into a graph."""
    global _capture_stream
    if _capture_stream is None:
        _capture_stream = torch.cuda.Stream()
    return _capture_stream


def capture(torch, fn):
    """A HIP graph of fn()'s launches (the library launches on the current
    stream, which is the capture stream inside the context). Replaying it
    removes the Python call overhead between kernels; it records only the
    library's kernel nodes (no memset or fill nodes: run fn() once eagerly
    on capture_stream() first)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=capture_stream(torch)):
        fn()
    return g


def eager_on_capture_stream(torch, cases):
    """One eager call of each case on the capture stream (workspaces and the
    library's once-per-device set-up happen outside the graphs)."""
    s = capture_stream(torch)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in cases:
            c.launch()
    torch.cuda.synchronize()


def case_summary(c):
    ms = c.avg_ms
    d = {"ms": round(ms, 6)}
    if c.kind == "gemv":
        gbs = c.bytes / (ms * 1e-3) / 1e9
        d.update(gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4), bytes=c.bytes)
    else:
        tf = c.flops / (ms * 1e-3) / 1e12
        peak = F16_PEAK_TFLOPS if c.kind == "gemm_f16" else F32_PEAK_TFLOPS
        d.update(tflops=round(tf, 1), frac=round(tf / peak, 4), flops=c.flops)
    return d


def traffic_for(case_name):
    """HBM bytes per launch of a case from the committed rocprofv3 counter
    summary, or None when it is missing or any library source changed since
    the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return t.get("cases", {}).get(case_name, {}).get("hbm_bytes_per_launch")


def roofline_entry(c):
    """Roofline figures of one case: GEMVs against HBM, GEMMs against their
    matrix-core peak."""
    ms = c.avg_ms
    if c.kind == "gemv":
        ach = c.bytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_for(c.name),
                "algorithmic_bytes_per_launch": c.bytes, "avg_launch_ms": round(ms, 6)}
    peak = F16_PEAK_TFLOPS if c.kind == "gemm_f16" else F32_PEAK_TFLOPS
    ach = c.flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 4), "traffic": None, "flops_per_launch": c.flops,
            "avg_launch_ms": round(ms, 6)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inputs, gpu_outputs, min_seconds):
    """The fp64 CPU oracle on the same host bytes as the GPU GEMV calls: all
    rows of every call, repeated until at least `min_seconds` of wall time
    (a bounded sample), plus a parity check of the GPU outputs against it;
    then a shorter sample on one thread."""
    import oracle

    orc = oracle.get()
    gemv = [(n, v) for n, v in inputs.items() if v[0] in ("q4_0", "q4_k")]
    if not gemv:
        return None, None

    def sample(seconds, check):
        tot_bytes, passes, worst = 0, 0, 0.0
        t0 = time.perf_counter()
        while True:
            for name, (fmt, W, x, N, K) in gemv:
                ref = orc.gemv_q4_0(W, x, N, K) if fmt == "q4_0" else orc.gemv_q4_k(W, x, N, K)
                b = x.shape[0]
                tot_bytes += W.nbytes + b * K * 4 + b * N * 4
                if check and passes == 0 and name in gpu_outputs:
                    rel, nmax = oracle.errors(gpu_outputs[name], ref)
                    worst = max(worst, rel, nmax)
            passes += 1
            if time.perf_counter() - t0 >= seconds:
                break
        return tot_bytes, passes, time.perf_counter() - t0, worst

    threads = orc.threads
    tot_bytes, passes, tot_s, worst = sample(min_seconds, True)
    orc.set_threads(1)
    b1, p1, s1, _ = sample(min_seconds / 4, False)
    orc.set_threads(threads)
    names = ", ".join(n for n, _ in gemv)
    return ({"value": round(tot_bytes / tot_s / 1e9, 3), "unit": "GB/s", "cores": threads,
             "kind": "oracle",
             "sample": f"{passes} passes over all rows of the step's {len(gemv)} GEMV calls "
                       f"({names}); {tot_s:.1f} s wall on {threads} threads; fp64 "
                       "dequantize-then-multiply",
             "single_thread": {"value": round(b1 / s1 / 1e9, 3), "unit": "GB/s",
                               "sample": f"{p1} passes, {s1:.1f} s wall on 1 thread"},
             "cpu_model": cpu_model()},
            worst)


def measure_context(torch, cases, stream_sets, steps):
    """Context figures, taken after the timed steps (see the module doc)."""
    import ctypes

    import block_quantized_matmul_amd as bq

    ctx = {}

    def graph_ms(fn, n):
        # outside the capture, on the capture stream: library set-up
        # (hipBLASLt's, the binding's workspaces) and warm-up
        s = capture_stream(torch)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(3):
                fn()
        torch.cuda.synchronize()
        g = capture(torch, lambda: [fn() for _ in range(n)])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    # Plain streaming read over the rotated Q4_K weight copies.
    probe = os.path.join(ROOT, "block_quantized_matmul_amd", "liblqmm_probe.so")
    ws = stream_sets.get("q4_k_28672x8192")
    if ws is not None and os.path.exists(probe):
        lib = ctypes.CDLL(probe)
        lib.lqmm_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.lqmm_probe_stream_read.restype = ctypes.c_int
        out = torch.zeros(4, dtype=torch.int32, device="cuda:0")
        nbytes = ws.copies[0].numel() * ws.copies[0].element_size()
        best, per_order = None, {}
        for blocks, order in ((0, "grid_stride"), (1, "wave_blocks")):
            for grid in (1024, 2048, 4096):
                def rd(grid=grid, blocks=blocks):
                    t = ws.next()
                    rc = lib.lqmm_probe_stream_read(t.data_ptr(), nbytes, out.data_ptr(), grid,
                                                    blocks, torch.cuda.current_stream().cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"streaming-read probe failed: {rc}")
                ms = graph_ms(rd, steps)
                gbs = nbytes / (ms * 1e-3) / 1e9
                per_order[order] = max(per_order.get(order, 0.0), round(gbs, 1))
                if best is None or gbs > best[0]:
                    best = (gbs, grid, ms, order)
        ctx["hbm_stream"] = {"gbs": round(best[0], 1), "frac": round(best[0] / HBM_PEAK_GBS, 4),
                             "bytes": nbytes, "ms": round(best[2], 6), "grid": best[1],
                             "order": best[3], "gbs_by_order": per_order,
                             "kernel": "16-byte non-temporal reads of every word once, over the "
                                       "rotated Q4_K weight copies (cold HBM), in grid-stride "
                                       "order (8 in flight per thread) or in 4 KB blocks per "
                                       "wave; best of both orders and grids 1024, 2048, 4096"}
    # GEMVs on one weight copy back to back: cache-resident, not HBM.
    warm = {}
    for c in cases:
        if c.kind == "gemv" and c.launch_warm is not None:
            ms = graph_ms(c.launch_warm, steps)
            warm[c.name] = {"ms": round(ms, 6), "gbs": round(c.bytes / (ms * 1e-3) / 1e9, 1)}
    if warm:
        ctx["warm_same_copy"] = warm
    # A decode layer's GEMV chain (Q4_0 QKV, O, gate/up, down at batch 1, each
    # reading the previous output) over 8 layers of distinct weights (cold:
    # 784 MB), replayed from one HIP graph against the same launches from
    # Python one by one.
    try:
        from block_quantized_matmul_amd.chain import DecodeChain
        ch = DecodeChain(torch, layers=8, seed=1)
        for _ in range(3):
            ch.run()
        torch.cuda.synchronize()
        g = ch.capture()
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < 0.05:
            g.replay()
            torch.cuda.synchronize()
        reps = 10
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        e1.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / reps / len(ch.layers)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            ch.run()
        torch.cuda.synchronize()
        eager_us = (time.perf_counter() - t0) * 1e6 / reps / len(ch.layers)
        per_layer = ch.weight_bytes / len(ch.layers)
        ctx["decode_chain"] = {
            "layers": len(ch.layers), "gemvs_per_layer": 4,
            "weight_bytes_per_layer": per_layer,
            "graph_us_per_layer": round(graph_us, 2),
            "graph_gbs": round(per_layer / (graph_us * 1e-6) / 1e9, 1),
            "eager_us_per_layer": round(eager_us, 2),
            "what": "Q4_0 batch-1 GEMVs QKV 12288x4096, O 4096x4096, gate/up 22016x4096, down "
                    "4096x11008 through the allocation-free entry point, one HIP graph per pass "
                    "over 8 layers; eager = the same calls from Python with one sync per pass"}
        del ch, g
    except Exception as e:  # context only
        ctx["decode_chain"] = {"error": f"{type(e).__name__}: {e}"}
    # Host wall time per call, one call at a time (binding and launch included).
    calls = {}
    for c in cases:
        if c.name in ("q4_0_gemv_4096x4096_b1", "q4_0_gemv_4096x4096_b4"):
            for _ in range(20):
                c.launch()
            torch.cuda.synchronize()
            n = 200
            t0 = time.perf_counter()
            for _ in range(n):
                c.launch()
            torch.cuda.synchronize()
            calls[c.name] = round((time.perf_counter() - t0) / n * 1e6, 2)
    if calls:
        ctx["host_wall_us_per_call"] = calls
    # The vendor library's GEMMs at the same shapes (reference points, not
    # this library): dense fp16 weights (twice the Q8_0 bytes), rotated cold
    # copies; and the fp32 GEMM.
    vend = {}
    gq = next((c for c in cases if c.name == "q8_0_gemm_512x14336x4096"), None)
    if gq is not None:
        M, N, K = 512, 14336, 4096
        X = torch.randn(M, K, dtype=torch.float16, device="cuda:0")
        Y = torch.empty(M, N, dtype=torch.float16, device="cuda:0")
        R = max(2, math.ceil(ROTATE_BYTES / (N * K * 2)))
        Wf = Rot([torch.randn(N, K, dtype=torch.float16, device="cuda:0") for _ in range(R)])
        ms = graph_ms(lambda: torch.matmul(X, Wf.next().t(), out=Y), steps)
        tf = 2 * M * N * K / (ms * 1e-3) / 1e12
        vend["fp16_gemm_512x14336x4096"] = {
            "ms": round(ms, 6), "tflops": round(tf, 1), "frac": round(tf / F16_PEAK_TFLOPS, 4),
            "call": "torch.matmul(X fp16 [512x4096], W fp16 [14336x4096] transposed view)"}
        del Wf, X, Y
    gs = next((c for c in cases if c.name == "sgemm_2048"), None)
    if gs is not None:
        n = 2048
        R = max(2, math.ceil(ROTATE_BYTES / (2 * n * n * 4)))
        AB = Rot([(torch.rand(n, n, device="cuda:0") * 2 - 1, torch.rand(n, n, device="cuda:0") * 2 - 1)
                  for _ in range(R)])
        C = torch.empty(n, n, device="cuda:0")

        def mm():
            A, B = AB.next()
            torch.matmul(A, B, out=C)
        ms = graph_ms(mm, steps)
        tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
        vend["fp32_gemm_2048"] = {"ms": round(ms, 6), "tflops": round(tf, 1),
                                  "frac": round(tf / F32_PEAK_TFLOPS, 4),
                                  "call": "torch.matmul(A fp32, B fp32), TF32 off",
                                  "allow_tf32": bool(torch.backends.cuda.matmul.allow_tf32)}
        del AB, C
    if vend:
        ctx["vendor_gemm"] = vend
    torch.cuda.empty_cache()
    return ctx


# ---- rocprofv3 summaries (host only) -------------------------------------------

def _short_kernel(name):
    import re
    name = re.sub(r"\(anonymous namespace\)::", "", name).replace("lqmm::", "")
    name = name.replace("void ", "")
    if name.endswith(")"):  # drop the argument list (the last balanced parentheses)
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    if name.startswith("Cijk_"):  # vendor GEMM kernels: keep the tile part of the name
        m = re.search(r"_MT\w+?_MI\w+?_", name)
        name = "vendor GEMM " + name.split("_")[1] + (" " + m.group(0).strip("_") if m else "")
    elif name.startswith("at::"):  # torch's set-up kernels: their template name only
        name = name.split("<")[0] + " (torch)"
    return name


def _find(dirpath, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(dirpath, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {dirpath}")
    return hits[-1]


def _pct(v, p):
    """p-th percentile of the sorted list v (linear interpolation)."""
    if len(v) == 1:
        return v[0]
    i = (len(v) - 1) * p / 100.0
    lo = int(math.floor(i))
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (i - lo)


def summarize_trace(trace_dir, bench_log, out_md, command):
    """Markdown summary of a `rocprofv3 --kernel-trace --stats` run of this
    benchmark. The timed launches lie between the two marker kernels; they
    run case-major in the order of the JSON line's "cases", the same number
    per case, so each case's launches are identified by position. For each
    case: launches, kernel, mean / median / p10 / p90 duration, and the
    throughput of the mean against the peak. All other launches (settle,
    warmup, context) are listed apart, per kernel."""
    import csv
    line = None
    for l in open(bench_log):
        l = l.strip()
        if l.startswith("{") and '"metric"' in l:
            line = json.loads(l)
    if line is None:
        raise SystemExit(f"no JSON line in {bench_log}")
    order = list(line["cases"].keys())
    rows = list(csv.DictReader(open(_find(trace_dir, "kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"] for r in rows]
    b = max(i for i, n in enumerate(names) if "timed_region_begin_marker" in n)
    e = min(i for i, n in enumerate(names) if "timed_region_end_marker" in n and i > b)
    timed = rows[b + 1:e]
    per = len(timed) // len(order)
    if per * len(order) != len(timed) or per == 0:
        raise SystemExit(f"{len(timed)} timed launches do not split over {len(order)} cases")
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
    out = []
    out.append(f"# Kernel trace of `bench.py`: {line['config']['workload']}\n\n")
    out.append("Command, from the repository root on one MI355X after "
               "`cd /tmp && export TMPDIR=/tmp` (paths relative to the repository):\n\n")
    out.append(f"```\n{command}\n```\n\n")
    out.append(f"Timed region: {len(timed)} launches, {per} per case, between the marker "
               f"kernels (steps {line['steps']}, warmup {line['warmup']}). Durations are kernel "
               "start to end from the trace; `bench us` is the same case's mean launch time "
               "from the HIP events of the bench line (graph replay: it includes the gaps "
               "between launches).\n\n")
    out.append("| case | kernel | launches | mean us | median us | p10 us | p90 us | bench us "
               "| mean rate | of peak |\n|---|---|---:|---:|---:|---:|---:|---:|---:|---:|\n")
    summary = {}
    for ci, case in enumerate(order):
        rs = timed[ci * per:(ci + 1) * per]
        kn = sorted(set(_short_kernel(r["Kernel_Name"]) for r in rs))
        d = sorted(dur(r) for r in rs)
        mean = sum(d) / len(d)
        cs = line["cases"][case]
        if "bytes" in cs:
            rate = cs["bytes"] / (mean * 1e-6) / 1e9
            rate_s, frac = f"{rate:.0f} GB/s", rate / HBM_PEAK_GBS
        else:
            rate = cs["flops"] / (mean * 1e-6) / 1e12
            peak = F16_PEAK_TFLOPS if case.startswith("q8_0") else F32_PEAK_TFLOPS
            rate_s, frac = f"{rate:.1f} TFLOP/s", rate / peak
        summary[case] = {"mean_us": mean, "frac": frac}
        out.append(f"| {case} | `{' + '.join(kn)}` | {len(d)} | {mean:.2f} | {_pct(d, 50):.2f} | "
                   f"{_pct(d, 10):.2f} | {_pct(d, 90):.2f} | {cs['ms'] * 1e3:.2f} | {rate_s} | "
                   f"{frac:.3f} |\n")
    rf = line.get("roofline", {})
    if rf.get("case") in summary:
        out.append(f"\nThe bench line's `roofline` names {rf['case']}: {rf['frac']:.3f} of peak from "
                   f"the HIP events, {summary[rf['case']]['frac']:.3f} from the trace mean.\n")
    other = {}
    for r in rows[:b] + rows[e + 1:]:
        other.setdefault(_short_kernel(r["Kernel_Name"]), []).append(dur(r))
    out.append("\nOther launches (settle and warmup replays before the timed region, context "
               "figures after it; the GEMVs' `warm_same_copy` launches here are cache-resident):\n\n"
               "| kernel | launches | mean us | median us |\n|---|---:|---:|---:|\n")
    for k in sorted(other, key=lambda k: -sum(other[k])):
        d = sorted(other[k])
        out.append(f"| `{k}` | {len(d)} | {sum(d) / len(d):.2f} | {_pct(d, 50):.2f} |\n")
    with open(out_md, "w") as f:
        f.write("".join(out))
    print("".join(out))


def _counter_per_dispatch(csv_path, counter):
    """{dispatch id: (kernel name, summed value of `counter`)}."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter:
            k = r["Dispatch_Id"]
            name, v = per.get(k, (r["Kernel_Name"], 0.0))
            per[k] = (name, v + float(r["Counter_Value"]))
    return per


def summarize_series(trace_dir, bench_log, out_md, command):
    """Markdown summary of how each case's launch durations evolve over its
    timed graph (launches in order, means of consecutive blocks of ten),
    next to the same kernel's launches in the settle and warmup replays
    before the timed region. Launches are identified as in summarize_trace."""
    import csv
    line = None
    for l in open(bench_log):
        l = l.strip()
        if l.startswith("{") and '"metric"' in l:
            line = json.loads(l)
    if line is None:
        raise SystemExit(f"no JSON line in {bench_log}")
    order = list(line["cases"].keys())
    rows = list(csv.DictReader(open(_find(trace_dir, "kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"] for r in rows]
    b = max(i for i, n in enumerate(names) if "timed_region_begin_marker" in n)
    e = min(i for i, n in enumerate(names) if "timed_region_end_marker" in n and i > b)
    timed = rows[b + 1:e]
    per = len(timed) // len(order)
    if per * len(order) != len(timed) or per == 0:
        raise SystemExit(f"{len(timed)} timed launches do not split over {len(order)} cases")
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
    out = [f"# Launch durations over the timed graphs: {', '.join(order)}\n\n",
           "Command, from the repository root on one MI355X after "
           "`cd /tmp && export TMPDIR=/tmp` (paths relative to the repository):\n\n",
           f"```\n{command}\n```\n\n",
           f"Each case's {per} timed launches run back to back in one HIP graph, the cases "
           "one after another in the order listed. Durations are kernel start to end from "
           "the trace, in us.\n\n",
           "| case | kernel | min | median | max | settle and warmup launches: count, median |\n"
           "|---|---|---:|---:|---:|---:|\n"]
    series = []
    for ci, case in enumerate(order):
        rs = timed[ci * per:(ci + 1) * per]
        kn = sorted(set(r["Kernel_Name"] for r in rs))
        d = [dur(r) for r in rs]
        pre = sorted(dur(r) for r in rows[:b] if r["Kernel_Name"] in kn)
        pre_s = f"{len(pre)}, {_pct(pre, 50):.2f}" if pre else "-"
        ds = sorted(d)
        out.append(f"| {case} | `{' + '.join(_short_kernel(k) for k in kn)}` | {ds[0]:.2f} | "
                   f"{_pct(ds, 50):.2f} | {ds[-1]:.2f} | {pre_s} |\n")
        blocks = [sum(d[i:i + 10]) / len(d[i:i + 10]) for i in range(0, len(d), 10)]
        series.append((case, blocks))
    out.append("\nMeans of consecutive blocks of ten timed launches, in launch order:\n\n")
    for case, blocks in series:
        out.append(f"- {case}: " + ", ".join(f"{v:.1f}" for v in blocks) + "\n")
    with open(out_md, "w") as f:
        f.write("".join(out))
    print(f"wrote {out_md}")


def summarize_traffic(pmc_dir, calib_mib, command):
    """HBM bytes per launch of every GEMV case, from one FETCH_SIZE run and
    one WRITE_SIZE run per case (PMC_DIR/<case>.fetch, PMC_DIR/<case>.write;
    KiB per dispatch). Each counter is scaled by what it reads for the
    calibration kernel in the same run (torch.neg over calib_mib MiB, which
    reads and writes that many bytes). The library's kernels are every
    dispatch named lqmm:: (the run holds only that case's launches)."""
    import glob
    expect_kib = calib_mib * 1024.0
    out = {"kernel_source_sha256": kernel_source_sha256(),
           "calibration": {"kernel": "torch.neg, float32, out of place",
                           "mib_read": calib_mib, "mib_written": calib_mib},
           "command": command, "cases": {}}
    for d in sorted(glob.glob(os.path.join(pmc_dir, "*.fetch"))):
        case = os.path.basename(d)[:-len(".fetch")]
        res = {}
        for counter, sub in (("FETCH_SIZE", ".fetch"), ("WRITE_SIZE", ".write")):
            per = _counter_per_dispatch(_find(os.path.join(pmc_dir, case + sub),
                                              "counter_collection.csv"), counter)
            kern = [v for n, v in per.values() if "lqmm::" in n and "probe" not in n]
            cal = [v for n, v in per.values() if "neg_kernel" in n]
            kname = sorted(set(_short_kernel(n) for n, v in per.values() if "lqmm::" in n))
            if not kern or not cal:
                raise SystemExit(f"{case}: no {counter} dispatches of the kernel or calibration")
            scale = expect_kib / (sum(cal) / len(cal))
            res[counter] = (sum(kern) / len(kern), len(kern), scale, kname)
        fk, nf, fs, kname = res["FETCH_SIZE"]
        wk, nw, wsc, _ = res["WRITE_SIZE"]
        out["cases"][case] = {
            "kernel": " + ".join(kname), "dispatches": {"fetch": nf, "write": nw},
            "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
            "fetch_scale": round(fs, 4), "write_scale": round(wsc, 4),
            "hbm_bytes_per_launch": int(round((fk * fs + wk * wsc) * 1024))}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def summarize_counters(pmc_dir, out_md, command):
    """Markdown summary of rocprofv3 `--kernel-trace --pmc` passes over the
    GEMM cases (PMC_DIR/pass<n>/...): per library kernel, the mean per
    dispatch of every counter collected, the mean kernel duration from the
    same pass's trace, and ratios stated with their formulas. Counter values
    are summed over the GPU's instances by rocprofv3."""
    import csv
    import glob
    per_kernel = {}  # kernel -> {counter: [values per dispatch]}
    durs = {}        # kernel -> [us]
    for pdir in sorted(glob.glob(os.path.join(pmc_dir, "pass*"))):
        vals = {}
        for r in csv.DictReader(open(_find(pdir, "counter_collection.csv"))):
            if "lqmm::" not in r["Kernel_Name"]:
                continue
            key = (r["Dispatch_Id"], r["Counter_Name"])
            k = _short_kernel(r["Kernel_Name"])
            vals.setdefault(k, {}).setdefault(key, 0.0)
            vals[k][key] += float(r["Counter_Value"])
        for k, d in vals.items():
            for (_, cn), v in d.items():
                per_kernel.setdefault(k, {}).setdefault(cn, []).append(v)
        for r in csv.DictReader(open(_find(pdir, "kernel_trace.csv"))):
            if "lqmm::" in r["Kernel_Name"]:
                k = _short_kernel(r["Kernel_Name"])
                durs.setdefault(k, []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    mean = lambda v: sum(v) / len(v)
    out = ["# Matrix-core and LDS counters of the GEMM kernels\n\n",
           "Commands, from the repository root on one MI355X after "
           "`cd /tmp && export TMPDIR=/tmp` (one rocprofv3 pass per counter group, "
           "paths relative to the repository):\n\n", f"```\n{command}\n```\n\n",
           "Means per dispatch over every launch of the kernel in the passes (warmup and "
           "timed launches of the cases, cold weights). Durations are from the kernel trace "
           "taken in the same passes.\n\n"]
    for k in sorted(per_kernel):
        c = {cn: mean(v) for cn, v in per_kernel[k].items()}
        n = max(len(v) for v in per_kernel[k].values())
        d = mean(durs.get(k, [float("nan")]))
        out.append(f"## `{k}`\n\n{n} dispatches per counter; mean duration {d:.2f} us.\n\n"
                   "| counter | mean per dispatch |\n|---|---:|\n")
        for cn in sorted(c):
            out.append(f"| {cn} | {c[cn]:,.0f} |\n")
        out.append("\n")
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs (its ratio to the
        # duration is 8x the shader clock); one XCD's cycles times the 1024
        # SIMDs (256 CUs x 4) are the SIMD-cycles of the launch.
        ratios = []
        g = c.get("GRBM_GUI_ACTIVE")
        if g:
            ratios.append(("shader clock, GHz: GRBM_GUI_ACTIVE / 8 XCDs / duration",
                           g / 8 / (d * 1e3)))
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            ratios.append(("matrix cores busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 "
                           "x 1024 SIMDs)", c["SQ_VALU_MFMA_BUSY_CYCLES"] / (g / 8 * 1024)))
        for mops, peak in (("SQ_INSTS_VALU_MFMA_MOPS_F16", F16_PEAK_TFLOPS),
                           ("SQ_INSTS_VALU_MFMA_MOPS_F32", F32_PEAK_TFLOPS)):
            if c.get(mops):
                ratios.append((f"TFLOP/s through the matrix cores: {mops} x 512 / duration",
                               c[mops] * 512 / (d * 1e-6) / 1e12))
                ratios.append((f"  the same against the {peak:g} TFLOP/s peak (2.4 GHz)",
                               c[mops] * 512 / (d * 1e-6) / 1e12 / peak))
                if c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
                    ratios.append((f"  busy cycles per 512 matrix-core flops: "
                                   f"SQ_VALU_MFMA_BUSY_CYCLES / {mops}",
                                   c["SQ_VALU_MFMA_BUSY_CYCLES"] / c[mops]))
        if c.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in c:
            ratios.append(("LDS bank-conflict share: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
                           c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]))
        if ratios:
            out.append("| ratio | value |\n|---|---:|\n")
            for name, v in ratios:
                out.append(f"| {name} | {v:.4g} |\n")
            out.append("\n")
    with open(out_md, "w") as f:
        f.write("".join(out))
    print("".join(out))


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_series:
        summarize_series(*args.summarize_series)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_traffic:
        pmc_dir, calib_mib, command = args.summarize_traffic
        summarize_traffic(pmc_dir, int(calib_mib), command)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(no multi-GPU path is implemented).", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_quantized_matmul_amd as bq
    bq.load()  # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    only = set(s for s in args.cases.split(",") if s)

    t_setup = time.perf_counter()
    cases, inputs, stream_sets = build_cases(torch, only)
    torch.cuda.synchronize()
    print(f"[bench] {len(cases)} cases set up in {time.perf_counter() - t_setup:.1f} s",
          file=sys.stderr, flush=True)

    if args.calib_copy_mib:
        # Counter calibration: a plain elementwise kernel that reads and
        # writes a known number of bytes.
        n = args.calib_copy_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] calibration kernel over {args.calib_copy_mib} MiB x3 done",
              file=sys.stderr, flush=True)

    # The K timed steps run case-major: every hot-path call is captured K
    # times back to back in one HIP graph (each launch on the next weight
    # copy), and the graphs are replayed in step order, each bracketed by HIP
    # events on the launch stream. This is the same work as K step-major
    # passes, with the graph-launch overhead spread over K launches; the
    # events give each call's average launch duration inside the timed region.
    step = [c for c in cases if c.section == "step"]
    gemv = [c for c in step if c.kind == "gemv"]
    order = gemv + [c for c in step if c.kind != "gemv"]
    extra = [c for c in cases if c.section == "next"]
    # One eager call of each case before any capture, on the capture stream:
    # the binding's split-K workspaces and the library's once-per-device
    # set-up happen outside the graphs.
    for c in order:
        c.launch()
    eager_on_capture_stream(torch, order)
    if args.eager:
        run = {c.name: (lambda c=c, n=args.steps: [c.launch() for _ in range(n)]) for c in order}
        warm = {c.name: (lambda c=c, n=args.warmup: [c.launch() for _ in range(n)]) for c in order}
    else:
        run, warm = {}, {}
        for c in order:
            g = capture(torch, lambda c=c: [c.launch() for _ in range(args.steps)])
            run[c.name] = g.replay
            if args.warmup:
                gw = capture(torch, lambda c=c: [c.launch() for _ in range(args.warmup)])
                warm[c.name] = gw.replay
    # Settle: replay the steps untimed until --settle-ms of wall time has
    # passed, so that the clocks have ramped up whatever --warmup is.
    settle_passes = 0
    if args.settle_ms > 0:
        settle = {c.name: (warm.get(c.name) or run[c.name]) for c in order}
        t_settle = time.perf_counter()
        while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
            for c in order:
                settle[c.name]()
            torch.cuda.synchronize()
            settle_passes += 1
    for c in order:
        if c.name in warm:
            warm[c.name]()
    # One untimed replay of every timed graph: a graph's first replay also
    # uploads it to the device, which must not land in the timed region.
    if not args.eager:
        for c in order:
            run[c.name]()
    torch.cuda.synchronize()
    # Marker kernels bracket the timed region in kernel traces (outside the
    # events, so they are not timed).
    marker = None
    if os.path.exists(PROBE_LIB):
        import ctypes
        plib = ctypes.CDLL(PROBE_LIB)
        plib.lqmm_probe_marker.argtypes = [ctypes.c_int, ctypes.c_void_p]
        plib.lqmm_probe_marker.restype = ctypes.c_int
        marker = lambda w: plib.lqmm_probe_marker(w, torch.cuda.current_stream().cuda_stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)]
    if marker:
        marker(0)
    t0 = time.perf_counter()
    ev[0].record()
    for i, c in enumerate(order):
        run[c.name]()
        ev[i + 1].record()
    if marker:
        marker(1)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    # The further format x phase pairs, after the timed steps and timed the
    # same way (a settle of up to 50 ms of replays, then a graph of --steps
    # launches per case between HIP events).
    if extra:
        xrun = {}
        for c in extra:
            c.launch()
        eager_on_capture_stream(torch, extra)
        for c in extra:
            xrun[c.name] = capture(torch, lambda c=c: [c.launch() for _ in range(args.steps)])
            xrun[c.name].replay()  # first replay (upload) untimed
            xw = capture(torch, lambda c=c: [c.launch() for _ in range(max(args.warmup, 5))])
            t_settle = time.perf_counter()
            while True:
                xw.replay()
                torch.cuda.synchronize()
                if (time.perf_counter() - t_settle) * 1e3 >= min(args.settle_ms, 50.0):
                    break
        xev = [torch.cuda.Event(enable_timing=True) for _ in range(len(extra) + 1)]
        xev[0].record()
        for i, c in enumerate(extra):
            xrun[c.name].replay()
            xev[i + 1].record()
        torch.cuda.synchronize()
        for i, c in enumerate(extra):
            c.avg_ms = xev[i].elapsed_time(xev[i + 1]) / args.steps
            print(f"[bench] {c.name}: {case_summary(c)}", file=sys.stderr, flush=True)
    for i, c in enumerate(order):
        c.avg_ms = ev[i].elapsed_time(ev[i + 1]) / args.steps
        print(f"[bench] {c.name}: {case_summary(c)}", file=sys.stderr, flush=True)
    ms_per_step = sum(c.avg_ms for c in order)
    # the dominant GEMV kernel: the GEMV case with the longest launch
    roof = sorted(gemv, key=lambda c: -c.avg_ms)[:1]

    gpu_out = {c.name: c.make_out() for c in gemv}

    gemv_bytes = sum(c.bytes for c in gemv)
    gemv_ms = sum(c.avg_ms for c in gemv)
    value = gemv_bytes / (gemv_ms * 1e-3) / 1e9 if gemv else None

    line = {
        "metric": METRIC,
        "value": round(value, 1) if value else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "llama_layer_set: Q4_0 GEMV 1024x1024 b1; "
                        "Q4_0 GEMV K=4096 N=4096/11008/12288 b1+b4; "
                        "Q4_K GEMV N=28672 K=8192 b1+b8; Q8_0xf16 GEMM 512x14336x4096; "
                        "fp32 GEMM 2048^3",
            "weights": "cold HBM (rotated copies >= 512 MiB per set)",
            "value_is": "GEMV algorithmic bytes / GEMV share of the timed steps (case-major)",
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4) if value else None,
            "wall_ms_per_step_host": round(wall_ms / max(1, args.steps), 4),
            "settle": {"ms": args.settle_ms, "passes": settle_passes},
        },
    }
    if roof:
        line["roofline"] = dict(roofline_entry(roof[0]), case=roof[0].name)
    line["rooflines"] = {c.name: roofline_entry(c) for c in order}
    for kind, key, peak in (("gemm_f16", "prefill_gemm", F16_PEAK_TFLOPS),
                            ("gemm_f32", "fp32_gemm", F32_PEAK_TFLOPS)):
        gc = next((c for c in cases if c.kind == kind), None)
        if gc is not None:
            tf = gc.flops / (gc.avg_ms * 1e-3) / 1e12
            line[key] = {"tflops": round(tf, 1), "peak": peak, "frac": round(tf / peak, 4),
                         "ms": round(gc.avg_ms, 6)}
    line["cases"] = {c.name: case_summary(c) for c in order}
    if extra:
        line["next_formats"] = {c.name: dict(case_summary(c), roofline=roofline_entry(c))
                                for c in extra}
    if not args.no_context:
        try:
            line["context"] = measure_context(torch, cases, stream_sets, args.steps)
        except Exception as e:  # context only: never costs the measurement above
            line["context"] = {"error": f"{type(e).__name__}: {e}"}

    if not args.no_cpu_baseline:
        base, worst = cpu_baseline(inputs, gpu_out, args.cpu_seconds)
        line["cpu_baseline"] = base
        if worst is not None:
            line["parity_vs_oracle_max_err"] = float(f"{worst:.3e}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
