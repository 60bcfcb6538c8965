#!/usr/bin/env python3
"""Benchmark of the block-quantized matmul hot path on one MI355X.

One step runs every hot-path call once, each on synthetic Llama-shaped layer
inputs already resident in HBM:
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
  roofline       the largest decode GEMV (Q4_K 28672 x 8192, batch 1) against
                 the 8 TB/s HBM peak, timed the same way inside the steps;
                 traffic from the committed rocprofv3 counter summary;
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
ROOFLINE_CASE = "q4_k_gemv_28672x8192_b1"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_q4_k_gemv_28672x8192_b1.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # The GPU raises its clocks over the first tens of milliseconds of
    # sustained work; 100 untimed steps (about 40 ms) reach the steady state
    # that a serving loop runs in.
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    p.add_argument("--cases", default="", help="comma-separated subset of case names")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="wall time of the CPU-oracle baseline sample (whole passes)")
    p.add_argument("--summarize-trace", nargs=4, metavar=("STATS_CSV", "OUT_MD", "COMMAND", "TITLE"),
                   help="host only: write a markdown summary of a rocprofv3 kernel_stats.csv")
    p.add_argument("--summarize-traffic", nargs=5,
                   metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_MIB", "CMD_FETCH", "CMD_WRITE"),
                   help="host only: write the roofline kernel's HBM traffic summary from two "
                        "rocprofv3 --pmc counter_collection.csv files")
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
    def __init__(self, name, kind, bytes_, flops, launch, nrot, make_out, launch_warm=None):
        self.name, self.kind = name, kind
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
    return cases, inputs, stream_sets


def capture(torch, fn):
    """A HIP graph of fn()'s launches (the library launches on the current
    stream, which is the capture stream inside the context). Replaying it
    removes the Python call overhead between kernels; it records only kernel
    nodes (no memset nodes)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


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
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    src = os.path.join(ROOT, "block_quantized_matmul_amd", "csrc", "gemv.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if t.get("case") != case_name or t.get("kernel_source_sha256") != h:
        return None
    return t.get("hbm_bytes_per_launch")


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
        for _ in range(3):  # outside the capture: library set-up (hipBLASLt's) and warm-up
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


def summarize_trace(stats_csv, out_md, command, title):
    """Markdown table of a `rocprofv3 --kernel-trace --stats` kernel_stats.csv."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    with open(out_md, "w") as f:
        f.write(f"# {title}\n\n")
        f.write("Command, run from the repository root on one MI355X after "
                "`cd /tmp && export TMPDIR=/tmp` (paths relative to the repository):\n\n")
        f.write(f"```\n{command}\n```\n\n")
        f.write("| kernel | calls | avg us | min us | max us | share % |\n"
                "|---|---:|---:|---:|---:|---:|\n")
        for r in rows:
            f.write(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | "
                    f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                    f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |\n")


def _counter_means(csv_path, counter, pick):
    """Mean per-dispatch value of `counter` over the dispatches whose kernel
    name satisfies pick(name)."""
    import csv
    import collections
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter and pick(r["Kernel_Name"]):
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} dispatches matched in {csv_path}")
    return sum(per.values()) / len(per), len(per)


def summarize_traffic(fetch_csv, write_csv, calib_mib, commands):
    """HBM bytes per launch of the roofline kernel from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by what the same counter
    reads for the calibration kernel (reads and writes calib_mib MiB)."""
    kern = lambda n: "gemv_stream_kernel<lqmm::(anonymous namespace)::FmtQ4_K" in n
    calib = lambda n: "neg_kernel" in n
    f_k, nf = _counter_means(fetch_csv, "FETCH_SIZE", kern)
    w_k, nw = _counter_means(write_csv, "WRITE_SIZE", kern)
    f_c, _ = _counter_means(fetch_csv, "FETCH_SIZE", calib)
    w_c, _ = _counter_means(write_csv, "WRITE_SIZE", calib)
    expect_kib = calib_mib * 1024.0
    fs, ws = expect_kib / f_c, expect_kib / w_c
    src = os.path.join(ROOT, "block_quantized_matmul_amd", "csrc", "gemv.hip")
    out = {
        "case": ROOFLINE_CASE,
        "kernel": "gemv_stream_kernel<FmtQ4_K, ...> (batch 1, rows streamed through LDS)",
        "kernel_source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
        "dispatches": {"fetch": nf, "write": nw},
        "fetch_kib_per_dispatch": round(f_k, 1),
        "write_kib_per_dispatch": round(w_k, 1),
        "calibration": {"kernel": "torch.neg, float32, out of place", "mib_read": calib_mib,
                        "mib_written": calib_mib, "fetch_kib": round(f_c, 1),
                        "write_kib": round(w_c, 1), "fetch_scale": round(fs, 4),
                        "write_scale": round(ws, 4)},
        "hbm_bytes_per_launch": int(round((f_k * fs + w_k * ws) * 1024)),
        "commands": commands,
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main():
    args = parse()
    if args.summarize_trace:
        stats, out_md, command, title = args.summarize_trace
        summarize_trace(stats, out_md, command, title)
        return
    if args.summarize_traffic:
        fetch_csv, write_csv, calib_mib, cmd_fetch, cmd_write = args.summarize_traffic
        summarize_traffic(fetch_csv, write_csv, int(calib_mib), [cmd_fetch, cmd_write])
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
    gemv = [c for c in cases if c.kind == "gemv"]
    order = gemv + [c for c in cases if c.kind != "gemv"]
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
    for c in order:
        if c.name in warm:
            warm[c.name]()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i, c in enumerate(order):
        run[c.name]()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    for i, c in enumerate(order):
        c.avg_ms = ev[i].elapsed_time(ev[i + 1]) / args.steps
        print(f"[bench] {c.name}: {case_summary(c)}", file=sys.stderr, flush=True)
    ms_per_step = sum(c.avg_ms for c in order)
    roof = [c for c in gemv if c.name == ROOFLINE_CASE]

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
            "workload": "llama_layer_set: Q4_0 GEMV K=4096 N=4096/11008/12288 b1+b4; "
                        "Q4_K GEMV N=28672 K=8192 b1+b8; Q8_0xf16 GEMM 512x14336x4096; "
                        "fp32 GEMM 2048^3",
            "weights": "cold HBM (rotated copies >= 512 MiB per set)",
            "value_is": "GEMV algorithmic bytes / GEMV share of the timed steps (case-major)",
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4) if value else None,
            "wall_ms_per_step_host": round(wall_ms / max(1, args.steps), 4),
        },
    }
    if roof:
        rc = roof[0]
        ach = rc.bytes / (rc.avg_ms * 1e-3) / 1e9
        line["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                            "traffic": traffic_for(ROOFLINE_CASE),
                            "kernel": "gemv_stream_kernel<FmtQ4_K, ...> (" + ROOFLINE_CASE + ")",
                            "algorithmic_bytes_per_launch": rc.bytes,
                            "avg_launch_ms": round(rc.avg_ms, 6)}
    for kind, key, peak in (("gemm_f16", "prefill_gemm", F16_PEAK_TFLOPS),
                            ("gemm_f32", "fp32_gemm", F32_PEAK_TFLOPS)):
        gc = next((c for c in cases if c.kind == kind), None)
        if gc is not None:
            tf = gc.flops / (gc.avg_ms * 1e-3) / 1e12
            line[key] = {"tflops": round(tf, 1), "peak": peak, "frac": round(tf / peak, 4),
                         "ms": round(gc.avg_ms, 6)}
    line["cases"] = {c.name: case_summary(c) for c in order}
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
