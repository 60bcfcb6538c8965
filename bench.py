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
                 the step's GEMV launches / their summed kernel time (GB/s);
  roofline       the largest decode GEMV (Q4_K 28672 x 8192, batch 1) against
                 the 8 TB/s HBM peak, timed with HIP events on the launch
                 stream; traffic from the committed rocprofv3 counter summary;
  prefill_gemm   Q8_0 x fp16 GEMM TFLOP/s against the 2.5 PFLOP/s f16 peak;
  cases          every call: kernel time, GB/s or TFLOP/s, roofline fraction;
  cpu_baseline   the fp64 CPU oracle on the same GEMV inputs (host cores).

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
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--reps", type=int, default=50, help="launches per case for per-kernel timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    p.add_argument("--cases", default="", help="comma-separated subset of case names")
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
    def __init__(self, name, kind, bytes_, flops, launch, nrot, make_out):
        self.name, self.kind = name, kind
        self.bytes, self.flops = bytes_, flops
        self.launch = launch          # launch(): one call on the next weight copy
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

            cases.append(Case(name, "gemv", alg, 2 * b * N * 4096, launch, R,
                              lambda y=y: y.cpu().numpy()))
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

            cases.append(Case(name, "gemv", alg, 2 * b * ck.N * ck.K, launch, R,
                              lambda y=y: y.cpu().numpy()))
            inputs[name] = ("q4_k", ck.W, ck.x[:b].copy(), ck.N, ck.K)

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
    return cases, inputs


def capture(torch, fn):
    """A HIP graph of fn()'s launches (the library launches on the current
    stream, which is the capture stream inside the context). Replaying it
    removes the Python call overhead between kernels; it records only kernel
    nodes (no memset nodes)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def time_case(torch, c, reps, warm, use_graph):
    """Average duration of one launch over `reps` back-to-back launches
    (rotating weight copies), bracketed by HIP events on the launch stream.
    Inter-kernel gaps are included, so this is never below the kernel time."""
    for _ in range(warm):
        c.launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if use_graph:
        g = capture(torch, lambda: [c.launch() for _ in range(reps)])
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
    else:
        e0.record()
        for _ in range(reps):
            c.launch()
        e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


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


def cpu_baseline(inputs, gpu_outputs):
    """The fp64 oracle on the same host bytes as the GPU GEMV cases (all
    rows; a bounded sample of a few seconds of CPU work), plus a parity check
    of the GPU outputs against it."""
    import numpy as np

    import oracle

    orc = oracle.get()
    tot_bytes, tot_s, worst = 0, 0.0, 0.0
    done = []
    for name, (fmt, W, x, N, K) in inputs.items():
        if fmt not in ("q4_0", "q4_k"):
            continue
        t0 = time.perf_counter()
        ref = orc.gemv_q4_0(W, x, N, K) if fmt == "q4_0" else orc.gemv_q4_k(W, x, N, K)
        dt = time.perf_counter() - t0
        b = x.shape[0]
        tot_bytes += W.nbytes + b * K * 4 + b * N * 4
        tot_s += dt
        done.append(name)
        if name in gpu_outputs:
            rel, nmax = oracle.errors(gpu_outputs[name], ref)
            worst = max(worst, rel, nmax)
    if not done:
        return None, None
    return ({"value": round(tot_bytes / tot_s / 1e9, 3), "unit": "GB/s", "cores": orc.threads,
             "kind": "oracle",
             "sample": f"all rows of the step's {len(done)} GEMV calls ({', '.join(done)}), "
                       f"{tot_s:.1f} s of CPU time, fp64 dequantize-then-multiply"},
            worst)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on exactly one GPU; --gpus {args.gpus} is not supported by this "
              "single-GPU build (the multi-GPU sharding is a design note only).", file=sys.stderr)
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
    cases, inputs = build_cases(torch, only)
    torch.cuda.synchronize()
    print(f"[bench] {len(cases)} cases set up in {time.perf_counter() - t_setup:.1f} s",
          file=sys.stderr, flush=True)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {args.calib_copy_mib} MiB x3 done", file=sys.stderr,
              flush=True)

    # per-kernel timing (cold HBM through rotation)
    for c in cases:
        c.avg_ms = time_case(torch, c, args.reps, warm=min(5, c.nrot), use_graph=not args.eager)
        print(f"[bench] {c.name}: {case_summary(c)}", file=sys.stderr, flush=True)

    # whole steps
    gemv = [c for c in cases if c.kind == "gemv"]
    others = [c for c in cases if c.kind != "gemv"]
    order = gemv + others
    def step():
        for c in order:
            c.launch()

    # Four captured steps, replayed in turn, so that a weight copy is reused
    # only after four steps (> 1 GB of other traffic).
    graphs = [] if args.eager else [capture(torch, step) for _ in range(4)]

    def run_step(i):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step()

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        run_step(i)
    e1.record()
    e1.synchronize()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / max(1, args.steps)

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
        "dtype": "f16*f16->f32 (q4/q8 weights dequantized exactly; fp32 GEMM in f32)",
        "data": "synthetic",
        "config": {
            "workload": "llama_layer_set: Q4_0 GEMV K=4096 N=4096/11008/12288 b1+b4; "
                        "Q4_K GEMV N=28672 K=8192 b1+b8; Q8_0xf16 GEMM 512x14336x4096; "
                        "fp32 GEMM 2048^3",
            "weights": "cold HBM (rotated copies >= 512 MiB per set)",
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4) if value else None,
        },
    }
    rc = next((c for c in cases if c.name == ROOFLINE_CASE), None)
    if rc is not None:
        ach = rc.bytes / (rc.avg_ms * 1e-3) / 1e9
        line["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                            "traffic": traffic_for(ROOFLINE_CASE),
                            "kernel": "gemv_kernel<FmtQ4_K,1,R> (" + ROOFLINE_CASE + ")",
                            "algorithmic_bytes_per_launch": rc.bytes,
                            "avg_launch_ms": round(rc.avg_ms, 6)}
    gc = next((c for c in cases if c.kind == "gemm_f16"), None)
    if gc is not None:
        tf = gc.flops / (gc.avg_ms * 1e-3) / 1e12
        line["prefill_gemm"] = {"tflops": round(tf, 1), "peak": F16_PEAK_TFLOPS,
                                "frac": round(tf / F16_PEAK_TFLOPS, 4), "ms": round(gc.avg_ms, 6)}
    line["cases"] = {c.name: case_summary(c) for c in cases}

    if not args.no_cpu_baseline:
        base, worst = cpu_baseline(inputs, gpu_out)
        line["cpu_baseline"] = base
        if worst is not None:
            line["parity_vs_oracle_max_err"] = float(f"{worst:.3e}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
