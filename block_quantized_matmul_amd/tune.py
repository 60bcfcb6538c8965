"""Launch-configuration sweep for one GEMV or GEMM shape on the current GPU.

"Resumo Tecnico: Llamas na Web", section "Biblioteca de Kernels Portatil em
Desempenho", picks tile and workgroup sizes by sweeping configurations on the
target devices. Here the planner in the library chooses a launch for each
call; this tool runs the planner's tuning overrides (LQMM_TUNE_*, read on
every call) over a grid of values for one shape, times each variant the way
the benchmark does (cold weights rotated over >= 512 MiB of copies, HIP graph
of back-to-back launches between HIP events), checks every variant's output
against the default plan's, and prints a table, optionally as JSON and
markdown.

    python -m block_quantized_matmul_amd.tune --case q4_0_gemv_4096x4096_b1 \\
        --md profiles/tuning_q4_0_gemv_4096x4096_b1.md

Cases are the benchmark's shapes (synth.CONFIGS). Variants that the library
refuses for the shape (an override it cannot honour) are reported as such.
"""
from __future__ import annotations

import argparse
import itertools
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

ROTATE_BYTES = 512 * 2**20

# Override grids per kernel family: name -> list of {env: value} variants.
# The planner's default is always timed first ("default").
GEMV_SMALL = [dict(LQMM_TUNE_GEMV_SMALL="1", LQMM_TUNE_GEMV_SMALL_WAVES=str(w),
                   LQMM_TUNE_GEMV_SMALL_U=str(u), LQMM_TUNE_GEMV_SPLITK=str(s))
              for w, u, s in itertools.product((1, 2, 4, 8, 16), (1, 2), (1, 2, 4))]
GEMV_VALU = ([dict(LQMM_TUNE_GEMV_SMALL="0", LQMM_TUNE_GEMV_STREAM="1")] +
             [dict(LQMM_TUNE_GEMV_SMALL="0", LQMM_TUNE_GEMV_STREAM="0",
                   LQMM_TUNE_GEMV_R=str(r), LQMM_TUNE_GEMV_U=str(u),
                   LQMM_TUNE_GEMV_Q4_0_PAIR=str(p))
              for r, u, p in itertools.product((1, 2), (1, 2, 4), (0, 1))])
# (activations in LDS: also one or two super-chunks per row per chunk and the
# ring depth; activations in registers: a fixed ring)
GEMV_MFMA = ([dict(LQMM_TUNE_GEMV_SMALL="0", LQMM_TUNE_GEMV_WHOLE="0", LQMM_TUNE_GEMV_XREGS="0",
                   LQMM_TUNE_GEMV_KS=str(ks), LQMM_TUNE_GEMV_DEPTH=str(d), LQMM_TUNE_GEMV_U=str(u))
              for ks, d, u in itertools.product((1, 2, 4, 8), (2, 3, 4, 6), (1, 2))] +
             [dict(LQMM_TUNE_GEMV_SMALL="0", LQMM_TUNE_GEMV_WHOLE="0", LQMM_TUNE_GEMV_XREGS="1",
                   LQMM_TUNE_GEMV_KS=str(ks)) for ks in (1, 2, 4, 8)])
GEMV_WHOLE = [dict(LQMM_TUNE_GEMV_SMALL="0", LQMM_TUNE_GEMV_WHOLE=w) for w in ("0", "1")]
GEMM_Q8 = [dict(LQMM_TUNE_GEMM_WAVES=str(w)) for w in (7, 8)]


def _variants(kind, batch, fmt):
    if kind == "gemm":
        return GEMM_Q8 if fmt == "q8_0" else []
    if fmt in ("q8_0", "q6_k", "q2_k", "i4g32", "q1_0"):  # the small-problem kernel only
        return [v for v in GEMV_SMALL if v["LQMM_TUNE_GEMV_SPLITK"] != "4"]
    out = list(GEMV_SMALL) if batch <= 4 else []
    out += GEMV_VALU if batch <= 2 else []
    out += GEMV_WHOLE + GEMV_MFMA if batch >= 3 else []
    return out


def _setup(torch, name):
    """(kind, fmt, launch(), out tensor) for a benchmark shape; launch() runs
    one call on the next cold weight copy."""
    import numpy as np

    import block_quantized_matmul_amd as bq
    import synth

    kind = synth.CONFIGS[name]["kind"]
    c = synth.make(name)
    dev = torch.device("cuda:0")

    def rot(arr):
        t = torch.from_numpy(np.ascontiguousarray(arr).reshape(-1)).to(dev)
        n = max(2, math.ceil(ROTATE_BYTES / t.numel() / t.element_size()))
        return [t] + [t.clone() for _ in range(n - 1)]

    it = itertools.count()
    if kind in ("q4_0", "q4_k", "q8_0_gemv", "q6_k", "q2_k", "q1_0"):
        fmt = {"q8_0_gemv": "q8_0"}.get(kind, kind)
        fn = {"q4_0": bq.lqmm_gemv_q4_0, "q4_k": bq.lqmm_gemv_q4_k, "q8_0": bq.lqmm_gemv_q8_0,
              "q6_k": bq.lqmm_gemv_q6_k, "q2_k": bq.lqmm_gemv_q2_k, "q1_0": bq.lqmm_gemv_q1_0}[fmt]
        Ws, x = rot(c.W), torch.from_numpy(c.x.copy()).to(dev)
        y = torch.empty((c.batch, c.N), dtype=torch.float32, device=dev)
        return "gemv", fmt, c.batch, lambda: fn(Ws[next(it) % len(Ws)], x, c.N, out=y), y
    if kind == "i4g32":
        Wq, sc, z = rot(c.Wq.view(np.int32)), rot(c.scales), rot(c.zeros)
        x = torch.from_numpy(c.x.copy()).to(dev)
        y = torch.empty((c.batch, c.N), dtype=torch.float32, device=dev)

        def launch():
            i = next(it) % len(Wq)
            bq.lqmm_gemv_i4g32(Wq[i], sc[i].view(c.N, -1), z[i].view(c.N, -1), x, c.N, out=y)
        return "gemv", "i4g32", c.batch, launch, y
    if kind in ("q8_0", "q4_0_gemm", "q4_k_gemm"):
        fmt = {"q8_0": "q8_0", "q4_0_gemm": "q4_0", "q4_k_gemm": "q4_k"}[kind]
        fn = {"q8_0": bq.lqmm_gemm_q8_0_f16, "q4_0": bq.lqmm_gemm_q4_0_f16,
              "q4_k": bq.lqmm_gemm_q4_k_f16}[fmt]
        Ws, X = rot(c.W), torch.from_numpy(c.X).to(dev)
        Y = torch.empty((c.M, c.N), dtype=torch.float16, device=dev)
        return "gemm", fmt, c.M, lambda: fn(Ws[next(it) % len(Ws)], X, c.N, out=Y), Y
    raise SystemExit(f"no sweep for {name} ({kind})")


def _time(torch, launch, steps, reps=3):
    # warm-up calls on the capture stream: the binding's per-stream workspace
    # is allocated there, outside the graph (no zero fill recorded into it)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            launch()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(steps):
            launch()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.05:  # clocks up
        g.replay()
        torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return sorted(out)[len(out) // 2]


def sweep(name, steps=50, variants=None):
    import torch

    import block_quantized_matmul_amd as bq

    bq.load()
    torch.cuda.set_device(0)
    kind, fmt, rows, launch, out = _setup(torch, name)
    base_env = {k: v for k, v in os.environ.items() if k.startswith("LQMM_TUNE_")}
    for k in base_env:
        del os.environ[k]
    launch()
    torch.cuda.synchronize()
    ref = out.float().cpu()
    scale = float(ref.abs().max()) or 1.0
    results = []
    for v in [{}] + (variants if variants is not None else _variants(kind, rows, fmt)):
        for k in [k for k in os.environ if k.startswith("LQMM_TUNE_")]:
            del os.environ[k]
        os.environ.update(v)
        label = " ".join(f"{k[len('LQMM_TUNE_'):]}={val}" for k, val in v.items()) or "default"
        try:
            launch()
            torch.cuda.synchronize()
        except bq.LqmmError as e:
            results.append({"variant": label, "env": v, "status": f"refused: {e}"})
            continue
        err = float((out.float().cpu() - ref).abs().max()) / scale
        ms = _time(torch, launch, steps)
        results.append({"variant": label, "env": v, "us": round(ms * 1e3, 3),
                        "max_diff_vs_default": err, "status": "ok" if err <= 2e-3 else "MISMATCH"})
        print(f"[tune] {name} {label}: {ms * 1e3:.2f} us (diff {err:.1e})", file=sys.stderr,
              flush=True)
    for k in [k for k in os.environ if k.startswith("LQMM_TUNE_")]:
        del os.environ[k]
    os.environ.update(base_env)
    return {"case": name, "kind": kind, "format": fmt, "steps": steps, "results": results}


def to_markdown(rep, command):
    ok = [r for r in rep["results"] if r.get("status") == "ok"]
    best = min(ok, key=lambda r: r["us"]) if ok else None
    default = next((r for r in rep["results"] if r["variant"] == "default"), None)
    lines = [f"# Launch sweep: {rep['case']}\n\n",
             "Command, from the repository root on one MI355X (paths relative to the "
             "repository):\n\n", f"```\n{command}\n```\n\n"]
    if best and default and "us" in default:
        lines.append(f"Default plan {default['us']:.2f} us; best variant `{best['variant']}` "
                     f"{best['us']:.2f} us. Cold weights, graph of {rep['steps']} launches, median "
                     "of three replays.\n\n")
    lines.append("| variant | us | max diff vs default | status |\n|---|---:|---:|---|\n")
    for r in sorted(rep["results"], key=lambda r: r.get("us", 1e9)):
        us = f"{r['us']:.2f}" if "us" in r else "-"
        diff = f"{r['max_diff_vs_default']:.1e}" if "max_diff_vs_default" in r else "-"
        lines.append(f"| `{r['variant']}` | {us} | {diff} | {r['status']} |\n")
    return "".join(lines)


def main():
    p = argparse.ArgumentParser(description=__doc__,
                                formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--case", required=True)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--json", default="")
    p.add_argument("--md", default="")
    p.add_argument("--family", default="", choices=["", "small", "valu", "mfma", "whole"],
                   help="sweep one family of overrides only")
    args = p.parse_args()
    fam = {"small": GEMV_SMALL, "valu": GEMV_VALU, "mfma": GEMV_MFMA, "whole": GEMV_WHOLE}
    rep = sweep(args.case, args.steps, fam.get(args.family))
    if args.json:
        with open(args.json, "w") as f:
            json.dump(rep, f, indent=1)
    if args.md:
        cmd = "python -m block_quantized_matmul_amd.tune " + " ".join(sys.argv[1:])
        with open(args.md, "w") as f:
            f.write(to_markdown(rep, cmd))
    print(json.dumps({"case": rep["case"], "variants": len(rep["results"])}))


if __name__ == "__main__":
    main()
