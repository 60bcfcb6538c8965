"""Build liblqmm.so (HIP, gfx950) in-tree with hipcc, and the benchmark's
streaming-read probe (liblqmm_probe.so).

Each source is compiled to an object in parallel, then the objects are linked
into the shared library.

Usage: python -m block_quantized_matmul_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblqmm.so")
SOURCES = ["api.hip", "gemv.hip", "gemv_small.hip", "gemv_small_more.hip", "gemm_q8_0.hip",
           "gemm_lds.hip", "sgemm.hip", "gemv_whole.hip"]
PROBE_LIB = os.path.join(HERE, "liblqmm_probe.so")
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {what}")
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                    and "not a recognized feature" not in l)
    if verbose and err.strip():
        sys.stderr.write(err + "\n")


def _hipcc(sources, lib, verbose):
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in sources]
    jobs = [([HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o], s, verbose)
            for s, o in zip(sources, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for f in [ex.submit(_run, *j) for j in jobs]:
            f.result()
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
         os.path.basename(lib), verbose)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _hipcc(PROBE_SOURCES, PROBE_LIB, verbose)
    return _hipcc(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
