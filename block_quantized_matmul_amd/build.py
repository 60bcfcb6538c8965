"""Build liblqmm.so (HIP, gfx950) in-tree with hipcc, and the benchmark's
streaming-read probe (liblqmm_probe.so).

Usage: python -m block_quantized_matmul_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblqmm.so")
SOURCES = ["api.hip", "gemv.hip", "gemm_q8_0.hip", "sgemm.hip"]
PROBE_LIB = os.path.join(HERE, "liblqmm_probe.so")
PROBE_SOURCES = ["probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc(sources, lib, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l
                    and "not a recognized feature" not in l)
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _hipcc(PROBE_SOURCES, PROBE_LIB, verbose)
    return _hipcc(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
