"""Helpers for the GPU parity tests: device copies and the pass criteria."""
from __future__ import annotations

import sys

import numpy as np

import oracle

# Tolerances: both metrics (relative Frobenius, max-abs normalized by max|ref|)
TOL_FP32 = (1e-5, 1e-4)     # fp32 GEMM
TOL_QUANT = (2e-3, 2e-3)    # fp16-MFMA GEMM and quantized GEMVs


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def announce(msg: str):
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()
    sys.stderr.write(f"[gpu-case] {msg}\n")
    sys.stderr.flush()


def assert_close(G, R, tol, what=""):
    rel_fro, nmax = oracle.errors(G, R)
    assert rel_fro <= tol[0] and nmax <= tol[1], (
        f"{what}: rel_fro={rel_fro:.3e} (tol {tol[0]:.0e}) nmax={nmax:.3e} (tol {tol[1]:.0e})")
    return rel_fro, nmax
