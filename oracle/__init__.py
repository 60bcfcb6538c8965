"""CPU oracle for the block-quantized matmul hot path (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product library never loads it, and it shares no
code with the HIP path. The arithmetic lives in ``lqmm_oracle.c`` (plain C,
IEEE double, OpenMP over output rows); this module compiles it with gcc and
wraps it with ctypes and numpy arrays.

Every function returns float64 results of the dequantize-then-multiply
definition; see the header of ``lqmm_oracle.c`` for the block layouts and the
passages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lqmm_oracle.c")
LIB = os.path.join(HERE, "liblqmm_oracle.so")

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra"]


def build(mutant: int = 0, out: str | None = None) -> str:
    """Compile the oracle with gcc. ``mutant`` != 0 plants a known mistake
    (used only by the test that checks the pins catch it)."""
    out = out or LIB
    cmd = ["gcc", *_CFLAGS, f"-DLQMM_ORACLE_MUTANT={int(mutant)}", SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_i64 = ctypes.c_int64
_p = ctypes.c_void_p


class Oracle:
    """ctypes view of one built oracle library."""

    def __init__(self, path: str = LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.lqmm_oracle_f16_to_f64.restype = ctypes.c_double
        lib.lqmm_oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.lqmm_oracle_f16_array_to_f64.argtypes = [_p, _p, _i64]
        for name in ("lqmm_oracle_dequant_q4_0", "lqmm_oracle_dequant_q8_0",
                     "lqmm_oracle_dequant_q4_k", "lqmm_oracle_dequant_q6_k",
                     "lqmm_oracle_dequant_q2_k", "lqmm_oracle_dequant_q1_0"):
            getattr(lib, name).argtypes = [_p, _i64, _i64, _p]
        lib.lqmm_oracle_dequant_i4g32.argtypes = [_p, _p, _p, _i64, _i64, _p]
        for name in ("lqmm_oracle_gemv_q4_0", "lqmm_oracle_gemv_q4_k", "lqmm_oracle_gemv_q8_0",
                     "lqmm_oracle_gemv_q6_k", "lqmm_oracle_gemv_q2_k", "lqmm_oracle_gemv_q1_0"):
            getattr(lib, name).argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _i64]
        lib.lqmm_oracle_gemv_i4g32.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64]
        for name in ("lqmm_oracle_gemm_q8_0_f16", "lqmm_oracle_gemm_q4_0_f16",
                     "lqmm_oracle_gemm_q4_k_f16"):
            getattr(lib, name).argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _i64]
        lib.lqmm_oracle_sgemm.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _i64]
        lib.lqmm_oracle_mutant.restype = ctypes.c_int
        lib.lqmm_oracle_threads.restype = ctypes.c_int
        lib.lqmm_oracle_set_threads.argtypes = [ctypes.c_int]
        lib.lqmm_oracle_set_threads.restype = None
        self.lib = lib

    @property
    def threads(self) -> int:
        """OpenMP threads the oracle's loops use."""
        return self.lib.lqmm_oracle_threads()

    def set_threads(self, n: int) -> None:
        """Run the oracle's loops on n OpenMP threads."""
        self.lib.lqmm_oracle_set_threads(int(n))

    @property
    def mutant(self) -> int:
        return self.lib.lqmm_oracle_mutant()

    # -- decoders -----------------------------------------------------------
    def f16_to_f64(self, bits) -> np.ndarray:
        h = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
        out = np.empty(h.shape, np.float64)
        self.lib.lqmm_oracle_f16_array_to_f64(h.ctypes.data, out.ctypes.data, h.size)
        return out

    def _dequant(self, fn, W, N, K):
        W = np.ascontiguousarray(W, dtype=np.uint8)
        out = np.empty((N, K), np.float64)
        getattr(self.lib, fn)(W.ctypes.data, N, K, out.ctypes.data)
        return out

    def dequant_q4_0(self, W, N, K):
        return self._dequant("lqmm_oracle_dequant_q4_0", W, N, K)

    def dequant_q8_0(self, W, N, K):
        return self._dequant("lqmm_oracle_dequant_q8_0", W, N, K)

    def dequant_q4_k(self, W, N, K):
        return self._dequant("lqmm_oracle_dequant_q4_k", W, N, K)

    def dequant_q6_k(self, W, N, K):
        return self._dequant("lqmm_oracle_dequant_q6_k", W, N, K)

    def dequant_q2_k(self, W, N, K):
        return self._dequant("lqmm_oracle_dequant_q2_k", W, N, K)

    def dequant_q1_0(self, W, N, K):
        return self._dequant("lqmm_oracle_dequant_q1_0", W, N, K)

    def dequant_i4g32(self, Wq, scales, zeros, N, K):
        Wq = np.ascontiguousarray(Wq, dtype=np.uint32)
        sc = np.ascontiguousarray(scales, dtype=np.float32)
        z = np.ascontiguousarray(zeros, dtype=np.float32)
        out = np.empty((N, K), np.float64)
        self.lib.lqmm_oracle_dequant_i4g32(Wq.ctypes.data, sc.ctypes.data, z.ctypes.data, N, K,
                                           out.ctypes.data)
        return out

    # -- products -----------------------------------------------------------
    @staticmethod
    def _sel(idx):
        if idx is None:
            return None, 0, None
        a = np.ascontiguousarray(np.asarray(idx, dtype=np.int64))
        return a, a.size, a.ctypes.data

    def _gemv(self, fn, W, x, N, K, rows):
        W = np.ascontiguousarray(W, dtype=np.uint8)
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
        assert x.shape[1] == K
        b = x.shape[0]
        keep, nr, rp = self._sel(rows)
        R = nr if rows is not None else N
        y = np.empty((b, R), np.float64)
        getattr(self.lib, fn)(W.ctypes.data, x.ctypes.data, y.ctypes.data, N, K, b, rp, nr)
        del keep
        return y

    def gemv_q4_0(self, W, x, N, K, rows=None) -> np.ndarray:
        """y[b, n] = sum_k W[n, k] x[b, k]; returns (batch, N or len(rows))."""
        return self._gemv("lqmm_oracle_gemv_q4_0", W, x, N, K, rows)

    def gemv_q4_k(self, W, x, N, K, rows=None) -> np.ndarray:
        return self._gemv("lqmm_oracle_gemv_q4_k", W, x, N, K, rows)

    def gemv_q8_0(self, W, x, N, K, rows=None) -> np.ndarray:
        return self._gemv("lqmm_oracle_gemv_q8_0", W, x, N, K, rows)

    def gemv_q6_k(self, W, x, N, K, rows=None) -> np.ndarray:
        return self._gemv("lqmm_oracle_gemv_q6_k", W, x, N, K, rows)

    def gemv_q2_k(self, W, x, N, K, rows=None) -> np.ndarray:
        return self._gemv("lqmm_oracle_gemv_q2_k", W, x, N, K, rows)

    def gemv_q1_0(self, W, x, N, K, rows=None) -> np.ndarray:
        return self._gemv("lqmm_oracle_gemv_q1_0", W, x, N, K, rows)

    def gemv_i4g32(self, Wq, scales, zeros, x, N, K, rows=None) -> np.ndarray:
        """The int4 group-32 layout: Wq uint32 words (N*K/8), scales and zeros
        float32 (N, K/32); returns (batch, N or len(rows))."""
        Wq = np.ascontiguousarray(Wq, dtype=np.uint32)
        sc = np.ascontiguousarray(scales, dtype=np.float32)
        z = np.ascontiguousarray(zeros, dtype=np.float32)
        x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
        assert x.shape[1] == K
        b = x.shape[0]
        keep, nr, rp = self._sel(rows)
        R = nr if rows is not None else N
        y = np.empty((b, R), np.float64)
        self.lib.lqmm_oracle_gemv_i4g32(Wq.ctypes.data, sc.ctypes.data, z.ctypes.data,
                                        x.ctypes.data, y.ctypes.data, N, K, b, rp, nr)
        del keep
        return y

    def _gemm(self, fn, W, X, N, K, cols):
        W = np.ascontiguousarray(W, dtype=np.uint8)
        Xb = np.ascontiguousarray(np.asarray(X, dtype=np.float16)).view(np.uint16)
        M = Xb.shape[0]
        assert Xb.shape[1] == K
        keep, nc, cp = self._sel(cols)
        C = nc if cols is not None else N
        Y = np.empty((M, C), np.float64)
        getattr(self.lib, fn)(W.ctypes.data, Xb.ctypes.data, Y.ctypes.data, M, N, K, cp, nc)
        del keep
        return Y

    def gemm_q8_0_f16(self, W, X, N, K, cols=None) -> np.ndarray:
        """Y[m, n] = sum_k X[m, k] W[n, k]; X is fp16 (M, K); returns float64
        (M, N or len(cols))."""
        return self._gemm("lqmm_oracle_gemm_q8_0_f16", W, X, N, K, cols)

    def gemm_q4_0_f16(self, W, X, N, K, cols=None) -> np.ndarray:
        return self._gemm("lqmm_oracle_gemm_q4_0_f16", W, X, N, K, cols)

    def gemm_q4_k_f16(self, W, X, N, K, cols=None) -> np.ndarray:
        return self._gemm("lqmm_oracle_gemm_q4_k_f16", W, X, N, K, cols)

    def sgemm(self, A, B, rows=None) -> np.ndarray:
        """C = A @ B in double; A (M, K) fp32, B (K, N) fp32."""
        A = np.ascontiguousarray(A, dtype=np.float32)
        B = np.ascontiguousarray(B, dtype=np.float32)
        M, K = A.shape
        K2, N = B.shape
        assert K == K2
        keep, nr, rp = self._sel(rows)
        R = nr if rows is not None else M
        C = np.empty((R, N), np.float64)
        self.lib.lqmm_oracle_sgemm(A.ctypes.data, B.ctypes.data, C.ctypes.data, M, N, K, rp, nr)
        del keep
        return C


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from the unmodified source (compiled on first use if
    the library is missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default


def errors(G, R):
    """(rel_fro, nmax): ||G-R||_F / ||R||_F and max|G-R| / max|R|, in double."""
    G = np.asarray(G, np.float64)
    R = np.asarray(R, np.float64)
    diff = G - R
    rr = np.linalg.norm(R)
    mr = np.max(np.abs(R)) if R.size else 0.0
    rel_fro = float(np.linalg.norm(diff) / rr) if rr > 0 else float(np.linalg.norm(diff))
    nmax = float(np.max(np.abs(diff)) / mr) if mr > 0 else float(np.max(np.abs(diff), initial=0.0))
    return rel_fro, nmax
