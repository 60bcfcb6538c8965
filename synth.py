"""Seeded synthetic inputs for the block-quantized matmul hot path.

This module is shared by the tests, the benchmark and the smoke check. It
holds the random draws and the byte packing of the block formats, and none of
the arithmetic being checked: it never dequantizes a weight and never
multiplies anything. Both the HIP library and the CPU oracle read the bytes it
produces.

Workloads: synthetic Llama-shaped layers with the value distributions of the
benchmark configurations (the pages measure whole models whose weights are not
available; these seeded layers stand in for them):

* Q4_0 decode GEMV: fp16 scale d = |N(0,1)| * 0.02, codes q ~ U{0..15},
  x ~ N(0,1) fp32.
* Q8_0 x fp16 prefill GEMM: d = |N(0,1)| * 0.01, q ~ U{-127..127},
  X ~ N(0,1) rounded to fp16.
* Q4_K decode GEMV: d, dmin = |N(0,1)| * 0.01, 6-bit sc, m ~ U{0..63},
  q ~ U{0..15}, x ~ N(0,1) fp32.
* fp32 GEMM: A, B ~ U(-1, 1).
* The other format x phase pairs: Q8_0 decode GEMV (the Q8_0 draws, x ~
  N(0,1) fp32); Q4_0 and Q4_K x fp16 prefill GEMMs (the GEMV weight draws,
  X ~ N(0,1) rounded to fp16).
* Q6_K decode GEMV: d = |N(0,1)| * 0.002, int8 scales ~ U{-128..127}, 6-bit
  q ~ U{0..63}, x ~ N(0,1) fp32.
* Q2_K decode GEMV: d, dmin = |N(0,1)| * 0.01, 4-bit sc, m ~ U{0..15}, 2-bit
  q ~ U{0..3}, x ~ N(0,1) fp32.
* q1_0 decode GEMV (1-bit codes): d = |N(0,1)| * 0.02, codes c ~ U{0, 1}
  (weights -d or +d), x ~ N(0,1) fp32.
* int4 group-32 GEMV (GPTQ/AWQ-style layout): fp32 scales |N(0,1)| * 0.02,
  signed codes s ~ U{-8..7}, fp32 zero points ~ U{-8..7} (integers),
  x ~ N(0,1) fp32.

Every case draws from ``numpy.random.default_rng(seed)`` in the order: scales
(d, then dmin), codes (q, then sc, m), activations. fp16 values are rounded
from float64 with IEEE round-to-nearest-even (``astype(np.float16)``).

Byte layouts (llama.cpp / GGUF style; the pages name the formats, not their
bytes): see ``pack_q4_0``, ``pack_q8_0``, ``pack_q4_k``, ``pack_q6_k`` and
``pack_q2_k``; the 1-bit q1_0 reading: ``pack_q1_0``; the int4 layout of the
pages' int4 matmul: ``pack_i4g32``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

Q4_0_BYTES = 18   # per 32 weights
Q8_0_BYTES = 34   # per 32 weights
Q4_K_BYTES = 144  # per 256 weights
Q6_K_BYTES = 210  # per 256 weights
Q2_K_BYTES = 84   # per 256 weights
Q1_0_BYTES = 6    # per 32 weights


def _f16_bytes(a: np.ndarray) -> np.ndarray:
    """Little-endian bytes of an fp16 array, shape (..., 2)."""
    return np.ascontiguousarray(a.astype("<f2")).view(np.uint8).reshape(a.shape + (2,))


def pack_q4_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack Q4_0 blocks.

    d: (N, K/32) float16 scales. q: (N, K) codes in 0..15.
    Block = [d (2 bytes LE)][qs[16]]; weight j of the block sits in the low
    nibble of qs[j] for j < 16 and in the high nibble of qs[j-16] otherwise.
    Returns (N, K/32*18) uint8.
    """
    N, K = q.shape
    nb = K // 32
    qb = q.astype(np.uint8).reshape(N, nb, 32)
    qs = (qb[..., :16] & 0xF) | ((qb[..., 16:] & 0xF) << 4)
    blk = np.concatenate([_f16_bytes(d.reshape(N, nb)), qs], axis=-1)
    return np.ascontiguousarray(blk.reshape(N, nb * Q4_0_BYTES))


def pack_q8_0(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack Q8_0 blocks: [d (2 bytes LE)][q[32] as two's-complement int8].

    d: (N, K/32) float16. q: (N, K) int8. Returns (N, K/32*34) uint8.
    """
    N, K = q.shape
    nb = K // 32
    qb = q.astype(np.int8).view(np.uint8).reshape(N, nb, 32)
    blk = np.concatenate([_f16_bytes(d.reshape(N, nb)), qb], axis=-1)
    return np.ascontiguousarray(blk.reshape(N, nb * Q8_0_BYTES))


def pack_q4_k_scales(sc: np.ndarray, m: np.ndarray) -> np.ndarray:
    """Pack eight 6-bit (sc, m) pairs into the 12 scale bytes of a Q4_K block.

    Bytes 0-3: sc[0..3] in bits 0-5, bits 4-5 of sc[4..7] in bits 6-7.
    Bytes 4-7: m[0..3] in bits 0-5, bits 4-5 of m[4..7] in bits 6-7.
    Bytes 8-11: bits 0-3 of sc[4..7] (low nibble), bits 0-3 of m[4..7]
    (high nibble). sc, m: (..., 8) integers in 0..63. Returns (..., 12) uint8.
    """
    sc = sc.astype(np.uint8)
    m = m.astype(np.uint8)
    b0 = (sc[..., 0:4] & 63) | ((sc[..., 4:8] >> 4) << 6)
    b1 = (m[..., 0:4] & 63) | ((m[..., 4:8] >> 4) << 6)
    b2 = (sc[..., 4:8] & 15) | ((m[..., 4:8] & 15) << 4)
    return np.concatenate([b0, b1, b2], axis=-1).astype(np.uint8)


def pack_q4_k(d, dmin, sc, m, q) -> np.ndarray:
    """Pack Q4_K super-blocks of 256 weights (144 bytes each).

    Layout: [d (2)][dmin (2)][scales (12)][qs (128)]. Sub-block s holds
    weights 32s..32s+31; its codes are the low nibbles (even s) or high
    nibbles (odd s) of qs[32*(s//2) .. 32*(s//2)+31].
    d, dmin: (N, K/256) float16; sc, m: (N, K/256, 8) in 0..63;
    q: (N, K) in 0..15. Returns (N, K/256*144) uint8.
    """
    N, K = q.shape
    nsb = K // 256
    qb = q.astype(np.uint8).reshape(N, nsb, 4, 2, 32)
    qs = ((qb[:, :, :, 0, :] & 0xF) | ((qb[:, :, :, 1, :] & 0xF) << 4)).reshape(N, nsb, 128)
    blk = np.concatenate(
        [_f16_bytes(d.reshape(N, nsb)), _f16_bytes(dmin.reshape(N, nsb)),
         pack_q4_k_scales(sc.reshape(N, nsb, 8), m.reshape(N, nsb, 8)), qs],
        axis=-1)
    return np.ascontiguousarray(blk.reshape(N, nsb * Q4_K_BYTES))


def pack_q6_k(d, sc, q) -> np.ndarray:
    """Pack Q6_K super-blocks of 256 weights (210 bytes each).

    Layout: [ql (128)][qh (64)][scales (16, int8)][d (2)]. Weight
    k = 128h + 32j + l (h < 2, j < 4, l < 32): its low 4 bits are the low
    (j < 2) or high (j >= 2) nibble of ql[64h + l + 32*(j % 2)], its high 2
    bits are bits 2j..2j+1 of qh[32h + l]; its scale is scales[k // 16].
    d: (N, K/256) float16; sc: (N, K/256, 16) int8; q: (N, K) in 0..63.
    Returns (N, K/256*210) uint8.
    """
    N, K = q.shape
    nsb = K // 256
    qb = q.astype(np.uint8).reshape(N, nsb, 2, 4, 32)     # [h, j, l]
    low, high = qb & 15, qb >> 4
    ql = (low[:, :, :, 0:2, :] | (low[:, :, :, 2:4, :] << 4)).reshape(N, nsb, 128)
    qh = np.zeros((N, nsb, 2, 32), np.uint8)
    for j in range(4):
        qh |= (high[:, :, :, j, :] & 3) << (2 * j)
    blk = np.concatenate([ql, qh.reshape(N, nsb, 64),
                          sc.astype(np.int8).view(np.uint8).reshape(N, nsb, 16),
                          _f16_bytes(d.reshape(N, nsb))], axis=-1)
    return np.ascontiguousarray(blk.reshape(N, nsb * Q6_K_BYTES))


def pack_q2_k(d, dmin, sc, m, q) -> np.ndarray:
    """Pack Q2_K super-blocks of 256 weights (84 bytes each).

    Layout: [scales (16)][qs (64)][d (2)][dmin (2)]; scales[g] holds the
    4-bit scale sc (low nibble) and min m (high nibble) of weights 16g..16g+15.
    Weight k = 128h + 32j + l is bits 2j..2j+1 of qs[32h + l].
    d, dmin: (N, K/256) float16; sc, m: (N, K/256, 16) in 0..15;
    q: (N, K) in 0..3. Returns (N, K/256*84) uint8.
    """
    N, K = q.shape
    nsb = K // 256
    qb = q.astype(np.uint8).reshape(N, nsb, 2, 4, 32)     # [h, j, l]
    qs = np.zeros((N, nsb, 2, 32), np.uint8)
    for j in range(4):
        qs |= (qb[:, :, :, j, :] & 3) << (2 * j)
    scales = (sc.astype(np.uint8) & 15) | ((m.astype(np.uint8) & 15) << 4)
    blk = np.concatenate([scales.reshape(N, nsb, 16), qs.reshape(N, nsb, 64),
                          _f16_bytes(d.reshape(N, nsb)), _f16_bytes(dmin.reshape(N, nsb))],
                         axis=-1)
    return np.ascontiguousarray(blk.reshape(N, nsb * Q2_K_BYTES))


def pack_q1_0(d: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Pack q1_0 blocks: [d (2 bytes LE)][32 code bits in 4 bytes], the bit
    of weight j at bit j % 8 of byte j // 8 (least significant bit first).

    d: (N, K/32) float16 scales. c: (N, K) codes in {0, 1}.
    Returns (N, K/32 * 6) uint8.
    """
    N, K = c.shape
    nb = K // 32
    bits = np.packbits(c.astype(np.uint8).reshape(N, nb, 32), axis=-1, bitorder="little")
    blk = np.concatenate([_f16_bytes(d.reshape(N, nb)), bits], axis=-1)
    return np.ascontiguousarray(blk.reshape(N, nb * Q1_0_BYTES))


def pack_i4g32(s: np.ndarray) -> np.ndarray:
    """Pack signed 4-bit codes, eight per 32-bit word: code (n, k) is nibble
    (n*K + k) % 8 (bits 4i..4i+3) of word (n*K + k) // 8, two's complement.
    s: (N, K) integers in -8..7, N*K a multiple of 8. Returns (N*K/8,) uint32.
    """
    nib = (s.astype(np.int64).reshape(-1, 8) & 15).astype(np.uint32)
    shifts = (4 * np.arange(8)).astype(np.uint32)
    return np.bitwise_or.reduce(nib << shifts, axis=1).astype(np.uint32)


def _half_normal_f16(rng, shape, scale):
    return (np.abs(rng.standard_normal(shape)) * scale).astype(np.float16)


@dataclasses.dataclass
class Q4_0Case:
    W: np.ndarray      # (N, K/32*18) uint8
    x: np.ndarray      # (batch, K) float32
    d: np.ndarray      # (N, K/32) float16
    q: np.ndarray      # (N, K) uint8
    N: int
    K: int
    batch: int


@dataclasses.dataclass
class Q4_KCase:
    W: np.ndarray      # (N, K/256*144) uint8
    x: np.ndarray      # (batch, K) float32
    d: np.ndarray
    dmin: np.ndarray
    sc: np.ndarray     # (N, K/256, 8)
    m: np.ndarray      # (N, K/256, 8)
    q: np.ndarray      # (N, K)
    N: int
    K: int
    batch: int


@dataclasses.dataclass
class Q8_0Case:
    W: np.ndarray      # (N, K/32*34) uint8
    X: np.ndarray      # (M, K) float16
    d: np.ndarray
    q: np.ndarray      # (N, K) int8
    M: int
    N: int
    K: int


@dataclasses.dataclass
class Q8_0GemvCase:
    W: np.ndarray      # (N, K/32*34) uint8
    x: np.ndarray      # (batch, K) float32
    d: np.ndarray
    q: np.ndarray      # (N, K) int8
    N: int
    K: int
    batch: int


@dataclasses.dataclass
class Q1_0Case:
    W: np.ndarray      # (N, K/32*6) uint8
    x: np.ndarray      # (batch, K) float32
    d: np.ndarray      # (N, K/32) float16
    c: np.ndarray      # (N, K) uint8 codes in {0, 1}
    N: int
    K: int
    batch: int


@dataclasses.dataclass
class GemmCase:
    """A quantized weight matrix (any block format) times fp16 activations."""
    W: np.ndarray      # (N, bytes per row) uint8
    X: np.ndarray      # (M, K) float16
    w: object          # the weight draws (a Q4_0Case or Q4_KCase with batch 0)
    M: int
    N: int
    K: int


@dataclasses.dataclass
class Q6_KCase:
    W: np.ndarray      # (N, K/256*210) uint8
    x: np.ndarray
    d: np.ndarray      # (N, K/256) float16
    sc: np.ndarray     # (N, K/256, 16) int8
    q: np.ndarray      # (N, K) in 0..63
    N: int
    K: int
    batch: int


@dataclasses.dataclass
class Q2_KCase:
    W: np.ndarray      # (N, K/256*84) uint8
    x: np.ndarray
    d: np.ndarray
    dmin: np.ndarray
    sc: np.ndarray     # (N, K/256, 16) in 0..15
    m: np.ndarray      # (N, K/256, 16) in 0..15
    q: np.ndarray      # (N, K) in 0..3
    N: int
    K: int
    batch: int


@dataclasses.dataclass
class I4G32Case:
    Wq: np.ndarray     # (N*K/8,) uint32
    scales: np.ndarray  # (N, K/32) float32
    zeros: np.ndarray   # (N, K/32) float32
    s: np.ndarray      # (N, K) int8 in -8..7
    x: np.ndarray
    N: int
    K: int
    batch: int


@dataclasses.dataclass
class SgemmCase:
    A: np.ndarray      # (M, K) float32
    B: np.ndarray      # (K, N) float32
    M: int
    N: int
    K: int


def q4_0_case(N: int, K: int, batch: int = 1, seed: int = 0, scale: float = 0.02) -> Q4_0Case:
    assert K % 32 == 0
    rng = np.random.default_rng(seed)
    d = _half_normal_f16(rng, (N, K // 32), scale)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    return Q4_0Case(pack_q4_0(d, q), x, d, q, N, K, batch)


def q4_k_case(N: int, K: int, batch: int = 1, seed: int = 0, scale: float = 0.01) -> Q4_KCase:
    assert K % 256 == 0
    rng = np.random.default_rng(seed)
    nsb = K // 256
    d = _half_normal_f16(rng, (N, nsb), scale)
    dmin = _half_normal_f16(rng, (N, nsb), scale)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    sc = rng.integers(0, 64, size=(N, nsb, 8), dtype=np.uint8)
    m = rng.integers(0, 64, size=(N, nsb, 8), dtype=np.uint8)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    return Q4_KCase(pack_q4_k(d, dmin, sc, m, q), x, d, dmin, sc, m, q, N, K, batch)


def q8_0_case(M: int, N: int, K: int, seed: int = 0, scale: float = 0.01) -> Q8_0Case:
    assert K % 32 == 0
    rng = np.random.default_rng(seed)
    d = _half_normal_f16(rng, (N, K // 32), scale)
    q = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    X = rng.standard_normal((M, K)).astype(np.float16)
    return Q8_0Case(pack_q8_0(d, q), X, d, q, M, N, K)


def q8_0_gemv_case(N: int, K: int, batch: int = 1, seed: int = 0,
                   scale: float = 0.01) -> Q8_0GemvCase:
    assert K % 32 == 0
    rng = np.random.default_rng(seed)
    d = _half_normal_f16(rng, (N, K // 32), scale)
    q = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    return Q8_0GemvCase(pack_q8_0(d, q), x, d, q, N, K, batch)


def q4_0_gemm_case(M: int, N: int, K: int, seed: int = 0) -> GemmCase:
    w = q4_0_case(N, K, 0, seed)
    X = np.random.default_rng(seed + 7919).standard_normal((M, K)).astype(np.float16)
    return GemmCase(w.W, X, w, M, N, K)


def q4_k_gemm_case(M: int, N: int, K: int, seed: int = 0) -> GemmCase:
    w = q4_k_case(N, K, 0, seed)
    X = np.random.default_rng(seed + 7919).standard_normal((M, K)).astype(np.float16)
    return GemmCase(w.W, X, w, M, N, K)


def q6_k_case(N: int, K: int, batch: int = 1, seed: int = 0, scale: float = 0.002) -> Q6_KCase:
    assert K % 256 == 0
    rng = np.random.default_rng(seed)
    nsb = K // 256
    d = _half_normal_f16(rng, (N, nsb), scale)
    q = rng.integers(0, 64, size=(N, K), dtype=np.uint8)
    sc = rng.integers(-128, 128, size=(N, nsb, 16)).astype(np.int8)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    return Q6_KCase(pack_q6_k(d, sc, q), x, d, sc, q, N, K, batch)


def q2_k_case(N: int, K: int, batch: int = 1, seed: int = 0, scale: float = 0.01) -> Q2_KCase:
    assert K % 256 == 0
    rng = np.random.default_rng(seed)
    nsb = K // 256
    d = _half_normal_f16(rng, (N, nsb), scale)
    dmin = _half_normal_f16(rng, (N, nsb), scale)
    q = rng.integers(0, 4, size=(N, K), dtype=np.uint8)
    sc = rng.integers(0, 16, size=(N, nsb, 16), dtype=np.uint8)
    m = rng.integers(0, 16, size=(N, nsb, 16), dtype=np.uint8)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    return Q2_KCase(pack_q2_k(d, dmin, sc, m, q), x, d, dmin, sc, m, q, N, K, batch)


def q1_0_case(N: int, K: int, batch: int = 1, seed: int = 0, scale: float = 0.02) -> Q1_0Case:
    assert K % 32 == 0
    rng = np.random.default_rng(seed)
    d = _half_normal_f16(rng, (N, K // 32), scale)
    c = rng.integers(0, 2, size=(N, K), dtype=np.uint8)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    return Q1_0Case(pack_q1_0(d, c), x, d, c, N, K, batch)


def i4g32_case(N: int, K: int, batch: int = 1, seed: int = 0, scale: float = 0.02) -> I4G32Case:
    assert K % 32 == 0
    rng = np.random.default_rng(seed)
    scales = (np.abs(rng.standard_normal((N, K // 32))) * scale).astype(np.float32)
    s = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    zeros = rng.integers(-8, 8, size=(N, K // 32)).astype(np.float32)
    x = rng.standard_normal((batch, K)).astype(np.float32)
    return I4G32Case(pack_i4g32(s), scales, zeros, s, x, N, K, batch)


def sgemm_case(M: int, N: int, K: int, seed: int = 0) -> SgemmCase:
    rng = np.random.default_rng(seed)
    A = rng.uniform(-1.0, 1.0, (M, K)).astype(np.float32)
    B = rng.uniform(-1.0, 1.0, (K, N)).astype(np.float32)
    return SgemmCase(A, B, M, N, K)


# The benchmark configurations, by what they are.
CONFIGS = {
    # Q4_0 GEMV, 1024 out x 1024 in, batch 1, seed 0 (the small parity case)
    "q4_0_gemv_1024": dict(kind="q4_0", N=1024, K=1024, batch=1),
    # dense fp32 tiled GEMM, M = N = K = 2048
    "sgemm_2048": dict(kind="sgemm", M=2048, N=2048, K=2048),
    # Q4_0 decode GEMV at 7B-layer shapes, K = 4096
    "q4_0_gemv_4096x4096_b1": dict(kind="q4_0", N=4096, K=4096, batch=1),
    "q4_0_gemv_4096x4096_b4": dict(kind="q4_0", N=4096, K=4096, batch=4),
    "q4_0_gemv_11008x4096_b1": dict(kind="q4_0", N=11008, K=4096, batch=1),
    "q4_0_gemv_11008x4096_b4": dict(kind="q4_0", N=11008, K=4096, batch=4),
    "q4_0_gemv_12288x4096_b1": dict(kind="q4_0", N=12288, K=4096, batch=1),
    "q4_0_gemv_12288x4096_b4": dict(kind="q4_0", N=12288, K=4096, batch=4),
    # Q8_0 x fp16 prefill GEMM, 512 tokens, N = 14336, K = 4096
    "q8_0_gemm_512x14336x4096": dict(kind="q8_0", M=512, N=14336, K=4096),
    # Q4_K GEMV at a 70B FFN shape, K = 8192, N = 28672
    "q4_k_gemv_28672x8192_b1": dict(kind="q4_k", N=28672, K=8192, batch=1),
    "q4_k_gemv_28672x8192_b8": dict(kind="q4_k", N=28672, K=8192, batch=8),
    # the other format x phase pairs at the same layer shapes
    "q8_0_gemv_4096x4096_b1": dict(kind="q8_0_gemv", N=4096, K=4096, batch=1),
    "q8_0_gemv_11008x4096_b1": dict(kind="q8_0_gemv", N=11008, K=4096, batch=1),
    "q8_0_gemv_12288x4096_b4": dict(kind="q8_0_gemv", N=12288, K=4096, batch=4),
    "q4_0_gemm_512x14336x4096": dict(kind="q4_0_gemm", M=512, N=14336, K=4096),
    "q4_k_gemm_512x14336x4096": dict(kind="q4_k_gemm", M=512, N=14336, K=4096),
    # more block formats: 6-bit and 2-bit K-quants, the int4 group-32 layout
    "q6_k_gemv_11008x4096_b1": dict(kind="q6_k", N=11008, K=4096, batch=1),
    "q2_k_gemv_11008x4096_b1": dict(kind="q2_k", N=11008, K=4096, batch=1),
    "i4g32_gemv_11008x4096_b1": dict(kind="i4g32", N=11008, K=4096, batch=1),
    "q1_0_gemv_11008x4096_b1": dict(kind="q1_0", N=11008, K=4096, batch=1),
}


def make(name: str, seed: int = 0):
    c = dict(CONFIGS[name])
    kind = c.pop("kind")
    if kind == "q4_0":
        return q4_0_case(c["N"], c["K"], c["batch"], seed)
    if kind == "q4_k":
        return q4_k_case(c["N"], c["K"], c["batch"], seed)
    if kind == "q8_0":
        return q8_0_case(c["M"], c["N"], c["K"], seed)
    if kind == "sgemm":
        return sgemm_case(c["M"], c["N"], c["K"], seed)
    if kind == "q8_0_gemv":
        return q8_0_gemv_case(c["N"], c["K"], c["batch"], seed)
    if kind == "q4_0_gemm":
        return q4_0_gemm_case(c["M"], c["N"], c["K"], seed)
    if kind == "q4_k_gemm":
        return q4_k_gemm_case(c["M"], c["N"], c["K"], seed)
    if kind == "q6_k":
        return q6_k_case(c["N"], c["K"], c["batch"], seed)
    if kind == "q1_0":
        return q1_0_case(c["N"], c["K"], c["batch"], seed)
    if kind == "q2_k":
        return q2_k_case(c["N"], c["K"], c["batch"], seed)
    if kind == "i4g32":
        return i4g32_case(c["N"], c["K"], c["batch"], seed)
    raise KeyError(name)
