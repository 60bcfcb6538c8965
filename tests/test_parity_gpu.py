"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on
the same seeded inputs, element by element.

Bars: relative Frobenius and normalized max-abs error <= 1e-5 / 1e-4 for the
fp32 GEMM and <= 2e-3 for the quantized GEMVs and the Q8_0 x fp16 GEMM;
bit-exact where the arithmetic is exact (one-hot activations, identity
matrices). Full benchmark sizes are checked in the launch configuration the
benchmark uses (the library picks it from the shape), on all outputs where
the oracle is cheap and on sampled outputs otherwise.
"""
import numpy as np
import pytest

import block_quantized_matmul_amd as bq
import synth
from gpu_util import TOL_FP32, TOL_QUANT, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bq.load()


def _run_q4_0(c):
    y = bq.lqmm_gemv_q4_0(dev(c.W.reshape(-1)), dev(c.x), c.N)
    return host(y)


def _run_q4_k(c):
    y = bq.lqmm_gemv_q4_k(dev(c.W.reshape(-1)), dev(c.x), c.N)
    return host(y)


# ----------------------------------------------------------------- Q4_0 GEMV
Q4_0_SMALL = [(1, 32, 1), (7, 32, 3), (5, 64, 2), (13, 96, 1), (33, 288, 5), (64, 1024, 8),
              (100, 4096, 4), (1, 4096, 9), (3, 9216, 8), (257, 2048, 16), (2, 160, 7),
              (1000, 512, 1), (31, 8192, 2), (17, 1024, 17), (40, 18432, 18), (129, 4096, 3),
              (16, 512, 16), (3, 36864, 3),
              # matrix-core path through the coalesced kernel (K a multiple of
              # 256): one super-chunk, ragged tiles, several slices and K-split
              # launches
              (257, 256, 5), (33, 768, 16), (300, 2048, 3), (17, 512, 40), (1, 256, 3),
              (3, 36864, 4), (4096, 4096, 4)]


# Each shape with the planner's choice, and with the small-problem kernel
# switched off (so that the shapes it takes also reach the other kernels).
@pytest.mark.parametrize("small", ["default", "0"])
@pytest.mark.parametrize("N,K,B", Q4_0_SMALL)
def test_q4_0_small(orc, monkeypatch, small, N, K, B):
    if small != "default":
        monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", small)
    c = synth.q4_0_case(N, K, B, seed=N * 7 + K + B)
    announce(f"q4_0 gemv N={N} K={K} batch={B}")
    y = _run_q4_0(c)
    ref = orc.gemv_q4_0(c.W, c.x, N, K)
    assert_close(y, ref, TOL_QUANT, f"q4_0 {N}x{K} b{B}")


@pytest.mark.parametrize("pair", [0, 1])
@pytest.mark.parametrize("N,K,B", [(1, 64, 1), (7, 128, 2), (13, 96, 1), (33, 4096, 1),
                                   (1000, 512, 1), (64, 1024, 2), (2, 160, 2),
                                   # K split over launches that accumulate into y
                                   (5, 73728, 1), (5, 73728, 2), (3, 73760, 1)])
def test_q4_0_dot2_units(orc, monkeypatch, pair, N, K, B):
    # the dot2 path (batch <= 2) with one block per unit and with two (taken
    # only when K % 64 == 0), forced through the planner's tuning override
    # (the small-problem kernel, which would take most of these, is off)
    monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", "0")
    monkeypatch.setenv("LQMM_TUNE_GEMV_Q4_0_PAIR", str(pair))
    c = synth.q4_0_case(N, K, B, seed=N * 5 + K + B + pair)
    announce(f"q4_0 gemv N={N} K={K} batch={B} pair={pair}")
    y = _run_q4_0(c)
    ref = orc.gemv_q4_0(c.W, c.x, N, K)
    assert_close(y, ref, TOL_QUANT, f"q4_0 {N}x{K} b{B} pair={pair}")


@pytest.mark.parametrize("name", ["q4_0_gemv_1024", "q4_0_gemv_4096x4096_b1",
                                  "q4_0_gemv_4096x4096_b4", "q4_0_gemv_11008x4096_b1",
                                  "q4_0_gemv_11008x4096_b4", "q4_0_gemv_12288x4096_b1",
                                  "q4_0_gemv_12288x4096_b4"])
def test_q4_0_configs(orc, name):
    c = synth.make(name)
    announce(f"{name}")
    y = _run_q4_0(c)
    ref = orc.gemv_q4_0(c.W, c.x, c.N, c.K)
    assert_close(y, ref, TOL_QUANT, name)


@pytest.mark.parametrize("pair", [0, 1])
def test_q4_0_one_hot_exact(orc, monkeypatch, pair):
    """One-hot activations extract weight columns. dot2 path (batch <= 2),
    with one or two blocks per unit: bit-exact (x = 1 is exact in fp16 and
    every partial sum is an exact small integer). Matrix-core path (batch >=
    3): the weight is rounded once to fp16, so the result is exactly the
    fp16-rounded column."""
    monkeypatch.setenv("LQMM_TUNE_GEMV_Q4_0_PAIR", str(pair))
    c = synth.make("q4_0_gemv_1024")
    ks = [0, 1, 15, 16, 17, 31, 32, 500, 1007, 1023]
    x = np.zeros((len(ks), c.K), np.float32)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    announce("q4_0 one-hot exactness")
    W = dev(c.W.reshape(-1))
    ref = orc.gemv_q4_0(c.W, x, c.N, c.K)
    for i in range(0, len(ks), 2):
        y = host(bq.lqmm_gemv_q4_0(W, dev(x[i:i + 2]), c.N))
        assert np.array_equal(y, ref[i:i + 2].astype(np.float32))
    y = host(bq.lqmm_gemv_q4_0(W, dev(x), c.N))
    assert np.array_equal(y, ref.astype(np.float16).astype(np.float32))


def test_q4_0_subnormal_scales(orc, monkeypatch):
    """Subnormal fp16 scales are honoured (not flushed)."""
    N, K = 64, 256
    rng = np.random.default_rng(5)
    d = rng.integers(1, 1024, size=(N, K // 32)).astype(np.uint16).view(np.float16)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    W = synth.pack_q4_0(d, q)
    x = np.eye(K, dtype=np.float32)[[0, 20, 77, 255]]
    announce("q4_0 subnormal scales")
    ref = orc.gemv_q4_0(W, x, N, K)
    # dot2 arithmetic (exact): the small-problem kernel at two and (forced)
    # four rows, and the other batch-1/2 kernels
    for small in ("", "0"):
        if small:
            monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", small)
        for i in (0, 2):
            y = host(bq.lqmm_gemv_q4_0(dev(W.reshape(-1)), dev(x[i:i + 2]), N))
            assert np.array_equal(y, ref[i:i + 2].astype(np.float32))
    monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", "1")
    y = host(bq.lqmm_gemv_q4_0(dev(W.reshape(-1)), dev(x), N))
    assert np.array_equal(y, ref.astype(np.float32))
    # the matrix cores (each weight rounded once to fp16)
    monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", "0")
    y = host(bq.lqmm_gemv_q4_0(dev(W.reshape(-1)), dev(x), N))
    assert np.array_equal(y, ref.astype(np.float16).astype(np.float32))
    xr = rng.standard_normal((2, K)).astype(np.float32)
    y2 = host(bq.lqmm_gemv_q4_0(dev(W.reshape(-1)), dev(xr), N))
    assert_close(y2, orc.gemv_q4_0(W, xr, N, K), TOL_QUANT, "subnormal random x")
    monkeypatch.delenv("LQMM_TUNE_GEMV_SMALL")
    y2 = host(bq.lqmm_gemv_q4_0(dev(W.reshape(-1)), dev(xr), N))
    assert_close(y2, orc.gemv_q4_0(W, xr, N, K), TOL_QUANT, "subnormal random x, small kernel")


@pytest.mark.parametrize("fmt", ["q4_0", "q4_k"])
def test_batch_rows_are_independent(orc, fmt):
    """Each output row depends only on its own activation row: within the dot2
    path (batch <= 2) and within the matrix-core path (batch >= 3) a row's
    result is bitwise the same whatever the other rows hold; across the two
    paths results agree within the parity tolerance."""
    if fmt == "q4_0":
        c, fn = synth.q4_0_case(300, 4096, 4, seed=9), bq.lqmm_gemv_q4_0
    else:
        c, fn = synth.q4_k_case(300, 4096, 4, seed=9), bq.lqmm_gemv_q4_k
    announce(f"{fmt} batch row independence")
    W = dev(c.W.reshape(-1))
    y4 = host(fn(W, dev(c.x), c.N))            # matrix cores
    y2 = host(fn(W, dev(c.x[:2]), c.N))        # dot2
    for b in range(4):
        y1 = host(fn(W, dev(c.x[b]), c.N))     # dot2, batch 1
        if b < 2:
            assert np.array_equal(y1, y2[b])
        rep = np.repeat(c.x[b:b + 1], 3, axis=0)
        y3 = host(fn(W, dev(rep), c.N))        # matrix cores, other rows equal
        assert np.array_equal(y3[0], y4[b]) and np.array_equal(y3[2], y4[b])
        assert_close(y4[b], y1, TOL_QUANT, f"row {b} across paths")


# ----------------------------------------------------------------- Q4_K GEMV
Q4_K_SMALL = [(1, 256, 1), (3, 512, 2), (17, 768, 8), (5, 256, 9), (9, 8704, 8),
              (70, 2048, 3), (129, 4096, 5), (2, 1280, 4), (40, 16384, 1), (257, 256, 6),
              (33, 4608, 16), (18, 2048, 19), (48, 18432, 12),
              # dot2 path with K split over three launches
              (3, 147456, 1)]


@pytest.mark.parametrize("small", ["default", "0"])
@pytest.mark.parametrize("N,K,B", Q4_K_SMALL)
def test_q4_k_small(orc, monkeypatch, small, N, K, B):
    if small != "default":
        monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", small)
    c = synth.q4_k_case(N, K, B, seed=N * 3 + K + B)
    announce(f"q4_k gemv N={N} K={K} batch={B}")
    y = _run_q4_k(c)
    ref = orc.gemv_q4_k(c.W, c.x, N, K)
    assert_close(y, ref, TOL_QUANT, f"q4_k {N}x{K} b{B}")


# Matrix-core coalesced kernel in both of its forms, forced through the
# planner's tuning overrides: activations in registers (k-slices of one to
# four 256-weight super-chunks, slices partly or wholly past the row end,
# ragged tiles, up to 16 activation rows) and activations staged in LDS.
COAL_CASES = [("q4_k", 17, 256, 3, {}), ("q4_k", 33, 768, 8, {}), ("q4_k", 100, 2304, 5, {}),
              ("q4_k", 70, 7936, 16, {}), ("q4_k", 300, 8192, 8, {}),
              ("q4_k", 40, 1024, 4, {"LQMM_TUNE_GEMV_KS": "1"}),
              ("q4_k", 41, 2048, 6, {"LQMM_TUNE_GEMV_KS": "2"}),
              ("q4_k", 129, 4096, 3, {"LQMM_TUNE_GEMV_KS": "4"}),
              ("q4_0", 17, 256, 3, {}), ("q4_0", 33, 768, 16, {}), ("q4_0", 257, 2304, 4, {}),
              ("q4_0", 70, 7936, 8, {}), ("q4_0", 71, 7936, 9, {}), ("q4_0", 300, 4096, 4, {}),
              ("q4_0", 40, 1024, 8, {"LQMM_TUNE_GEMV_KS": "1"}),
              ("q4_0", 65, 3072, 5, {"LQMM_TUNE_GEMV_KS": "2"})]


@pytest.mark.parametrize("xregs", [0, 1])
@pytest.mark.parametrize("fmt,N,K,B,env", COAL_CASES)
def test_coal_forms(orc, monkeypatch, xregs, fmt, N, K, B, env):
    monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", "0")
    monkeypatch.setenv("LQMM_TUNE_GEMV_WHOLE", "0")
    monkeypatch.setenv("LQMM_TUNE_GEMV_XREGS", str(xregs))  # 1 forces it where it fits
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    make = synth.q4_k_case if fmt == "q4_k" else synth.q4_0_case
    c = make(N, K, B, seed=N + K * 3 + B + xregs)
    announce(f"{fmt} gemv N={N} K={K} batch={B} xregs={xregs} {env}")
    y = _run_q4_k(c) if fmt == "q4_k" else _run_q4_0(c)
    ref = (orc.gemv_q4_k if fmt == "q4_k" else orc.gemv_q4_0)(c.W, c.x, N, K)
    assert_close(y, ref, TOL_QUANT, f"{fmt} {N}x{K} b{B} xregs={xregs} {env}")


# Matrix-core kernel that requests each workgroup's whole weight share at
# once, forced through the planner's override: one to sixteen super-chunks
# per row (a wave's second super-chunk past the row end), ragged tiles, one
# to three tiles per CU, 3 to 16 activation rows and passes of 16 + 4.
WHOLE_CASES = [("q4_0", 17, 256, 3), ("q4_0", 257, 2304, 4), ("q4_0", 4097, 4096, 4),
               ("q4_0", 12288, 4096, 4), ("q4_0", 11008, 4096, 4), ("q4_0", 300, 4096, 8),
               ("q4_0", 100, 1024, 16), ("q4_0", 65, 2048, 20),
               ("q4_k", 33, 768, 5), ("q4_k", 4100, 4096, 4), ("q4_k", 700, 3840, 3),
               ("q4_k", 5000, 4096, 6)]


@pytest.mark.parametrize("fmt,N,K,B", WHOLE_CASES)
def test_whole_share_kernel(orc, monkeypatch, fmt, N, K, B):
    monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", "0")
    monkeypatch.setenv("LQMM_TUNE_GEMV_WHOLE", "1")
    make = synth.q4_k_case if fmt == "q4_k" else synth.q4_0_case
    c = make(N, K, B, seed=N + K * 7 + B)
    announce(f"{fmt} gemv whole-share kernel N={N} K={K} batch={B}")
    y = _run_q4_k(c) if fmt == "q4_k" else _run_q4_0(c)
    ref = (orc.gemv_q4_k if fmt == "q4_k" else orc.gemv_q4_0)(c.W, c.x, N, K)
    assert_close(y, ref, TOL_QUANT, f"{fmt} whole {N}x{K} b{B}")


@pytest.mark.parametrize("fmt", ["q4_0", "q4_k"])
def test_whole_share_matches_coalesced(monkeypatch, fmt):
    """Both kernels dequantize every weight the same way and multiply the
    same fp16 operands; only the order of the fp32 additions differs."""
    make = synth.q4_k_case if fmt == "q4_k" else synth.q4_0_case
    c = make(3000, 4096, 4, seed=93)
    W, x = dev(c.W.reshape(-1)), dev(c.x)
    call = bq.lqmm_gemv_q4_k if fmt == "q4_k" else bq.lqmm_gemv_q4_0
    monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", "0")
    announce(f"{fmt} whole-share kernel against the coalesced kernel")
    out = {}
    for whole in ("0", "1"):
        monkeypatch.setenv("LQMM_TUNE_GEMV_WHOLE", whole)
        out[whole] = host(call(W, x, c.N)).astype(np.float64)
    assert np.max(np.abs(out["1"] - out["0"])) <= 1e-5 * np.abs(out["0"]).max()


# Batch 1-2 Q4_K: the kernel that streams rows through LDS (the default at
# K <= 8192 with two weight rows per wave or more) and the register-loading
# kernel, forced through the planner's override: one super-block per row,
# more rows than waves, rows of one chunk and of two (16 + 1, 16 + 15 and
# 16 + 16 super-blocks), one and two activation rows; the last shape takes
# the register-loading kernel either way (K > 8192).
STREAM_CASES = [(1, 256, 1), (5, 1280, 2), (2049, 512, 1), (300, 4352, 1), (77, 7936, 2),
                (4100, 4096, 1), (4097, 8192, 1), (3, 8192, 2), (300, 8192, 2), (33, 8448, 1)]


@pytest.mark.parametrize("stream", [0, 1])
@pytest.mark.parametrize("N,K,B", STREAM_CASES)
def test_q4_k_dot2_forms(orc, monkeypatch, stream, N, K, B):
    monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", "0")
    monkeypatch.setenv("LQMM_TUNE_GEMV_STREAM", str(stream))
    c = synth.q4_k_case(N, K, B, seed=N + 5 * K + B + stream)
    announce(f"q4_k gemv N={N} K={K} batch={B} stream={stream}")
    y = _run_q4_k(c)
    ref = orc.gemv_q4_k(c.W, c.x, N, K)
    assert_close(y, ref, TOL_QUANT, f"q4_k {N}x{K} b{B} stream={stream}")


@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("fmt,K", [("q4_k", 8192), ("q4_0", 4096)])
def test_stream_matches_register_kernel(monkeypatch, fmt, K, B):
    """Both batch-1/2 kernels give lane l units l, l + 64, ... of a row, in
    that order, and reduce the lanes the same way: their outputs are the same
    bits (Q4_0 in two-block units)."""
    make = synth.q4_k_case if fmt == "q4_k" else synth.q4_0_case
    c = make(300, K, B, seed=77 + K + B)
    W, x = dev(c.W.reshape(-1)), dev(c.x)
    call = bq.lqmm_gemv_q4_k if fmt == "q4_k" else bq.lqmm_gemv_q4_0
    monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", "0")
    monkeypatch.setenv("LQMM_TUNE_GEMV_Q4_0_PAIR", "1")
    announce(f"{fmt} stream vs register kernel, K={K}")
    ys = []
    for stream in (1, 0):
        monkeypatch.setenv("LQMM_TUNE_GEMV_STREAM", str(stream))
        ys.append(host(call(W, x, c.N)))
    assert np.array_equal(ys[0], ys[1])


# Batch 1-2 Q4_0 in two-block units: streamed (forced) and register-loading;
# K = 4160 (rows over one chunk) and K = 4128 (K % 64 != 0, single-block
# units) take the register-loading kernel either way.
Q4_0_STREAM_CASES = [(1, 64, 1), (300, 2048, 1), (8193, 1024, 1), (9000, 4096, 1), (77, 4160, 1),
                     (40, 4128, 1), (300, 4096, 2), (8193, 2048, 2)]


@pytest.mark.parametrize("stream", [0, 1])
@pytest.mark.parametrize("N,K,B", Q4_0_STREAM_CASES)
def test_q4_0_dot2_forms(orc, monkeypatch, stream, N, K, B):
    monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", "0")
    monkeypatch.setenv("LQMM_TUNE_GEMV_STREAM", str(stream))
    monkeypatch.setenv("LQMM_TUNE_GEMV_Q4_0_PAIR", "1")
    c = synth.q4_0_case(N, K, B, seed=N + 7 * K + stream)
    announce(f"q4_0 gemv N={N} K={K} batch={B} stream={stream}")
    y = _run_q4_0(c)
    ref = orc.gemv_q4_0(c.W, c.x, N, K)
    assert_close(y, ref, TOL_QUANT, f"q4_0 {N}x{K} b{B} stream={stream}")


@pytest.mark.parametrize("name", ["q4_k_gemv_28672x8192_b1", "q4_k_gemv_28672x8192_b8"])
def test_q4_k_configs(orc, name):
    c = synth.make(name)
    announce(name)
    y = _run_q4_k(c)
    ref = orc.gemv_q4_k(c.W, c.x, c.N, c.K)
    assert_close(y, ref, TOL_QUANT, name)


def test_q4_k_one_hot_exact(orc):
    """dot2 path (batch <= 2): one-hot columns are bit-exact. Matrix-core
    path: d*sc, dmin*m and the weight d*sc*q - dmin*m are each rounded to fp16
    once (round to nearest, relative error <= 2^-11 each), so every entry obeys
    |err| <= 2^-11 (|d sc q| + |dmin m| + |w|) + 2^-24 (fp16 subnormal step)."""
    c = synth.q4_k_case(300, 2048, 1, seed=31)
    ks = [0, 31, 32, 63, 64, 200, 255, 256, 1500, 2047]
    x = np.zeros((len(ks), c.K), np.float32)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    announce("q4_k one-hot exactness")
    W = dev(c.W.reshape(-1))
    ref = orc.gemv_q4_k(c.W, x, c.N, c.K)
    for i in range(0, len(ks), 2):
        y = host(bq.lqmm_gemv_q4_k(W, dev(x[i:i + 2]), c.N))
        assert np.array_equal(y, ref[i:i + 2].astype(np.float32))
    y = host(bq.lqmm_gemv_q4_k(W, dev(x), c.N)).astype(np.float64)
    for i, k in enumerate(ks):
        sb, s = k // 256, (k % 256) // 32
        a = np.abs(c.d[:, sb].astype(np.float64) * c.sc[:, sb, s] * c.q[:, k])
        m = np.abs(c.dmin[:, sb].astype(np.float64) * c.m[:, sb, s])
        bound = 2.0 ** -11 * (a + m + np.abs(ref[i])) * 1.001 + 2.0 ** -24
        assert np.all(np.abs(y[i] - ref[i]) <= bound), k


def test_q4_k_extreme_codes(orc):
    """sc, m at 0 and 63, q at 0 and 15, subnormal d and dmin."""
    N, K = 48, 512
    rng = np.random.default_rng(8)
    nsb = K // 256
    d = rng.integers(1, 0x3C00, size=(N, nsb)).astype(np.uint16).view(np.float16)
    dmin = rng.integers(1, 0x0400, size=(N, nsb)).astype(np.uint16).view(np.float16)
    sc = rng.choice([0, 1, 62, 63], size=(N, nsb, 8)).astype(np.uint8)
    m = rng.choice([0, 1, 62, 63], size=(N, nsb, 8)).astype(np.uint8)
    q = rng.choice([0, 15], size=(N, K)).astype(np.uint8)
    W = synth.pack_q4_k(d, dmin, sc, m, q)
    x = rng.standard_normal((3, K)).astype(np.float32)
    announce("q4_k extreme codes")
    y = host(bq.lqmm_gemv_q4_k(dev(W.reshape(-1)), dev(x), N))
    assert_close(y, orc.gemv_q4_k(W, x, N, K), TOL_QUANT, "q4_k extremes")


# Small problems: the latency-bound kernel (one round trip to memory), with K
# split across workgroups where a row slice exceeds one wave (long K) or
# where the tuning override forces it (LQMM_TUNE_GEMV_SPLITK), including
# the configuration shapes; ragged N, K % 64 == 32 (single-block Q4_0
# units), one to four activation rows (three and four forced), one to
# sixteen waves per workgroup, one and two units per lane.
SMALL_CASES = [
    ("q4_0", 1024, 1024, 1, {}),
    ("q4_0", 1024, 1024, 1, {"LQMM_TUNE_GEMV_SPLITK": "2"}),
    ("q4_0", 1024, 1024, 1, {"LQMM_TUNE_GEMV_SPLITK": "4"}),
    ("q4_0", 4096, 4096, 1, {}),
    ("q4_0", 4096, 4096, 1, {"LQMM_TUNE_GEMV_SPLITK": "2"}),
    ("q4_0", 4096, 4096, 2, {"LQMM_TUNE_GEMV_SMALL_WAVES": "8"}),
    ("q4_0", 4096, 4096, 4, {"LQMM_TUNE_GEMV_SMALL": "1", "LQMM_TUNE_GEMV_SPLITK": "4"}),
    ("q4_0", 4096, 4096, 3, {"LQMM_TUNE_GEMV_SMALL": "1"}),
    ("q4_0", 777, 1056, 2, {"LQMM_TUNE_GEMV_SPLITK": "4"}),
    ("q4_0", 33, 96, 1, {"LQMM_TUNE_GEMV_SMALL": "1"}),
    ("q4_0", 100, 8192, 2, {}),
    ("q4_0", 50, 16384, 3, {"LQMM_TUNE_GEMV_SMALL": "1", "LQMM_TUNE_GEMV_SMALL_U": "2"}),
    ("q4_0", 129, 2048, 4, {"LQMM_TUNE_GEMV_SMALL": "1", "LQMM_TUNE_GEMV_SMALL_WAVES": "1"}),
    ("q4_0", 129, 2048, 2, {"LQMM_TUNE_GEMV_SMALL_WAVES": "2", "LQMM_TUNE_GEMV_SPLITK": "8"}),
    ("q4_0", 3000, 2048, 1, {"LQMM_TUNE_GEMV_SMALL_WAVES": "16", "LQMM_TUNE_GEMV_SPLITK": "2"}),
    ("q4_k", 1000, 4096, 1, {}),
    ("q4_k", 513, 8192, 2, {}),
    ("q4_k", 513, 8192, 4, {"LQMM_TUNE_GEMV_SMALL": "1"}),
    ("q4_k", 300, 2048, 2, {"LQMM_TUNE_GEMV_SPLITK": "8"}),
    ("q4_k", 64, 16384, 1, {}),
    ("q4_k", 7, 256, 3, {"LQMM_TUNE_GEMV_SMALL": "1", "LQMM_TUNE_GEMV_SPLITK": "2"}),
    ("q4_k", 90, 4352, 4, {"LQMM_TUNE_GEMV_SMALL": "1", "LQMM_TUNE_GEMV_SMALL_U": "2",
                           "LQMM_TUNE_GEMV_SPLITK": "2"}),
    ("q4_k", 1100, 2048, 2, {"LQMM_TUNE_GEMV_SMALL_WAVES": "16"}),
]


@pytest.mark.parametrize("fmt,N,K,B,env", SMALL_CASES)
def test_small_kernel(orc, monkeypatch, fmt, N, K, B, env):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    make = synth.q4_k_case if fmt == "q4_k" else synth.q4_0_case
    c = make(N, K, B, seed=3 * N + K + B + len(env))
    announce(f"{fmt} small gemv N={N} K={K} batch={B} {env}")
    y = _run_q4_k(c) if fmt == "q4_k" else _run_q4_0(c)
    ref = (orc.gemv_q4_k if fmt == "q4_k" else orc.gemv_q4_0)(c.W, c.x, N, K)
    assert_close(y, ref, TOL_QUANT, f"{fmt} small {N}x{K} b{B} {env}")


@pytest.mark.parametrize("fmt", ["q4_0", "q4_k"])
def test_small_split_fixed_order(monkeypatch, fmt):
    """Split-K results are added in slice order, whatever order the
    workgroups finish in: repeated calls are bitwise equal (the second and
    later ones also rely on the arrival counters being back at zero), and so
    are calls with other workgroup widths (each slice's partial sums do not
    depend on them)."""
    make = synth.q4_k_case if fmt == "q4_k" else synth.q4_0_case
    c = make(1000, 4096, 2, seed=12)
    call = bq.lqmm_gemv_q4_k if fmt == "q4_k" else bq.lqmm_gemv_q4_0
    W, x = dev(c.W.reshape(-1)), dev(c.x)
    monkeypatch.setenv("LQMM_TUNE_GEMV_SPLITK", "4")
    announce(f"{fmt} split-K fixed order")
    ys = [host(call(W, x, c.N)) for _ in range(4)]
    for nw in ("1", "2", "4"):
        monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL_WAVES", nw)
        ys.append(host(call(W, x, c.N)))
    for y in ys[1:]:
        assert np.array_equal(y, ys[0])


def test_small_split_needs_workspace(monkeypatch):
    """A forced split-K plan without a workspace is refused; without the
    override the planner runs a plan that needs none."""
    c = synth.q4_0_case(256, 4096, 1, seed=4)
    W, x = dev(c.W.reshape(-1)), dev(c.x)
    announce("split-K workspace errors")
    monkeypatch.setenv("LQMM_TUNE_GEMV_SPLITK", "2")
    with pytest.raises(bq.LqmmError) as e:
        bq.lqmm_gemv_q4_0(W, x, c.N, workspace=False)
    assert e.value.status == 4
    import torch
    small_ws = torch.zeros(64, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(bq.LqmmError):
        bq.lqmm_gemv_q4_0(W, x, c.N, workspace=small_ws)
    monkeypatch.delenv("LQMM_TUNE_GEMV_SPLITK")
    y = host(bq.lqmm_gemv_q4_0(W, x, c.N, workspace=False))
    y2 = host(bq.lqmm_gemv_q4_0(W, x, c.N))
    assert np.array_equal(y, y2)


# Activation scale: the GEMVs round x to fp16 unscaled, so their relative
# error must not grow when x is small (down to the fp16 subnormal range,
# 1e-4 * N(0,1)) or large (1e3 * N(0,1), up to ~5e3). Every batch-1/2/4
# kernel form is forced through the planner's overrides: the streamed and
# register-loading dot2 kernels (Q4_0 in one- and two-block units), the
# matrix-core kernels (activations in LDS, in registers, and the kernel that
# requests a workgroup's whole weight share at once), and the small-problem
# kernel with and without split-K.
SCALED_FORMS = [
    ("q4_0", 1, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "1", "LQMM_TUNE_GEMV_Q4_0_PAIR": "1"}),
    ("q4_0", 1, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "0", "LQMM_TUNE_GEMV_Q4_0_PAIR": "1"}),
    ("q4_0", 1, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "0", "LQMM_TUNE_GEMV_Q4_0_PAIR": "0"}),
    ("q4_0", 2, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "1", "LQMM_TUNE_GEMV_Q4_0_PAIR": "1"}),
    ("q4_0", 2, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "0", "LQMM_TUNE_GEMV_Q4_0_PAIR": "0"}),
    ("q4_0", 4, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_WHOLE": "0", "LQMM_TUNE_GEMV_XREGS": "0"}),
    ("q4_0", 4, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_WHOLE": "0", "LQMM_TUNE_GEMV_XREGS": "1"}),
    ("q4_0", 4, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_WHOLE": "1"}),
    ("q4_k", 1, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "1"}),
    ("q4_k", 1, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "0"}),
    ("q4_k", 2, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "1"}),
    ("q4_k", 2, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "0"}),
    ("q4_k", 4, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_WHOLE": "0", "LQMM_TUNE_GEMV_XREGS": "0"}),
    ("q4_k", 4, {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_WHOLE": "0", "LQMM_TUNE_GEMV_XREGS": "1"}),
    ("q4_0", 1, {"LQMM_TUNE_GEMV_SMALL": "1"}),
    ("q4_0", 4, {"LQMM_TUNE_GEMV_SMALL": "1", "LQMM_TUNE_GEMV_SPLITK": "2"}),
    ("q4_k", 2, {"LQMM_TUNE_GEMV_SMALL": "1"}),
    ("q4_k", 4, {"LQMM_TUNE_GEMV_SMALL": "1", "LQMM_TUNE_GEMV_SPLITK": "2"}),
]


@pytest.mark.parametrize("scale", [1e-4, 1e-2, 1e3])
@pytest.mark.parametrize("fmt,B,env", SCALED_FORMS)
def test_activation_scale(orc, monkeypatch, scale, fmt, B, env):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    N, K = (300, 4096) if fmt == "q4_0" else (300, 8192)
    make = synth.q4_k_case if fmt == "q4_k" else synth.q4_0_case
    c = make(N, K, B, seed=int(N + K + B + 1e4 * scale) % 100003)
    x = (c.x.astype(np.float64) * scale).astype(np.float32)
    announce(f"{fmt} gemv N={N} K={K} batch={B} x*{scale:g} {env}")
    call = bq.lqmm_gemv_q4_k if fmt == "q4_k" else bq.lqmm_gemv_q4_0
    y = host(call(dev(c.W.reshape(-1)), dev(x), N))
    ref = (orc.gemv_q4_k if fmt == "q4_k" else orc.gemv_q4_0)(c.W, x, N, K)
    assert_close(y, ref, TOL_QUANT, f"{fmt} {N}x{K} b{B} x*{scale:g} {env}")


# ------------------------------------------------------------- Q8_0 GEMM
Q8_0_SMALL = [(1, 1, 32), (3, 5, 64), (17, 130, 96), (128, 128, 64), (130, 257, 320),
              (64, 200, 4096), (256, 512, 1024), (1, 300, 32),
              # ragged in every dimension at once: partial output tiles and a
              # last K step holding a single block
              (129, 257, 160), (300, 513, 224), (512, 768, 4128),
              # odd numbers of 64-wide K steps
              (70, 300, 192), (33, 257, 448)]


@pytest.mark.parametrize("M,N,K", Q8_0_SMALL)
def test_q8_0_small(orc, M, N, K):
    c = synth.q8_0_case(M, N, K, seed=M + N + K)
    announce(f"q8_0 gemm M={M} N={N} K={K}")
    Y = host(bq.lqmm_gemm_q8_0_f16(dev(c.W.reshape(-1)), dev(c.X), N)).astype(np.float64)
    ref = orc.gemm_q8_0_f16(c.W, c.X, N, K)
    assert_close(Y, ref, TOL_QUANT, f"q8_0 {M}x{N}x{K}")


@pytest.mark.parametrize("waves", [7, 8])
@pytest.mark.parametrize("M,N,K", [(300, 513, 224), (129, 481, 4096), (512, 1000, 128)])
def test_q8_0_tile_widths(orc, monkeypatch, waves, M, N, K):
    # the K % 64 == 0 kernel in both of its tile widths (224 and 256 columns),
    # forced through the planner's tuning override
    monkeypatch.setenv("LQMM_TUNE_GEMM_WAVES", str(waves))
    c = synth.q8_0_case(M, N, K, seed=M + N + K + waves)
    announce(f"q8_0 gemm M={M} N={N} K={K} waves={waves}")
    Y = host(bq.lqmm_gemm_q8_0_f16(dev(c.W.reshape(-1)), dev(c.X), N)).astype(np.float64)
    ref = orc.gemm_q8_0_f16(c.W, c.X, N, K)
    assert_close(Y, ref, TOL_QUANT, f"q8_0 {M}x{N}x{K} waves={waves}")


def test_q8_0_config_full(orc):
    """The prefill configuration at full size, every output element against
    the oracle (about 3e10 multiply-adds in fp64 on the host cores)."""
    c = synth.make("q8_0_gemm_512x14336x4096")
    announce("q8_0 gemm 512x14336x4096 (all elements)")
    Y = host(bq.lqmm_gemm_q8_0_f16(dev(c.W.reshape(-1)), dev(c.X), c.N)).astype(np.float64)
    assert np.isfinite(Y).all()
    ref = orc.gemm_q8_0_f16(c.W, c.X, c.N, c.K)
    assert_close(Y, ref, TOL_QUANT, "q8_0 config (all elements)")


def test_q8_0_one_hot_exact(orc):
    """A one-hot X row returns fp16(d*q) exactly: one rounding of the weight,
    exact products and sums."""
    c = synth.q8_0_case(8, 96, 256, seed=3)
    X = np.zeros((8, c.K), np.float16)
    for i, k in enumerate([0, 5, 31, 32, 100, 200, 254, 255]):
        X[i, k] = 1.0
    announce("q8_0 one-hot exactness")
    Y = host(bq.lqmm_gemm_q8_0_f16(dev(c.W.reshape(-1)), dev(X), c.N))
    ref = orc.gemm_q8_0_f16(c.W, X, c.N, c.K)
    assert np.array_equal(Y, ref.astype(np.float16))


# --------------------------------------------------------------- fp32 GEMM
SGEMM_SMALL = [(1, 1, 1), (3, 5, 7), (17, 33, 65), (127, 129, 130), (128, 128, 128),
               (200, 64, 3), (64, 256, 1000), (5, 300, 33)]


@pytest.mark.parametrize("M,N,K", SGEMM_SMALL)
def test_sgemm_small(orc, M, N, K):
    s = synth.sgemm_case(M, N, K, seed=M * N + K)
    announce(f"sgemm M={M} N={N} K={K}")
    C = host(bq.lqmm_sgemm(dev(s.A), dev(s.B)))
    ref = orc.sgemm(s.A, s.B)
    assert_close(C, ref, TOL_FP32, f"sgemm {M}x{N}x{K}")


def test_sgemm_config_full(orc):
    """The fp32 configuration at full size (2048^3), every element."""
    s = synth.make("sgemm_2048")
    announce("sgemm 2048^3 (all elements)")
    C = host(bq.lqmm_sgemm(dev(s.A), dev(s.B)))
    assert np.isfinite(C).all()
    ref = orc.sgemm(s.A, s.B)
    assert_close(C, ref, TOL_FP32, "sgemm config (all elements)")


def test_sgemm_identity_exact():
    rng = np.random.default_rng(2)
    A = rng.uniform(-1, 1, (150, 130)).astype(np.float32)
    I = np.eye(130, dtype=np.float32)
    announce("sgemm identity exactness")
    C = host(bq.lqmm_sgemm(dev(A), dev(I)))
    assert np.array_equal(C, A)


def test_errors_raise_on_device():
    import torch
    W = torch.zeros(18 * 4, dtype=torch.uint8, device="cuda:0")
    x = torch.zeros((1, 48), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError):
        bq.lqmm_gemv_q4_0(W, x, 4)
    # a contiguous view whose data pointer is only 4-byte aligned: the
    # library itself rejects it
    xs = torch.zeros((1, 33), dtype=torch.float32, device="cuda:0")[:, 1:]
    with pytest.raises(bq.LqmmError) as e:
        bq.lqmm_gemv_q4_0(W[:18 * 4], xs, 4)
    assert e.value.status == 3
    # a strided (non-contiguous) activation is refused by the binding
    xn = torch.zeros((2, 64), dtype=torch.float32, device="cuda:0")[:, ::2]
    with pytest.raises(ValueError):
        bq.lqmm_gemv_q4_0(W, xn, 4)


_THREADS_SCRIPT = r"""
import sys, threading
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import block_quantized_matmul_amd as bq
import synth

torch.cuda.set_device(0)
a = synth.q4_0_case(1000, 4096, 1, seed=1)
k = synth.q4_k_case(700, 8192, 8, seed=2)
g = synth.q8_0_case(130, 300, 512, seed=3)
s = synth.sgemm_case(150, 130, 70, seed=4)
d = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
calls = [
    lambda: bq.lqmm_gemv_q4_0(d(a.W.reshape(-1)), d(a.x), a.N),
    lambda: bq.lqmm_gemv_q4_k(d(k.W.reshape(-1)), d(k.x), k.N),
    lambda: bq.lqmm_gemv_q4_k(d(k.W.reshape(-1)), d(k.x[:1]), k.N),
    lambda: bq.lqmm_gemm_q8_0_f16(d(g.W.reshape(-1)), d(g.X), g.N),
    lambda: bq.lqmm_sgemm(d(s.A), d(s.B)),
] * 2
out = [None] * len(calls)
start = threading.Barrier(len(calls))

def work(i):
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        start.wait()   # every thread's first call to the library at once
        out[i] = calls[i]()
    st.synchronize()

ts = [threading.Thread(target=work, args=(i,)) for i in range(len(calls))]
for t in ts: t.start()
for t in ts: t.join()
torch.cuda.synchronize()
for i, c in enumerate(calls):
    ref = c().cpu().numpy()
    assert np.array_equal(out[i].cpu().numpy(), ref), i
print("threads ok", len(calls))
"""


def test_concurrent_first_calls(tmp_path):
    """Ten host threads make their first library calls at the same moment, on
    their own streams, in a fresh process (so every kernel's once-per-device
    set-up races): each result equals the same call made again serially."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = tmp_path / "threads.py"
    script.write_text(_THREADS_SCRIPT)
    announce("concurrent first calls (subprocess)")
    r = subprocess.run([sys.executable, str(script), root], capture_output=True, text=True,
                       timeout=110)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "threads ok" in r.stdout


def test_decode_chain_graph_replays(orc):
    """The decode-layer GEMV chain captured in one HIP graph: every replay
    (with eager work and synchronizations between replays) reproduces the
    eager pass bit for bit, and the chain's first GEMV matches the oracle."""
    import torch
    from block_quantized_matmul_amd.chain import LAYER, DecodeChain
    announce("decode chain graph replays")
    ch = DecodeChain(torch, layers=1, seed=3)
    ch.run()
    torch.cuda.synchronize()
    eager = [host(o).copy() for o in ch.outs]
    g = ch.capture()
    scratch = torch.randn(1 << 16, device="cuda:0")
    for i in range(3):
        for o in ch.outs:
            o.fill_(float("nan"))
        scratch.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(ch.outs, eager):
            assert np.array_equal(host(o), e), i
    assert np.isfinite(eager[-1]).all()
    N, K = LAYER[0][1], LAYER[0][2]
    W0 = host(ch.layers[0][0]).reshape(N, -1)
    ref = orc.gemv_q4_0(W0, host(ch.x), N, K)
    assert_close(eager[0], ref, TOL_QUANT, "chain qkv")
