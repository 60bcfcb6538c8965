"""GPU parity for the other format x phase pairs and the further block formats:
Q8_0 decode GEMV, Q4_0 and Q4_K prefill GEMMs, Q6_K, Q2_K and 1-bit q1_0
decode GEMVs and the int4 group-32 GEMV, through the C ABI against the CPU oracle on the same
seeded inputs. Bars as for the other quantized paths (2e-3 on both metrics);
bit-exact where the arithmetic is exact (one-hot activations)."""
import numpy as np
import pytest

import block_quantized_matmul_amd as bq
import synth
from gpu_util import TOL_QUANT, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bq.load()


def _i4_dev(c):
    return (dev(c.Wq.view(np.int32)), dev(c.scales), dev(c.zeros))


def run_gemv(fmt, c, x=None):
    x = c.x if x is None else x
    if fmt == "i4g32":
        Wq, sc, z = _i4_dev(c)
        return host(bq.lqmm_gemv_i4g32(Wq, sc, z, dev(x), c.N))
    fn = {"q8_0": bq.lqmm_gemv_q8_0, "q6_k": bq.lqmm_gemv_q6_k, "q2_k": bq.lqmm_gemv_q2_k,
          "q1_0": bq.lqmm_gemv_q1_0}[fmt]
    return host(fn(dev(c.W.reshape(-1)), dev(x), c.N))


def ref_gemv(orc, fmt, c, x=None):
    x = c.x if x is None else x
    if fmt == "i4g32":
        return orc.gemv_i4g32(c.Wq, c.scales, c.zeros, x, c.N, c.K)
    return {"q8_0": orc.gemv_q8_0, "q6_k": orc.gemv_q6_k, "q2_k": orc.gemv_q2_k,
            "q1_0": orc.gemv_q1_0}[fmt](
        c.W, x, c.N, c.K)


MAKE = {"q8_0": synth.q8_0_gemv_case, "q6_k": synth.q6_k_case, "q2_k": synth.q2_k_case,
        "i4g32": synth.i4g32_case, "q1_0": synth.q1_0_case}

# ragged N; one block or super-block per row up to long rows (split-K); one to
# nine activation rows (passes of four)
GEMV_CASES = [
    ("q8_0", 1, 32, 1), ("q8_0", 7, 96, 3), ("q8_0", 300, 4096, 1), ("q8_0", 129, 8192, 2),
    ("q8_0", 33, 4128, 5), ("q8_0", 1000, 2048, 4), ("q8_0", 5000, 4096, 2), ("q8_0", 17, 16384, 9),
    ("q6_k", 1, 256, 1), ("q6_k", 13, 512, 3), ("q6_k", 300, 4096, 2), ("q6_k", 70, 16384, 1),
    ("q6_k", 5000, 4096, 1), ("q6_k", 41, 2304, 6),
    ("q2_k", 1, 256, 1), ("q2_k", 13, 512, 4), ("q2_k", 300, 4096, 1), ("q2_k", 70, 16384, 2),
    ("q2_k", 5000, 4096, 1), ("q2_k", 41, 2304, 7),
    ("i4g32", 1, 32, 1), ("i4g32", 9, 96, 2), ("i4g32", 300, 4096, 1), ("i4g32", 129, 8192, 3),
    ("i4g32", 5000, 4096, 1), ("i4g32", 33, 4160, 5),
    ("q1_0", 1, 32, 1), ("q1_0", 7, 96, 2), ("q1_0", 300, 4096, 1), ("q1_0", 129, 8192, 3),
    ("q1_0", 5000, 4096, 4), ("q1_0", 33, 4128, 5), ("q1_0", 17, 16384, 1),
]


def dequant(orc, fmt, c):
    if fmt == "i4g32":
        return orc.dequant_i4g32(c.Wq, c.scales, c.zeros, c.N, c.K)
    return getattr(orc, f"dequant_{fmt}")(c.W, c.N, c.K)


@pytest.mark.parametrize("fmt,N,K,B", GEMV_CASES)
def test_gemv_formats(orc, fmt, N, K, B):
    """Outputs of more than 256 elements: the 2e-3 bars. Fewer: each element
    within (2^-11 + 2^-9) * sum_k |x w| + 2^-24 |y|. x is rounded to fp16
    (at most 2^-11 relative per element), and the codes' fp16 bias (1024 to
    1152 times the block scale) cancels in the fp32 sums, which adds at most
    K/2 roundings of 2^-24 of that bias: 2^-9 sum |x w| for q1_0, whose
    weights are +-d, less for the other formats on these draws. One dot
    product of these weights can cancel by a factor of tens to hundreds
    (q1_0 1 x 32: |y| = 0.013 against sum |x w| = 0.42), so no relative bar
    holds on a single element."""
    c = MAKE[fmt](N, K, B, seed=N + 3 * K + B)
    announce(f"{fmt} gemv N={N} K={K} batch={B}")
    y, ref = run_gemv(fmt, c).astype(np.float64), ref_gemv(orc, fmt, c)
    if N * B > 256:
        assert_close(y, ref, TOL_QUANT, f"{fmt} {N}x{K} b{B}")
        return
    bound = (2.0 ** -11 + 2.0 ** -9) * (np.abs(c.x.astype(np.float64))
                                        @ np.abs(dequant(orc, fmt, c)).T)
    assert np.all(np.abs(y - ref) <= bound + 2.0 ** -24 * np.abs(ref)), \
        np.max(np.abs(y - ref) / bound)


@pytest.mark.parametrize("name", ["q8_0_gemv_4096x4096_b1", "q8_0_gemv_11008x4096_b1",
                                  "q8_0_gemv_12288x4096_b4", "q6_k_gemv_11008x4096_b1",
                                  "q2_k_gemv_11008x4096_b1", "i4g32_gemv_11008x4096_b1",
                                  "q1_0_gemv_11008x4096_b1"])
def test_gemv_format_configs(orc, name):
    c = synth.make(name)
    fmt = name.split("_gemv")[0]
    announce(name)
    assert_close(run_gemv(fmt, c), ref_gemv(orc, fmt, c), TOL_QUANT, name)


@pytest.mark.parametrize("fmt", ["q8_0", "q6_k", "q2_k", "i4g32", "q1_0"])
def test_gemv_formats_one_hot_exact(orc, fmt):
    """One-hot activations extract weight columns: the codes become exact
    fp16 integers, the bias removal is exact, and the block scales are
    applied in fp32 with one rounding, so the columns equal the oracle's
    rounded to fp32."""
    K = 512
    c = MAKE[fmt](70, K, 1, seed=5)
    ks = [0, 1, 15, 16, 31, 32, 100, 255, 256, 300, 511]
    announce(f"{fmt} one-hot exactness")
    for i in range(0, len(ks), 4):
        x = np.zeros((len(ks[i:i + 4]), K), np.float32)
        for r, k in enumerate(ks[i:i + 4]):
            x[r, k] = 1.0
        y = run_gemv(fmt, c, x)
        ref = ref_gemv(orc, fmt, c, x)
        assert np.array_equal(y, ref.astype(np.float32)), ks[i:i + 4]


@pytest.mark.parametrize("scale", [1e-4, 1e3])
@pytest.mark.parametrize("fmt", ["q8_0", "q6_k", "q2_k", "i4g32", "q1_0"])
def test_gemv_formats_activation_scale(orc, fmt, scale):
    c = MAKE[fmt](200, 4096, 2, seed=11)
    x = (c.x.astype(np.float64) * scale).astype(np.float32)
    announce(f"{fmt} gemv x*{scale:g}")
    assert_close(run_gemv(fmt, c, x), ref_gemv(orc, fmt, c, x), TOL_QUANT, f"{fmt} x*{scale:g}")


# ---------------------------------------------------------- Q4_0 / Q4_K GEMMs
GEMM_MAKE = {"q4_0": synth.q4_0_gemm_case, "q4_k": synth.q4_k_gemm_case}


def run_gemm(fmt, c, X=None):
    X = c.X if X is None else X
    fn = bq.lqmm_gemm_q4_0_f16 if fmt == "q4_0" else bq.lqmm_gemm_q4_k_f16
    return host(fn(dev(c.W.reshape(-1)), dev(X), c.N)).astype(np.float64)


def ref_gemm(orc, fmt, c, X=None):
    X = c.X if X is None else X
    fn = orc.gemm_q4_0_f16 if fmt == "q4_0" else orc.gemm_q4_k_f16
    return fn(c.W, X, c.N, c.K)


# ragged M and N (partial 128 x 128 tiles), K % 64 == 32 (Q4_0: a last step of
# one block), one step, many steps
GEMM_CASES = [("q4_0", 1, 1, 32), ("q4_0", 3, 5, 64), ("q4_0", 130, 257, 96),
              ("q4_0", 128, 128, 4096), ("q4_0", 300, 513, 1056), ("q4_0", 64, 200, 4096),
              ("q4_k", 1, 1, 256), ("q4_k", 3, 5, 256), ("q4_k", 130, 257, 768),
              ("q4_k", 128, 128, 4096), ("q4_k", 300, 513, 2304), ("q4_k", 64, 200, 8192)]


@pytest.mark.parametrize("fmt,M,N,K", GEMM_CASES)
def test_gemm_q4(orc, fmt, M, N, K):
    """Outputs of more than 256 elements: the 2e-3 bars. Fewer: each element
    within the fp16 rounding bound, 2^-11 * sum_k |X w| (every weight rounded
    once) + 2^-11 |Y| (the output), since a single dot product of these
    weights can cancel by a factor of several hundred and no fp16 weight
    representation meets a relative bar on it (1 x 1 x 256 Q4_K: |Y| = 0.64
    against sum |X w| = 282)."""
    c = GEMM_MAKE[fmt](M, N, K, seed=M + N + K)
    announce(f"{fmt} gemm M={M} N={N} K={K}")
    Y, ref = run_gemm(fmt, c), ref_gemm(orc, fmt, c)
    if M * N > 256:
        assert_close(Y, ref, TOL_QUANT, f"{fmt} gemm {M}x{N}x{K}")
        return
    deq = orc.dequant_q4_0 if fmt == "q4_0" else orc.dequant_q4_k
    absw = np.abs(deq(c.W, N, K))
    bound = 2.0 ** -11 * (np.abs(c.X.astype(np.float64)) @ absw.T) * 1.001 + 2.0 ** -11 * np.abs(ref)
    assert np.all(np.abs(Y - ref) <= bound + 2.0 ** -24), np.max(np.abs(Y - ref) / bound)


@pytest.mark.parametrize("fmt", ["q4_0", "q4_k"])
def test_gemm_q4_config_full(orc, fmt):
    """The prefill shape (512 x 14336 x 4096), every element."""
    c = synth.make(f"{fmt}_gemm_512x14336x4096")
    announce(f"{fmt} gemm 512x14336x4096 (all elements)")
    Y = run_gemm(fmt, c)
    assert np.isfinite(Y).all()
    assert_close(Y, ref_gemm(orc, fmt, c), TOL_QUANT, f"{fmt} gemm config")


def test_gemm_q4_0_one_hot_exact(orc):
    """One-hot X rows return fp16(d * (q - 8)): one rounding of the weight,
    exact products and sums, and the same rounding of the output."""
    c = synth.q4_0_gemm_case(8, 96, 256, seed=3)
    X = np.zeros((8, c.K), np.float16)
    for i, k in enumerate([0, 5, 15, 16, 31, 32, 200, 255]):
        X[i, k] = 1.0
    announce("q4_0 gemm one-hot exactness")
    Y = host(bq.lqmm_gemm_q4_0_f16(dev(c.W.reshape(-1)), dev(X), c.N))
    assert np.array_equal(Y, ref_gemm(orc, "q4_0", c, X).astype(np.float16))


def test_gemm_q4_k_one_hot_exact(orc):
    """One-hot X rows return fp16(d * sc * q - dmin * m): the weight formed in
    fp32 (exact here: these fields need at most 23 significant bits) and
    rounded once to fp16, then exact products and sums and the same rounding
    of the output."""
    c = synth.q4_k_gemm_case(8, 96, 512, seed=4)
    ks = [0, 31, 32, 63, 64, 255, 256, 511]
    X = np.zeros((8, c.K), np.float16)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    announce("q4_k gemm one-hot exactness")
    Y = host(bq.lqmm_gemm_q4_k_f16(dev(c.W.reshape(-1)), dev(X), c.N))
    assert np.array_equal(Y, ref_gemm(orc, "q4_k", c, X).astype(np.float16))


def test_new_entry_argument_errors():
    import torch
    W = torch.zeros(34 * 4, dtype=torch.uint8, device="cuda:0")
    x = torch.zeros((1, 48), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError):  # K not a multiple of 32
        bq.lqmm_gemv_q8_0(W, x, 4)
    # a long Q8_0 row needs the split-K workspace: refused without it
    Wl = torch.zeros(34 * 512, dtype=torch.uint8, device="cuda:0")
    xl = torch.zeros((1, 16384), dtype=torch.float32, device="cuda:0")
    with pytest.raises(bq.LqmmError) as e:
        bq.lqmm_gemv_q8_0(Wl, xl, 1, workspace=False)
    assert e.value.status == 4
    X = torch.zeros((2, 100), dtype=torch.float16, device="cuda:0")
    with pytest.raises(ValueError):
        bq.lqmm_gemm_q4_k_f16(torch.zeros(144, dtype=torch.uint8, device="cuda:0"), X, 1)
