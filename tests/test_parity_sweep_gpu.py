"""GPU parity over seeded random shapes: the quantized GEMVs (Q4_0, Q4_K) with
the planner's own choice and with the small-problem kernel switched off, the
prefill GEMMs (Q8_0, Q4_0, Q4_K x fp16) and the fp32 GEMM, each against the
CPU oracle on the same inputs. The shapes are drawn once from a fixed seed
(ragged N and M, K from one block up to long rows, one to seventeen
activation rows), so that tails, split-K plans and batch passes are reached
at sizes no hand-picked case names.

The further block formats (Q8_0, Q6_K, Q2_K, q1_0 and the int4 group-32
layout) run through their decode GEMVs the same way.

Outputs of more than 256 elements take the usual bars (2e-3 for the
quantized paths, 1e-5 / 1e-4 for fp32). Smaller outputs are checked per
element against a rounding bound, since one dot product can cancel by a large
factor and no relative bar holds on a single element:
- GEMVs: x is rounded to fp16 (2^-11 relative) and the codes' fp16 bias
  cancels in fp32 sums: (2^-11 + 2^-9) * sum_k |x w| + 2^-24 |y|.
- fp16 GEMMs: each weight is rounded to fp16 once and the output once:
  2^-9 * sum_k |x w| + 2^-10 |y|.
- fp32 GEMM: K fp32 additions: K * 2^-23 * sum_k |a b|.
"""
import numpy as np
import pytest

import block_quantized_matmul_amd as bq
import synth
from gpu_util import TOL_FP32, TOL_QUANT, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu

# multiply-adds per case, so that the oracle finishes each in well under a
# second on the host cores
MAX_MACS = 3e8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bq.load()


def _log_uniform(rng, hi):
    """An integer in [1, hi], log-uniform (small and large sizes alike)."""
    return max(1, min(hi, int(round(float(np.exp(rng.uniform(0.0, np.log(hi + 0.5))))))))


def _gemv_draws():
    rng = np.random.default_rng(20241)
    out = []
    for i in range(24):
        fmt = "q4_0" if i % 2 == 0 else "q4_k"
        blk = 32 if fmt == "q4_0" else 256
        # a third of each format's draws may take rows of up to 36864 weights
        kmax = 36864 if i % 6 in (0, 3) else 8192
        K = blk * int(rng.integers(1, kmax // blk + 1))
        B = int(rng.choice([1, 1, 1, 2, 2, 3, 4, 5, 8, 9, 16, 17]))
        N = _log_uniform(rng, max(1, min(20000, int(MAX_MACS // (K * B)))))
        out.append((fmt, N, K, B))
    return out


def _gemm_draws():
    rng = np.random.default_rng(20242)
    out = []
    for i in range(18):
        fmt = ("q8_0", "q8_0", "q4_0", "q4_k", "q8_0", "sgemm")[i % 6]
        blk = {"q8_0": 32, "q4_0": 32, "q4_k": 256, "sgemm": 1}[fmt]
        kmax = 700 if fmt == "sgemm" else 8192
        K = blk * int(rng.integers(1, kmax // blk + 1))
        M = _log_uniform(rng, 700)
        N = _log_uniform(rng, max(1, min(3000, int(MAX_MACS // (K * M)))))
        out.append((fmt, M, N, K))
    return out


def _format_draws():
    rng = np.random.default_rng(20243)
    out = []
    for i in range(15):
        fmt = ("q8_0", "q6_k", "q2_k", "q1_0", "i4g32")[i % 5]
        blk = 256 if fmt in ("q6_k", "q2_k") else 32
        K = blk * int(rng.integers(1, 16384 // blk + 1))
        B = int(rng.choice([1, 1, 2, 3, 4, 5, 9]))
        N = _log_uniform(rng, max(1, min(20000, int(MAX_MACS // (K * B)))))
        out.append((fmt, N, K, B))
    return out


GEMV_DRAWS = _gemv_draws()
GEMM_DRAWS = _gemm_draws()
FORMAT_DRAWS = _format_draws()


def _ids(draws):
    return ["-".join(str(v) for v in d) for d in draws]


@pytest.mark.parametrize("small", ["default", "0"])
@pytest.mark.parametrize("fmt,N,K,B", GEMV_DRAWS, ids=_ids(GEMV_DRAWS))
def test_gemv_random_shapes(orc, monkeypatch, small, fmt, N, K, B):
    if small != "default":
        monkeypatch.setenv("LQMM_TUNE_GEMV_SMALL", small)
    make = synth.q4_0_case if fmt == "q4_0" else synth.q4_k_case
    c = make(N, K, B, seed=N * 11 + K * 3 + B)
    announce(f"sweep {fmt} gemv N={N} K={K} batch={B} small={small}")
    fn = bq.lqmm_gemv_q4_0 if fmt == "q4_0" else bq.lqmm_gemv_q4_k
    y = host(fn(dev(c.W.reshape(-1)), dev(c.x), N)).astype(np.float64)
    ref = getattr(orc, f"gemv_{fmt}")(c.W, c.x, N, K)
    assert np.isfinite(y).all()
    if N * B > 256:
        assert_close(y, ref, TOL_QUANT, f"{fmt} {N}x{K} b{B}")
        return
    w = getattr(orc, f"dequant_{fmt}")(c.W, N, K)
    bound = (2.0 ** -11 + 2.0 ** -9) * (np.abs(c.x.astype(np.float64)) @ np.abs(w).T)
    assert np.all(np.abs(y - ref) <= bound + 2.0 ** -24 * np.abs(ref)), \
        float(np.max(np.abs(y - ref) / (bound + 1e-300)))


@pytest.mark.parametrize("fmt,M,N,K", GEMM_DRAWS, ids=_ids(GEMM_DRAWS))
def test_gemm_random_shapes(orc, fmt, M, N, K):
    announce(f"sweep {fmt} gemm M={M} N={N} K={K}")
    if fmt == "sgemm":
        s = synth.sgemm_case(M, N, K, seed=M * 5 + N + K)
        C = host(bq.lqmm_sgemm(dev(s.A), dev(s.B))).astype(np.float64)
        ref = orc.sgemm(s.A, s.B)
        assert np.isfinite(C).all()
        if M * N > 256:
            assert_close(C, ref, TOL_FP32, f"sgemm {M}x{N}x{K}")
            return
        bound = K * 2.0 ** -23 * (np.abs(s.A.astype(np.float64)) @ np.abs(s.B.astype(np.float64)))
        assert np.all(np.abs(C - ref) <= bound)
        return
    seed = M * 7 + N + K
    if fmt == "q8_0":
        c = synth.q8_0_case(M, N, K, seed=seed)
        fn, ref_fn = bq.lqmm_gemm_q8_0_f16, orc.gemm_q8_0_f16
    else:
        c = getattr(synth, f"{fmt}_gemm_case")(M, N, K, seed=seed)
        fn, ref_fn = getattr(bq, f"lqmm_gemm_{fmt}_f16"), getattr(orc, f"gemm_{fmt}_f16")
    Y = host(fn(dev(c.W.reshape(-1)), dev(c.X), N)).astype(np.float64)
    ref = ref_fn(c.W, c.X, N, K)
    assert np.isfinite(Y).all()
    if M * N > 256:
        assert_close(Y, ref, TOL_QUANT, f"{fmt} gemm {M}x{N}x{K}")
        return
    w = getattr(orc, f"dequant_{fmt}")(c.W, N, K)
    bound = 2.0 ** -9 * (np.abs(c.X.astype(np.float64)) @ np.abs(w).T)
    assert np.all(np.abs(Y - ref) <= bound + 2.0 ** -10 * np.abs(ref))


FORMAT_MAKE = {"q8_0": synth.q8_0_gemv_case, "q6_k": synth.q6_k_case, "q2_k": synth.q2_k_case,
               "q1_0": synth.q1_0_case, "i4g32": synth.i4g32_case}


@pytest.mark.parametrize("fmt,N,K,B", FORMAT_DRAWS, ids=_ids(FORMAT_DRAWS))
def test_format_gemv_random_shapes(orc, fmt, N, K, B):
    c = FORMAT_MAKE[fmt](N, K, B, seed=N * 13 + K + B)
    announce(f"sweep {fmt} gemv N={N} K={K} batch={B}")
    if fmt == "i4g32":
        y = bq.lqmm_gemv_i4g32(dev(c.Wq.view(np.int32)), dev(c.scales), dev(c.zeros), dev(c.x), N)
        ref = orc.gemv_i4g32(c.Wq, c.scales, c.zeros, c.x, N, K)
    else:
        y = getattr(bq, f"lqmm_gemv_{fmt}")(dev(c.W.reshape(-1)), dev(c.x), N)
        ref = getattr(orc, f"gemv_{fmt}")(c.W, c.x, N, K)
    y = host(y).astype(np.float64)
    assert np.isfinite(y).all()
    if N * B > 256:
        assert_close(y, ref, TOL_QUANT, f"{fmt} {N}x{K} b{B}")
        return
    w = (orc.dequant_i4g32(c.Wq, c.scales, c.zeros, N, K) if fmt == "i4g32"
         else getattr(orc, f"dequant_{fmt}")(c.W, N, K))
    bound = (2.0 ** -11 + 2.0 ** -9) * (np.abs(c.x.astype(np.float64)) @ np.abs(w).T)
    assert np.all(np.abs(y - ref) <= bound + 2.0 ** -24 * np.abs(ref)), \
        float(np.max(np.abs(y - ref) / (bound + 1e-300)))


# Every kernel family forced through the planner's tuning overrides on random
# shapes (the planner falls back where a forced form does not fit the shape):
# the matrix-core kernels at any batch, with activations in registers or in
# LDS, the whole-share kernel and the MFMA-layout kernel; the vector-ALU
# kernels (register-loading and streamed) at any batch.
FORCED = {
    "mfma": {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_MFMA": "1"},
    "mfma_xregs": {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_MFMA": "1",
                   "LQMM_TUNE_GEMV_WHOLE": "0", "LQMM_TUNE_GEMV_XREGS": "1"},
    "mfma_lds": {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_MFMA": "1",
                 "LQMM_TUNE_GEMV_WHOLE": "0", "LQMM_TUNE_GEMV_XREGS": "0"},
    "mfma_whole": {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_MFMA": "1",
                   "LQMM_TUNE_GEMV_WHOLE": "1"},
    "mfma_layout": {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_MFMA": "1",
                    "LQMM_TUNE_GEMV_LDSK": "0"},
    "valu_regs": {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_MFMA": "0",
                  "LQMM_TUNE_GEMV_STREAM": "0"},
    "valu_stream": {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_MFMA": "0",
                    "LQMM_TUNE_GEMV_STREAM": "1"},
}


def _forced_draws():
    rng = np.random.default_rng(20244)
    out = []
    for i in range(16):
        fmt = "q4_0" if i % 2 == 0 else "q4_k"
        blk = 32 if fmt == "q4_0" else 256
        K = blk * int(rng.integers(1, 16384 // blk + 1))
        B = int(rng.choice([1, 2, 3, 4, 7, 8, 16]))
        N = _log_uniform(rng, max(1, min(5000, int(MAX_MACS // (K * B)))))
        out.append((fmt, N, K, B))
    return out


FORCED_DRAWS = _forced_draws()


@pytest.mark.parametrize("form", sorted(FORCED))
@pytest.mark.parametrize("fmt,N,K,B", FORCED_DRAWS, ids=_ids(FORCED_DRAWS))
def test_gemv_forced_forms_random_shapes(orc, monkeypatch, form, fmt, N, K, B):
    for k, v in FORCED[form].items():
        monkeypatch.setenv(k, v)
    make = synth.q4_0_case if fmt == "q4_0" else synth.q4_k_case
    c = make(N, K, B, seed=N * 17 + K * 5 + B)
    announce(f"sweep {fmt} gemv N={N} K={K} batch={B} forced={form}")
    fn = bq.lqmm_gemv_q4_0 if fmt == "q4_0" else bq.lqmm_gemv_q4_k
    try:
        y = host(fn(dev(c.W.reshape(-1)), dev(c.x), N)).astype(np.float64)
    except bq.LqmmError as e:  # an override the planner cannot honour for this shape
        pytest.skip(f"refused: {e}")
    ref = getattr(orc, f"gemv_{fmt}")(c.W, c.x, N, K)
    assert np.isfinite(y).all()
    if N * B > 256:
        assert_close(y, ref, TOL_QUANT, f"{fmt} {N}x{K} b{B} {form}")
        return
    w = getattr(orc, f"dequant_{fmt}")(c.W, N, K)
    bound = (2.0 ** -11 + 2.0 ** -9) * (np.abs(c.x.astype(np.float64)) @ np.abs(w).T)
    assert np.all(np.abs(y - ref) <= bound + 2.0 ** -24 * np.abs(ref)), \
        float(np.max(np.abs(y - ref) / (bound + 1e-300)))
