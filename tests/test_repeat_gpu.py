"""Repeatability on the GPU: every kernel family, reached through its entry
point with the planner's choice or a forced form, gives bitwise-equal results
over repeated calls.

Between the repeats other work runs (a different library call on other data,
and torch work that touches other memory), and one repeat runs on a second
stream, so the calls meet different cache contents and timing. No kernel here
adds in an order that depends on timing: in-workgroup k-slices add in slice
order, split-K partials are added by the last arrival in slice order, and the
GEMMs own their output tiles. Any difference would show an unordered
reduction or a race.
"""
import numpy as np
import pytest

import block_quantized_matmul_amd as bq
import synth
from gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu

REPEATS = 5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bq.load()


def _gemv(fn, c):
    W, x = dev(c.W.reshape(-1)), dev(c.x)
    return lambda: fn(W, x, c.N)


def _gemm(fn, c):
    W, X = dev(c.W.reshape(-1)), dev(c.X)
    return lambda: fn(W, X, c.N)


def _i4(c):
    Wq, sc, z, x = dev(c.Wq.view(np.int32)), dev(c.scales), dev(c.zeros), dev(c.x)
    return lambda: bq.lqmm_gemv_i4g32(Wq, sc, z, x, c.N)


def _sgemm(c):
    A, B = dev(c.A), dev(c.B)
    return lambda: bq.lqmm_sgemm(A, B)


# (label, builder, environment): each label names the kernel the shape and
# the overrides select
CASES = [
    ("q4_0 1024x1024 b1 small-problem", lambda: _gemv(bq.lqmm_gemv_q4_0, synth.make("q4_0_gemv_1024")), {}),
    ("q4_0 4096x4096 b1 small split-K 4", lambda: _gemv(bq.lqmm_gemv_q4_0, synth.q4_0_case(4096, 4096, 1, seed=5)),
     {"LQMM_TUNE_GEMV_SPLITK": "4"}),
    ("q4_0 4096x4096 b4 whole share", lambda: _gemv(bq.lqmm_gemv_q4_0, synth.make("q4_0_gemv_4096x4096_b4")), {}),
    ("q4_0 12288x4096 b4 coalesced", lambda: _gemv(bq.lqmm_gemv_q4_0, synth.q4_0_case(12288, 4096, 4, seed=6)),
     {"LQMM_TUNE_GEMV_WHOLE": "0"}),
    ("q4_0 12288x4096 b1 streamed", lambda: _gemv(bq.lqmm_gemv_q4_0, synth.q4_0_case(12288, 4096, 1, seed=7)),
     {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "1"}),
    ("q4_0 12288x4096 b2 register-loading", lambda: _gemv(bq.lqmm_gemv_q4_0, synth.q4_0_case(12288, 4096, 2, seed=8)),
     {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_STREAM": "0"}),
    ("q4_0 300x4000 b5 generic matrix-core", lambda: _gemv(bq.lqmm_gemv_q4_0, synth.q4_0_case(300, 4000, 5, seed=9)),
     {"LQMM_TUNE_GEMV_SMALL": "0"}),
    ("q4_k 4096x8192 b8 activations in registers", lambda: _gemv(bq.lqmm_gemv_q4_k, synth.q4_k_case(4096, 8192, 8, seed=10)),
     {"LQMM_TUNE_GEMV_SMALL": "0", "LQMM_TUNE_GEMV_XREGS": "1"}),
    ("q4_k 14336x4096 b1 streamed", lambda: _gemv(bq.lqmm_gemv_q4_k, synth.q4_k_case(14336, 4096, 1, seed=11)), {}),
    ("q8_0 gemv 4096x4096 b1", lambda: _gemv(bq.lqmm_gemv_q8_0, synth.q8_0_gemv_case(4096, 4096, 1, seed=12)), {}),
    ("q6_k gemv 2048x4096 b2", lambda: _gemv(bq.lqmm_gemv_q6_k, synth.q6_k_case(2048, 4096, 2, seed=13)), {}),
    ("q2_k gemv 2048x4096 b1", lambda: _gemv(bq.lqmm_gemv_q2_k, synth.q2_k_case(2048, 4096, 1, seed=14)), {}),
    ("q1_0 gemv 2048x8192 b3", lambda: _gemv(bq.lqmm_gemv_q1_0, synth.q1_0_case(2048, 8192, 3, seed=15)), {}),
    ("i4g32 gemv 2048x4096 b1", lambda: _i4(synth.i4g32_case(2048, 4096, 1, seed=16)), {}),
    ("q8_0 gemm 256x2048x4096", lambda: _gemm(bq.lqmm_gemm_q8_0_f16, synth.q8_0_case(256, 2048, 4096, seed=17)), {}),
    ("q8_0 gemm ragged K 200x300x1056", lambda: _gemm(bq.lqmm_gemm_q8_0_f16, synth.q8_0_case(200, 300, 1056, seed=18)), {}),
    ("q4_0 gemm 256x2048x4096", lambda: _gemm(bq.lqmm_gemm_q4_0_f16, synth.q4_0_gemm_case(256, 2048, 4096, seed=19)), {}),
    ("q4_k gemm 256x2048x4096", lambda: _gemm(bq.lqmm_gemm_q4_k_f16, synth.q4_k_gemm_case(256, 2048, 4096, seed=20)), {}),
    ("sgemm 513x511x509", lambda: _sgemm(synth.sgemm_case(513, 511, 509, seed=21)), {}),
]


@pytest.mark.parametrize("label,build,env", CASES, ids=[c[0] for c in CASES])
def test_repeat_bitwise(monkeypatch, label, build, env):
    import torch
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    announce(f"repeat {label}")
    call = build()
    other = _gemv(bq.lqmm_gemv_q4_k, synth.q4_k_case(2048, 4096, 3, seed=99))
    junk = torch.randn(1 << 22, device="cuda:0")
    side = torch.cuda.Stream()
    ys = []
    for i in range(REPEATS):
        if i == REPEATS - 1:
            with torch.cuda.stream(side):
                out = call()
            side.synchronize()
        else:
            out = call()
        ys.append(host(out).copy())
        other()
        junk.mul_(0.5).add_(1.0)
    torch.cuda.synchronize()
    for i, y in enumerate(ys[1:], 1):
        assert np.array_equal(y, ys[0], equal_nan=True), f"{label}: repeat {i} differs"
    assert np.isfinite(ys[0]).all(), label
