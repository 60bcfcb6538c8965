"""The allocation-free Q4_0 GEMV entry point (lqmm_gemv_q4_0_noalloc) through
the C ABI: the same outputs as lqmm_gemv_q4_0 given a workspace, on split-K
plans (which use the library's static per-GPU scratch) and on plans without
one; two calls in a row, the second smaller; oversized forced splits are
refused."""
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


def _pair(c):
    """(allocation-free result, lqmm_gemv_q4_0 result with a workspace)."""
    import torch
    W, x = dev(c.W.reshape(-1)), dev(c.x)
    y0 = torch.full((c.x.shape[0], c.N), float("nan"), dtype=torch.float32, device="cuda:0")
    bq.lqmm_gemv_q4_0_noalloc(W, x, c.N, out=y0)
    y1 = bq.lqmm_gemv_q4_0(W, x, c.N)
    return host(y0), host(y1)


@pytest.mark.parametrize("shapes", [
    # split-K plans: K = 16384 (four slices), then K = 8192 (two), smaller
    [(300, 16384, 2), (100, 8192, 1)],
    # a plan without split-K, then a split-K one
    [(4096, 4096, 1), (64, 16384, 2)],
])
def test_noalloc_matches_workspace_entry(orc, shapes):
    for i, (N, K, B) in enumerate(shapes):
        c = synth.q4_0_case(N, K, B, seed=17 * N + K + B)
        announce(f"noalloc q4_0 N={N} K={K} batch={B} (call {i + 1})")
        y0, y1 = _pair(c)
        assert np.array_equal(y0, y1)
        assert_close(y0, orc.gemv_q4_0(c.W, c.x, N, K), TOL_QUANT, f"noalloc {N}x{K} b{B}")


def test_noalloc_forced_split(orc, monkeypatch):
    """A forced split within the scratch runs (counters cleared by the call);
    one needing more than LQMM_NOALLOC_SCRATCH_BYTES is refused, and the next
    call still works."""
    monkeypatch.setenv("LQMM_TUNE_GEMV_SPLITK", "4")
    c = synth.q4_0_case(1024, 1024, 1, seed=3)
    announce("noalloc forced split 1024x1024")
    y0, y1 = _pair(c)
    assert np.array_equal(y0, y1)
    assert_close(y0, orc.gemv_q4_0(c.W, c.x, c.N, c.K), TOL_QUANT, "noalloc forced split")
    # 64 slices of one unit at 4096 x 4096, two rows: 2 MiB of partial sums
    monkeypatch.setenv("LQMM_TUNE_GEMV_SPLITK", "64")
    big = synth.q4_0_case(4096, 4096, 2, seed=5)
    announce("noalloc oversized split")
    with pytest.raises(bq.LqmmError) as e:
        bq.lqmm_gemv_q4_0_noalloc(dev(big.W.reshape(-1)), dev(big.x), big.N)
    assert e.value.status == 4
    monkeypatch.setenv("LQMM_TUNE_GEMV_SPLITK", "2")
    c2 = synth.q4_0_case(500, 2048, 2, seed=6)
    y0, y1 = _pair(c2)
    assert np.array_equal(y0, y1)
