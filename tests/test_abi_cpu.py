"""The C-ABI library loads, exports every symbol include/lqmm.h declares, and
reports argument errors before touching a GPU (CPU only; no compute calls)."""
import ctypes
import os
import re
import subprocess

import pytest

import block_quantized_matmul_amd as bq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lqmm.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN = 0, 1, 2, 3


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lqmm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bq.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return bq.load()


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("lqmm_sgemm", "lqmm_gemv_q4_0", "lqmm_gemm_q8_0_f16", "lqmm_gemv_q4_k"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bq.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lqmm_[a-z0-9_]+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name
        getattr(lib, name)
    assert set(bq.EXPORTS) == set(_declared())


def test_probe_library_loads(lib):
    # the bench's streaming-read probe: its own library, built with liblqmm.so
    probe = os.path.join(os.path.dirname(bq.library_path()), "liblqmm_probe.so")
    assert os.path.exists(probe)
    out = subprocess.run(["nm", "-D", "--defined-only", probe],
                         capture_output=True, text=True, check=True).stdout
    assert re.search(r"\bT lqmm_probe_stream_read$", out, flags=re.M)
    ctypes.CDLL(probe).lqmm_probe_stream_read


def test_library_does_not_link_the_oracle(lib):
    out = subprocess.run(["nm", "-D", bq.library_path()], capture_output=True, text=True).stdout
    assert "oracle" not in out
    deps = subprocess.run(["ldd", bq.library_path()], capture_output=True, text=True).stdout
    assert "oracle" not in deps


def test_status_strings(lib):
    for s in range(7):
        assert bq.lqmm_status_string(s).startswith("LQMM_")
    assert "unknown" in bq.lqmm_status_string(99)
    assert bq.lqmm_version() >= 100


def test_workspace_query(lib, monkeypatch):
    """The split-K workspace the planner may ask for, the largest over the
    GEMV formats and over devices (one wave per workgroup, one unit per lane
    at most): none when one wave covers a row slice of 64 units; otherwise
    one arrival counter per row block (256-byte aligned) and S * batch * N
    fp32 partial sums."""
    monkeypatch.delenv("LQMM_TUNE_GEMV_SPLITK", raising=False)
    def need(rows_per_wave, N, S, B):
        blocks = (N + rows_per_wave - 1) // rows_per_wave
        return (blocks * 4 + 255) // 256 * 256 + S * B * N * 4
    # K = 1024: every format's row fits one wave slice (Q8_0: 32 units)
    assert bq.lqmm_gemv_workspace_bytes(1024, 1024, 1) == 0
    # K = 4096: Q8_0 and the int4 layout (32-weight units, 128 per row) split
    # in two slices of 64 units, one row per wave
    assert bq.lqmm_gemv_workspace_bytes(4096, 4096, 1) == need(1, 4096, 2, 1)
    # K = 8192: 256 units of 32 weights, four slices
    assert bq.lqmm_gemv_workspace_bytes(100, 8192, 2) == need(1, 100, 4, 2)
    # K = 16384: eight slices
    assert bq.lqmm_gemv_workspace_bytes(64, 16384, 1) == need(1, 64, 8, 1)
    # more than four activation rows: passes of four
    assert bq.lqmm_gemv_workspace_bytes(100, 8192, 5) == need(1, 100, 4, 4)
    # a forced split at the 1024 x 1024 configuration: two slices of 16
    # 32-weight units (16 lanes per row, 4 rows per wave)
    monkeypatch.setenv("LQMM_TUNE_GEMV_SPLITK", "2")
    assert bq.lqmm_gemv_workspace_bytes(1024, 1024, 1) == need(4, 1024, 2, 1)


def test_workspace_alignment_checked(lib):
    f = lib.lqmm_gemv_q4_0
    assert f(A16, A16, A16, 8, 64, 1, A8, 4096, None) == ERR_ALIGN


# Fake but 16-byte aligned addresses: validation rejects the call before any
# HIP call, so they are never dereferenced.
A16 = 0x10000
A8 = 0x10008


@pytest.mark.parametrize("fn", ["lqmm_gemv_q4_0", "lqmm_gemv_q4_k"])
def test_gemv_argument_errors(lib, fn):
    f = getattr(lib, fn)
    blk = 32 if fn.endswith("q4_0") else 256
    assert f(None, A16, A16, 8, blk, 1, None, 0, None) == ERR_NULL
    assert f(A16, None, A16, 8, blk, 1, None, 0, None) == ERR_NULL
    assert f(A16, A16, None, 8, blk, 1, None, 0, None) == ERR_NULL
    assert f(A16, A16, A16, 0, blk, 1, None, 0, None) == ERR_SHAPE
    assert f(A16, A16, A16, -5, blk, 1, None, 0, None) == ERR_SHAPE
    assert f(A16, A16, A16, 8, 0, 1, None, 0, None) == ERR_SHAPE
    assert f(A16, A16, A16, 8, blk + 16, 1, None, 0, None) == ERR_SHAPE
    assert f(A16, A16, A16, 8, blk, 0, None, 0, None) == ERR_SHAPE
    assert f(A16, A16, A16, 8, (1 << 31) + blk, 1, None, 0, None) == ERR_SHAPE
    assert f(A8, A16, A16, 8, blk, 1, None, 0, None) == ERR_ALIGN
    assert f(A16, A8, A16, 8, blk, 1, None, 0, None) == ERR_ALIGN
    assert f(A16, A16, A8, 8, blk, 1, None, 0, None) == ERR_ALIGN


def test_gemm_argument_errors(lib):
    f = lib.lqmm_gemm_q8_0_f16
    assert f(None, A16, A16, 4, 4, 32, None) == ERR_NULL
    assert f(A16, A16, A16, 0, 4, 32, None) == ERR_SHAPE
    assert f(A16, A16, A16, 4, 0, 32, None) == ERR_SHAPE
    assert f(A16, A16, A16, 4, 4, 48, None) == ERR_SHAPE
    assert f(A16, A16, A16, 4, 4, 1 << 22, None) == ERR_SHAPE  # K limit of the GEMM
    assert f(A16, A8, A16, 4, 4, 32, None) == ERR_ALIGN


def test_sgemm_argument_errors(lib):
    f = lib.lqmm_sgemm
    assert f(A16, A16, None, 4, 4, 4, None) == ERR_NULL
    assert f(A16, A16, A16, 4, 0, 4, None) == ERR_SHAPE
    assert f(A16, A16, A16, 4, 4, -1, None) == ERR_SHAPE
    assert f(A16, A8, A16, 4, 4, 4, None) == ERR_ALIGN


def test_host_paths_from_many_threads(lib):
    """Sixteen host threads at once (ctypes releases the GIL, so the calls run
    concurrently in the library): the planner behind the workspace query
    gives every thread the answer a single thread gets, and the argument
    checks return their status codes. Without a GPU, well-formed calls reach
    the per-device set-up (std::call_once) and fail with LQMM_ERR_DEVICE."""
    import random
    import threading

    shapes = [(n, k, b) for n in (1, 100, 1024, 4096, 11008, 28672)
              for k in (32, 256, 1024, 4096, 8192, 16384) for b in (1, 2, 4, 8, 16)]
    expect = {s: bq.lqmm_gemv_workspace_bytes(*s) for s in shapes}
    buf = ctypes.create_string_buffer(4096 + 16)
    base = (ctypes.addressof(buf) + 15) // 16 * 16
    f = lib.lqmm_gemv_q4_0
    errors = []
    no_gpu = not os.path.exists("/dev/kfd")

    def work(seed):
        rng = random.Random(seed)
        for _ in range(1500):
            s = rng.choice(shapes)
            got = bq.lqmm_gemv_workspace_bytes(*s)
            if got != expect[s]:
                errors.append(("workspace", s, got, expect[s]))
            if f(None, base, base, 1, 32, 1, None, 0, None) != ERR_NULL:
                errors.append("null")
            if f(base, base, base, 1, 33, 1, None, 0, None) != ERR_SHAPE:
                errors.append("shape")
            if f(base + 4, base, base, 1, 32, 1, None, 0, None) != ERR_ALIGN:
                errors.append("align")
            if no_gpu and f(base, base, base, 2, 64, 1, None, 0, None) != 5:
                errors.append("device")

    ts = [threading.Thread(target=work, args=(i,)) for i in range(16)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors[:5]
