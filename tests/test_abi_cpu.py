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


def test_workspace_query(lib):
    assert bq.lqmm_gemv_workspace_bytes(4096, 4096, 1) == 0


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
