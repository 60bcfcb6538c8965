"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs of the CPU oracle
and of the C ABI's host code (CPU only).

- The oracle (oracle/lqmm_oracle.c) is built with gcc and both sanitizers
  together with tests/sanitize/oracle_check.c, which calls every exported
  oracle function on ragged shapes with exactly-sized buffers, with and
  without row/column subsets, with leak detection on.
- The library's sources are built with the sanitizers on their host code
  only (device code is compiled as usual; no GPU sanitizer is involved) and
  linked with tests/sanitize/abi_check.c, which calls every entry point with
  arguments the boundary must reject and checks the documented status, and,
  with no GPU visible, well-formed calls that must fail with LQMM_ERR_DEVICE.

Any sanitizer report aborts the check program (-fno-sanitize-recover=all) and
fails the test. Builds go to a temporary directory.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "block_quantized_matmul_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(SAN, "oracle_check.c"), os.path.join(ROOT, "oracle", "lqmm_oracle.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "oracle sanitizer run: ok" in r.stdout


def _gpu_visible():
    return os.path.exists("/dev/kfd") and bool(os.environ.get("HIP_VISIBLE_DEVICES", "x"))


def test_abi_host_code_under_asan_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not available")
    import sys
    sys.path.insert(0, ROOT)
    from block_quantized_matmul_amd import build as bqbuild

    # host code instrumented; every -fsanitize= goes to the host pass only
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in bqbuild.FLAGS if f != "-O3"] + ["-O1"] + host_san

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        _run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(bqbuild.SOURCES))) as ex:
        objs = list(ex.map(compile_one, bqbuild.SOURCES))
    drv = str(tmp_path / "abi_check.o")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(SAN, "abi_check.c"), "-o", drv])
    exe = str(tmp_path / "abi_check")
    _run([CLANG + "++", "-fsanitize=address,undefined", drv, *objs,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
          "-o", exe])
    args = [] if _gpu_visible() else ["nodevice"]
    r = _run([exe, *args], env=ENV, timeout=300)
    assert "abi sanitizer run: ok" in r.stdout
