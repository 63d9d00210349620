"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The double-precision oracle (oracle/ne_oracle.c) built with gcc -fsanitize=address,undefined
  and driven on small shapes by tests/sanitize/oracle_driver.c (exact-size buffers, so any access
  past an array is reported).
* The library's host code (the C ABI's argument validation in api.hip and the launch helpers it
  reaches) built with hipcc, the sanitizers on the host pass only (-Xarch_host before each
  -fsanitize=), driven through every rejection path by tests/sanitize/abi_driver.cpp; every call
  there returns before any launch, so no GPU is needed.
Any sanitizer report makes the program exit non-zero.
"""
import concurrent.futures
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "causal_gqa_flashattention_ne_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        subprocess.run(["gcc", "-std=c99", "-g", "-O1", "-fopenmp", "-fno-omit-frame-pointer",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        os.path.join(ROOT, "oracle", "ne_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                        "-lm", "-o", exe], check=True, capture_output=True)
        _run(exe)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_validation_under_asan_ubsan():
    from causal_gqa_flashattention_ne_amd import build as b
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    flags = [f for f in b.FLAGS if f != "-fPIC"] + san
    with tempfile.TemporaryDirectory() as d:
        def comp(src):
            obj = os.path.join(d, src + ".o")
            subprocess.run([HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj], check=True,
                           capture_output=True)
            return obj
        with concurrent.futures.ThreadPoolExecutor(len(b.SOURCES)) as ex:
            objs = list(ex.map(comp, b.SOURCES))
        # the driver is host code: clang++ compiles it and links everything with the sanitizer
        # runtimes and the HIP runtime
        exe = os.path.join(d, "abi_driver")
        subprocess.run([CLANG, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-I" + os.path.join(ROOT, "include"), os.path.join(HERE, "abi_driver.cpp")] + objs +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                       check=True, capture_output=True)
        _run(exe)
