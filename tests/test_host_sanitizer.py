"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The library is built a second time with the host sanitizers (device code as
usual) and the argument-check tests of test_abi.py run against that build in
a child process with the shared ASan runtime preloaded: any out-of-bounds
access, use after free, signed overflow or other undefined behaviour in the
plan checks, the workspace arithmetic or the error reporting aborts it.
"""
import os
import subprocess
import sys

import pytest

from sequence_approximate_attention_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def sanitized_env(lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = B.asan_runtime()
    env["SPAVA_LIBRARY"] = lib
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    try:
        B.hipcc()
        B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    return B.build_host_sanitized(str(tmp_path_factory.mktemp("host_sanitized")))


def test_sanitizer_reports_planted_overflow(tmp_path):
    # The harness itself: a planted signed overflow in host code built with
    # the same flags must abort the child under the same environment.
    src = tmp_path / "planted.hip"
    src.write_text('#include <cstdio>\nextern "C" int planted(int x) { return x + 2147483647; }\n')
    so = tmp_path / "libplanted.so"
    r = subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", str(src), "-o", str(so),
                        *B.HOST_SANITIZE, *B.HOST_SANITIZE_LINK], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("hipcc could not build the planted library: " + r.stderr[-500:])
    code = f"import ctypes; print(ctypes.CDLL({str(so)!r}).planted(5))"
    r = subprocess.run([sys.executable, "-c", code], env=sanitized_env(str(so)), capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and "runtime error" in r.stderr, r.stdout + r.stderr


def test_abi_checks_are_clean_under_host_sanitizers(sanitized_lib):
    # -s: a sanitizer report goes to stderr just before the abort, which
    # pytest's own capture would lose.
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=sanitized_env(sanitized_lib), cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
