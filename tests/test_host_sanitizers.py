"""The host-side argument validation of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): the library is rebuilt with the host
code instrumented, and the host ABI tests run against it in a child process
with the sanitizer runtime preloaded.  Any report aborts that process."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from adaptive_block_sparse_amd import build as B  # noqa: E402


def _stale():
    if not os.path.exists(B.SAN_LIB):
        return True
    t = os.path.getmtime(B.SAN_LIB)
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)]
    srcs.append(os.path.join(ROOT, "include", "abs.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def san_lib():
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    if _stale():
        B.build_sanitized()
    return B.SAN_LIB


def test_sanitized_library_is_instrumented(san_lib):
    syms = subprocess.run(["nm", "-D", "--undefined-only", san_lib], capture_output=True,
                          text=True).stdout
    assert "__asan_report_load" in syms or "__asan_loadN" in syms
    assert "__ubsan_handle_" in syms


def test_host_abi_tests_pass_under_the_sanitizers(san_lib):
    env = B.host_sanitizer_env()
    assert os.path.exists(env["LD_PRELOAD"])
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr, tail
    # the child really ran against the sanitized build
    probe = subprocess.run([sys.executable, "-c",
                            "import adaptive_block_sparse_amd as A; print(A.LIB_PATH)"],
                           env=env, cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert probe.stdout.strip() == san_lib, probe.stderr[-2000:]
