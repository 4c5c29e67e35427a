"""Compile the HIP sources into the in-tree shared library libabs.so (gfx950).

Run ``python -m adaptive_block_sparse_amd.build``.  hipcc cross-compiles for
gfx950 without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libabs.so")
SOURCES = ["api.hip", "route.hip", "attend.hip", "noalloc.hip"]
# measurement aid (sustained MFMA rate and clock), a library of its own
PROBE_LIB = os.path.join(HERE, "libabs_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = os.environ.get("ABS_OFFLOAD_ARCH", "gfx950")


def hipcc_command(out: str = LIB, sources=None):
    sources = SOURCES if sources is None else sources
    return ["/opt/rocm/bin/hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-shared", "-Wall", "-Wno-unused-function",
            # no packed-fp32 instructions anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in sources], "-o", out]


def _compile(lib: str, sources, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = hipcc_command(tmp, sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer build of the same
# sources, for the CPU tests of the argument validation paths (device code is
# built as usual, without sanitizers).  Load it with the sanitizer runtime
# preloaded (host_sanitizer_env) and ABS_LIBRARY pointing at it.
SAN_LIB = os.path.join(HERE, "libabs_san.so")
SAN_FLAGS = ("-O1 -g -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined "
             "-Xarch_host -fno-omit-frame-pointer -shared-libsan")


def build_sanitized(verbose: bool = False) -> str:
    tmp = SAN_LIB + ".tmp"
    cmd = [c for c in hipcc_command(tmp) if c != "-O3"]
    cmd[1:1] = SAN_FLAGS.split()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def host_sanitizer_env() -> dict:
    """Environment for a process that loads SAN_LIB: the ASan runtime
    preloaded (the Python interpreter is not instrumented), leak checks off,
    any report fatal."""
    asan = subprocess.run(["/opt/rocm/bin/hipcc", "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ABS_LIBRARY=SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env


def build(verbose: bool = False) -> str:
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return _compile(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
