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


def build(verbose: bool = False) -> str:
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return _compile(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
