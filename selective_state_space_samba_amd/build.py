"""Build the HIP library (libsamba_scan.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsamba_scan.so")
MAIN = os.path.join(CSRC, "samba_scan.hip")
# the benchmark's measurement of the vector-ALU issue rates (not part of the scan's C ABI)
PROBE_LIB = os.path.join(PKG, "libsamba_probe.so")
PROBE = os.path.join(CSRC, "peak_probe.hip")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-shared", "-fPIC",
    # packed fp32 instructions are disabled on purpose (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                  glob.glob(os.path.join(PKG, "..", "include", "*.h")))


def _hipcc(src: str, lib: str, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + ["-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build_library(verbose: bool = False) -> str:
    _hipcc(MAIN, LIB, verbose)
    _hipcc(PROBE, PROBE_LIB, verbose)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in sources())


if __name__ == "__main__":
    print(build_library(verbose=True))
