"""Build the gfx950 BitLinear library (libbitlinear.so) in-tree with hipcc."""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbitlinear.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Quantisation decisions must be exact: IEEE division, no contraction.
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # Keep the compiler from forming packed fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


HEADER = os.path.join(os.path.dirname(PKG), "include", "bitlinear.h")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def source_sha256() -> str:
    """SHA-256 over the library's sources (kernels, internal headers, the C
    ABI header) and the compile flags; embedded in the library at build time
    so that a loader can tell a stale build from a current one."""
    h = hashlib.sha256()
    files = sources() + sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + [HEADER]
    for f in files:
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    h.update(" ".join(HIP_FLAGS).encode())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, f'-DBL_SOURCE_SHA256="{source_sha256()}"', *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libbitlinear.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
