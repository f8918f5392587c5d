"""Build libemu_fp8gemm.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "emu_kernels.hip"), os.path.join(CSRC, "emu_api.cpp")]
OUTPUT = os.path.join(PKG, "libemu_fp8gemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-fno-fast-math", "-ffp-contract=off",
    # hipcc -O3 may form packed binary32 instructions on its own; keep them out
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-DEMU_BUILDING_LIBRARY",
    f"-I{os.path.join(ROOT, 'include')}",
]


def build(output: str = OUTPUT, extra_flags=None, verbose: bool = False) -> str:
    tmp = output + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libemu_fp8gemm.so")
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
