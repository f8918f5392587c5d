"""Build libemu_fp8gemm.so for gfx950 with hipcc (in-tree, next to this file).

The main kernel's variants (block width x format pair) are separate
translation units of emu_variant.hip (and of emu_cin_variant.hip for the
chains from incoming accumulators), compiled in parallel and linked with the
dispatcher, the combine kernel, the deferred-infinity kernels
(emu_specials.hip), the no-allocation entry point (emu_noalloc.hip) and the
C ABI."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUTPUT = os.path.join(PKG, "libemu_fp8gemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-fno-fast-math", "-ffp-contract=off",
    # hipcc -O3 may form packed binary32 instructions on its own; keep them out
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-DEMU_BUILDING_LIBRARY",
    f"-I{os.path.join(ROOT, 'include')}",
]

# (block width, x format, w format): e5m2 x e5m2 is rejected by the ABI.
VARIANTS = [(b, xf, wf) for b in (32, 16) for xf, wf in ((0, 0), (0, 1), (1, 0))]


def _units(objdir: str):
    units = [(os.path.join(CSRC, "emu_kernels.hip"), os.path.join(objdir, "emu_kernels.o"), []),
             (os.path.join(CSRC, "emu_specials.hip"), os.path.join(objdir, "emu_specials.o"), []),
             (os.path.join(CSRC, "emu_noalloc.hip"), os.path.join(objdir, "emu_noalloc.o"), []),
             (os.path.join(CSRC, "emu_api.cpp"), os.path.join(objdir, "emu_api.o"), [])]
    for b, xf, wf in VARIANTS:
        defs = [f"-DEMU_VARIANT_BLK={b}", f"-DEMU_VARIANT_XF={xf}", f"-DEMU_VARIANT_WF={wf}"]
        units.append((os.path.join(CSRC, "emu_variant.hip"), os.path.join(objdir, f"emu_variant_{b}_{xf}{wf}.o"), defs))
        units.append((os.path.join(CSRC, "emu_cin_variant.hip"), os.path.join(objdir, f"emu_cin_{b}_{xf}{wf}.o"),
                      defs))
    return units


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libemu_fp8gemm.so")


def build(output: str = OUTPUT, extra_flags=None, verbose: bool = False, jobs: int | None = None) -> str:
    jobs = jobs or min(8, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="emu_build_") as objdir:
        units = _units(objdir)
        cmds = [[HIPCC, *FLAGS, *(extra_flags or []), *defs, "-c", src, "-o", obj] for src, obj, defs in units]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = output + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[obj for _, obj, _ in units], "-o", tmp], verbose)
    os.replace(tmp, output)
    return output


MICROBENCH_OUTPUT = os.path.join(PKG, "libemu_microbench.so")


def build_microbench(output: str = MICROBENCH_OUTPUT, verbose: bool = False) -> str:
    """The issue-rate microbenchmark (measurement only, not part of the GEMM)."""
    tmp = output + ".tmp"
    _run([HIPCC, *FLAGS, "-shared", os.path.join(CSRC, "microbench.hip"), "-o", tmp], verbose)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_microbench(verbose=True))
