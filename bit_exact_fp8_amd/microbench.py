"""Issue rates of the main kernel's VALU instructions on one MI355X, and of
its term loop's mix: the measured side of the integer-VALU ceiling.

    python -m bit_exact_fp8_amd.microbench [--iters N]

Prints one JSON line per instruction: lane operations per second over the
whole chip (HIP events around one launch of 8 waves per SIMD) and that rate
as a fraction of the spec rate of 16 lanes per SIMD per clock at 2.4 GHz
(1,024 SIMDs: 3.93e13 lane operations per second).  The sustained clock is
read separately from rocprofv3's GRBM_GUI_ACTIVE over the same launches."""
from __future__ import annotations

import argparse
import ctypes
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libemu_microbench.so")
SIMDS = 256 * 4
SPEC_LANE_OPS = SIMDS * 16 * 2.4e9  # 16 lanes per SIMD per clock at 2.4 GHz
BLOCKS = 2048          # 8 waves on each of the 1,024 SIMDs
PER_ITER = 32          # instructions per loop iteration per wave


def load():
    if not os.path.exists(LIBRARY):
        raise RuntimeError(f"{LIBRARY} is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIBRARY)
    lib.mb_op_count.restype = ctypes.c_int
    lib.mb_op_name.argtypes = [ctypes.c_int]
    lib.mb_op_name.restype = ctypes.c_char_p
    lib.mb_issue_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.mb_issue_rate.restype = ctypes.c_int
    return lib


def measure(iters: int = 20000):
    """One row per instruction (op kernels) and one for each term mix (the
    last two ops: binary32 and binary16 operands): wave instructions and
    lane operations per second over the chip, the rate as a fraction of 16
    lanes per SIMD per clock at 2.4 GHz, and, for the term mixes, the
    multiply-add and GEMM-op rates they stand for (5 instructions per 2
    multiply-adds)."""
    lib = load()
    rows = []
    n = lib.mb_op_count()
    for op in range(n + 2):
        ms = ctypes.c_double()
        rc = lib.mb_issue_rate(op, iters, BLOCKS, ms)
        if rc != 0:
            raise RuntimeError(f"microbenchmark {op} failed with HIP error {rc}")
        per_iter = PER_ITER if op < n else 4 * 8 * 5
        wave_instr = BLOCKS * 4 * per_iter * iters
        rate = wave_instr / (ms.value * 1e-3)
        row = {"instruction": lib.mb_op_name(op).decode(), "ms": ms.value, "instructions_per_s": rate,
               "lane_ops_per_s": rate * 64, "of_spec_16_lanes_2.4GHz": rate * 64 / SPEC_LANE_OPS,
               "cycles_per_wave_instruction": SIMDS * 2.4e9 / rate}
        if op >= n:
            macs = rate * 64 * 2 / 5
            row.update({"term_mix_macs_per_s": macs, "term_mix_gemm_ops_per_s": 2 * macs})
        rows.append(row)
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--iters", type=int, default=20000)
    args = ap.parse_args()
    rows = measure(args.iters)
    for r in rows:
        print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
