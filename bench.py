"""Benchmark of the bit-exact emulated FP8 GEMM on one MI355X.

One step is one emulated scaled GEMM over the whole workload (decode, block
chains, epilogue; and the split combination when the workload splits), with
the FP8 operands, scales, output and workspace already resident in HBM.
Prints one JSON line.

Metric: emulated GEMM-ops/s = 2*M*N*K / t, and the fraction of the
integer-VALU ceiling.

roofline.peak (bound "alu") is the VALU issue ceiling of the path's term
loop: every multiply-add needs one truncating FMA, and half of a byte
permute, a sign-pair bitop and a 16-bit dot product (2.5 instructions per
lane), and that mix issues at 3.40 cycles per wave instruction on gfx950
(measured, profiles/issue_ceiling.md), so the chip's 1,024 SIMDs at 2.4 GHz
issue at most 1,024 x 2.4e9 / 3.40 x 64 / 2.5 multiply-adds per second:
37.0e12 GEMM-ops/s.  Everything else the kernel issues (decode, block
maxima, per-block prologue and epilogue, addressing) counts against it.
roofline.issue_peak prices the kernel's own instructions (3.05 lane slots per
multiply-add, counted in its assembly) at that rate: 30.3e12 GEMM-ops/s.
roofline.frac_vs_R is the achieved rate over the op-count model R,
which charges 7 packed 16-bit integer operations per multiply-add (exponent
add, block maximum, alignment distance, significand product, shift-truncate,
sign, accumulate): 256 x 64 x 2.4e9 x 2 / 7 x 2 = 22.47e12 GEMM-ops/s; the
kernel fuses several of those into one instruction, so it can exceed R.

cpu_baseline: the CPU oracle, untuned, timed on the host on a bounded sample
of the same workload (whole rows of the output), and checked bit for bit
against the GPU's output on that sample.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from bit_exact_fp8_amd import api  # noqa: E402
from bit_exact_fp8_amd.inputs import (FP8_DTYPES, OUT_DTYPES, WORKLOADS, make_operands,  # noqa: E402
                                      scale_bits)

SIMDS, CLOCK = 256 * 4, 2.4e9
TERM_MIX_CYCLES = 3.38                     # cycles per wave instruction of the term mix (measured; see below)
TERM_LOOP_SLOTS_PER_MAC = 2.5              # fma + (perm + bitop3 + dot2c) / 2
R_MODEL = 256 * 64 * 2.4e9 * 2 / 7 * 2    # op-count model R: 7 packed 16-bit ops per MAC at 16 lanes per clock
METRIC = "bit-exact emulated FP8 GEMM ops/s (2MNK/s) and % of int-VALU roofline"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """sha256 over the GEMM library's sources (csrc/emu_* and fp_round.h,
    sorted by name)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_exact_fp8_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith("emu_") or name == "fp_round.h":
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    one exists for this workload and the current kernel source."""
    path = os.path.join(PROFILE_DIR, f"traffic_main_kernel_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
        digest = kernel_source_digest()
        if d.get("kernel_source_sha256") != digest:
            return None
        return d.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None


def load_issue_ceiling():
    """The term loop's issue ceiling at measured instruction rates, from the
    committed microbenchmark summary, or None."""
    path = os.path.join(PROFILE_DIR, "issue_ceiling.json")
    try:
        with open(path) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def peak_alu(ceiling) -> tuple[float, float]:
    """(term-loop issue ceiling in GEMM-ops/s, the term mix's cycles per wave
    instruction it rests on): from the committed microbenchmark summary, or
    the last measured 3.38 cycles."""
    cyc = (ceiling or {}).get("term_mix_cycles_per_wave_instruction") or TERM_MIX_CYCLES
    return SIMDS * CLOCK / cyc * 64 / TERM_LOOP_SLOTS_PER_MAC * 2, cyc


def oracle_threads() -> int:
    """Threads for the oracle: the host's cores, at most 16 (one GPU's share
    of its host)."""
    return min(16, os.cpu_count() or 1)


def cpu_baseline(wl, x, w, y_gpu, budget_s: float, profile: str = "hopper"):
    """Time the oracle on whole output rows, sized to about budget_s seconds."""
    import oracle
    orc = oracle.default()
    threads = oracle_threads()
    xs, ws = x.numpy(), w.numpy()
    sx, sw = scale_bits(wl.scale_x), scale_bits(wl.scale_w)
    # probe the rate on a small sample
    rows_probe = min(wl.M, threads)
    cols_probe = min(wl.N, 256)
    t0 = time.perf_counter()
    orc.scaled_mm(xs[:rows_probe], wl.xfmt, ws[:cols_probe], wl.wfmt, sx, sw, wl.out, wl.fast, wl.split_S,
                  profile=profile, threads=threads)
    dt = max(time.perf_counter() - t0, 1e-3)
    rate = rows_probe * cols_probe * wl.K / dt  # MAC/s
    rows = int(max(threads, min(wl.M, budget_s * rate / (wl.N * wl.K))))
    rows = max(threads, (rows // threads) * threads)
    rows = min(rows, wl.M)
    t0 = time.perf_counter()
    acc, y = orc.scaled_mm(xs[:rows], wl.xfmt, ws, wl.wfmt, sx, sw, wl.out, wl.fast, wl.split_S,
                           profile=profile, threads=threads)
    dt = time.perf_counter() - t0
    ops = 2 * rows * wl.N * wl.K
    same = bool(np.array_equal(y, y_gpu[:rows]))
    return {"value": ops / dt, "unit": "GEMM-ops/s", "cores": threads, "kind": "oracle",
            "sample": f"output rows 0..{rows - 1} (all {wl.N} columns, K={wl.K}) of the workload, "
                      f"{ops / 2:.3g} MACs in {dt:.1f} s",
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "gpu_bit_exact_on_sample": same}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rates():
    """The CPU oracle's own rates on the host, no GPU involved: the C oracle
    on one thread over the tiny workload and a row sample of the projection,
    the same on all threads (up to 16) over the projection, and the exact
    Python (Fraction) specification on one thread over the tiny workload,
    checked bit for bit against the C oracle there."""
    import oracle
    from oracle import spec
    orc = oracle.default()
    threads = oracle_threads()
    res = {"cpu": cpu_model(), "host_threads": os.cpu_count(), "threads_used": threads}

    def timed(fn, min_s=1.0):
        reps, t0 = 0, time.perf_counter()
        while True:
            out = fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                return out, dt / reps

    for name, rows, nthreads, key in (("tiny", None, 1, "c_oracle_1thread_tiny"),
                                      ("proj_64x5760x1920", 16, 1, "c_oracle_1thread_proj"),
                                      ("proj_64x5760x1920", None, threads, "c_oracle_all_threads_proj")):
        wl = WORKLOADS[name]
        x, w = make_operands(wl, 0)
        xs = x.numpy() if rows is None else x.numpy()[:rows]
        m = xs.shape[0]
        _, dt = timed(lambda: orc.scaled_mm(xs, wl.xfmt, w.numpy(), wl.wfmt, scale_bits(wl.scale_x),
                                            scale_bits(wl.scale_w), wl.out, wl.fast, wl.split_S, threads=nthreads))
        res[key] = {"gemm_ops_per_s": 2 * m * wl.N * wl.K / dt, "threads": nthreads,
                    "sample": f"{m} x {wl.N} x {wl.K}", "seconds": dt}
    wl = WORKLOADS["tiny"]
    x, w = make_operands(wl, 0)
    t0 = time.perf_counter()
    _, ys = spec.scaled_mm(x.numpy().tolist(), wl.xfmt, w.numpy().tolist(), wl.wfmt, scale_bits(wl.scale_x),
                           scale_bits(wl.scale_w), wl.out, wl.fast, wl.split_S)
    dt = time.perf_counter() - t0
    _, yc = orc.scaled_mm(x.numpy(), wl.xfmt, w.numpy(), wl.wfmt, scale_bits(wl.scale_x),
                          scale_bits(wl.scale_w), wl.out, wl.fast, wl.split_S, threads=1)
    res["python_spec_1thread_tiny"] = {"gemm_ops_per_s": 2 * wl.M * wl.N * wl.K / dt, "threads": 1,
                                       "sample": f"{wl.M} x {wl.N} x {wl.K}", "seconds": dt,
                                       "equals_c_oracle": bool(np.array_equal(np.array(ys, dtype=np.uint32),
                                                                              yc.astype(np.uint32)))}
    print(json.dumps({"oracle_rates": res}), flush=True)


def copy_reference(mib: int):
    """A plain device-to-device copy of a known size: reads and writes
    mib MiB once each.  Profiling it gives the scale of the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) for the same run conditions."""
    dev = torch.device("cuda:0")
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_reference_bytes": n, "dispatches": 3}), flush=True)


def output_bits(t):
    t = t.cpu()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy().astype(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32)


def cpu_baseline_incoming(wl, x, w, c_bits, acc_gpu, budget_s: float, profile: str = "hopper"):
    """The oracle's chains from incoming accumulators, timed on whole output
    rows sized to about budget_s seconds (one thread: the entry point is not
    threaded)."""
    import oracle
    orc = oracle.default()
    xs, ws = x.numpy(), w.numpy()
    t0 = time.perf_counter()
    orc.accumulate_c(xs[:1], wl.xfmt, ws[:256], wl.wfmt, c_bits[:1, :256], profile=profile)
    rate = 256 * wl.K / max(time.perf_counter() - t0, 1e-3)
    rows = int(max(1, min(wl.M, budget_s * rate / (wl.N * wl.K))))
    t0 = time.perf_counter()
    acc = orc.accumulate_c(xs[:rows], wl.xfmt, ws, wl.wfmt, c_bits[:rows], profile=profile)
    dt = time.perf_counter() - t0
    ops = 2 * rows * wl.N * wl.K
    return {"value": ops / dt, "unit": "GEMM-ops/s", "cores": 1, "kind": "oracle",
            "sample": f"output rows 0..{rows - 1} (all {wl.N} columns, K={wl.K}), chains from incoming "
                      f"accumulators, {ops / 2:.3g} MACs in {dt:.1f} s",
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "gpu_bit_exact_on_sample": bool(np.array_equal(acc, acc_gpu[:rows]))}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixed_8192", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile", type=int, default=-1, help="force a tile configuration (tuning)")
    ap.add_argument("--profile", default="hopper", choices=sorted(api.PROFILE),
                    help="arithmetic profile (hopper is the pages' default)")
    ap.add_argument("--inf-density", type=float, default=0.0, metavar="P",
                    help="replace a fraction P of the e5m2 operand's codes by +-Inf (specials throughput)")
    ap.add_argument("--out", default=None, choices=sorted(OUT_DTYPES),
                    help="override the workload's output type (FP8 outputs use scale_result 1)")
    ap.add_argument("--incoming-acc", action="store_true",
                    help="time emu_accumulate_c (chains from incoming accumulators) instead of emu_scaled_mm")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--oracle-rates", action="store_true",
                    help="only time the CPU oracle (C on 1 and all threads, Python spec on 1) on the host")
    ap.add_argument("--f4-census", action="store_true",
                    help="only count, on the host, the blocks an exact int8 matrix-core path could take")
    args = ap.parse_args()

    if args.oracle_rates:
        oracle_rates()
        return
    if args.f4_census:
        from bit_exact_fp8_amd import census
        census.main()
        return

    if args.copy_reference:
        copy_reference(args.copy_reference)
        return

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(one process, one MI355X).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)

    wl = WORKLOADS[args.workload]
    if args.out:
        wl = dataclasses.replace(wl, out=args.out)
    if args.incoming_acc and (not wl.fast or wl.split_S != 1):
        print("bench.py: --incoming-acc needs a fast-accumulation workload with split_S = 1", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    log(f"[bench] generating {wl.name} inputs (seed {args.seed})")
    x, w = make_operands(wl, args.seed)
    if args.inf_density > 0:
        if "e5m2" not in (wl.xfmt, wl.wfmt):
            print("bench.py: --inf-density needs an e5m2 operand", file=sys.stderr)
            sys.exit(2)
        t = w if wl.wfmt == "e5m2" else x
        gen = torch.Generator().manual_seed(args.seed + 2000)
        hit = torch.rand(t.shape, generator=gen) < args.inf_density
        signs = torch.randint(0, 2, t.shape, generator=gen, dtype=torch.uint8) << 7
        t[hit] = signs[hit] | 0x7C
        log(f"[bench] {int(hit.sum())} infinities in {'w' if t is w else 'x'}")
    xd = x.to(dev).view(FP8_DTYPES[wl.xfmt])
    wd = w.to(dev).view(FP8_DTYPES[wl.wfmt])
    sxd = torch.tensor([wl.scale_x], dtype=torch.float32, device=dev)
    swd = torch.tensor([wl.scale_w], dtype=torch.float32, device=dev)
    out = torch.empty((wl.M, wl.N), dtype=OUT_DTYPES[wl.out], device=dev)
    ws_bytes = api.workspace_bytes(wl.M, wl.N, wl.K, wl.split_S, wl.fast, args.profile)
    wsbuf = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    lib = api._lib()
    plan = api.plan_options(tile=args.tile if args.tile >= 0 else None)
    stream = torch.cuda.current_stream(dev)
    call_args = (xd.data_ptr(), api.FP8_FORMAT[xd.dtype], wl.K, wd.data_ptr(), api.FP8_FORMAT[wd.dtype], wl.K,
                 wl.M, wl.N, wl.K, sxd.data_ptr(), swd.data_ptr(), None, out.data_ptr(), api.OUT_DTYPE[out.dtype],
                 wl.N, int(wl.fast), wl.split_S, api.PROFILE[args.profile], wsbuf.data_ptr(), ws_bytes,
                 stream.cuda_stream, plan)

    def step():
        st = lib.emu_scaled_mm(*call_args)
        if st != 0:
            raise api.EmuError(st, lib.emu_last_error_message().decode())

    if args.incoming_acc:
        # incoming accumulators of a chain's size: N(0, 1) * 2^12, binary32
        gen = torch.Generator().manual_seed(args.seed + 3000)
        c_in = (torch.randn((wl.M, wl.N), generator=gen) * 4096.0).to(dev)
        out = torch.empty((wl.M, wl.N), dtype=torch.float32, device=dev)
        cin_args = (xd.data_ptr(), api.FP8_FORMAT[xd.dtype], wl.K, wd.data_ptr(), api.FP8_FORMAT[wd.dtype], wl.K,
                    wl.M, wl.N, wl.K, c_in.data_ptr(), wl.N, out.data_ptr(), wl.N, api.PROFILE[args.profile],
                    stream.cuda_stream, plan)

        def step():  # noqa: F811 -- the timed call of this mode
            st = lib.emu_accumulate_c(*cin_args)
            if st != 0:
                raise api.EmuError(st, lib.emu_last_error_message().decode())

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    log(f"[bench] timing {args.steps} steps")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ev_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    launch_ms = float(np.mean(ev_ms))
    ops = wl.gemm_ops
    value = ops * args.steps / wall
    achieved = ops / (launch_ms * 1e-3)

    default_call = args.inf_density == 0 and args.profile == "hopper" and not args.out and not args.incoming_acc
    traffic = load_traffic(wl.name) if default_call else None
    ceiling = load_issue_ceiling()
    peak, mix_cycles = peak_alu(ceiling)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "GEMM-ops/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {**wl.describe(), "profile": args.profile, "parallelism": "single GPU",
                   **({"inf_density": args.inf_density} if args.inf_density > 0 else {}),
                   **({"entry_point": "emu_accumulate_c", "out": "fp32 accumulator"} if args.incoming_acc else {})},
        "roofline": {
            "bound": "alu",
            "achieved": achieved / 1e12,
            "achieved_tmac_per_s": achieved / 2e12,
            "peak": peak / 1e12,
            "unit": "T GEMM-ops/s",
            "frac": achieved / peak,
            "peak_basis": f"term-loop issue ceiling: 1024 SIMDs x 2.4 GHz / {mix_cycles:.2f} cycles per wave "
                          "instruction (measured mix) x 64 lanes / 2.5 instructions per multiply-add x 2",
            "traffic": traffic,
            "R": R_MODEL / 1e12,
            "frac_vs_R": achieved / R_MODEL,
            "launch_ms": launch_ms,
            "launch_ms_min": float(np.min(ev_ms)),
            "launch_ms_median": float(np.median(ev_ms)),
        },
    }
    if default_call and wl.name == "mixed_8192" and ceiling and ceiling.get("gemm_ops_per_s"):
        # the kernel's own instruction mix at the term mix's issue rate (the
        # 8192^3 kernel: counted in its assembly)
        result["roofline"]["issue_peak"] = ceiling["gemm_ops_per_s"] / 1e12
        result["roofline"]["issue_frac"] = achieved / ceiling["gemm_ops_per_s"]
    if not args.no_cpu_baseline:
        log("[bench] cpu_baseline: timing the oracle on a sample")
        if args.incoming_acc:
            result["cpu_baseline"] = cpu_baseline_incoming(wl, x, w, output_bits(c_in), output_bits(out),
                                                           args.cpu_budget, args.profile)
        else:
            result["cpu_baseline"] = cpu_baseline(wl, x, w, output_bits(out), args.cpu_budget, args.profile)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
