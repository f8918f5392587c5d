"""Issue-rate model of the main kernel's stage loop on gfx950.

    python -m bit_exact_fp8_amd.issue_model [--rates RATES.json]

Compiles one main-kernel variant to gfx950 assembly (the library's own
flags), cuts the chosen kernel into basic blocks, and counts the VALU
instructions one wave issues per stage of its K walk: the stage loop's
blocks once, its inner self-loop (the per-block term loop) as many times as
it runs per stage, and the two sides of the stage's x / w decode split in
the proportion of waves that take each.  Divided by the multiply-adds one
wave does per stage, that is the kernel's VALU instructions per multiply-add
by opcode.

With the measured issue rate of each opcode (bit_exact_fp8_amd.microbench,
instructions per second over the whole chip at 8 waves per SIMD), the model
prices the stage: the time the chip needs to issue those instructions back
to back, one opcode class after another, gives the kernel's issue ceiling
in GEMM-ops/s.  Matrix-core (v_mfma) and LDS instructions run on their own
units and are counted but not priced.  Measurement and analysis only: the
GEMM library does not use this module.
"""
from __future__ import annotations

import argparse
import collections
import json
import os
import re
import subprocess
import tempfile

from . import build

# The 64x64-output matrix-core tile for 32-product blocks, e4m3fn x e5m2,
# fast accumulation (the kernel of the 8192^3 workload).
DEFAULT_KERNEL = "main_kernelILi0ELi1ELi64ELi64ELi4ELi4ELi1ELi0ELb1ELi32ELi1EE"
SIMDS = 256 * 4
CLOCK = 2.4e9

TERMINATORS = ("s_branch", "s_cbranch_", "s_endpgm", "s_setpc_b64")


def assemble(blk: int = 32, xf: int = 0, wf: int = 1) -> str:
    """gfx950 assembly of emu_variant.hip for one block width and format
    pair, with the library's compile flags."""
    flags = [f for f in build.FLAGS if f not in ("-fPIC",)]
    with tempfile.TemporaryDirectory(prefix="emu_asm_") as d:
        out = os.path.join(d, "variant.s")
        cmd = [build.HIPCC, *flags, f"-DEMU_VARIANT_BLK={blk}", f"-DEMU_VARIANT_XF={xf}",
               f"-DEMU_VARIANT_WF={wf}", "--offload-device-only", "-S",
               os.path.join(build.CSRC, "emu_variant.hip"), "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
        return open(out).read()


def kernel_lines(asm: str, key: str) -> list[str]:
    """The instruction and label lines of the kernel whose symbol holds key."""
    lines = asm.split("\n")
    start = next(i for i, l in enumerate(lines) if re.match(r"^_Z\S*" + re.escape(key) + r"\S*:", l))
    body = []
    for l in lines[start + 1:]:
        if l.startswith(".Lfunc_end"):
            break
        t = l.split(";")[0].strip()
        if t and (t.endswith(":") or not t.startswith(".")):
            body.append(t)
    return body


def basic_blocks(body: list[str]):
    """[(label, [instructions])], cut at labels and after terminators."""
    blocks, cur = [], None
    for t in body:
        if t.endswith(":"):
            cur = (t[:-1], [])
            blocks.append(cur)
            continue
        if cur is None:
            cur = ("entry", [])
            blocks.append(cur)
        cur[1].append(t)
        if t.startswith(TERMINATORS):
            cur = (f"{cur[0]}+{len(blocks)}", [])
            blocks.append(cur)
    return [b for b in blocks if b[1]]


def target(ins: str):
    m = re.search(r"(\.LBB\d+_\d+)", ins)
    return m.group(1) if m else None


def stage_weights(blocks, inner_trips: int, then_share: float):
    """Per-stage execution weights of the stage loop's blocks: the loop is
    the union of the backward branches (block j to an earlier or the same
    block i) whose span i..j holds an s_barrier, from the smallest i to the
    largest j (the compiler may rotate the loop so that it is entered in its
    middle); a block branching to itself is the inner loop (inner_trips runs
    per stage); the sides of an exec-mask if / else (a block with s_xor_b64
    of exec ending in s_cbranch_execz) weigh then_share and 1 - then_share."""
    labels = [b[0] for b in blocks]
    index = {lab: i for i, lab in enumerate(labels)}
    barrier = [any(x.startswith("s_barrier") for x in b[1]) for b in blocks]
    spans = []
    for j, (_, ins) in enumerate(blocks):
        for x in ins:
            i = index.get(target(x)) if x.startswith(TERMINATORS) else None
            if i is not None and i <= j and any(barrier[i:j + 1]):
                spans.append((i, j))
    head = min(i for i, _ in spans)
    latch = max(j for _, j in spans)
    w = {}
    i = head
    while i <= latch:
        lab, ins = blocks[i]
        w[lab] = w.get(lab, 1.0)
        last = ins[-1]
        if target(last) == lab:
            w[lab] = float(inner_trips)
        if last.startswith("s_cbranch_execz") and any(x.startswith("s_xor_b64") and "exec" in x for x in ins):
            else_lab = target(last)
            j = i + 1
            while j <= latch and blocks[j][0] != else_lab:
                w[blocks[j][0]] = then_share
                j += 1
            # the else side runs up to its own execz skip target
            k = j
            end_lab = None
            while k <= latch:
                w[blocks[k][0]] = 1.0 - then_share
                lastk = blocks[k][1][-1]
                if lastk.startswith("s_cbranch_execz"):
                    end_lab = target(lastk)
                    break
                k += 1
            k += 1
            while k <= latch and blocks[k][0] != end_lab:
                w[blocks[k][0]] = 1.0 - then_share
                k += 1
            i = k
            continue
        i += 1
    return w


def opcode_counts(blocks, weights):
    counts = collections.Counter()
    for lab, ins in blocks:
        if lab not in weights:
            continue
        for x in ins:
            counts[x.split()[0]] += weights[lab]
    return counts


def normalise(op: str) -> str:
    """Opcode without its encoding suffix (_e32, _e64, _sdwa, _dpp)."""
    return re.sub(r"_(e32|e64|sdwa|dpp)$", "", op)


def model(rates: dict | None, kernel: str = DEFAULT_KERNEL, inner_trips: int = 8, then_share: float = 0.5,
          macs_per_wave_stage: int = 64 * 16 * 32, asm: str | None = None) -> dict:
    blocks = basic_blocks(kernel_lines(asm or assemble(), kernel))
    w = stage_weights(blocks, inner_trips, then_share)
    counts = opcode_counts(blocks, w)
    valu = {normalise(k): 0.0 for k in counts}
    for k, v in counts.items():
        valu[normalise(k)] += v
    valu = {k: v for k, v in valu.items() if k.startswith("v_") and not k.startswith("v_mfma")}
    mfma = sum(v for k, v in counts.items() if k.startswith("v_mfma"))
    lds = sum(v for k, v in counts.items() if k.startswith("ds_"))
    total = sum(valu.values())
    res = {"kernel": kernel, "valu_per_wave_stage": total, "mfma_per_wave_stage": mfma,
           "lds_per_wave_stage": lds, "macs_per_wave_stage": macs_per_wave_stage,
           "valu_lane_slots_per_mac": total * 64 / macs_per_wave_stage,
           "valu_by_opcode": dict(sorted(valu.items(), key=lambda kv: -kv[1]))}
    if rates:
        # seconds the chip needs to issue one wave-stage's instructions on
        # every SIMD: instructions / (chip instructions per second / SIMDs)
        missing = [k for k in valu if k not in rates]
        default = max(rates.values())  # unmeasured opcodes at the fastest measured rate (an upper bound)
        t = sum(v / ((rates.get(k, default)) / SIMDS) for k, v in valu.items())
        mac_rate = macs_per_wave_stage * SIMDS / t
        res.update({"issue_ceiling_gemm_ops_per_s": 2 * mac_rate, "unmeasured_opcodes": missing,
                    "wave_stage_issue_cycles": t * CLOCK})
    return res


TERM_LOOP_SLOTS_PER_MAC = 2.5  # fma + (perm + bitop3 + dot2c) / 2 per multiply-add


def ceilings(rates: dict, term_mix_rate: float, kernel: str = DEFAULT_KERNEL, asm: str | None = None) -> dict:
    """The issue ceilings of a kernel from measured rates: the term loop alone
    at the term mix's rate (2.5 instructions per multiply-add), the kernel's
    own instructions per multiply-add at that rate, and the per-class
    additive estimate (each opcode class at its own measured rate)."""
    m = model(rates, kernel, asm=asm)
    cyc = SIMDS * CLOCK / term_mix_rate  # cycles per wave instruction of the term mix
    term_ceiling = SIMDS * CLOCK / cyc * 64 / TERM_LOOP_SLOTS_PER_MAC * 2
    own = SIMDS * CLOCK / cyc * 64 / m["valu_lane_slots_per_mac"] * 2
    return {
        "term_mix_cycles_per_wave_instruction": cyc,
        "term_loop_ceiling_gemm_ops_per_s": term_ceiling,
        "kernel_valu_per_wave_stage": m["valu_per_wave_stage"],
        "kernel_macs_per_wave_stage": m["macs_per_wave_stage"],
        "kernel_valu_lane_slots_per_mac": m["valu_lane_slots_per_mac"],
        "gemm_ops_per_s": own,
        "additive_per_class_estimate_gemm_ops_per_s": m.get("issue_ceiling_gemm_ops_per_s"),
        "unmeasured_opcodes": m.get("unmeasured_opcodes", []),
        "rates_cycles_per_wave_instruction": {k: round(SIMDS * CLOCK / v, 3) for k, v in rates.items()},
        "valu_by_opcode_per_wave_stage": m["valu_by_opcode"],
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--rates", help="JSON lines of bit_exact_fp8_amd.microbench (instruction rates)")
    ap.add_argument("--kernel", default=DEFAULT_KERNEL)
    ap.add_argument("--json", help="write the issue ceilings (needs --rates) to this file")
    args = ap.parse_args()
    rates, term_mix = None, None
    if args.rates:
        rates = {}
        for line in open(args.rates):
            line = line.strip()
            if line.startswith("{"):
                d = json.loads(line)
                if "instructions_per_s" not in d:
                    continue
                if d["instruction"].startswith("term mix:"):
                    term_mix = d["instructions_per_s"]
                elif not d["instruction"].startswith("term mix"):
                    rates[d["instruction"]] = d["instructions_per_s"]
    if args.json:
        if not rates or term_mix is None:
            raise SystemExit("--json needs --rates with the term mix row")
        out = {"about": "Issue ceilings of the 8192^3 main kernel (64x64 matrix-core tile, e4m3fn x e5m2, "
                        "32-product blocks): instruction rates from python3 -m bit_exact_fp8_amd.microbench "
                        "--iters 20000 on one MI355X, instruction counts from this module on the same sources.",
               **ceilings(rates, term_mix, args.kernel)}
        with open(args.json, "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
    print(json.dumps(model(rates, args.kernel)), flush=True)


if __name__ == "__main__":
    main()
