"""Seeded synthetic inputs for the emulated FP8 GEMM.

This module holds none of the emulated arithmetic: it only draws FP8 operand
codes and scales.  Both the HIP path's tests and the CPU oracle's tests use it,
so that the two sides see the same bytes.

Recipe (the pages' own example in the user guide, section 3 "A first GEMM",
draws ``(torch.randn(M, K) * 40).clamp(-448, 448).to(torch.float8_e4m3fn)``
for the input first and then the weight the same way):

* one CPU ``torch.Generator`` seeded per workload and seed; x [M, K] is drawn
  first, then w [N, K];
* values are ``randn * sigma``, clamped to the format's largest finite value,
  then cast with torch's round-to-nearest-even cast;
* optional injected codes are written on the uint8 view with a second
  generator seeded at ``seed + 1000``: exact zeros (0x00 or 0x80 with equal
  probability) and subnormals (random sign, exponent field 0, mantissa uniform
  over the nonzero codes); the zero and subnormal masks are disjoint.

The pages measured Evo 2 projections on "Gaussian and adversarial data"; the
model weights and datasets are not available, so these Gaussian workloads
stand in for them, using the pages' shapes where the pages give one.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

FP8_DTYPES = {"e4m3fn": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FP8_MAX = {"e4m3fn": 448.0, "e5m2": 57344.0}
MANTISSA_BITS = {"e4m3fn": 3, "e5m2": 2}
OUT_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32,
              "e4m3fn": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    xfmt: str = "e4m3fn"
    wfmt: str = "e4m3fn"
    x_sigma: float = 40.0
    w_sigma: float = 40.0
    zero_frac: float = 0.0
    subnormal_frac: float = 0.0
    scale_x: float = 1 / 64
    scale_w: float = 1 / 32
    fast: bool = True
    split_S: int = 1
    out: str = "bf16"
    note: str = field(default="", compare=False)

    @property
    def gemm_ops(self) -> int:
        return 2 * self.M * self.N * self.K

    def describe(self) -> dict:
        return {
            "workload": self.name, "M": self.M, "N": self.N, "K": self.K,
            "x": self.xfmt, "w": self.wfmt, "fast_accum": self.fast, "split_S": self.split_S,
            "out": self.out, "scale_x": self.scale_x, "scale_w": self.scale_w,
        }


# The five workloads: sizes, value distributions and modes.
WORKLOADS = {
    "tiny": Workload("tiny", 16, 64, 256, note="tiny fast-accumulation GEMM"),
    "proj_64x5760x1920": Workload(
        "proj_64x5760x1920", 64, 5760, 1920,
        note="the user guide's example projection shape, M=64, K=1920, N=5760"),
    "slow_256x4096x4096": Workload(
        "slow_256x4096x4096", 256, 4096, 4096, zero_frac=0.05, subnormal_frac=0.05,
        scale_x=1 / 128, scale_w=1 / 16, fast=False, out="fp32",
        note="slow accumulation, 5% zeros and 5% subnormals"),
    "splitk_16x256x65536_s8": Workload(
        "splitk_16x256x65536_s8", 16, 256, 65536, x_sigma=8.0, w_sigma=8.0,
        scale_x=1 / 32, scale_w=1 / 32, split_S=8,
        note="split-K into 8 contiguous partials, serial combination"),
    "mixed_8192": Workload(
        "mixed_8192", 8192, 8192, 8192, wfmt="e5m2", x_sigma=40.0, w_sigma=1000.0,
        zero_frac=0.01, subnormal_frac=0.01, scale_x=1 / 256, scale_w=1 / 256,
        note="large e4m3 x e5m2 GEMM, 1% zeros and 1% subnormals of both signs"),
    # the validation page's own bench shape (its results table: the Evo 2 1B
    # projection at M = 2048), on the user guide's recipe
    "proj_2048x5760x1920": Workload(
        "proj_2048x5760x1920", 2048, 5760, 1920,
        note="the validation page's bench shape, the Evo 2 1B projection at M=2048"),
}
WORKLOAD_ORDER = ["tiny", "proj_64x5760x1920", "slow_256x4096x4096", "splitk_16x256x65536_s8",
                  "mixed_8192", "proj_2048x5760x1920"]


def fp8_codes(values: torch.Tensor, fmt: str) -> torch.Tensor:
    """Clamp to the format's range, cast with torch (RNE), return the uint8 codes."""
    lim = FP8_MAX[fmt]
    return values.clamp(-lim, lim).to(FP8_DTYPES[fmt]).view(torch.uint8)


def inject(codes: torch.Tensor, fmt: str, zero_frac: float, subnormal_frac: float,
           gen: torch.Generator) -> torch.Tensor:
    """Overwrite a random subset of codes with exact zeros and subnormals."""
    if zero_frac <= 0 and subnormal_frac <= 0:
        return codes
    u = torch.rand(codes.shape, generator=gen)
    zero_mask = u < zero_frac
    sub_mask = (u >= zero_frac) & (u < zero_frac + subnormal_frac)
    signs = torch.randint(0, 2, codes.shape, generator=gen, dtype=torch.uint8) << 7
    mbits = MANTISSA_BITS[fmt]
    mant = torch.randint(1, 1 << mbits, codes.shape, generator=gen, dtype=torch.uint8)
    out = codes.clone()
    out[zero_mask] = signs[zero_mask]
    out[sub_mask] = signs[sub_mask] | mant[sub_mask]
    return out


def make_operands(wl: Workload, seed: int = 0, M: int | None = None, N: int | None = None,
                  K: int | None = None):
    """(x codes uint8 [M, K], w codes uint8 [N, K]) on the CPU for a workload.
    M, N, K may be overridden to draw a smaller problem with the same recipe."""
    M = wl.M if M is None else M
    N = wl.N if N is None else N
    K = wl.K if K is None else K
    gen = torch.Generator().manual_seed(int(seed))
    x = fp8_codes(torch.randn(M, K, generator=gen) * wl.x_sigma, wl.xfmt)
    w = fp8_codes(torch.randn(N, K, generator=gen) * wl.w_sigma, wl.wfmt)
    gen2 = torch.Generator().manual_seed(int(seed) + 1000)
    x = inject(x, wl.xfmt, wl.zero_frac, wl.subnormal_frac, gen2)
    w = inject(w, wl.wfmt, wl.zero_frac, wl.subnormal_frac, gen2)
    return x.contiguous(), w.contiguous()


def random_codes(shape, fmt: str, gen: torch.Generator, finite: bool = True) -> torch.Tensor:
    """Uniformly random codes over all 256 patterns (finite ones only if asked)."""
    c = torch.randint(0, 256, shape, generator=gen, dtype=torch.int32).to(torch.uint8)
    if finite:
        if fmt == "e4m3fn":
            c = torch.where((c & 0x7F) == 0x7F, c & 0xF0, c)
        else:
            c = torch.where((c & 0x7C) == 0x7C, c & 0xF3, c)
    return c


def scale_bits(v: float) -> int:
    return int(np.array(v, dtype=np.float32).view(np.uint32))
