"""CPU oracle for the emulated FP8 scaled GEMM -- TEST INFRASTRUCTURE ONLY.

Two independent implementations of the arithmetic described in the mmaemu
v0.1 documentation pages (user guide, FAQ, limitations, validation evidence):

* ``emu_oracle.c`` -- plain C, exact int64 integers with explicit exponents,
  threaded over output rows.  Loaded here through ctypes.
* ``spec.py`` -- a pure-Python ``fractions.Fraction`` formulation for tiny
  inputs, used to pin the C oracle (it also accepts an unbounded number of
  retained bits).

Parity unpinned, as the header of ``emu_oracle.c`` lists: the canonical NaN
bit patterns, the pairwise split tree for S >= 4 and the alignment of a
subnormal incoming accumulator, which the pages leave open.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never does, and this
package imports nothing from it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "emu_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

FMT = {"e4m3fn": 0, "e5m2": 1}
OUT = {"bf16": 0, "fp16": 1, "fp32": 2, "e4m3fn": 3, "e5m2": 4}
ONE = 0x3F800000  # binary32 1.0: the default scale_result
CLS_ZERO, CLS_FINITE, CLS_INF, CLS_NAN = 0, 1, 2, 3

LAYOUT = {"contiguous": 0, "round-robin": 1}
COMBINE = {"serial": 0, "pairwise": 1}

# The default (hopper) profile: 32-product blocks, 13 retained fraction bits,
# slow accumulation restarting every 128, split-K in contiguous runs of
# 128-wide k-tiles added serially (validation page: H100 claims table and
# scope table).
HOPPER = dict(B=32, F=13, Q=128, W=128, layout="contiguous", combine="serial")
# The RTX 4060 (ada) profiles: 16-product blocks, 13 retained fraction bits
# (validation page, scope table "Ada instruction model" and claims table),
# slow accumulation every 128 along each split's sequence, 64-wide k-tiles
# dealt round-robin to the splits, partials added serially or pairwise
# (limitations page, corrections table; validation page, claims table).
ADA_SERIAL = dict(B=16, F=13, Q=128, W=64, layout="round-robin", combine="serial")
ADA_PAIRWISE = dict(ADA_SERIAL, combine="pairwise")
PROFILES = {"hopper": HOPPER, "ada-serial": ADA_SERIAL, "ada-pairwise": ADA_PAIRWISE}


def resolve_profile(profile=None) -> dict:
    """A profile name, or a dict of overrides of the hopper profile."""
    if profile is None:
        return dict(HOPPER)
    if isinstance(profile, str):
        return dict(PROFILES[profile])
    return dict(HOPPER, **profile)

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-fvisibility=hidden", "-pthread"]


def build(path: str = LIBRARY, mutant: int = 0) -> str:
    """Compile the C oracle (optionally a numbered mutant) with gcc."""
    cmd = ["gcc", *CFLAGS, f"-DORACLE_MUTANT={int(mutant)}", SOURCE, "-o", path, "-lm"]
    subprocess.run(cmd, check=True)
    return path


_I64P = ctypes.POINTER(ctypes.c_int64)
_U32P = ctypes.POINTER(ctypes.c_uint32)
_U8P = ctypes.POINTER(ctypes.c_uint8)
_IP = ctypes.POINTER(ctypes.c_int)


class Oracle:
    """ctypes view of one build of emu_oracle.c."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path) or (path == LIBRARY and os.path.getmtime(path) < os.path.getmtime(SOURCE)):
            build(path)
        self.path = path
        L = self.lib = ctypes.CDLL(path)
        L.oracle_mutant_id.restype = ctypes.c_int
        L.oracle_decode.argtypes = [ctypes.c_uint8, ctypes.c_int, _IP, _IP, _IP, _IP]
        for name in ("oracle_mul_f32", "oracle_add_f32", "oracle_epilogue_f32"):
            getattr(L, name).argtypes = [ctypes.c_uint32, ctypes.c_uint32]
            getattr(L, name).restype = ctypes.c_uint32
        L.oracle_encode_output.argtypes = [ctypes.c_uint32, ctypes.c_int]
        L.oracle_encode_output.restype = ctypes.c_uint32
        L.oracle_output_from_acc.argtypes = [ctypes.c_uint32] * 4 + [ctypes.c_int]
        L.oracle_output_from_acc.restype = ctypes.c_uint32
        L.oracle_chain_exact.argtypes = [
            _U8P, ctypes.c_int, ctypes.c_int64, _U8P, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            _IP, _I64P, _IP]
        L.oracle_block_step.argtypes = [_IP, _IP, _IP, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_int, _IP, _I64P, _IP]
        L.oracle_points.argtypes = [
            _U8P, ctypes.c_int, ctypes.c_int64, _U8P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, _I64P, _I64P, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, _U32P, _U32P]
        L.oracle_scaled_mm.argtypes = [
            _U8P, ctypes.c_int, ctypes.c_int64, _U8P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, _U32P, _U32P, ctypes.c_int]
        L.oracle_accumulate_c.argtypes = [
            _U8P, ctypes.c_int, ctypes.c_int64, _U8P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, _U32P, ctypes.c_int, ctypes.c_int, _U32P]

    @property
    def mutant(self) -> int:
        return self.lib.oracle_mutant_id()

    # ---- scalar helpers ------------------------------------------------
    def decode(self, code: int, fmt: str):
        c, s, e, m = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        self.lib.oracle_decode(code, FMT[fmt], c, s, e, m)
        return c.value, s.value, e.value, m.value

    def mul_f32(self, a: int, b: int) -> int:
        return self.lib.oracle_mul_f32(a, b)

    def add_f32(self, a: int, b: int) -> int:
        return self.lib.oracle_add_f32(a, b)

    def epilogue_f32(self, acc: int, alpha: int) -> int:
        return self.lib.oracle_epilogue_f32(acc, alpha)

    def encode_output(self, y32: int, out: str) -> int:
        return self.lib.oracle_encode_output(y32, OUT[out])

    def output_from_acc(self, acc: int, sx: int, sw: int, out: str, sr: int = ONE) -> int:
        return self.lib.oracle_output_from_acc(acc, sx, sw, sr, OUT[out])

    def block_step(self, prods, F=13, c=(0, 0, 0)):
        """prods: list of (sign, g, P); c: (neg, mag, q).  Returns (neg, mag, q)."""
        n = len(prods)
        g = (ctypes.c_int * max(n, 1))(*[p[1] for p in prods])
        P = (ctypes.c_int * max(n, 1))(*[p[2] for p in prods])
        s = (ctypes.c_int * max(n, 1))(*[p[0] for p in prods])
        neg, mag, q = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int()
        rc = self.lib.oracle_block_step(g, P, s, n, F, c[0], c[1], c[2], neg, mag, q)
        assert rc == 0
        return neg.value, mag.value, q.value

    def chain_exact(self, x, xfmt, w, wfmt, m, n, k0, k1, B=32, F=13):
        x = np.ascontiguousarray(x, dtype=np.uint8)
        w = np.ascontiguousarray(w, dtype=np.uint8)
        neg, mag, q = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int()
        rc = self.lib.oracle_chain_exact(_u8(x), FMT[xfmt], x.shape[1], _u8(w), FMT[wfmt], w.shape[1],
                                         m, n, k0, k1, B, F, neg, mag, q)
        assert rc == 0
        return neg.value, mag.value, q.value

    # ---- matrix entry points -------------------------------------------
    def scaled_mm(self, x, xfmt, w, wfmt, sx_bits, sw_bits, out="bf16", fast=True, S=1,
                  profile=None, threads=None, sr_bits=ONE):
        """x: uint8 [M,K], w: uint8 [N,K] (codes).  Returns (acc uint32 [M,N],
        y uint32 [M,N] holding the output bit patterns).  sr_bits: the
        binary32 scale_result, used by FP8 outputs only."""
        pf = resolve_profile(profile)
        x = np.ascontiguousarray(x, dtype=np.uint8)
        w = np.ascontiguousarray(w, dtype=np.uint8)
        M, K = x.shape
        N = w.shape[0]
        assert w.shape[1] == K
        acc = np.zeros((M, N), dtype=np.uint32)
        y = np.zeros((M, N), dtype=np.uint32)
        threads = threads or os.cpu_count() or 1
        rc = self.lib.oracle_scaled_mm(_u8(x), FMT[xfmt], max(K, 1), _u8(w), FMT[wfmt], max(K, 1),
                                       M, N, K, sx_bits, sw_bits, sr_bits, OUT[out], int(fast), S,
                                       pf["B"], pf["F"], pf["Q"], pf["W"], LAYOUT[pf["layout"]],
                                       COMBINE[pf["combine"]], _u32(acc), _u32(y), threads)
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return acc, y

    def points(self, x, xfmt, w, wfmt, ms, ns, sx_bits, sw_bits, out="bf16", fast=True, S=1,
               profile=None, sr_bits=ONE):
        """Accumulator and output at the listed (m, n) points only."""
        pf = resolve_profile(profile)
        x = np.ascontiguousarray(x, dtype=np.uint8)
        w = np.ascontiguousarray(w, dtype=np.uint8)
        K = x.shape[1]
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        acc = np.zeros(len(ms), dtype=np.uint32)
        y = np.zeros(len(ms), dtype=np.uint32)
        rc = self.lib.oracle_points(_u8(x), FMT[xfmt], max(K, 1), _u8(w), FMT[wfmt], max(K, 1), K,
                                    len(ms), ms.ctypes.data_as(_I64P), ns.ctypes.data_as(_I64P),
                                    sx_bits, sw_bits, sr_bits, OUT[out], int(fast), S,
                                    pf["B"], pf["F"], pf["Q"], pf["W"], LAYOUT[pf["layout"]],
                                    COMBINE[pf["combine"]], _u32(acc), _u32(y))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return acc, y


    def accumulate_c(self, x, xfmt, w, wfmt, c_in, profile=None):
        """The fast-accumulation chain of every output started from the
        incoming binary32 accumulators c_in (uint32 bit patterns [M, N])
        instead of +0; one split.  Returns the accumulators (uint32 [M, N])."""
        pf = resolve_profile(profile)
        x = np.ascontiguousarray(x, dtype=np.uint8)
        w = np.ascontiguousarray(w, dtype=np.uint8)
        M, K = x.shape
        N = w.shape[0]
        c_in = np.ascontiguousarray(c_in, dtype=np.uint32)
        assert c_in.shape == (M, N)
        acc = np.zeros((M, N), dtype=np.uint32)
        rc = self.lib.oracle_accumulate_c(_u8(x), FMT[xfmt], max(K, 1), _u8(w), FMT[wfmt], max(K, 1),
                                          M, N, K, _u32(c_in), pf["B"], pf["F"], _u32(acc))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return acc


def _u8(a):
    return a.ctypes.data_as(_U8P)


def _u32(a):
    return a.ctypes.data_as(_U32P)


_DEFAULT = None


def default() -> Oracle:
    """The oracle built from emu_oracle.c (compiled on first use if needed)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def f32_bits(v: float) -> int:
    return int(np.array(v, dtype=np.float32).view(np.uint32))
