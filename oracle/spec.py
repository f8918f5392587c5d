"""Exact rational specification of the emulated FP8 GEMM -- TEST INFRASTRUCTURE ONLY.

A second, independent formulation of what ``emu_oracle.c`` computes, written
with ``fractions.Fraction`` values instead of integer mantissas.  It is meant
for tiny inputs (pure-Python loops) and serves to pin the C oracle:

* it accepts ``F=None`` (no truncation at all), which must give the exact sum
  of the products for any block width;
* it rounds to binary formats from exact rationals with its own
  round-to-nearest-even, instead of the host's IEEE arithmetic.

Sources are the mmaemu v0.1 documentation pages: the user guide (sections 1
and 3), the limitations page (corrections table) and the validation page
(scope table and claims tables).  Readings where the pages are silent are
the same as in ``emu_oracle.c`` and are listed in the design notes.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

# ---------------------------------------------------------------------------
# Formats: (exponent bits, mantissa bits, bias, has_inf)
FORMATS = {"e4m3fn": (4, 3, 7, False), "e5m2": (5, 2, 15, True)}

NAN, INF, ZERO, FIN = "nan", "inf", "zero", "finite"


def decode(code: int, fmt: str):
    """(kind, sign, field_exponent, value) of an FP8 code.

    The field exponent of a subnormal is the format's emin = 1 - bias
    (validation page, claims table, row on subnormal inputs)."""
    ebits, mbits, bias, has_inf = FORMATS[fmt]
    sign = (code >> 7) & 1
    ef = (code >> mbits) & ((1 << ebits) - 1)
    mf = code & ((1 << mbits) - 1)
    emax_field = (1 << ebits) - 1
    if has_inf and ef == emax_field:
        return (INF if mf == 0 else NAN), sign, None, None
    if not has_inf and ef == emax_field and mf == (1 << mbits) - 1:
        return NAN, sign, None, None
    if ef == 0:
        e = 1 - bias
        frac = Fraction(mf, 1 << mbits)
    else:
        e = ef - bias
        frac = 1 + Fraction(mf, 1 << mbits)
    mag = frac * Fraction(2) ** e
    if mag == 0:
        return ZERO, sign, e, Fraction(0)
    return FIN, sign, e, (-mag if sign else mag)


def floor_log2(v: Fraction) -> int:
    """floor(log2 v) for a positive rational, exactly."""
    assert v > 0
    n, d = v.numerator, v.denominator
    e = n.bit_length() - d.bit_length()
    # now 2^(e-1) < n/d < 2^(e+1); fix up
    if Fraction(2) ** e > v:
        e -= 1
    assert Fraction(2) ** e <= v < Fraction(2) ** (e + 1)
    return e


def trunc_to_quantum(v: Fraction, quantum: Fraction) -> Fraction:
    """Cut v toward zero to a multiple of quantum (sign-magnitude truncation)."""
    k = abs(v) / quantum
    t = k.numerator // k.denominator
    return t * quantum if v >= 0 else -t * quantum


def block(c: Fraction, prods, F):
    """One block step.  prods: list of (value, alignment exponent) for the
    nonzero products; c the incoming accumulator (0 means +0).

    E = max(alignment exponents, c's exponent if c != 0); every term and c
    are cut toward zero to multiples of 2^(E-F); their exact sum is cut toward
    zero to F+1 significant bits; a zero sum is +0.  F=None keeps everything
    exact.  c's exponent is floor(log2|c|), or -126 (binary32's emin) for a
    subnormal c: the reading that takes a binary32 c as the pages take
    subnormal FP8 inputs (only a caller's incoming accumulator is that small)."""
    exps = [g for _, g in prods]
    if c != 0:
        exps.append(max(floor_log2(abs(c)), -126))
    if not exps:
        return Fraction(0)
    if F is None:
        return c + sum((v for v, _ in prods), Fraction(0))
    E = max(exps)
    quantum = Fraction(2) ** (E - F)
    total = trunc_to_quantum(c, quantum) + sum((trunc_to_quantum(v, quantum) for v, _ in prods),
                                               Fraction(0))
    if total == 0:
        return Fraction(0)
    lead = floor_log2(abs(total))
    return trunc_to_quantum(total, Fraction(2) ** (lead - F))


def chain(xrow, xfmt, wrow, wfmt, k0, k1, B, F, ks=None, c0=Fraction(0)):
    """Blocks of B consecutive products (of range(k0, k1), or of the ordered
    index list ks), each stepping the accumulator, which starts at c0."""
    ks = list(range(k0, k1)) if ks is None else list(ks)
    c = c0
    for i in range(0, len(ks), B):
        prods = []
        for k in ks[i:i + B]:
            ka, sa, ea, va = decode(int(xrow[k]), xfmt)
            kb, sb, eb, vb = decode(int(wrow[k]), wfmt)
            if ka == FIN and kb == FIN:
                prods.append((va * vb, ea + eb))
        c = block(c, prods, F)
    return c


def split_indices(K, S, W, layout):
    """The ordered k indices of every split.  contiguous: runs of
    ceil(ceil(K/W)/S) tiles of width W; round-robin: tile t goes to split
    t mod S, in increasing t."""
    tiles = [list(range(t * W, min((t + 1) * W, K))) for t in range(-(-K // W))]
    if layout == "round-robin":
        return [[k for t in range(s, len(tiles), S) for k in tiles[t]] for s in range(S)]
    tps = -(-len(tiles) // S) if tiles else 0
    return [[k for t in tiles[s * tps:(s + 1) * tps] for k in t] for s in range(S)]


def combine(parts, scheme):
    """serial: ((p0 + p1) + p2) + ...; pairwise: p_0 after the stride-halving
    tree over the next power of two >= S (for S = 3: (p0 + p2) + p1)."""
    if scheme == "serial":
        acc = parts[0]
        for p in parts[1:]:
            acc = round_nearest_even(acc + p)
        return acc
    S = len(parts)
    P = 1
    while P < S:
        P *= 2

    def value(i, h):  # p_i after the levels with stride >= h
        if h == P:
            return parts[i]
        left = value(i, 2 * h)
        if i + h < S:
            return round_nearest_even(left + value(i + h, 2 * h))
        return left

    return value(0, 1)


# ---------------------------------------------------------------------------
# Binary rounding from exact rationals.
BINARY32 = (24, -126, 127)
BINARY16 = (11, -14, 15)
BFLOAT16 = (8, -126, 127)


def round_nearest_even(v: Fraction, fmt=BINARY32):
    """IEEE round-to-nearest-even of an exact rational, subnormals kept.
    Returns a Fraction, or +-math.inf on overflow.  The sign of a zero result
    is the caller's business."""
    p, emin, emax = fmt
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = max(floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    k = a / quantum
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        return -math.inf if v < 0 else math.inf
    return -r if v < 0 else r


def f32_bits_of(v, negative_zero=False) -> int:
    if isinstance(v, float) and math.isinf(v):
        return 0xFF800000 if v < 0 else 0x7F800000
    if v == 0:
        return 0x80000000 if negative_zero else 0
    f = float(v)  # exact: v is a binary32 value
    return struct.unpack("<I", struct.pack("<f", f))[0]


def f32_value(bits: int):
    f = struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]
    if math.isnan(f) or math.isinf(f):
        return f
    return Fraction(f)


CANON_NAN_32 = 0x7FFFFFFF
CANON_NAN_16 = 0x7FFF


def encode16(v, fmt, negative_zero=False) -> int:
    """Bits of a value exactly representable in bf16 / binary16."""
    p, emin, emax = fmt
    ebits = 8 if fmt == BFLOAT16 else 5
    bias = (1 << (ebits - 1)) - 1
    mbits = p - 1
    if isinstance(v, float) and math.isinf(v):
        return (0x8000 if v < 0 else 0) | (((1 << ebits) - 1) << mbits)
    sign = 0x8000 if (v < 0 or (v == 0 and negative_zero)) else 0
    if v == 0:
        return sign
    a = abs(v)
    e = floor_log2(a)
    if e < emin:
        m = a / Fraction(2) ** (emin - mbits)
        assert m.denominator == 1
        return sign | int(m)
    m = a / Fraction(2) ** (e - mbits) - (1 << mbits)
    assert m.denominator == 1
    return sign | ((e + bias) << mbits) | int(m)


E4M3FN = (4, -6, 8)
E5M2 = (3, -14, 15)
FP8_MAX = {"e4m3fn": Fraction(448), "e5m2": Fraction(57344)}
CANON_NAN_8 = 0x7F


def encode8(v, out, negative_zero=False) -> int:
    """Bits of a value exactly representable in the FP8 output format."""
    p, emin, _ = E4M3FN if out == "e4m3fn" else E5M2
    bias, mbits = (7, 3) if out == "e4m3fn" else (15, 2)
    sign = 0x80 if (v < 0 or (v == 0 and negative_zero)) else 0
    if v == 0:
        return sign
    a = abs(v)
    e = floor_log2(a)
    if e < emin:
        m = a / Fraction(2) ** (emin - mbits)
        assert m.denominator == 1
        return sign | int(m)
    m = a / Fraction(2) ** (e - mbits) - (1 << mbits)
    assert m.denominator == 1
    return sign | ((e + bias) << mbits) | int(m)


def epilogue_bits(acc_bits: int, sx_bits: int, sw_bits: int, out: str, sr_bits: int = 0x3F800000) -> int:
    """alpha = RN32(sx*sw); y32 = RN32(acc*alpha + (+0)); then RN to the output.
    FP8 outputs: y' = RN32(y32 * scale_result), |y'| clamped to the format's
    largest finite value, then RN to the format."""
    acc, sx, sw = f32_value(acc_bits), f32_value(sx_bits), f32_value(sw_bits)
    neg_sx, neg_sw = bool(sx_bits >> 31), bool(sw_bits >> 31)

    def is_nan(v):
        return isinstance(v, float) and math.isnan(v)

    def is_inf(v):
        return isinstance(v, float) and math.isinf(v)

    nan = False
    # alpha
    if is_nan(sx) or is_nan(sw) or (is_inf(sx) and sw == 0) or (is_inf(sw) and sx == 0):
        nan = True
        alpha, alpha_neg = None, False
    elif is_inf(sx) or is_inf(sw):
        alpha_neg = neg_sx ^ neg_sw
        alpha = -math.inf if alpha_neg else math.inf
    else:
        alpha = round_nearest_even(sx * sw)
        alpha_neg = neg_sx ^ neg_sw
    # y32
    acc_neg = bool(acc_bits >> 31)
    y_neg_zero = False
    y = None
    if nan or is_nan(acc) or (is_inf(acc) and alpha == 0) or (is_inf(alpha) and acc == 0):
        nan = True
    elif is_inf(acc) or is_inf(alpha):
        y = -math.inf if (acc_neg ^ alpha_neg) else math.inf
    else:
        exact = acc * alpha
        if exact == 0:
            y = Fraction(0)  # (+-0) + (+0) = +0
        else:
            y = round_nearest_even(exact)
            y_neg_zero = (y == 0) and exact < 0
    if out in FP8_MAX:
        if nan:
            return CANON_NAN_8
        sr = f32_value(sr_bits)
        sr_neg = bool(sr_bits >> 31)
        y_neg = (y < 0) or y_neg_zero
        if is_nan(sr) or (is_inf(y) and sr == 0) or (y == 0 and is_inf(sr)):
            return CANON_NAN_8
        if is_inf(y) or is_inf(sr):
            yp, yp_negzero = (-math.inf if (y_neg ^ sr_neg) else math.inf), False
        else:
            exact = y * sr
            if exact == 0:
                yp, yp_negzero = Fraction(0), y_neg ^ sr_neg
            else:
                yp = round_nearest_even(exact)
                yp_negzero = (yp == 0) and exact < 0
        neg = (yp < 0) or yp_negzero
        a = FP8_MAX[out] if is_inf(yp) else min(abs(yp), FP8_MAX[out])
        r = round_nearest_even(a, E4M3FN if out == "e4m3fn" else E5M2)
        return encode8(-r if neg else r, out, negative_zero=neg)
    if out == "fp32":
        return CANON_NAN_32 if nan else f32_bits_of(y, y_neg_zero)
    if nan:
        return CANON_NAN_16
    fmt = BFLOAT16 if out == "bf16" else BINARY16
    if isinstance(y, float):
        return encode16(y, fmt)
    r = round_nearest_even(y, fmt)
    return encode16(r, fmt, negative_zero=(y_neg_zero or (r == 0 and y < 0)))


# ---------------------------------------------------------------------------
def special(xrow, xfmt, wrow, wfmt, K):
    """'nan', '+inf', '-inf' or None for one output, from its whole rows."""
    nan = pos = neg = False
    for k in range(K):
        ka, sa, _, va = decode(int(xrow[k]), xfmt)
        kb, sb, _, vb = decode(int(wrow[k]), wfmt)
        if ka == NAN or kb == NAN:
            nan = True
        elif ka == INF or kb == INF:
            if ka == ZERO or kb == ZERO:
                nan = True
            elif sa ^ sb:
                neg = True
            else:
                pos = True
    if nan or (pos and neg):
        return "nan"
    if pos:
        return "+inf"
    if neg:
        return "-inf"
    return None


def accumulator(xrow, xfmt, wrow, wfmt, K, fast=True, S=1, B=32, F=13, Q=128, W=128,
                layout="contiguous", scheme="serial"):
    """Accumulator of one output as a Fraction (F may be None only with fast
    accumulation and S = 1), or a special string."""
    sp = special(xrow, xfmt, wrow, wfmt, K)
    if sp is not None:
        return sp
    parts = []
    for ks in split_indices(K, S, W, layout):
        if not ks:
            parts.append(Fraction(0))
        elif fast:
            parts.append(chain(xrow, xfmt, wrow, wfmt, 0, 0, B, F, ks=ks))
        else:
            a = Fraction(0)
            for i in range(0, len(ks), Q):
                a = round_nearest_even(a + chain(xrow, xfmt, wrow, wfmt, 0, 0, B, F, ks=ks[i:i + Q]))
            parts.append(a)
    if F is None:
        assert fast and S == 1, "unbounded bits only for one fast chain"
        return parts[0]
    return combine(parts, scheme)


def accumulator_c_bits(xrow, xfmt, wrow, wfmt, K, c_bits, B=32, F=13) -> int:
    """The fast chain of one output from the incoming binary32 accumulator
    c_bits (one split), as bits.  Readings as in emu_oracle.c: K = 0 returns
    c unchanged (NaN canonical); NaN c gives NaN; an infinite c stays, unless
    the products give NaN or the opposite infinity (then NaN); -0 enters as
    +0."""
    c = f32_value(c_bits)
    if isinstance(c, float) and math.isnan(c):
        return CANON_NAN_32
    if K == 0:
        return c_bits
    sp = special(xrow, xfmt, wrow, wfmt, K)
    if isinstance(c, float):  # an infinity
        if sp == "nan" or (sp is not None and (sp == "-inf") != (c < 0)):
            return CANON_NAN_32
        return c_bits
    if sp is not None:
        return {"nan": CANON_NAN_32, "+inf": 0x7F800000, "-inf": 0xFF800000}[sp]
    return f32_bits_of(chain(xrow, xfmt, wrow, wfmt, 0, K, B, F, c0=c))


def accumulator_bits(*args, **kw) -> int:
    a = accumulator(*args, **kw)
    if a == "nan":
        return CANON_NAN_32
    if a == "+inf":
        return 0x7F800000
    if a == "-inf":
        return 0xFF800000
    return f32_bits_of(a)


def scaled_mm(x, xfmt, w, wfmt, sx_bits, sw_bits, out="bf16", fast=True, S=1, B=32, F=13, Q=128, W=128,
              layout="contiguous", scheme="serial", sr_bits=0x3F800000):
    """Tiny whole-matrix evaluation: returns (acc bits, output bits) as lists of lists."""
    M, K = len(x), (len(x[0]) if len(x) else 0)
    N = len(w)
    accs, ys = [], []
    for m in range(M):
        ra, ry = [], []
        for n in range(N):
            a = accumulator_bits(x[m], xfmt, w[n], wfmt, K, fast, S, B, F, Q, W, layout, scheme)
            ra.append(a)
            ry.append(epilogue_bits(a, sx_bits, sw_bits, out, sr_bits))
        accs.append(ra)
        ys.append(ry)
    return accs, ys
