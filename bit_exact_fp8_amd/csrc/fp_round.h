// fp_round.h -- IEEE 754 roundings in integer arithmetic, for host and device.
//
// The epilogue of the emulated GEMM rounds twice (mmaemu limitations page,
// corrections table: y is one fused multiply-add of acc and alpha with a +0
// addend, rounded once; validation page, claims table: bf16/fp16 outputs
// rounded from the fp32 value).  These
// routines do those roundings on bit patterns with integer operations only,
// so the result never depends on the GPU's floating-point mode register
// (rounding mode, denormal flushing) or on how the compiler treats float
// code.  Round to nearest, ties to even; subnormals kept; overflow to
// infinity (FP8 outputs: saturation); NaN results canonical (0x7FFFFFFF,
// 0x7FFF, 0x7F).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define EMU_HD __host__ __device__ __forceinline__
#else
#define EMU_HD inline
#endif

namespace emu {

constexpr uint32_t kCanonNan32 = 0x7FFFFFFFu;
constexpr uint16_t kCanonNan16 = 0x7FFFu;

EMU_HD int clz64(uint64_t v)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return v ? __clzll((long long)v) : 64;
#else
    return v ? __builtin_clzll(v) : 64;
#endif
}

// RN32(a*b) of two binary32 values.  zero_plus: an exactly zero product
// gives +0 (the fma(acc, alpha, +0) rule) instead of the signed zero of a
// plain multiplication.
EMU_HD uint32_t mul_round_f32(uint32_t a, uint32_t b, bool zero_plus)
{
    const uint32_t sign = (a ^ b) & 0x80000000u;
    const uint32_t ea = (a >> 23) & 0xFFu, eb = (b >> 23) & 0xFFu;
    const uint32_t fa = a & 0x7FFFFFu, fb = b & 0x7FFFFFu;
    const bool a_nan = ea == 0xFFu && fa, b_nan = eb == 0xFFu && fb;
    const bool a_inf = ea == 0xFFu && !fa, b_inf = eb == 0xFFu && !fb;
    const bool a_zero = ea == 0 && !fa, b_zero = eb == 0 && !fb;
    if (a_nan || b_nan) return kCanonNan32;
    if ((a_inf && b_zero) || (b_inf && a_zero)) return kCanonNan32;
    if (a_inf || b_inf) return sign | 0x7F800000u;
    if (a_zero || b_zero) return zero_plus ? 0u : sign;

    // value = sig * 2^(exp - 23); subnormals have exponent -126, no hidden bit
    const uint64_t sa = ea ? (fa | 0x800000u) : fa;
    const uint64_t sb = eb ? (fb | 0x800000u) : fb;
    const int xa = ea ? (int)ea - 127 : -126;
    const int xb = eb ? (int)eb - 127 : -126;
    const uint64_t P = sa * sb;              // exact, < 2^48
    const int e0 = xa + xb - 46;             // value = P * 2^e0
    const int lead = 63 - clz64(P) + e0;     // exponent of the leading bit
    const int qexp = (lead < -126 ? -126 : lead) - 23;  // quantum of the result
    const int shift = qexp - e0;             // low bits of P to drop
    uint64_t mant;
    if (shift <= 0) {
        mant = P << (-shift);
    } else if (shift >= 64) {
        mant = 0;                            // P < 2^48 <= half a quantum
    } else {
        mant = P >> shift;
        const uint64_t rem = P & ((1ull << shift) - 1);
        const uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (mant & 1))) mant += 1;
    }
    // ((qexp + 149) << 23) + mant encodes normal and subnormal results alike,
    // including a rounding carry into the next binade.
    const int64_t enc = ((int64_t)(qexp + 149) << 23) + (int64_t)mant;
    if (mant == 0) return sign;  // a nonzero product rounded to zero keeps its sign
    if (enc >= 0x7F800000ll) return sign | 0x7F800000u;
    return sign | (uint32_t)enc;
}

// alpha = RN32(scale_x * scale_w)
EMU_HD uint32_t mul_f32(uint32_t a, uint32_t b) { return mul_round_f32(a, b, false); }

// y32 = RN32(acc * alpha + (+0))
EMU_HD uint32_t epilogue_f32(uint32_t acc, uint32_t alpha) { return mul_round_f32(acc, alpha, true); }

EMU_HD uint32_t canon_f32(uint32_t f)
{
    return ((f & 0x7FFFFFFFu) > 0x7F800000u) ? kCanonNan32 : f;
}

// binary32 -> bfloat16, round to nearest even
EMU_HD uint16_t f32_to_bf16(uint32_t f)
{
    if ((f & 0x7FFFFFFFu) > 0x7F800000u) return kCanonNan16;
    const uint32_t r = f + 0x7FFFu + ((f >> 16) & 1u);
    return (uint16_t)(r >> 16);
}

// binary32 -> binary16, round to nearest even, subnormals kept
EMU_HD uint16_t f32_to_f16(uint32_t f)
{
    const uint32_t s = (f >> 16) & 0x8000u;
    const uint32_t a = f & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return kCanonNan16;
    if (a >= 0x477FF000u) return (uint16_t)(s | 0x7C00u);  // |f| >= 65520 rounds to infinity
    const uint32_t e = a >> 23;
    if (e >= 113) {  // |f| >= 2^-14: normal binary16
        const uint32_t m = a & 0x7FFFFFu;
        uint32_t h = ((e - 112) << 10) | (m >> 13);
        const uint32_t rem = m & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;  // carry may reach the exponent
        return (uint16_t)(s | h);
    }
    if (e == 0) return (uint16_t)s;  // binary32 subnormal: far below half of 2^-24
    // subnormal binary16: quantum 2^-24; value = sig * 2^(e - 150)
    const uint32_t sig = (a & 0x7FFFFFu) | 0x800000u;
    const uint32_t shift = 126 - e;  // >= 14
    if (shift >= 25) return (uint16_t)s;  // below 2^-25 (ties at 2^-25 go to even 0)
    uint32_t h = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1u))) h += 1;
    return (uint16_t)(s | h);
}

// binary32 -> FP8 (E4: e4m3fn, else e5m2) with saturation (validation page,
// scope table row "Epilogue" and claims table: FP8 outputs saturate to the
// format's largest finite value): |f| at or above 448 (e4m3fn) / 57344
// (e5m2), infinities included, gives the signed largest finite value; other
// values round to nearest even, subnormals kept, the sign of zero kept; NaN
// gives 0x7F.
template <bool E4>
EMU_HD uint8_t f32_to_fp8_sat(uint32_t f)
{
    constexpr int MB = E4 ? 3 : 2;                             // mantissa bits
    constexpr int BIAS = E4 ? 7 : 15;
    constexpr int EMIN = 1 - BIAS;                             // -6, -14
    constexpr uint32_t MAXF = E4 ? 0x43E00000u : 0x47600000u;  // 448.0f, 57344.0f
    constexpr uint32_t MAXC = E4 ? 0x7Eu : 0x7Bu;
    const uint32_t s = (f >> 24) & 0x80u;
    const uint32_t a = f & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7Fu;
    if (a >= MAXF) return (uint8_t)(s | MAXC);
    if (a < 0x00800000u) return (uint8_t)s;  // binary32 subnormal: far below the FP8 subnormals
    const int e = (int)(a >> 23) - 127;
    const uint32_t sig = (a & 0x7FFFFFu) | 0x800000u;        // value = sig * 2^(e - 23)
    // quantum 2^((e < EMIN ? EMIN : e) - MB): drop `shift` low bits of sig
    const int shift = 23 - MB + (e < EMIN ? EMIN - e : 0);
    if (shift >= 25) return (uint8_t)s;                      // below half the smallest subnormal
    uint32_t q = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1;
    // subnormal: the code is q (q = 2^MB is the smallest normal's code);
    // normal: a rounding carry moves into the exponent field by itself
    const uint32_t code = (e < EMIN) ? q : ((uint32_t)(e + BIAS) << MB) + q - (1u << MB);
    return (uint8_t)(s | code);
}

}  // namespace emu
