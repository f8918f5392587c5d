// emu_chain.h -- one block step of the emulated accumulation in integer
// arithmetic, for host and device: the exponent-speculation walk's
// continuation (c_step) and its recomputation of a block whose speculated
// exponent was wrong (block_step_codes).
//
// The block step (mmaemu v0.1 pages: validation page, scope table row
// "Hopper preset" and claims table; user guide section 1): E is the largest
// alignment exponent among the block's nonzero products (field exponents,
// subnormals at emin) and the incoming accumulator c; every term and c are
// cut toward zero to multiples of 2^(E-13); the exact sum is cut toward zero
// to 14 significant bits; a zero sum is +0.
#pragma once

#include <stdint.h>

#include "fp_round.h"

namespace emu {

// Accumulators are binary32 bit patterns of at most 14 significant bits in
// the normal range, or +0.  Ebits is E + 127 (the biased exponent of 2^E).

// The signed sum S of a block's truncated terms at exponent Ebits, plus the
// truncated c, cut to 14 significant bits: the new accumulator.
EMU_HD uint32_t c_step(uint32_t c, int32_t S, uint32_t Ebits)
{
    int32_t T = S;
    const uint32_t cf = (c >> 23) & 0xFFu;
    if (cf) {
        // |c| = mc * 2^(cf - 150); the quantum is 2^(Ebits - 140); cf <= Ebits
        const uint32_t mc = (c & 0x7FFFFFu) | 0x800000u;
        const uint32_t sh = Ebits - cf + 10u;
        const int32_t tc = sh >= 32u ? 0 : (int32_t)(mc >> sh);
        T += (c >> 31) ? -tc : tc;
    }
    if (T == 0) return 0u;
    const uint32_t sign = T < 0 ? 0x80000000u : 0u;
    uint32_t a = (uint32_t)(T < 0 ? -T : T);  // < 2^21
    const int L = 31 - __builtin_clz(a);
    if (L > 13) a = (a >> (L - 13)) << (L - 13);
    // value a * 2^(Ebits - 140): exponent field L + Ebits - 13
    return sign | ((uint32_t)(L + (int)Ebits - 13) << 23) | ((a << (23 - L)) & 0x7FFFFFu);
}

// FP8 code -> (class, sign, field exponent with emin for subnormals, integer
// significand with 3 fraction bits: E5M2's 2 bits doubled).  cls: 0 zero,
// 1 finite, 2 infinity, 3 NaN.
EMU_HD void fp8_fields(uint32_t code, bool e5m2, int &cls, uint32_t &s, int &e, uint32_t &M)
{
    s = (code >> 7) & 1u;
    if (!e5m2) {
        const uint32_t ef = (code >> 3) & 15u, mf = code & 7u;
        if (ef == 15u && mf == 7u) { cls = 3; e = 0; M = 0; return; }
        e = ef ? (int)ef - 7 : -6;
        M = ef ? 8u + mf : mf;
    } else {
        const uint32_t ef = (code >> 2) & 31u, mf = code & 3u;
        if (ef == 31u) { cls = mf ? 3 : 2; e = 0; M = 0; return; }
        e = ef ? (int)ef - 15 : -14;
        M = 2u * (ef ? 4u + mf : mf);
    }
    cls = M ? 1 : 0;
}

// The block step from codes held in words (code i in byte i % 4 of word
// i / 4, 32 codes: 8 words per operand; codes past the block are zero): the
// products x[i] * w[i] of finite codes, incoming accumulator c.
EMU_HD uint32_t block_step_words(uint32_t c, const uint32_t *xw, bool x_e5m2, const uint32_t *ww, bool w_e5m2)
{
    int G = -1000;
#pragma unroll 1
    for (int i = 0; i < 32; ++i) {
        int ca, cb, ea, eb;
        uint32_t sa, sb, Ma, Mb;
        fp8_fields((xw[i >> 2] >> (8 * (i & 3))) & 0xFFu, x_e5m2, ca, sa, ea, Ma);
        fp8_fields((ww[i >> 2] >> (8 * (i & 3))) & 0xFFu, w_e5m2, cb, sb, eb, Mb);
        if (ca == 1 && cb == 1 && ea + eb > G) G = ea + eb;  // zero products are excluded
    }
    const uint32_t cf = (c >> 23) & 0xFFu;
    if (G == -1000 && !cf) return 0u;  // nothing in the block: +0
    int E = G;
    if (cf && (int)cf - 127 > E) E = (int)cf - 127;
    int32_t S = 0;
#pragma unroll 1
    for (int i = 0; i < 32; ++i) {
        int ca, cb, ea, eb;
        uint32_t sa, sb, Ma, Mb;
        fp8_fields((xw[i >> 2] >> (8 * (i & 3))) & 0xFFu, x_e5m2, ca, sa, ea, Ma);
        fp8_fields((ww[i >> 2] >> (8 * (i & 3))) & 0xFFu, w_e5m2, cb, sb, eb, Mb);
        if (ca != 1 || cb != 1) continue;
        // P * 2^(g - 6) cut to the quantum 2^(E - 13): shift by E - g - 7 (>= -7)
        const uint32_t P = Ma * Mb;
        const int sh = E - (ea + eb) - 7;
        const int32_t t = sh >= 8 ? 0 : (sh >= 0 ? (int32_t)(P >> sh) : (int32_t)(P << -sh));
        S += (sa ^ sb) ? -t : t;
    }
    return c_step(c, S, (uint32_t)(E + 127));
}

// The block step from codes: products of x[i] and w[i] for i < n (n <= 32;
// finite codes only), incoming accumulator c.
EMU_HD uint32_t block_step_codes(uint32_t c, const uint8_t *x, bool x_e5m2, const uint8_t *w, bool w_e5m2, int n)
{
    uint32_t xw[8] = {0, 0, 0, 0, 0, 0, 0, 0}, ww[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < n; ++i) {
        xw[i >> 2] |= (uint32_t)x[i] << (8 * (i & 3));
        ww[i >> 2] |= (uint32_t)w[i] << (8 * (i & 3));
    }
    return block_step_words(c, xw, x_e5m2, ww, w_e5m2);
}

}  // namespace emu
