// emu_main_kernel.h -- the main kernel of the bit-exact emulated FP8 GEMM
// (gfx950), as templates; emu_variant.hip instantiates one block width and
// format pair per translation unit.
//
// The arithmetic (mmaemu v0.1 pages: user guide section 1; validation page,
// scope table rows "Hopper preset", "Ada instruction model", "Slow
// accumulation", "Split-K", "Split-K on the H100 PCIe", "Epilogue", claims
// tables; limitations page, corrections table): products are added in blocks
// of 32 (hopper) or 16 (RTX 4060 profiles) along each split's k-list; each
// block and the incoming accumulator c are aligned to the block's largest
// exponent E (field exponents, subnormals at emin, zero products excluded);
// every term and c are cut toward zero to the quantum 2^(E-13); the exact sum
// is cut toward zero to 14 significant bits and becomes the new c (+0 when
// zero).
//
// How one block is computed here, per output (m, n):
//
//  pass 1  E from packed 16-bit exponent planes: g = ea + eb with one
//          v_pk_add_u16 per two products; the planes are biased so that
//          every sum is a positive normal binary16 pattern, whose order is
//          the integer order, and one v_pk_maximum3_f16 folds two pairs
//          into the running maximum.  (Or on the matrix cores, see the power
//          planes below.)
//  pass 2  with C = 1.5 * 2^(E-13+23), a binary32 fma in round-toward-zero
//          mode, fma(|a|, |b|, C), returns exactly C + trunc(|a*b| / 2^(E-13))
//          * 2^(E-13): the product is exact inside the fma, C pins the
//          result's binade to [2^(E+10), 2^(E+11)) whose ulp is the quantum,
//          and round-toward-zero is the truncation.  The truncated magnitude
//          (< 2^15) sits in the low 16 bits.  v_perm_b32 packs two of them,
//          the sign pair (+-1, +-1) comes from one v_bitop3_b32 on packed
//          sign masks, and v_dot2_i32_i16 applies the signs and accumulates.
//  c       the same fma turns c into its truncated magnitude.
//  block   T = signed sum (< 2^21, exact in an int); binary32(T) is exact and
//          clearing its 10 low mantissa bits cuts it toward zero to 14
//          significant bits; a multiplication by 2^(E-13), whose bits come
//          from C's, gives the new c (exact).
//
// Round-toward-zero is set once per wave at kernel entry.  Every floating
// point instruction whose rounding matters is written as inline assembly
// that takes a token produced by the mode switch, so the compiler can neither
// hoist it above the switch nor mix it with code that expects another mode.
// The only round-to-nearest steps in this kernel, the slow-accumulation chunk
// adds, switch the mode around themselves the same way.  All other floating
// point operations here are exact (FP8 and small-integer conversions,
// products of powers of two).  The epilogue rounds in integer arithmetic
// (fp_round.h).

#pragma once

#include <hip/hip_runtime.h>

#include "emu_internal.h"
#include "emu_output.h"
#include "fp_round.h"

namespace emu {

namespace {

constexpr int FMT_E4M3 = 0;
constexpr int FMT_E5M2 = 1;

constexpr int KB = 32;           // k per LDS stage (one 32-product block or two 16-product blocks)
constexpr int KP = KB / 2;       // packed pairs per stage
constexpr int CHUNK = 128;       // slow-accumulation restart
constexpr int A_STRIDE = KB + 4; // floats per LDS row of the value plane (16 B pad)
constexpr int P_STRIDE = KP + 4; // words per LDS row of the exponent planes
// Words per LDS row of the sign planes: an odd number of 8-byte pairs, so that
// 16 lanes reading 8 bytes from 16 consecutive rows (the 64x64 and 64x128
// tiles' w side) use all 32 banks once; rows are 8-byte aligned.  Tiles whose
// G lanes share an output read G slices of few rows, which no stride spreads
// over all banks; measured on MI355X (16 x 256 x 65536, 8 splits, A/B in one
// session) 16-product blocks run faster with the exponent planes' stride
// (0.151 against 0.155 ms) and 32-product blocks with this one (0.130 against
// 0.132 ms).
template <int G, int BLK>
constexpr int sign_stride() { return (G == 4 && BLK == 32) ? KP : (G == 1 || BLK == 32) ? KP + 2 : P_STRIDE; }
// Words per LDS row of the exponent planes.  With 4 lanes per chain and
// 32-product blocks, the 8 lanes a 16-byte LDS read serves at a time are 2
// rows x 4 slices of 16 bytes: rows 64 bytes apart put them on all 32 banks
// once (the same holds for the sign planes above, read 16 bytes at a time
// there).
template <int G, int BLK>
constexpr int exp_stride() { return (G == 4 && BLK == 32) ? KP : P_STRIDE; }
// Words per LDS row of a binary16 value plane.  4-lane tiles: with
// 32-product blocks a 16-byte read serves 8 lanes, 2 rows x 4 slices: rows
// 64 bytes apart put them on all 32 banks once; with 16-product blocks an
// 8-byte read serves 16 lanes, 4 rows x 4 slices of one 32-byte half row:
// rows 96 bytes apart (24 words: 0, 24, 16, 8 mod 32) do.  One lane per
// output (matrix-core tiles): 16 lanes read 8 bytes at one k from 16
// consecutive rows, which an odd number of 8-byte pairs (18 words) spreads
// over all banks.
template <int G, int BLK>
constexpr int half_stride() { return (G == 1) ? KP + 2 : (BLK == 32) ? KP : KP + 8; }

// Exponent planes (one u16 per code).  A nonzero code stores
// ex + 0x200 + bias, with ex its field exponent (emin for subnormals) and
// bias 64 for x, 63 for w, so that a product's plane sum is
// (g + 127) + 0x400: a positive normal binary16 pattern (the block maximum
// can use binary16 maximum instructions, whose order on such patterns is the
// integer order) whose low 9 bits are g + 127, directly comparable with the
// binary32 exponent field of c.  A zero code stores ZERO_PLANE = 0x208: a
// zero product's sum is then at most 0x208 + 0x200 + 79 = 0x400 + 87, below
// every real product (g >= -20, i.e. 0x400 + 107) and every nonzero c
// (|c| >= 2^-33, i.e. 0x400 + 94), and at least 0x400 + 16, which keeps the
// quantum 2^(E-13) a normal binary32 value.
constexpr uint32_t X_EBIAS = 64;
constexpr uint32_t W_EBIAS = 63;
constexpr uint32_t ZERO_PLANE = 0x208u;
constexpr uint32_t SUM_OFFSET = 0x400u;
// C = 1.5 * 2^(E + 10) has exponent field (E + 127) + 10 and fraction 0x400000.
// (M << 23) drops M's bit 9 and above, so the 0x400 offset of the maximum
// vanishes from C.
constexpr uint32_t C_OFFSET = (10u << 23) | 0x400000u;

// Exponent maximum on the matrix cores.  x codes become 2^(4*ex + 4), w codes
// 2^(4*ew + 4), zeros 0 (bf16 "power planes"), so the product of a nonzero
// pair is 2^(4*g + 8).  A 16x16x16 bf16 matrix instruction takes one
// quarter-block (8 consecutive k) twice: its lanes 32-63 read the same 8 codes
// as lanes 0-31, so it returns S = 2 * sum of 2^(4*g_k + 8) over the quarter's
// nonzero products, 16 exact binary32 terms.  With G = max g_k the largest
// term occurs at least twice and no term exceeds it, so
// 2^(4G+9) <= S <= 16 * 2^(4G+8) = 2^(4G+12), and the binary32 exponent field
// of S, 4G + 136 .. 4G + 139, shifted right by 2 is exactly G + 34.  Both
// bounds are representable and every partial sum of nonnegative terms lies
// between the largest term and S, so any accumulation order and any faithful
// rounding keep S inside them: the matrix instruction's own rounding cannot
// change the result.  A quarter with no nonzero product gives S = 0, i.e. 0
// after the shift, below every real product (G >= -20 -> 14).  The biased
// block maximum is then E + 127 = max over the quarters of (S >> 25) + 93,
// compared with c's binary32 exponent field (|c| >= 2^-33 -> 94 or more,
// c = 0 -> 0).
constexpr uint32_t X_POW_OFF = 4;
constexpr uint32_t W_POW_OFF = 4;
constexpr uint32_t POW_TO_EB = 93;
constexpr int PW_ROW = 4;  // words per (quarter, row) of a power plane: 8 bf16
// The two 8-byte chunks of a power-plane row are stored swapped for rows 8-15
// of every 16: the 16 lanes that read one chunk of 16 consecutive rows (rows
// 16 bytes apart) then cover all 32 banks once instead of every bank pair
// twice.
__device__ __forceinline__ int pw_chunk(int row, int chunk) { return chunk ^ ((row >> 3) & 1); }

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_add_u16(uint32_t a, uint32_t b)
{
    us2 r = __builtin_bit_cast(us2, a) + __builtin_bit_cast(us2, b);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    us2 r = __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b));
    return __builtin_bit_cast(uint32_t, r);
}

// max(a, b, c) per 16-bit half, on positive normal binary16 patterns
__device__ __forceinline__ uint32_t pk_max3_h(uint32_t a, uint32_t b, uint32_t c)
{
    h2 r = __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b)), __builtin_bit_cast(h2, c));
    return __builtin_bit_cast(uint32_t, r);
}

// min(a, 1) per 16-bit half (written out: the compiler would unpack it)
__device__ __forceinline__ uint32_t pk_min1_u16(uint32_t a)
{
    uint32_t r;
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(a), "s"(0x00010001u));
    return r;
}

// max(lo16(g), hi16(g), lo16(e)), valid in the low 16 bits
__device__ __forceinline__ uint32_t max3_lo_hi_u16(uint32_t g, uint32_t e)
{
    uint32_t r;
    asm("v_max3_u16 %0, %1, %1, %2 op_sel:[0,1,0,0]" : "=v"(r) : "v"(g), "v"(e));
    return r;
}


__device__ __forceinline__ uint32_t pk_mad_u16(uint32_t a, uint32_t b, uint32_t c)
{
    us2 r = __builtin_bit_cast(us2, a) * __builtin_bit_cast(us2, b) + __builtin_bit_cast(us2, c);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pk_mul_u16(uint32_t a, uint32_t b)
{
    us2 r = __builtin_bit_cast(us2, a) * __builtin_bit_cast(us2, b);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pk_shr_u16(uint32_t a, uint32_t sh)
{
    us2 r = __builtin_bit_cast(us2, a) >> (us2){(unsigned short)sh, (unsigned short)sh};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ int dot2_i16(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot2(__builtin_bit_cast(s2, a), __builtin_bit_cast(s2, b), c, false);
}

// max(v, v of the partner lane) on the low 16 bits, and v + v of the partner
// lane, for the quad DPP patterns 0xB1 (lane ^ 1) and 0x4E (lane ^ 2): each
// one DPP-modified instruction (v_max_u16_dpp, v_add_u32_dpp).
template <int CTRL>
__device__ __forceinline__ uint32_t quad_max_lo16(uint32_t v)
{
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
    return __builtin_elementwise_max((unsigned short)v, (unsigned short)o);
}

template <int CTRL>
__device__ __forceinline__ int quad_add(int v)
{
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// K4PL steps of 4 binary16 values (2 words each) from LDS: one 16-byte or
// 8-byte read.
template <int K4PL>
__device__ __forceinline__ uint4 load_half_slice(const uint32_t *p)
{
    if constexpr (K4PL == 2) return *reinterpret_cast<const uint4 *>(p);
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    return make_uint4(v.x, v.y, 0u, 0u);
}

// The sign pair (+-1, +-1) of two products from the packed 16-bit sign masks
// of their x and w codes (0xFFFF negative, 0 positive): (sa ^ sb) | 1 per
// half, one v_bitop3_b32 (truth table 0xBE: (a ^ b) | c).
__device__ __forceinline__ uint32_t sign_pair(uint32_t sa, uint32_t sb)
{
    return __builtin_amdgcn_bitop3_b32(sa, sb, 0x00010001u, 0xBE);
}

// ---- floating-point mode control -----------------------------------------
// MODE register bits [1:0]: binary32 rounding (0 nearest even, 3 toward zero).
__device__ __forceinline__ uint32_t mode_round_toward_zero()
{
    uint32_t tok;
    asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3\n\t"
                 "s_nop 1\n\t"
                 "s_mov_b32 %0, 0"
                 : "=s"(tok)::"memory");
    return tok;
}

// Switch to round-to-nearest-even once `dep` (a value computed in the current
// mode) exists; returns a token for instructions that need the new mode.
__device__ __forceinline__ uint32_t mode_round_nearest_after(uint32_t dep)
{
    uint32_t tok;
    asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\t"
                 "s_nop 1\n\t"
                 "s_mov_b32 %0, 0"
                 : "=s"(tok)
                 : "v"(dep)
                 : "memory");
    return tok;
}

__device__ __forceinline__ uint32_t mode_round_toward_zero_after(uint32_t dep)
{
    uint32_t tok;
    asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3\n\t"
                 "s_nop 1\n\t"
                 "s_mov_b32 %0, 0"
                 : "=s"(tok)
                 : "v"(dep)
                 : "memory");
    return tok;
}

// fma(|a|, |b|, c) in the current (round-toward-zero) mode, as raw bits.
__device__ __forceinline__ uint32_t fma_abs_rz(float a, float b, uint32_t c, uint32_t tok)
{
    uint32_t r;
    asm("v_fma_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c), "s"(tok));
    return r;
}

// The same with a and b the low (LO) or high (HI) binary16 halves of two
// registers: v_fma_mix_f32 widens them exactly and forms the same fused
// product and sum (FP8 values are exact in binary16, subnormals included).
__device__ __forceinline__ uint32_t fma_abs_rz_lo16(uint32_t a, uint32_t b, uint32_t c, uint32_t tok)
{
    uint32_t r;
    asm("v_fma_mix_f32 %0, |%1|, |%2|, %3 op_sel_hi:[1,1,0]" : "=v"(r) : "v"(a), "v"(b), "v"(c), "s"(tok));
    return r;
}
__device__ __forceinline__ uint32_t fma_abs_rz_hi16(uint32_t a, uint32_t b, uint32_t c, uint32_t tok)
{
    uint32_t r;
    asm("v_fma_mix_f32 %0, |%1|, |%2|, %3 op_sel:[1,1,0] op_sel_hi:[1,1,0]"
        : "=v"(r)
        : "v"(a), "v"(b), "v"(c), "s"(tok));
    return r;
}

// The block sum starts from C's own bits: 2^q, the block's quantum, is the
// unit in the last place of Cb = 1.5 * 2^(E+10), whose low 22 fraction bits
// are zero, so Cb's bits plus the integer sum n (|n| < 2^21: at most 32
// terms and c's, each below 2^15) are the bits of Cb + n * 2^q, inside Cb's
// binade [2^(E+10), 2^(E+11)).  The difference of two binary32 values in one
// binade is exact in any rounding mode: one subtraction gives n * 2^q.
__device__ __forceinline__ uint32_t sub_block_base(uint32_t sum_bits, uint32_t Cb, uint32_t tok)
{
    uint32_t r;
    asm("v_sub_f32 %0, %1, %2" : "=v"(r) : "v"(sum_bits), "v"(Cb), "s"(tok));
    return r;
}

// The incoming accumulator's term of a block sum, in units of the block's
// quantum: |c| cut toward zero by the RTZ fma against C (the low 16 bits of
// the result, below 2^15), times c's sign: the sign from c's bits read as a
// signed integer, clamped to [-1, 1] (-0 gives -1, which only multiplies a
// zero magnitude), and a signed 16-bit multiply, in one statement so that no
// wait is placed between its three dependent instructions; Cb's bits are
// added, the sum's start (see sub_block_base).  (A form with the sign as the
// 16-bit pair (+-1, 0) and a dot product takes one instruction more; on
// MI355X it measured slower in every kernel once the LDS planes were free of
// bank conflicts: 8192^3 hopper 43.4 against 42.3 ms.)
__device__ __forceinline__ int c_block_term(uint32_t c, uint32_t Cb, uint32_t tok)
{
    int acc;
    uint32_t sgn, r;
    asm("v_med3_i32 %1, %3, -1, 1\n\t"
        "v_fma_f32 %2, |%3|, 1.0, %4\n\t"
        "v_mad_i32_i16 %0, %2, %1, %4"
        : "=v"(acc), "=&v"(sgn), "=&v"(r)
        : "v"(c), "v"(Cb), "s"(tok));
    return acc;
}

// The same term where G lanes share a chain and it enters the block sum on
// one lane only: that lane clamps c's bits to [lo, hi] = [-1, 1], the others
// to [0, 0], so their term is 0 without a separate select; `base` is Cb's
// bits on that lane and 0 on the others, so that the chain's sum across its
// lanes starts from Cb once.
__device__ __forceinline__ int c_block_term_on(uint32_t c, uint32_t Cb, uint32_t tok, int lo, int hi, uint32_t base)
{
    int acc;
    uint32_t sgn, r;
    asm("v_med3_i32 %1, %3, %6, %7\n\t"
        "v_fma_f32 %2, |%3|, 1.0, %4\n\t"
        "v_mad_i32_i16 %0, %2, %1, %8"
        : "=v"(acc), "=&v"(sgn), "=&v"(r)
        : "v"(c), "v"(Cb), "s"(tok), "v"(lo), "v"(hi), "v"(base));
    return acc;
}

// a + b in the current (round-to-nearest-even) mode.
__device__ __forceinline__ uint32_t add_rn(uint32_t a, uint32_t b, uint32_t tok)
{
    uint32_t r;
    asm("v_add_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b), "s"(tok));
    return r;
}

// c cut toward zero to 14 significant bits from its exponent field (emin for
// a subnormal c): the low 10 fraction bits cleared.  A negative c that leaves
// nothing becomes -0, which enters later blocks as +0 does; the chain's end
// turns it into +0.
__device__ __forceinline__ uint32_t cut14(uint32_t c) { return c & 0xFFFFFC00u; }
// The same cut where a chain ends, as an instruction the compiler keeps in
// place (as plain code it may recompute it after every block of the chain).
__device__ __forceinline__ uint32_t cut14_at_exit(uint32_t c)
{
    uint32_t r;
    asm("v_and_b32 %0, 0xfffffc00, %1" : "=v"(r) : "v"(c));
    return r;
}

// ---- FP8 decoding -----------------------------------------------------------
// Four codes of a row (one 32-bit word, k ascending from the low byte) become
//   four signed binary32 values (exact hardware conversions, subnormals
//   included),
//   two exponent-plane pairs (u16 per code, see the plane constants above;
//   subnormals take the field exponent emin, validation page claims table),
//   two sign-mask pairs (u16 per code, 0xFFFF for a negative code, else 0).
// NaN / Inf codes decode to something finite or not; outputs they touch are
// overwritten by the specials rule, so their lanes' values do not matter.
template <int FMT>
__device__ __forceinline__ void cvt4(uint32_t w, float &v0, float &v1, float &v2, float &v3)
{
    if (FMT == FMT_E4M3) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
        v0 = lo[0]; v1 = lo[1]; v2 = hi[0]; v3 = hi[1];
    } else {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
        v0 = lo[0]; v1 = lo[1]; v2 = hi[0]; v3 = hi[1];
    }
}

// Two codes (bytes 0-1, or 2-3 with HI) of a word as two binary16 values
// (exact hardware conversions, subnormals included), code 0 in the low half.
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt2_h(uint32_t w)
{
    if (FMT == FMT_E4M3) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI));
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)w, 1.0f, HI));
}

// The magnitudes (sign bits cleared) of four packed codes; the decode and the
// special-code test share them.
__device__ __forceinline__ uint32_t code_mags(uint32_t w) { return w & 0x7F7F7F7Fu; }

// Spread magnitude bytes 0-1 (HI: 2-3) of a word into [mag0, 0, mag1, 0].
template <bool HI>
__device__ __forceinline__ uint32_t mag_pair(uint32_t m)
{
    return __builtin_amdgcn_perm(0u, m, HI ? 0x0C030C02u : 0x0C010C00u);
}

// Exponent-plane pair of two codes whose magnitudes are held as [mag0, 0,
// mag1, 0].
template <int FMT, uint32_t EBIAS>
__device__ __forceinline__ uint32_t plane_pair(uint32_t mag)
{
    constexpr uint32_t FBIAS = (FMT == FMT_E4M3) ? 7u : 15u;
    constexpr uint32_t SH = (FMT == FMT_E4M3) ? 3u : 2u;
    // nonzero: max(ef, 1) - FBIAS + 0x200 + EBIAS = (max(ef,1) + K) * 1 + ZERO_PLANE
    constexpr uint32_t K = 0x200u + EBIAS - FBIAS - ZERO_PLANE;
    const uint32_t ef = pk_shr_u16(mag, SH);
    const uint32_t nz = pk_min1_u16(mag);
    const uint32_t pl = pk_add_u16(__builtin_bit_cast(uint32_t, __builtin_elementwise_max(
                                       __builtin_bit_cast(us2, ef), (us2){1, 1})),
                                   K | (K << 16));
    return pk_mad_u16(pl, nz, ZERO_PLANE | (ZERO_PLANE << 16));
}

// Power-plane pair (bf16 bits of 2^(4*ex + OFF), 0 for a zero code) of two
// codes whose magnitudes are held as [mag0, 0, mag1, 0]; ex is the field
// exponent (emin for subnormals).  bf16 bits of 2^E are (E + 127) << 7, and
// E + 127 = 4*max(ef, 1) + (OFF + 127 - 4*FBIAS).  (The compiler splits the
// multiply-add into a shift and an add; one v_pk_mad_u16 written out saved 8
// instructions per chunk but measured slower on MI355X: 8192^3 40.5 against
// 39.9 ms, A/B in one session.)
template <int FMT, uint32_t OFF>
__device__ __forceinline__ uint32_t power_pair(uint32_t mag)
{
    constexpr uint32_t FBIAS = (FMT == FMT_E4M3) ? 7u : 15u;
    constexpr uint32_t SH = (FMT == FMT_E4M3) ? 3u : 2u;
    constexpr uint32_t K = (OFF + 127u - 4u * FBIAS) << 7;
    const uint32_t ef = pk_shr_u16(mag, SH);
    const uint32_t nz = pk_min1_u16(mag);
    const uint32_t efc = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, ef), (us2){1, 1}));
    return pk_mul_u16(pk_mad_u16(efc, 0x02000200u, K | (K << 16)), nz);
}

// Decode 16 consecutive codes of one row into the value and sign planes and
// the power plane (the two quarter-blocks the 16 codes cover, 8 codes each).
// H: binary16 values, written as four 8-byte pairs (the rows of such planes
// are 8-byte aligned).
template <int FMT, uint32_t OFF, bool H = false>
__device__ __forceinline__ void decode_chunk_pw(uint4 raw, float *va, uint32_t *vs, uint32_t *pq0, uint32_t *pq1,
                                                int row)
{
    const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[16];
    uint32_t h[8];
    uint32_t pp[8], sp[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w = words[q];
        if constexpr (H) {
            h[2 * q] = cvt2_h<FMT, false>(w);
            h[2 * q + 1] = cvt2_h<FMT, true>(w);
        } else {
            cvt4<FMT>(w, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
        const uint32_t m = code_mags(w);
        pp[2 * q] = power_pair<FMT, OFF>(mag_pair<false>(m));
        pp[2 * q + 1] = power_pair<FMT, OFF>(mag_pair<true>(m));
        const uint32_t t = w << 8;
        sp[2 * q] = __builtin_amdgcn_perm(t, w, 0x08080A0Au);
        sp[2 * q + 1] = __builtin_amdgcn_perm(t, w, 0x09090B0Bu);
    }
    if constexpr (H) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint32_t *>(va) + 2 * q) = make_uint2(h[2 * q], h[2 * q + 1]);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4 *>(va + 4 * q) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint2 *>(vs + 2 * q) = make_uint2(sp[2 * q], sp[2 * q + 1]);
    // the quarter's 8 codes fill the two chunks of its row
    *reinterpret_cast<uint2 *>(pq0 + 2 * pw_chunk(row, 0)) = make_uint2(pp[0], pp[1]);
    *reinterpret_cast<uint2 *>(pq0 + 2 * pw_chunk(row, 1)) = make_uint2(pp[2], pp[3]);
    *reinterpret_cast<uint2 *>(pq1 + 2 * pw_chunk(row, 0)) = make_uint2(pp[4], pp[5]);
    *reinterpret_cast<uint2 *>(pq1 + 2 * pw_chunk(row, 1)) = make_uint2(pp[6], pp[7]);
}

// Decode 16 consecutive codes of one row into the LDS planes.
template <int FMT, uint32_t EBIAS>
__device__ __forceinline__ void decode_chunk(uint4 raw, float *va, uint32_t *ve, uint32_t *vs)
{
    const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[16];
    uint32_t ep[8], sp[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w = words[q];
        cvt4<FMT>(w, v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        const uint32_t m = code_mags(w);
        ep[2 * q] = plane_pair<FMT, EBIAS>(mag_pair<false>(m));
        ep[2 * q + 1] = plane_pair<FMT, EBIAS>(mag_pair<true>(m));
        // v_perm selectors 8..11 replicate the top bit of bytes 1, 3 of the
        // second source and bytes 1, 3 of the first: with (w << 8, w) these
        // are the signs of codes 1, 3, 0, 2.
        const uint32_t t = w << 8;
        sp[2 * q] = __builtin_amdgcn_perm(t, w, 0x08080A0Au);
        sp[2 * q + 1] = __builtin_amdgcn_perm(t, w, 0x09090B0Bu);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4 *>(va + 4 * q) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
#pragma unroll
    for (int q = 0; q < 2; ++q)
        *reinterpret_cast<uint4 *>(ve + 4 * q) = make_uint4(ep[4 * q], ep[4 * q + 1], ep[4 * q + 2], ep[4 * q + 3]);
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint2 *>(vs + 2 * q) = make_uint2(sp[2 * q], sp[2 * q + 1]);
}

// decode_chunk with a binary16 value plane (8 words for the 16 codes).
// SWZ: each plane's 32 bytes for the chunk are two 16-byte blocks, stored
// at word offsets o0 and 4 - o0 (o0 = 0 or 4, see the 4-lane tiles' row
// swizzle in the kernel).
template <int FMT, uint32_t EBIAS, bool SWZ = false>
__device__ __forceinline__ void decode_chunk_h(uint4 raw, uint32_t *vh, uint32_t *ve, uint32_t *vs, int o0 = 0)
{
    const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t h[8], ep[8], sp[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t w = words[q];
        h[2 * q] = cvt2_h<FMT, false>(w);
        h[2 * q + 1] = cvt2_h<FMT, true>(w);
        const uint32_t m = code_mags(w);
        ep[2 * q] = plane_pair<FMT, EBIAS>(mag_pair<false>(m));
        ep[2 * q + 1] = plane_pair<FMT, EBIAS>(mag_pair<true>(m));
        const uint32_t t = w << 8;
        sp[2 * q] = __builtin_amdgcn_perm(t, w, 0x08080A0Au);
        sp[2 * q + 1] = __builtin_amdgcn_perm(t, w, 0x09090B0Bu);
    }
    if constexpr (SWZ) {
        const int o1 = 4 - o0;
        *reinterpret_cast<uint4 *>(vh + o0) = make_uint4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<uint4 *>(vh + o1) = make_uint4(h[4], h[5], h[6], h[7]);
        *reinterpret_cast<uint4 *>(ve + o0) = make_uint4(ep[0], ep[1], ep[2], ep[3]);
        *reinterpret_cast<uint4 *>(ve + o1) = make_uint4(ep[4], ep[5], ep[6], ep[7]);
        *reinterpret_cast<uint4 *>(vs + o0) = make_uint4(sp[0], sp[1], sp[2], sp[3]);
        *reinterpret_cast<uint4 *>(vs + o1) = make_uint4(sp[4], sp[5], sp[6], sp[7]);
        return;
    }
    *reinterpret_cast<uint4 *>(vh) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4 *>(vh + 4) = make_uint4(h[4], h[5], h[6], h[7]);
#pragma unroll
    for (int q = 0; q < 2; ++q)
        *reinterpret_cast<uint4 *>(ve + 4 * q) = make_uint4(ep[4 * q], ep[4 * q + 1], ep[4 * q + 2], ep[4 * q + 3]);
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint2 *>(vs + 2 * q) = make_uint2(sp[2 * q], sp[2 * q + 1]);
}

// Any NaN (E4M3FN: magnitude 0x7F) or Inf / NaN (E5M2: magnitude 0x7C and
// above) code among four packed codes: the high bit of each byte of the
// result.  A magnitude byte is at most 0x7F, so adding 1 or 4 carries into
// its high bit exactly for those codes and never into the next byte.
template <int FMT>
__device__ __forceinline__ uint32_t has_special(uint32_t v)
{
    return (code_mags(v) + (FMT == FMT_E4M3 ? 0x01010101u : 0x04040404u)) & 0x80808080u;
}

// Row flags of a 16-byte chunk that holds a special code: bit 0 always,
// bit 1 if one of them is a NaN (E4M3FN: every special; E5M2: magnitude
// above 0x7C, the infinity).
template <int FMT>
__device__ __forceinline__ uint32_t special_flags(uint4 raw)
{
    if (FMT == FMT_E4M3) return 3u;
    const uint32_t nan = (((raw.x & 0x7F7F7F7Fu) + 0x03030303u) | ((raw.y & 0x7F7F7F7Fu) + 0x03030303u) |
                          ((raw.z & 0x7F7F7F7Fu) + 0x03030303u) | ((raw.w & 0x7F7F7F7Fu) + 0x03030303u)) &
                         0x80808080u;
    return nan ? 3u : 1u;
}

// A chunk's row flags where `hit` marks special codes in it.  NaN / Inf codes
// are rare: with BRANCH (tiles whose waves decode only x or only w rows) the
// flags are formed only where a lane of the wave holds one -- the empty
// volatile statement keeps that a branch, which the compiler would otherwise
// turn into forming them for every chunk and selecting (2048 x 5760 x 1920
// 1.96 -> 1.92 ms, 8192^3 unchanged, A/B in one session); tiles whose waves
// decode both keep the select (the 32x16 tile measured 4% slower with the
// branch while its waves held both).
template <int FMT, bool BRANCH>
__device__ __forceinline__ void rare_flags(uint32_t &flag, uint32_t hit, uint4 raw)
{
    if constexpr (BRANCH) {
        if (__any(hit != 0)) {
            asm volatile("");
            if (hit) flag |= special_flags<FMT>(raw);
        }
    } else {
        if (hit) flag |= special_flags<FMT>(raw);
    }
}

// The k-list of one split: positions 0 .. len-1 along its k-tiles (width
// 2^shift; tile `first`, then every `stride`-th), k = tile * W + offset.
struct SplitSeq {
    int64_t first, stride, len;
    int shift;
    __device__ __forceinline__ int64_t k_of(int64_t pos) const
    {
        return ((first + (pos >> shift) * stride) << shift) + (pos & ((int64_t(1) << shift) - 1));
    }
};

__device__ __forceinline__ SplitSeq split_seq(const MainParams &p, int z)
{
    const int64_t W = int64_t(1) << p.tile_shift;
    const int64_t nt = (p.K + W - 1) >> p.tile_shift;
    SplitSeq q;
    q.shift = p.tile_shift;
    int64_t ntiles;
    if (p.round_robin) {
        q.first = z;
        q.stride = p.S;
        ntiles = (z < nt) ? (nt - z + p.S - 1) / p.S : 0;
    } else {
        q.first = (int64_t)z * p.tps;
        q.stride = 1;
        ntiles = (q.first < nt) ? ((p.tps < nt - q.first) ? p.tps : nt - q.first) : 0;
    }
    q.len = 0;
    if (ntiles > 0) {
        const int64_t last = q.first + (ntiles - 1) * q.stride;
        const int64_t tail = p.K - (last << p.tile_shift);
        q.len = ((ntiles - 1) << p.tile_shift) + (tail < W ? tail : W);
    }
    return q;
}

// Byte masks (the high bit of each byte) of four packed codes: zero, NaN
// and infinite codes.
__device__ __forceinline__ uint32_t zero_bytes(uint32_t v)
{
    return ~((v & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;
}
template <int FMT>
__device__ __forceinline__ uint32_t nan_bytes(uint32_t v)
{
    return ((v & 0x7F7F7F7Fu) + (FMT == FMT_E4M3 ? 0x01010101u : 0x03030303u)) & 0x80808080u;
}
template <int FMT>
__device__ __forceinline__ uint32_t inf_bytes(uint32_t v)
{
    if (FMT == FMT_E4M3) return 0u;
    return zero_bytes((v & 0x7F7F7F7Fu) ^ 0x7C7C7C7Cu);
}
// The non-finite result of one output over positions [p0, p1) of a split's
// k-list: NaN if a NaN code is in either row, if some k pairs an infinity
// with a zero, or if infinite products of both signs occur; otherwise the
// signed infinity; 0 (not a result: the range is finite) when no product
// there involves a NaN or Inf code.  Called only for outputs with a flagged
// row (xflag, wflag: the row holds such codes in this workgroup's range).
// The flagged rows are read 16 codes at a time; the other row only where a
// flagged chunk holds a NaN / Inf code, so the work per output is one pass
// over the flagged row(s), whatever the number of special codes.
template <int XF, int WF>
__device__ uint32_t special_scan(const uint8_t *xr, const uint8_t *wr, const SplitSeq &sq, int64_t p0, int64_t p1,
                             bool xflag, bool wflag)
{
    uint32_t bad = 0, pos = 0, neg = 0;
    for (int64_t q = p0; q < p1; q += 16) {
        const int64_t k = sq.k_of(q);
        uint4 xv = make_uint4(0, 0, 0, 0), wv = make_uint4(0, 0, 0, 0);
        uint32_t hit = 0;
        if (xflag) {
            xv = *reinterpret_cast<const uint4 *>(xr + k);
            hit |= has_special<XF>(xv.x) | has_special<XF>(xv.y) | has_special<XF>(xv.z) | has_special<XF>(xv.w);
        }
        if (wflag) {
            wv = *reinterpret_cast<const uint4 *>(wr + k);
            hit |= has_special<WF>(wv.x) | has_special<WF>(wv.y) | has_special<WF>(wv.z) | has_special<WF>(wv.w);
        }
        if (!hit) continue;
        if (!xflag) xv = *reinterpret_cast<const uint4 *>(xr + k);
        if (!wflag) wv = *reinterpret_cast<const uint4 *>(wr + k);
        const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w}, ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t a = xs[u], b = ws[u];
            const uint32_t ai = inf_bytes<XF>(a), bi = inf_bytes<WF>(b);
            const uint32_t inf = ai | bi;
            const uint32_t neg_sign = (a ^ b) & 0x80808080u;
            bad |= nan_bytes<XF>(a) | nan_bytes<WF>(b) | (ai & zero_bytes(b)) | (bi & zero_bytes(a));
            neg |= inf & neg_sign;
            pos |= inf & ~neg_sign;
        }
    }
    if (bad || (pos && neg)) return kCanonNan32;
    if (neg) return 0xFF800000u;
    return pos ? 0x7F800000u : 0u;
}

__device__ __forceinline__ void store_output(const MainParams &p, int64_t m, int64_t n, uint32_t acc,
                                             uint32_t alpha, uint32_t sr, int split)
{
    if (p.out_kind == OUT_ACC_F32) {  // the accumulator, or this split's partial
        float *o = reinterpret_cast<float *>(p.out) + split * p.split_stride;
        reinterpret_cast<uint32_t *>(o)[m * p.ldo + n] = canon_f32(acc);
        return;
    }
    store_epilogue(p.out_kind, p.out, m * p.ldo + n, acc, alpha, sr);
}

// XCD-aware tile order.  The workgroups of a launch are dealt round-robin to
// the 8 XCDs (workgroup id mod 8), each with its own L2.  When the tile
// count allows, ids are renumbered so that XCD j takes the j-th eighth of
// the tiles, and the tiles are walked in groups of TILE_GROUP tile-rows,
// column by column inside a group: the workgroups resident on one XCD then
// cover a compact block of tile-rows and tile-columns and share their
// operand rows in that XCD's L2.  A bijection on any grid.
constexpr int TILE_GROUP = 8;

__device__ __forceinline__ void tile_order(int &tile_m, int &tile_n)
{
    const int64_t nx = gridDim.x, ny = gridDim.y;
    const int64_t T = nx * ny;
    int64_t id = (int64_t)blockIdx.y * nx + blockIdx.x;
    if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
    const int64_t per_group = TILE_GROUP * nx;
    const int64_t g = id / per_group;
    const int64_t first = g * TILE_GROUP;
    const int64_t rows = (ny - first < TILE_GROUP) ? ny - first : TILE_GROUP;
    const int64_t r = id - g * per_group;
    tile_m = (int)(first + r % rows);
    tile_n = (int)(r / rows);
}

// ---- the main kernel ---------------------------------------------------------
// Workgroup tile BM x BN outputs of one split; thread tile RM x RN with rows
// tm + i*TM and columns tn + j*TN (interleaved, so that the lanes of a wave
// read consecutive, padded LDS rows).
// Minimum workgroups per CU the register allocation must allow for a thread
// tile: the launch bound's second argument, which the compiler caps at what
// the workgroup's LDS lets fit.  With the 256-thread workgroups of the tiles
// with one lane per output this is the minimum waves per SIMD (3: at most 168
// VGPRs).
// Without the bound of 3 for 4x4 tiles the compiler gave the 64x64
// matrix-core kernel of incoming accumulators 200 VGPRs (2 waves per SIMD),
// which cost it 9% on 8192^3 (49.3 against 44.7 ms, A/B in one session).
// 4x4 tiles of fast accumulation run 4 waves per SIMD (their LDS lets 4
// workgroups share a CU): with the term loop unrolled under step barriers
// they fit in 117 VGPRs without spills (8192^3 39.3-39.5 against 39.8 ms for
// 3 waves with the loop rolled, A/B in one session; the unrolled loop at 3
// waves measured 41.1 ms, and 4 waves with the rolled loop 0.5% slower than
// 3).  Slow accumulation and incoming accumulators would spill at 4 waves
// and keep 3.
// The 4-lane tiles with 32-product blocks in fast accumulation read their
// LDS words a stage ahead into registers (see LDS_PF in the kernel); a
// 512-thread workgroup of them is two waves per SIMD, the most their grids
// (one workgroup per CU) give, so their bound is 2 (up to 256 VGPRs; a
// 1024-thread workgroup stays within 128 by its size).
template <int RM, int RN, int ACC, int G = 1, int BLK = 32>
struct WavesPerSimd {
    static constexpr bool FOUR = RM * RN == 16 && ACC == 0;  // ACC_FAST
    static constexpr int value = (G == 4 && BLK == 32 && (ACC == 0 || ACC == 3))   ? 2
                                 : (RM * RN > 16)                                  ? 2
                                 : (RM * RN == 2 || (RM * RN == 16 && !FOUR)) ? 3
                                                                                   : 4;
};
// Most waves per SIMD the compiler may schedule for: those 4x4 tiles' own
// count, otherwise the hardware's 8.
template <int RM, int RN, int ACC>
struct MaxWavesPerSimd {
    static constexpr int value = (RM * RN == 16) ? WavesPerSimd<RM, RN, ACC>::value : 8;
};

// G lanes share each output chain (G = 1, 2 or 4): lane g of a chain takes
// the g-th of G equal slices of every block; the block maximum and the block
// sum are combined across the G lanes with quad DPP moves, and every lane of
// the chain then carries the same accumulator.
//
// BLK products per block (32: hopper; 16: the RTX 4060 profiles).  The LDS
// stage is always 32 k wide; with BLK = 16 it holds two blocks, stepped in
// order.
//
// MX: the block maximum comes from bf16 matrix instructions (see the power
// planes above) instead of packed VALU maxima.  Needs G = 1, RM = 4 or 2 and
// 4 / RM waves per 16-row band: the band's 16 x (16*RN) outputs are RN 16x16
// matrix-instruction tiles, and lane l owns columns l%16 + 16*j and rows
// 4*(l/16) + i, the layout of v_mfma_f32_16x16x16_bf16's result.  With RM = 2
// the band's two waves h = 0, 1 take rows 4*(l/16) + 2h + i (i = 0, 1): wave h
// feeds the instruction its own two rows of every four twice (A rows 4q + i
// are x rows 4q + 2h + (i & 1)), so that its results i and i + 2 are both row
// 4q + 2h + i and every result register is read (both waves issue the band's
// matrix instructions).  With results 2 and 3 unread, the compiler reused
// their registers while the instruction could still write them: measured on
// MI355X, wrong block maxima for every second row of the 32x16 tile with
// 16-product blocks.
// Accumulation styles (template parameter ACC): one chain per split; slow
// accumulation with the running binary32 sum in registers; slow
// accumulation with each 128-chunk's result stored as a partial.
constexpr int ACC_FAST = 0, ACC_SLOW = 1, ACC_SLOW_CHUNKS = 2, ACC_FAST_CIN = 3;

template <int XF, int WF, int BM, int BN, int RM, int RN, int G, int ACC, bool MX, int BLK, int SS>
__global__ __launch_bounds__((BM / RM) * (BN / RN) * G)
__attribute__((amdgpu_waves_per_eu(WavesPerSimd<RM, RN, ACC, G, BLK>::value, MaxWavesPerSimd<RM, RN, ACC>::value))) void main_kernel(
    MainParams p)
{
    static_assert(G == 1 || G == 2 || G == 4, "G lanes per chain: 1, 2 or 4");
    static_assert(BLK == 32 || BLK == 16, "blocks of 32 or 16 products");
    static_assert(!MX || ((RM == 4 || RM == 2) && G == 1 && BN == 16 * RN &&
                          (BM / 16) * (4 / RM) * 64 == (BM / RM) * (BN / RN)),
                  "matrix-instruction exponents need 4 / RM waves per 16-row band and RM x RN thread tiles");
    constexpr int TM = BM / RM, TN = BN / RN, NT = TM * TN * G;
    constexpr int NCHUNK = 2 * (BM + BN);  // 16-byte chunks per stage: two per row
    constexpr int CPT = (NCHUNK * SS + NT - 1) / NT;
    constexpr int NXC = 2 * BM * SS;  // x chunks per barrier round, numbered first
    // every wave decodes x rows only or w rows only
    constexpr bool FLAG_BRANCH = NXC % 64 == 0 && NT % 64 == 0;
    constexpr int NBS = KB / BLK;          // blocks per stage
    constexpr int QPB = BLK / 8;           // quarter-blocks (8 products) per block
    constexpr int WPB = BLK / 2;           // exponent-plane words per block
    constexpr int WPL = WPB / G;           // ... per lane
    constexpr int WU = (WPL >= 4) ? 4 : 2; // words per exponent-plane read
    constexpr int K4PL = BLK / 4 / G;      // groups of 4 products per lane and block
    static_assert(WPL % WU == 0 && K4PL >= 1, "block slice per lane");
    static_assert(SS >= 1, "stages per barrier");
    // Unroll of the per-block pass loops: whole blocks for thread tiles of
    // at most 4 outputs (immediate LDS offsets), except the two-stage 2x2
    // tile, whose four waves per SIMD would then spill registers (it keeps
    // an unroll of 2); none for larger thread tiles (registers).
    constexpr int PASS_UNROLL = (RM * RN > 4) ? 1 : (SS == 2 && RM * RN == 4) ? 2 : 8;
    // The 4x4 tiles of 4 waves per SIMD (256-thread workgroups; the one-wave
    // 16x64 tile's LDS leaves it at 2) unroll the term loop of a block as
    // well, with a scheduling barrier after every step: each step keeps its
    // own LDS reads (the register budget of the rolled loop), while every
    // address becomes a base plus an immediate offset (no per-step address
    // additions).
    constexpr bool STEP_FENCE = WavesPerSimd<RM, RN, ACC>::FOUR && NT == 256;
    constexpr int TERM_UNROLL = STEP_FENCE ? K4PL : PASS_UNROLL;
    // CIN: fast accumulation from incoming accumulators c_in instead of +0
    constexpr bool CIN = ACC == ACC_FAST_CIN;
    constexpr bool FAST = ACC == ACC_FAST || CIN, CHUNKS = ACC == ACC_SLOW_CHUNKS;
    constexpr bool RANGED = CHUNKS;  // a group of 128-chunks of the split's k-list per workgroup
    constexpr int PST = exp_stride<G, BLK>();
    // sign words read 16 bytes (two steps of 4 products) at a time
    constexpr bool SIGN16 = G == 4 && BLK == 32;
    // The 4-lane tiles, bound by LDS bandwidth rather than by the VALU, keep
    // their value planes in binary16 (half the bytes; the truncating products
    // then issue as v_fma_mix_f32, whose term mix is 12% slower to issue).
    constexpr bool V16 = G == 4 || (MX && RM == 2);
    constexpr int AHS = half_stride<G, BLK>();
    constexpr bool SLICE16 = V16 && K4PL <= 2;  // a lane's whole slice of a block in one read
    constexpr int XA = V16 ? BM * AHS : BM * A_STRIDE, XP = BM * PST;
    constexpr int WA = V16 ? BN * AHS : BN * A_STRIDE, WP = BN * PST;
    static_assert(!V16 || (G == 4 && K4PL <= 2 && !MX) || (G == 1 && MX), "binary16 value planes");
    constexpr int SST = sign_stride<G, BLK>();
    constexpr int XS = BM * SST, WS = BN * SST;
    // 4-lane tiles with 32-product blocks: every plane row is 64 bytes, four
    // 16-byte blocks, lane g of a chain reading block g.  The decode writes a
    // chunk (half a row) as two 16-byte stores per plane, 8 lanes at a time
    // from 4 consecutive rows: unswizzled, rows r and r + 2 put them on the
    // same banks.  Storing block b of row r at b ^ ((r >> 1) & 1) spreads
    // those 8 stores over all 32 banks, and every 8 lanes of a read (2 rows x
    // 4 blocks) still cover them once.
    constexpr bool SWZ = G == 4 && BLK == 32;
    static_assert(!SWZ || (PST == KP && AHS == KP && SST == KP && SIGN16 && SLICE16 && NBS == 1),
                  "swizzled 64-byte rows");
    auto swz = [&](int row) { return SWZ ? 4 * ((row >> 1) & 1) : 0; };  // word offset
    constexpr int XPW = 4 * BM * PW_ROW, WPW = 4 * BN * PW_ROW;  // power-plane words per stage

    // LDS planes of SS consecutive stages (k-list positions pos .. pos + 32*SS)
    __shared__ __attribute__((aligned(16))) float xa_all[SS * XA];
    __shared__ __attribute__((aligned(16))) uint32_t xe_all[MX ? 4 : SS * XP];
    __shared__ __attribute__((aligned(16))) uint32_t xs_all[SS * XS];
    __shared__ __attribute__((aligned(16))) float wa_all[SS * WA];
    __shared__ __attribute__((aligned(16))) uint32_t we_all[MX ? 4 : SS * WP];
    __shared__ __attribute__((aligned(16))) uint32_t wsg_all[SS * WS];
    __shared__ __attribute__((aligned(16))) uint32_t xp[MX ? SS * XPW : 4];
    __shared__ __attribute__((aligned(16))) uint32_t wp[MX ? SS * WPW : 4];
    __shared__ uint32_t flags[BM + BN + CHUNKS];  // per row (and, for stored chunks, their union)

    const int t = threadIdx.x;
    const int lane_g = t % G, slot = t / G;
    const int c_lo = lane_g == 0 ? -1 : 0, c_hi = lane_g == 0 ? 1 : 0;  // see c_block_term_on
    const int tn = slot % TN, tm = slot / TN;
    const int wave = t >> 6, lane = t & 63;
    // MX: the wave's 16-row band and, for RM = 2, its half of the band's rows
    constexpr int BAND_WAVES = MX ? 4 / RM : 1;
    const int band = wave / BAND_WAVES, half_rows = (RM == 2) ? 2 * (wave % BAND_WAVES) : 0;
    // local row of chain i, local column of chain j
    auto row_of = [&](int i) { return MX ? 16 * band + 4 * (lane >> 4) + half_rows + i : tm + i * TM; };
    auto col_of = [&](int j) { return MX ? (lane & 15) + 16 * j : tn + j * TN; };
    int tile_m, tile_n;
    tile_order(tile_m, tile_n);
    const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
    const int split = RANGED ? blockIdx.z / p.chunk_groups : blockIdx.z;
    const int group = RANGED ? blockIdx.z % p.chunk_groups : 0;
    const SplitSeq sq = split_seq(p, split);
    // positions [pos_begin, pos_end) of the split's k-list: all of them, or
    // one group of 128-chunks when chunk results are stored
    const int64_t span = (int64_t)p.chunks_per_group * CHUNK;
    const int64_t pos_begin = RANGED ? (int64_t)group * span : 0;
    const int64_t pos_end = RANGED ? ((pos_begin + span < sq.len) ? pos_begin + span : sq.len) : sq.len;

    for (int i = t; i < BM + BN + CHUNKS; i += NT) flags[i] = 0;

    // The 4-lane tiles with 32-product blocks (one output per thread) in fast
    // accumulation read a stage's six 16-byte LDS words -- exponents, binary16 values and signs of
    // the x and the w row, lane g's block g of each -- one stage ahead, into
    // registers: the reads of stage st + 1 are in flight while stage st
    // computes its chain.
    constexpr bool LDS_PF = SWZ && RM == 1 && RN == 1 && FAST;
    struct StageReads {
        uint4 ea, eb, ah, bh, sa, sb;
    };
    auto stage_reads = [&](int st) {
        StageReads r;
        const int ox = (4 * lane_g) ^ swz(tm), ow = (4 * lane_g) ^ swz(tn);
        const uint32_t *xh = reinterpret_cast<const uint32_t *>(xa_all + st * XA);
        const uint32_t *wh = reinterpret_cast<const uint32_t *>(wa_all + st * WA);
        r.ea = *reinterpret_cast<const uint4 *>(xe_all + st * XP + tm * PST + ox);
        r.eb = *reinterpret_cast<const uint4 *>(we_all + st * WP + tn * PST + ow);
        r.ah = *reinterpret_cast<const uint4 *>(xh + tm * AHS + ox);
        r.bh = *reinterpret_cast<const uint4 *>(wh + tn * AHS + ow);
        r.sa = *reinterpret_cast<const uint4 *>(xs_all + st * XS + tm * SST + ox);
        r.sb = *reinterpret_cast<const uint4 *>(wsg_all + st * WS + tn * SST + ow);
        return r;
    };

    uint32_t myflag[CPT];
    uint4 raw[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q) myflag[q] = 0;

    // Stages at sequence positions pos, pos + 32, ..., pos + 32*(SS-1) (each a
    // multiple of 32 inside one k-tile), 2 16-byte chunks per row and stage:
    // chunk idx = t + q*NT numbers the x chunks of all SS stages first
    // (stage idx / (2*BM), row (idx % (2*BM)) >> 1), then the w chunks (row
    // index BM + that of idx - NXC), half idx & 1.  With NXC a multiple of
    // 64, every wave decodes x rows only or w rows only (a wave holding both
    // runs both decode paths, one after the other).
    // A 32-wide stage never straddles a k-tile (tiles are 64 or 128 wide and
    // stages start at multiples of 32 of the k-list), and only the last
    // k-tile of K can be short, so a chunk is loaded when its k is below K;
    // codes past K, rows past M or N and stages past the k-list load as
    // zeros (zero products: neutral in every block).  Each thread's row
    // pointers (with its 16-byte half) and stage offsets are fixed for the
    // whole walk: small thread tiles keep them in registers, large ones
    // (whose register budget is tight) recompute them at every load.
    constexpr bool KEEP_ROWS = RM * RN <= 4;
    // (one stage per barrier: the same order as idx % NCHUNK, which the
    // 64x64 kernel keeps -- the general form cost it 1.9% on 8192^3)
    auto chunk_stage = [&](int idx) {
        if constexpr (SS == 1) return 0;
        return idx < NXC ? idx / (2 * BM) : (idx - NXC) / (2 * BN);
    };
    auto chunk_rowidx = [&](int idx) {
        if constexpr (SS == 1) return (idx % NCHUNK) >> 1;
        return idx < NXC ? (idx % (2 * BM)) >> 1 : BM + (((idx - NXC) % (2 * BN)) >> 1);
    };
    auto chunk_row_of = [&](int q) -> const uint8_t * {
        const int idx = t + q * NT;
        const int c = (SS == 1) ? idx % NCHUNK : idx;  // c: the half's parity
        const int r = (SS == 1) ? c >> 1 : chunk_rowidx(idx);
        const uint8_t *row = nullptr;
        if (idx < NCHUNK * SS) {
            if (r < BM) {
                if (m0 + r < p.M) row = p.x + (m0 + r) * p.ldx;
            } else if (n0 + (r - BM) < p.N) {
                row = p.w + (n0 + r - BM) * p.ldw;
            }
        }
        return row ? row + 16 * (c & 1) : nullptr;
    };
    const uint8_t *chunk_row[KEEP_ROWS ? CPT : 1];
    if constexpr (KEEP_ROWS) {
#pragma unroll
        for (int q = 0; q < CPT; ++q) chunk_row[q] = chunk_row_of(q);
    }
    // Several stages per barrier over a contiguous k-list (position sp is
    // k = k0 + sp): chunk q of this thread, at offset off = stage * 32 + half
    // from the barrier's first position pos, reads chunk_base[q] + k0 + pos
    // (its row pointer with the offset folded in) while off is below both the
    // k-list's end and K, measured from pos; chunks without a row get an
    // offset no bound reaches.
    constexpr bool MULTI = SS > 1 && KEEP_ROWS;
    const uint8_t *chunk_base[MULTI ? CPT : 1];
    int chunk_off[MULTI ? CPT : 1];
    if constexpr (MULTI) {
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int idx = t + q * NT;
            const int stk = chunk_stage(idx) * KB;
            chunk_base[q] = chunk_row[q] ? chunk_row[q] + stk : p.x;
            chunk_off[q] = chunk_row[q] ? stk + 16 * (idx & 1) : INT32_MAX;
        }
    }
    auto load_block = [&](int64_t pos) {
        if constexpr (SS == 1) {
            // one stage per barrier: every chunk sits at position pos (inside
            // the k-list: the callers check), whose k is the same for the
            // whole workgroup and is formed by scalar instructions.  (Reading
            // chunks without codes from a zero constant instead of zeroing
            // them made these loads flat ones, which also count as LDS
            // accesses: 8192^3 41.2 against 40.2 ms.)
            const int64_t k = sq.k_of(pos);
#pragma unroll
            for (int q = 0; q < CPT; ++q) {
                const int half = 16 * ((t + q * NT) & 1);
                const uint8_t *row = KEEP_ROWS ? chunk_row[KEEP_ROWS ? q : 0] : chunk_row_of(q);
                raw[q] = make_uint4(0, 0, 0, 0);
                if (row && k + half < p.K) raw[q] = *reinterpret_cast<const uint4 *>(row + k);
            }
        } else {
            if (MULTI && !p.round_robin) {
                // the contiguous k-list (uniform branch): one scalar bound
                const int64_t kp = (sq.first << sq.shift) + pos;
                int64_t lim = pos_end - pos;
                if (p.K - kp < lim) lim = p.K - kp;
                const int lim32 = (int)(lim < KB * SS ? lim : KB * SS);
#pragma unroll
                for (int q = 0; q < CPT; ++q) {
                    raw[q] = make_uint4(0, 0, 0, 0);
                    if (chunk_off[MULTI ? q : 0] < lim32)
                        raw[q] = *reinterpret_cast<const uint4 *>(chunk_base[MULTI ? q : 0] + kp);
                }
            } else {
#pragma unroll
                for (int q = 0; q < CPT; ++q) {
                    const int idx = t + q * NT;
                    const int half = 16 * (idx & 1);
                    raw[q] = make_uint4(0, 0, 0, 0);
                    const int64_t sp = pos + (int64_t)chunk_stage(idx) * KB;
                    const uint8_t *row = KEEP_ROWS ? chunk_row[KEEP_ROWS ? q : 0] : chunk_row_of(q);
                    if (row && sp < pos_end) {
                        const int64_t k = sq.k_of(sp);
                        if (k + half < p.K) raw[q] = *reinterpret_cast<const uint4 *>(row + k);
                    }
                }
            }
        }
    };

    uint32_t tok = mode_round_toward_zero();

    uint32_t c[RM][RN];
    constexpr bool RUNNING = ACC == ACC_SLOW;  // a running slow sum per output
    // Between blocks the chain may carry its block sum uncut (up to 21
    // significant bits): the next block reads c only through its exponent,
    // which the cut does not change, and through c truncated to a multiple of
    // 2^(E-13) with E >= c's exponent, which the cut's quantum 2^(ec-13)
    // divides, so truncating the uncut value gives the same multiple.  The
    // cut to 14 significant bits is then made where c leaves the chain.
    // Incoming accumulators keep c cut after every block (they select c
    // itself on some blocks).
    constexpr bool CUT_EACH_BLOCK = CIN;
    // The block sum starts from Cb's bits (the epilogue is then one
    // subtraction, see sub_block_base; where c stays cut after every block,
    // the cut follows it: n * 2^q is a normal binary32 value on every block
    // whose result is used, biased E >= 94, so cutting it and cutting n
    // before the scaling clear the same bits).  Where G lanes share a chain
    // only its first lane adds Cb's bits (masked by cb_on), with the incoming
    // c's term; the quad sums then give every lane of the chain Cb + n.
    const uint32_t cb_on = lane_g == 0 ? 0xFFFFFFFFu : 0u;
    uint32_t slow[RUNNING ? RM : 1][RUNNING ? RN : 1];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) c[i][j] = 0u;
    if constexpr (CIN) {
        // every lane of a chain starts from the output's c_in (it enters the
        // block sums once); NaN / Inf c_in start from +0 and are applied
        // at the end
#pragma unroll
        for (int i = 0; i < RM; ++i)
#pragma unroll
            for (int j = 0; j < RN; ++j) {
                const int64_t m = m0 + row_of(i), n = n0 + col_of(j);
                if (m < p.M && n < p.N) {
                    const uint32_t cb = __float_as_uint(p.c_in[m * p.ldc + n]);
                    c[i][j] = ((cb >> 23) & 0xFFu) == 0xFFu ? 0u : cb;
                }
            }
    }
    if (RUNNING) {
#pragma unroll
        for (int i = 0; i < (RUNNING ? RM : 1); ++i)
#pragma unroll
            for (int j = 0; j < (RUNNING ? RN : 1); ++j) slow[i][j] = 0u;
    }

    if (pos_begin < pos_end) load_block(pos_begin);
    for (int64_t pos = pos_begin; pos < pos_end; pos += (int64_t)KB * SS) {
        __syncthreads();  // previous stages' readers are done with the LDS planes
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int idx = t + q * NT;
            if (idx < NCHUNK * SS) {
                const int c = (SS == 1) ? idx % NCHUNK : idx;
                const int st = (SS == 1) ? idx / NCHUNK : chunk_stage(idx);
                const int r = (SS == 1) ? c >> 1 : chunk_rowidx(idx), half = c & 1;
                if (r < BM) {
                    const uint32_t hit = has_special<XF>(raw[q].x) | has_special<XF>(raw[q].y) |
                                         has_special<XF>(raw[q].z) | has_special<XF>(raw[q].w);
                    rare_flags<XF, FLAG_BRANCH>(myflag[q], hit, raw[q]);
                    float *xa = xa_all + st * XA;
                    uint32_t *xe = xe_all + (MX ? 0 : st * XP), *xs = xs_all + st * XS;
                    if (MX)
                        decode_chunk_pw<XF, X_POW_OFF, V16>(raw[q],
                                                            V16 ? reinterpret_cast<float *>(
                                                                      reinterpret_cast<uint32_t *>(xa) + r * AHS +
                                                                      8 * half)
                                                                : xa + r * A_STRIDE + 16 * half,
                                                       xs + r * SST + 8 * half,
                                                       xp + st * XPW + ((2 * half) * BM + r) * PW_ROW,
                                                       xp + st * XPW + ((2 * half + 1) * BM + r) * PW_ROW, r);
                    else if (V16)
                        decode_chunk_h<XF, X_EBIAS, SWZ>(raw[q], reinterpret_cast<uint32_t *>(xa) + r * AHS + 8 * half,
                                                         xe + r * PST + 8 * half, xs + r * SST + 8 * half, swz(r));
                    else
                        decode_chunk<XF, X_EBIAS>(raw[q], xa + r * A_STRIDE + 16 * half,
                                                  xe + r * PST + 8 * half, xs + r * SST + 8 * half);
                } else {
                    const int rw = r - BM;
                    const uint32_t hit = has_special<WF>(raw[q].x) | has_special<WF>(raw[q].y) |
                                         has_special<WF>(raw[q].z) | has_special<WF>(raw[q].w);
                    rare_flags<WF, FLAG_BRANCH>(myflag[q], hit, raw[q]);
                    float *wa = wa_all + st * WA;
                    uint32_t *we = we_all + (MX ? 0 : st * WP), *wsg = wsg_all + st * WS;
                    if (MX)
                        decode_chunk_pw<WF, W_POW_OFF, V16>(raw[q],
                                                            V16 ? reinterpret_cast<float *>(
                                                                      reinterpret_cast<uint32_t *>(wa) + rw * AHS +
                                                                      8 * half)
                                                                : wa + rw * A_STRIDE + 16 * half,
                                                       wsg + rw * SST + 8 * half,
                                                       wp + st * WPW + ((2 * half) * BN + rw) * PW_ROW,
                                                       wp + st * WPW + ((2 * half + 1) * BN + rw) * PW_ROW, rw);
                    else if (V16)
                        decode_chunk_h<WF, W_EBIAS, SWZ>(raw[q], reinterpret_cast<uint32_t *>(wa) + rw * AHS + 8 * half,
                                                         we + rw * PST + 8 * half, wsg + rw * SST + 8 * half, swz(rw));
                    else
                        decode_chunk<WF, W_EBIAS>(raw[q], wa + rw * A_STRIDE + 16 * half,
                                                  we + rw * PST + 8 * half, wsg + rw * SST + 8 * half);
                }
            }
        }
        __syncthreads();
        // prefetch the next stages; latency hidden by the compute below
        if (pos + (int64_t)KB * SS < pos_end) load_block(pos + (int64_t)KB * SS);

        [[maybe_unused]] StageReads nxt;
        if constexpr (LDS_PF) nxt = stage_reads(0);
        // all the stages of one barrier unrolled: every LDS address of the
        // stage's planes is then a per-thread base plus an immediate offset
        // (not for two stages of 2x2 thread tiles: unrolled, their four
        // waves per SIMD would spill registers)
#pragma unroll((SS == 2 && RM * RN == 4) ? 1 : SS)
        for (int st = 0; st < SS; ++st) {
        const int64_t spos = pos + (int64_t)st * KB;
        // Past the end of the k-list the stages hold zero codes.  In fast
        // accumulation such a block leaves c cut to 14 significant bits, the
        // cut its exit makes anyway, so the stages of one barrier run as one
        // straight block of code (the compiler can then start a stage's LDS
        // reads during the previous stage's arithmetic); slow accumulation
        // stops at the end (its chunk boundaries count positions).
        if (!FAST && spos >= pos_end) break;  // uniform across the workgroup
        [[maybe_unused]] StageReads cur;
        if constexpr (LDS_PF) {
            cur = nxt;
            if (st + 1 < SS) nxt = stage_reads(st + 1);
        }
        const float *xa = xa_all + st * XA, *wa = wa_all + st * WA;
        const uint32_t *xe = xe_all + (MX ? 0 : st * XP), *we = we_all + (MX ? 0 : st * WP);
        const uint32_t *xs = xs_all + st * XS, *wsg = wsg_all + st * WS;
#pragma unroll
        for (int hb = 0; hb < NBS; ++hb) {
            uint32_t Cb[RM][RN];
            int acc[RM][RN];
            if constexpr (MX) {
                // pass 1 on the matrix cores: per quarter-block, S for every output
                uint32_t smax[RM][RN];
#pragma unroll
                for (int qq = 0; qq < QPB; ++qq) {
                    const int qb = hb * QPB + qq;
                    // lanes 32-63 read the quarter again (its k 8-15 repeat k 0-7);
                    // with RM = 2, rows 4q + i of the instruction's A take the
                    // wave's rows 4q + half_rows + (i & 1)
                    const int arow = (RM == 2) ? ((lane & 12) | half_rows | (lane & 1)) : (lane & 15);
                    const s4 a = *reinterpret_cast<const s4 *>(xp + st * XPW + (qb * BM + 16 * band + arow) * PW_ROW +
                                                               2 * pw_chunk(arow, (lane >> 4) & 1));
#pragma unroll
                    for (int j = 0; j < RN; ++j) {
                        const s4 b = *reinterpret_cast<const s4 *>(wp + st * WPW + (qb * BN + 16 * j + (lane & 15)) *
                                                                                     PW_ROW +
                                                                   2 * pw_chunk(lane & 15, (lane >> 4) & 1));
                        const f4 d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < RM; ++i) {
                            // RM = 2: results i and i + 2 are the same row; reading
                            // both leaves no result register unread while the
                            // instruction may still be writing it
                            const uint32_t v = (RM == 2) ? max(__float_as_uint(d[i]), __float_as_uint(d[i + 2]))
                                                         : __float_as_uint(d[i]);
                            smax[i][j] = qq ? max(smax[i][j], v) : v;
                        }
                    }
                }
                // block prologue: C and the truncated incoming accumulator
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < RN; ++j) {
                        const uint32_t eb = max((smax[i][j] >> 25) + POW_TO_EB, (c[i][j] >> 23) & 0xFFu);
                        uint32_t cb = (eb << 23) + C_OFFSET;
                        // later uses derive from C itself (measured slower in
                        // the hopper incoming-accumulator kernel: left out there)
                        if constexpr (!(CIN && BLK == 32)) asm("" : "+v"(cb));
                        Cb[i][j] = cb;
                        acc[i][j] = c_block_term(c[i][j], Cb[i][j], tok);
                        if constexpr (CIN) c[i][j] = cut14(c[i][j]);
                    }
            } else {
                // pass 1: E per output, from this lane's slice of the block
                uint32_t gmax[RM][RN];
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < RN; ++j) gmax[i][j] = 0u;
#pragma unroll(PASS_UNROLL)
                for (int wo = hb * WPB + lane_g * WPL; wo < hb * WPB + (lane_g + 1) * WPL; wo += WU) {
                    if constexpr (WU == 4) {
                        uint4 ea[RM], eb[RN];
                        if constexpr (LDS_PF) {
                            ea[0] = cur.ea;
                            eb[0] = cur.eb;
                        } else {
#pragma unroll
                            for (int i = 0; i < RM; ++i)
                                ea[i] = *reinterpret_cast<const uint4 *>(xe + (tm + i * TM) * PST +
                                                                         (wo ^ swz(tm + i * TM)));
#pragma unroll
                            for (int j = 0; j < RN; ++j)
                                eb[j] = *reinterpret_cast<const uint4 *>(we + (tn + j * TN) * PST +
                                                                         (wo ^ swz(tn + j * TN)));
                        }
#pragma unroll
                        for (int i = 0; i < RM; ++i)
#pragma unroll
                            for (int j = 0; j < RN; ++j) {
                                uint32_t g = gmax[i][j];
                                g = pk_max3_h(g, pk_add_u16(ea[i].x, eb[j].x), pk_add_u16(ea[i].y, eb[j].y));
                                g = pk_max3_h(g, pk_add_u16(ea[i].z, eb[j].z), pk_add_u16(ea[i].w, eb[j].w));
                                gmax[i][j] = g;
                            }
                    } else {
                        uint2 ea[RM], eb[RN];
#pragma unroll
                        for (int i = 0; i < RM; ++i)
                            ea[i] = *reinterpret_cast<const uint2 *>(xe + (tm + i * TM) * PST + wo);
#pragma unroll
                        for (int j = 0; j < RN; ++j)
                            eb[j] = *reinterpret_cast<const uint2 *>(we + (tn + j * TN) * PST + wo);
#pragma unroll
                        for (int i = 0; i < RM; ++i)
#pragma unroll
                            for (int j = 0; j < RN; ++j)
                                gmax[i][j] = pk_max3_h(gmax[i][j], pk_add_u16(ea[i].x, eb[j].x),
                                                       pk_add_u16(ea[i].y, eb[j].y));
                    }
                }

                // block prologue: C and the truncated incoming accumulator.
                // The maximum of this lane's two plane halves and c's
                // exponent (every lane of a chain carries the same c), then
                // over the G lanes of the chain; only its low 9 bits reach C.
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < RN; ++j) {
                        const uint32_t ec = ((c[i][j] >> 23) & 0xFFu) | SUM_OFFSET;
                        uint32_t e = max3_lo_hi_u16(gmax[i][j], ec);
                        if (G >= 2) e = quad_max_lo16<0xB1>(e);
                        if (G == 4) e = quad_max_lo16<0x4E>(e);
                        uint32_t cb = (e << 23) + C_OFFSET;
                        asm("" : "+v"(cb));  // later uses derive from C itself
                        Cb[i][j] = cb;
                        // c enters the block sum once
                        acc[i][j] = (G == 1) ? c_block_term(c[i][j], Cb[i][j], tok)
                                             : c_block_term_on(c[i][j], Cb[i][j], tok, c_lo, c_hi, Cb[i][j] & cb_on);
                        if constexpr (CIN) c[i][j] = cut14(c[i][j]);
                    }
            }

            // pass 2: truncated terms, signs, accumulation (small thread tiles
            // unroll the whole block: its LDS reads then take immediate
            // offsets from one address per plane, and the reads of later
            // steps can overlap earlier arithmetic at 1-2 waves per SIMD)
            uint4 sa4[SIGN16 ? RM : 1], sb4[SIGN16 ? RN : 1];
            // binary16 values: the lane's whole slice of the block (K4PL steps
            // of 4 codes, 2 words each) in one read per row
            uint4 ah4[SLICE16 ? RM : 1], bh4[SLICE16 ? RN : 1];
            if constexpr (LDS_PF) {
                ah4[0] = cur.ah;
                bh4[0] = cur.bh;
            } else if constexpr (SLICE16) {
                const int k40 = hb * (BLK / 4) + lane_g * K4PL;
                const uint32_t *xh = reinterpret_cast<const uint32_t *>(xa);
                const uint32_t *wh = reinterpret_cast<const uint32_t *>(wa);
#pragma unroll
                for (int i = 0; i < RM; ++i)
                    ah4[i] = load_half_slice<K4PL>(xh + row_of(i) * AHS + ((2 * k40) ^ swz(row_of(i))));
#pragma unroll
                for (int j = 0; j < RN; ++j)
                    bh4[j] = load_half_slice<K4PL>(wh + col_of(j) * AHS + ((2 * k40) ^ swz(col_of(j))));
            }
#pragma unroll(TERM_UNROLL)
            for (int u = 0; u < K4PL; ++u) {
                const int k4 = hb * (BLK / 4) + lane_g * K4PL + u;
                float4 av[V16 ? 1 : RM], bv[V16 ? 1 : RN];
                uint2 ah2[V16 && !SLICE16 ? RM : 1], bh2[V16 && !SLICE16 ? RN : 1];  // step u's binary16 values
                uint2 sa[RM], sb[RN];
#pragma unroll
                for (int i = 0; i < RM; ++i) {
                    if constexpr (!V16) av[i] = *reinterpret_cast<const float4 *>(xa + row_of(i) * A_STRIDE + 4 * k4);
                    if constexpr (V16 && !SLICE16)
                        ah2[i] = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint32_t *>(xa) +
                                                                  row_of(i) * AHS + 2 * k4);
                    if constexpr (SIGN16) {
                        if ((u & 1) == 0)
                            sa4[i] = LDS_PF ? cur.sa
                                            : *reinterpret_cast<const uint4 *>(xs + row_of(i) * SST +
                                                                               ((2 * k4) ^ swz(row_of(i))));
                        sa[i] = (u & 1) ? make_uint2(sa4[i].z, sa4[i].w) : make_uint2(sa4[i].x, sa4[i].y);
                    } else {
                        sa[i] = *reinterpret_cast<const uint2 *>(xs + row_of(i) * SST + 2 * k4);
                    }
                }
#pragma unroll
                for (int j = 0; j < RN; ++j) {
                    if constexpr (!V16) bv[j] = *reinterpret_cast<const float4 *>(wa + col_of(j) * A_STRIDE + 4 * k4);
                    if constexpr (V16 && !SLICE16)
                        bh2[j] = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint32_t *>(wa) +
                                                                  col_of(j) * AHS + 2 * k4);
                    if constexpr (SIGN16) {
                        if ((u & 1) == 0)
                            sb4[j] = LDS_PF ? cur.sb
                                            : *reinterpret_cast<const uint4 *>(wsg + col_of(j) * SST +
                                                                               ((2 * k4) ^ swz(col_of(j))));
                        sb[j] = (u & 1) ? make_uint2(sb4[j].z, sb4[j].w) : make_uint2(sb4[j].x, sb4[j].y);
                    } else {
                        sb[j] = *reinterpret_cast<const uint2 *>(wsg + col_of(j) * SST + 2 * k4);
                    }
                }
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < RN; ++j) {
                        const uint32_t C = Cb[i][j];
                        uint32_t r0, r1, r2, r3;
                        if constexpr (V16) {
                            // step u's codes 0-1 and 2-3 as low / high halves
                            uint32_t x0, x1, y0, y1;
                            if constexpr (SLICE16) {
                                x0 = (u & 1) ? ah4[i].z : ah4[i].x;
                                x1 = (u & 1) ? ah4[i].w : ah4[i].y;
                                y0 = (u & 1) ? bh4[j].z : bh4[j].x;
                                y1 = (u & 1) ? bh4[j].w : bh4[j].y;
                            } else {
                                x0 = ah2[i].x;
                                x1 = ah2[i].y;
                                y0 = bh2[j].x;
                                y1 = bh2[j].y;
                            }
                            r0 = fma_abs_rz_lo16(x0, y0, C, tok);
                            r1 = fma_abs_rz_hi16(x0, y0, C, tok);
                            r2 = fma_abs_rz_lo16(x1, y1, C, tok);
                            r3 = fma_abs_rz_hi16(x1, y1, C, tok);
                        } else {
                            r0 = fma_abs_rz(av[i].x, bv[j].x, C, tok);
                            r1 = fma_abs_rz(av[i].y, bv[j].y, C, tok);
                            r2 = fma_abs_rz(av[i].z, bv[j].z, C, tok);
                            r3 = fma_abs_rz(av[i].w, bv[j].w, C, tok);
                        }
                        int a = acc[i][j];
                        a = dot2_i16(__builtin_amdgcn_perm(r1, r0, 0x05040100u), sign_pair(sa[i].x, sb[j].x), a);
                        a = dot2_i16(__builtin_amdgcn_perm(r3, r2, 0x05040100u), sign_pair(sa[i].y, sb[j].y), a);
                        acc[i][j] = a;
                    }
                if constexpr (STEP_FENCE) __builtin_amdgcn_sched_barrier(0);
            }

            if (G >= 2) {
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < RN; ++j) {
                        int a = quad_add<0xB1>(acc[i][j]);
                        if (G == 4) a = quad_add<0x4E>(a);
                        acc[i][j] = a;
                    }
            }

            // block epilogue: the exact sum scaled by 2^q (then cut to 14
            // significant bits where c must stay cut after every block)
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < RN; ++j) {
                    uint32_t cn = sub_block_base((uint32_t)acc[i][j], Cb[i][j], tok);
                    if constexpr (CUT_EACH_BLOCK) cn = cut14(cn);
                    if constexpr (CIN) {
                        // c (cut to 14 significant bits by the prologue) stays when
                        // the block exponent, biased, is below 94 -- no products
                        // (their plane sentinels sit at 93 and below) and c under
                        // 2^-33, where those sentinels would cut it wrongly -- or
                        // 166 and above -- c >= 2^39, whose quantum 2^(E-13)
                        // exceeds every product (< 2^25), and where C =
                        // 1.5 * 2^(E+10) would leave the binary32 range: in both
                        // cases the block step leaves c cut to 14 significant bits
                        // biased E in [94, 166) <=> Cb's top bits in [104, 176)
                        c[i][j] = (Cb[i][j] - (104u << 23) < (72u << 23)) ? cn : c[i][j];
                    } else {
                        c[i][j] = cn;
                    }
                }
        }

        // slow accumulation: every 128 positions of the split's k-list the
        // chunk result is added to the running sum, in order, or stored as a
        // partial for the combine kernel to add
        const bool chunk_end = ((spos + KB) & (CHUNK - 1)) == 0 || spos + KB >= pos_end;
        if (CHUNKS && chunk_end) {
            const int64_t part = (int64_t)split * p.cps + spos / CHUNK;
            uint32_t *o = reinterpret_cast<uint32_t *>(p.out) + part * p.split_stride;
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < RN; ++j) {
                    const int64_t m = m0 + row_of(i), n = n0 + col_of(j);
                    if (m < p.M && n < p.N && lane_g == 0) o[m * p.ldo + n] = cut14(c[i][j]);
                    c[i][j] = 0u;
                }
        } else if (RUNNING && chunk_end) {
            uint32_t dep = 0;
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < RN; ++j) dep |= c[i][j];
            const uint32_t tok_rn = mode_round_nearest_after(dep);
            uint32_t dep2 = 0;
#pragma unroll
            for (int i = 0; i < (RUNNING ? RM : 1); ++i)
#pragma unroll
                for (int j = 0; j < (RUNNING ? RN : 1); ++j) {
                    slow[i][j] = add_rn(slow[i][j], cut14(c[i][j]), tok_rn);
                    dep2 |= slow[i][j];
                    c[i][j] = 0u;
                }
            tok = mode_round_toward_zero_after(dep2);
        }
        // With 2 lanes per chain each stage stays a scheduling region of its
        // own: merged, the compiler's early LDS reads spill registers at this
        // tile's 4 waves per SIMD (measured 25% slower).
        if constexpr (G == 2) __builtin_amdgcn_sched_barrier(0);
        }  // stages
    }

    // rows holding NaN / Inf codes in this split's k-list (special_flags bits)
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
        const int idx = t + q * NT;
        if (idx < NCHUNK * SS && myflag[q]) {
            atomicOr(&flags[chunk_rowidx(idx)], myflag[q]);
            if (CHUNKS) atomicOr(&flags[BM + BN], myflag[q]);
        }
    }
    __syncthreads();

    if constexpr (CHUNKS) {
        // chunk partials: +0 for this group's chunks past the k-list; rows
        // with NaN / Inf codes overwrite the chunks that hold them
        const int c_lo = group * p.chunks_per_group;
        const int c_hi = (c_lo + p.chunks_per_group < p.cps) ? c_lo + p.chunks_per_group : p.cps;
        if ((int64_t)(c_hi - 1) * CHUNK < sq.len && !flags[BM + BN]) return;  // uniform: nothing to overwrite
#pragma unroll
        for (int i = 0; i < RM; ++i)
#pragma unroll
            for (int j = 0; j < RN; ++j) {
                const int rm = row_of(i), rn = col_of(j);
                const int64_t m = m0 + rm, n = n0 + rn;
                if (m >= p.M || n >= p.N || lane_g != 0) continue;
                const uint32_t f = flags[rm] | flags[BM + rn];
                for (int ch = c_lo; ch < c_hi; ++ch) {
                    uint32_t *o = reinterpret_cast<uint32_t *>(p.out) + ((int64_t)split * p.cps + ch) * p.split_stride;
                    const int64_t cs = (int64_t)ch * CHUNK;
                    if (cs >= sq.len) {
                        o[m * p.ldo + n] = 0u;
                    } else if (f) {
                        const int64_t ce = (cs + CHUNK < sq.len) ? cs + CHUNK : sq.len;
                        const uint32_t v = special_scan<XF, WF>(p.x + m * p.ldx, p.w + n * p.ldw, sq, cs, ce,
                                                                flags[rm] != 0, flags[BM + rn] != 0);
                        if (v) o[m * p.ldo + n] = v;
                    }
                }
            }
        return;
    }

    uint32_t alpha = 0, sr = 0x3F800000u;  // the scales are read only when the epilogue runs here
    if (p.out_kind != OUT_ACC_F32) {
        alpha = mul_f32(__float_as_uint(*p.scale_x), __float_as_uint(*p.scale_w));
        sr = scale_result_bits(p.scale_result);
    }
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) {
            const int rm = row_of(i), rn = col_of(j);
            const int64_t m = m0 + rm, n = n0 + rn;
            if (m >= p.M || n >= p.N || lane_g != 0) continue;
            uint32_t a = FAST ? (CUT_EACH_BLOCK ? c[i][j] : cut14_at_exit(c[i][j]))
                              : slow[RUNNING ? i : 0][RUNNING ? j : 0];
            const uint32_t f = flags[rm] | flags[BM + rn];
            if (f & 2u) a = kCanonNan32;  // a NaN code in either row wins
            else if (f && !p.defer_specials)  // infinities (or left to the fix-up kernel)
                a = special_scan<XF, WF>(p.x + m * p.ldx, p.w + n * p.ldw, sq, 0, sq.len, flags[rm] != 0,
                                         flags[BM + rn] != 0);
            if constexpr (CIN) {
                if (a == 0x80000000u && p.K > 0) a = 0u;  // a zero block result is +0
                // a NaN c_in gives NaN; an infinite one stays, unless the
                // products give NaN or the opposite infinity
                const uint32_t cb = __float_as_uint(p.c_in[m * p.ldc + n]);
                if (((cb >> 23) & 0xFFu) == 0xFFu) {
                    if (cb & 0x7FFFFFu) a = kCanonNan32;
                    else if (f && (a == kCanonNan32 || ((a >> 23) & 0xFFu) == 0xFFu) && a != cb) a = kCanonNan32;
                    else a = cb;
                }
            }
            store_output(p, m, n, a, alpha, sr, split);
        }
}

template <int XF, int WF, int BM, int BN, int RM, int RN, int G, bool MX, int BLK, int SS = 1>
hipError_t launch_cfg(const MainParams &p, int S, hipStream_t stream)
{
    constexpr int NT = (BM / RM) * (BN / RN) * G;
    dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM, S);
    if (p.fast)
        hipLaunchKernelGGL((main_kernel<XF, WF, BM, BN, RM, RN, G, ACC_FAST, MX, BLK, SS>), grid, dim3(NT), 0, stream,
                           p);
    else if (p.chunked)
        hipLaunchKernelGGL((main_kernel<XF, WF, BM, BN, RM, RN, G, ACC_SLOW_CHUNKS, MX, BLK, SS>), grid, dim3(NT), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((main_kernel<XF, WF, BM, BN, RM, RN, G, ACC_SLOW, MX, BLK, SS>), grid, dim3(NT), 0, stream,
                           p);
    return hipGetLastError();
}

// Stages per barrier for the 16x8 tile with 4 lanes per output.  Longer
// rounds halve the barrier rounds of long k-lists (16 x 256 x 65536 with 8
// splits: 16 stages 0.0858 against 0.0923 ms for 8, A/B in one session), but
// in fast accumulation every stage of the last round is computed, so the
// host counts one round as its stages plus about 1.3 stages of barrier and
// decode overhead (from that measurement) and takes the round that costs
// least for the longest split, the shorter on a tie.  32 stages fit the LDS
// (144 KB) with 32-product blocks only, and there they also even out the
// decode: 1,536 chunks per round, three for each of the 512 threads (16
// stages give half of them two and the other half one).
inline int g4_stages(const MainParams &p, int max_ss)
{
    const int64_t W = int64_t(1) << p.tile_shift;
    const int64_t nt = (p.K + W - 1) >> p.tile_shift;
    const int64_t tiles = p.round_robin ? (nt + p.S - 1) / p.S : p.tps;
    const int64_t len = (tiles * W < p.K) ? tiles * W : p.K;
    const int64_t stages = (len + KB - 1) / KB;
    int best = 8;
    int64_t best_cost = ((stages + 7) / 8) * (3 * 8 + 4);
    for (int ss = 16; ss <= max_ss; ss *= 2) {
        const int64_t cost = ((stages + ss - 1) / ss) * (3 * ss + 4);
        if (cost < best_cost) {
            best = ss;
            best_cost = cost;
        }
    }
    return best;
}

template <int XF, int WF, int BLK>
hipError_t launch_fmt(int cfg, const MainParams &p, int S, hipStream_t stream)
{
    switch (cfg) {
    case TILE_64x128: return launch_cfg<XF, WF, 64, 128, 4, 8, 1, false, BLK>(p, S, stream);
    case TILE_64x64: return launch_cfg<XF, WF, 64, 64, 4, 4, 1, false, BLK>(p, S, stream);
    case TILE_32x64: return launch_cfg<XF, WF, 32, 64, 2, 4, 1, false, BLK>(p, S, stream);
    case TILE_32x32: return launch_cfg<XF, WF, 32, 32, 2, 2, 1, false, BLK, 2>(p, S, stream);
    case TILE_16x16_G2: return launch_cfg<XF, WF, 16, 16, 1, 1, 2, false, BLK, 8>(p, S, stream);
    case TILE_16x16_G4: return launch_cfg<XF, WF, 16, 16, 1, 1, 4, false, BLK, 8>(p, S, stream);
    case TILE_64x64_MX: return launch_cfg<XF, WF, 64, 64, 4, 4, 1, true, BLK>(p, S, stream);
    case TILE_64x128_MX: return launch_cfg<XF, WF, 64, 128, 4, 8, 1, true, BLK>(p, S, stream);
    case TILE_16x8_G4:
        if constexpr (BLK == 32)
            if (g4_stages(p, 32) == 32) return launch_cfg<XF, WF, 16, 8, 1, 1, 4, false, BLK, 32>(p, S, stream);
        return g4_stages(p, 16) == 16 ? launch_cfg<XF, WF, 16, 8, 1, 1, 4, false, BLK, 16>(p, S, stream)
                                      : launch_cfg<XF, WF, 16, 8, 1, 1, 4, false, BLK, 8>(p, S, stream);
    case TILE_16x64_MX: return launch_cfg<XF, WF, 16, 64, 4, 4, 1, true, BLK>(p, S, stream);
    case TILE_32x32_S4: return launch_cfg<XF, WF, 32, 32, 2, 2, 1, false, BLK, 4>(p, S, stream);
    case TILE_32x32_MX_S4: return launch_cfg<XF, WF, 32, 32, 2, 2, 1, true, BLK, 4>(p, S, stream);
    case TILE_32x16_MX_S5: return launch_cfg<XF, WF, 32, 16, 2, 1, 1, true, BLK, 5>(p, S, stream);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

// All tile configurations of one block width and format pair.
template <int BLK, int XF, int WF>
hipError_t launch_variant(int cfg, const MainParams &p, int S, hipStream_t stream)
{
    return launch_fmt<XF, WF, BLK>(cfg, p, S, stream);
}

// Fast accumulation from incoming accumulators (ACC_FAST_CIN), every tile
// configuration; instantiated in a translation unit of its own
// (emu_cin_variant.hip), apart from the other main-kernel instantiations.
template <int XF, int WF, int BM, int BN, int RM, int RN, int G, bool MX, int BLK, int SS = 1>
hipError_t launch_cin_cfg(const MainParams &p, hipStream_t stream)
{
    constexpr int NT = (BM / RM) * (BN / RN) * G;
    dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM, 1);
    hipLaunchKernelGGL((main_kernel<XF, WF, BM, BN, RM, RN, G, ACC_FAST_CIN, MX, BLK, SS>), grid, dim3(NT), 0, stream,
                       p);
    return hipGetLastError();
}

template <int BLK, int XF, int WF>
hipError_t launch_variant_cin(int cfg, const MainParams &p, hipStream_t stream)
{
    switch (cfg) {
    case TILE_64x128: return launch_cin_cfg<XF, WF, 64, 128, 4, 8, 1, false, BLK>(p, stream);
    case TILE_64x64: return launch_cin_cfg<XF, WF, 64, 64, 4, 4, 1, false, BLK>(p, stream);
    case TILE_32x64: return launch_cin_cfg<XF, WF, 32, 64, 2, 4, 1, false, BLK>(p, stream);
    case TILE_32x32: return launch_cin_cfg<XF, WF, 32, 32, 2, 2, 1, false, BLK, 2>(p, stream);
    case TILE_16x16_G2: return launch_cin_cfg<XF, WF, 16, 16, 1, 1, 2, false, BLK, 8>(p, stream);
    case TILE_16x16_G4: return launch_cin_cfg<XF, WF, 16, 16, 1, 1, 4, false, BLK, 8>(p, stream);
    case TILE_64x64_MX: return launch_cin_cfg<XF, WF, 64, 64, 4, 4, 1, true, BLK>(p, stream);
    case TILE_64x128_MX: return launch_cin_cfg<XF, WF, 64, 128, 4, 8, 1, true, BLK>(p, stream);
    case TILE_16x8_G4:
        return g4_stages(p, 16) == 16 ? launch_cin_cfg<XF, WF, 16, 8, 1, 1, 4, false, BLK, 16>(p, stream)
                                      : launch_cin_cfg<XF, WF, 16, 8, 1, 1, 4, false, BLK, 8>(p, stream);
    case TILE_16x64_MX: return launch_cin_cfg<XF, WF, 16, 64, 4, 4, 1, true, BLK>(p, stream);
    case TILE_32x32_S4: return launch_cin_cfg<XF, WF, 32, 32, 2, 2, 1, false, BLK, 4>(p, stream);
    case TILE_32x32_MX_S4: return launch_cin_cfg<XF, WF, 32, 32, 2, 2, 1, true, BLK, 4>(p, stream);
    case TILE_32x16_MX_S5: return launch_cin_cfg<XF, WF, 32, 16, 2, 1, 1, true, BLK, 5>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace emu
