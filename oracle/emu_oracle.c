/*
 * emu_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU implementation of the emulated FP8 scaled GEMM
 *     y = (x @ w.T) * scale_x * scale_w
 * as the mmaemu v0.1 documentation pages describe it (user guide, FAQ,
 * limitations, validation evidence).  Only the test suite, the package smoke
 * check and the benchmark's cpu_baseline leg load this file's library.  It
 * shares no code, header, table or constant with the HIP library, and it
 * includes nothing from it.
 *
 * Arithmetic.  Every product and every block sum is an exact int64 integer
 * with an explicit power-of-two exponent.  The only floating-point steps are
 * the IEEE binary32 additions the pages name (slow-accumulation chunk adds and
 * the split-K combination), done with the host's IEEE arithmetic
 * (x86-64 SSE: round to nearest even, subnormals kept), and the epilogue's
 * roundings, which are written out below from the IEEE 754 definition of
 * round-to-nearest-even on an exact value.
 *
 * Readings taken where the pages are silent are marked "Reading:" and are
 * listed in the design notes of the repository.
 *
 * Parity unpinned (nothing on the pages fixes these, so no test can pin
 * them to more than this file's own reading): the canonical NaN bits of
 * binary32, binary16 and bfloat16 outputs (0x7FFFFFFF, 0x7FFF) and of FP8
 * outputs (0x7F); the pairwise split combination for S >= 4 (the pages fix
 * only S = 3; the stride-halving tree is taken); the alignment of a
 * subnormal incoming accumulator at binary32's emin.  The infinity and NaN
 * outcomes of products and incoming accumulators follow IEEE arithmetic,
 * which the tests pin, not the pages.  No result here is pinned to
 * recordings of the reference hardware.
 *
 * Mutants.  Building with -DORACLE_MUTANT=n (n > 0) plants one deliberate
 * mistake, so that the tests can show that their pins catch it.  The default
 * build (ORACLE_MUTANT 0) is the oracle.
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs binary32 arithmetic evaluated in binary32 (FLT_EVAL_METHOD 0)"
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* Mutant catalogue (see tests/test_oracle_mutants.py). */
#define MUT_FLOOR_NOT_TRUNC    1  /* floor of signed terms instead of truncation toward zero */
#define MUT_F12                2  /* 12 retained fraction bits instead of 13 */
#define MUT_F14                3  /* 14 retained fraction bits instead of 13 */
#define MUT_B16                4  /* 16-product blocks instead of 32 */
#define MUT_C_NOT_IN_MAX       5  /* incoming accumulator left out of the block maximum */
#define MUT_NORMALISED_EXP     6  /* product exponent floor(log2|p|) instead of the field sum */
#define MUT_NEG_ZERO_BLOCK     7  /* a block that sums to zero keeps the sign of the terms */
#define MUT_CHUNK64            8  /* slow chunks of 64 positions instead of 128 */
#define MUT_REVERSED_COMBINE   9  /* split partials added in reverse order */
#define MUT_SINGLE_ROUNDING   10  /* bf16/fp16 rounded straight from the exact product */
#define MUT_MUL_NOT_FMA       11  /* y32 = RN32(acc*alpha) keeping the product's zero sign */
#define MUT_NO_BLOCKSUM_TRUNC 12  /* block sum not cut back to 1+F significant bits */
#define MUT_SUBNORMAL_EXP     13  /* subnormal inputs take exponent emin-1 instead of emin */
#define MUT_SLOW_NO_RESTART   14  /* slow accumulation keeps chaining across chunks */
#define MUT_SPLIT_BALANCED    15  /* k-tiles divided floor/remainder instead of ceil-contiguous */
#define MUT_CANON_NAN         16  /* NaN output 0x7FC00000 / 0x7FC0 instead of 0x7FFFFFFF / 0x7FFF */
#define MUT_TRANSPOSED_W      17  /* w read as [K,N] row-major instead of [N,K] */
#define MUT_RR_AS_CONTIGUOUS  18  /* round-robin split layout taken as contiguous runs */
#define MUT_PAIRWISE_ADJACENT 19  /* pairwise combination over adjacent pairs, ((p0+p1)+p2)... */
#define MUT_RR_TILE_DOUBLED   20  /* round-robin k-tiles twice as wide as the profile's */
#define MUT_SR_FOLDED         21  /* scale_result folded into alpha instead of a separate multiply */
#define MUT_FP8_NO_SATURATION 22  /* FP8 outputs overflow to NaN / Inf instead of saturating */
#define MUT_C_OWN_EXPONENT    23  /* a binary32 subnormal c aligned at floor(log2|c|), not emin */
#define MUT_INF_TIMES_ZERO    24  /* an infinity times a zero taken as that infinity, not NaN */
#define MUT_INF_FIRST_SIGN    25  /* infinite products of both signs give the first one's sign */
#define MUT_C_INF_ABSORBS     26  /* an infinite c_in stays even against the opposite infinity */

/* ------------------------------------------------------------------------ */
/* Public constants (mirrored in oracle/__init__.py).                        */
enum { FMT_E4M3FN = 0, FMT_E5M2 = 1 };
enum { OUT_BF16 = 0, OUT_FP16 = 1, OUT_FP32 = 2, OUT_E4M3FN = 3, OUT_E5M2 = 4 };
enum { CLS_ZERO = 0, CLS_FINITE = 1, CLS_INF = 2, CLS_NAN = 3 };

enum { LAYOUT_CONTIGUOUS = 0, LAYOUT_ROUND_ROBIN = 1 };
enum { COMBINE_SERIAL = 0, COMBINE_PAIRWISE = 1 };

typedef struct {
    int B;        /* products per block */
    int F;        /* retained fraction bits */
    int Q;        /* slow-accumulation chunk length */
    int W;        /* split-K tile width */
    int layout;   /* LAYOUT_*: how the k-tiles are divided among the splits */
    int combine;  /* COMBINE_*: how the split partials are added */
} oracle_profile;

/* ------------------------------------------------------------------------ */
/* FP8 decoding.
 *
 * The two formats are the OCP 8-bit formats that torch calls float8_e4m3fn
 * and float8_e5m2 (user guide, section 3 "A first GEMM": E4M3 inputs clamped
 * to +-448; validation page, "Claims and their recordings": E4M3 x E5M2 and
 * E5M2 x E4M3 follow the same model).
 *
 * A finite code decodes to (-1)^s * M * 2^(e-3) with M an integer holding
 * three fraction bits.  For a subnormal code the exponent is the format's
 * emin, not the exponent of the leading bit (validation page, claims
 * table, row on subnormal inputs).  E5M2 has two
 * fraction bits; its M is doubled so both formats share the 2^(e-3) scale.
 */
typedef struct {
    int cls;  /* CLS_* */
    int s;    /* sign bit */
    int e;    /* field exponent (emin for subnormals) */
    int M;    /* integer significand with 3 fraction bits */
} fp8_val;

static fp8_val decode_fp8(uint8_t code, int fmt)
{
    fp8_val v;
    v.s = code >> 7;
    if (fmt == FMT_E4M3FN) {
        int ef = (code >> 3) & 15, mf = code & 7;
        if (ef == 15 && mf == 7) { v.cls = CLS_NAN; v.e = 0; v.M = 0; return v; }
        if (ef == 0) {
#if ORACLE_MUTANT == MUT_SUBNORMAL_EXP
            v.e = -7;
#else
            v.e = -6;  /* emin of E4M3 = 1 - bias 7 */
#endif
            v.M = mf;
        } else {
            v.e = ef - 7;
            v.M = 8 + mf;
        }
    } else {
        int ef = (code >> 2) & 31, mf = code & 3;
        if (ef == 31) { v.cls = (mf == 0) ? CLS_INF : CLS_NAN; v.e = 0; v.M = 0; return v; }
        if (ef == 0) {
#if ORACLE_MUTANT == MUT_SUBNORMAL_EXP
            v.e = -15;
#else
            v.e = -14;  /* emin of E5M2 = 1 - bias 15 */
#endif
            v.M = 2 * mf;
        } else {
            v.e = ef - 15;
            v.M = 2 * (4 + mf);
        }
    }
    v.cls = (v.M == 0) ? CLS_ZERO : CLS_FINITE;
    return v;
}

/* ------------------------------------------------------------------------ */
/* Products.
 *
 * A product of two finite nonzero inputs is exact: (-1)^s * P * 2^(g-6) with
 * P = Ma*Mb (at most 225) and g = ea + eb, the sum of the field exponents.
 * Reading: the alignment exponent of a product is this field sum, the product
 * is never renormalised (the claims table's row on subnormal inputs, which
 * places them at emin, only has content if the exponents come from the
 * fields).  A product with a zero factor is a zero product: it takes no part
 * in the block maximum (validation page, claims table, first row) and
 * contributes nothing.
 */
typedef struct {
    int cls;  /* CLS_ZERO or CLS_FINITE (specials are handled separately) */
    int s;
    int g;
    int P;
} product;

static int floor_log2_u64(uint64_t v)
{
    int l = -1;
    while (v) { v >>= 1; l++; }
    return l;
}

static product make_product(fp8_val a, fp8_val b)
{
    product p;
    p.s = a.s ^ b.s;
    if (a.cls != CLS_FINITE || b.cls != CLS_FINITE) {
        p.cls = CLS_ZERO; p.g = 0; p.P = 0;
        return p;
    }
    p.cls = CLS_FINITE;
    p.P = a.M * b.M;
    p.g = a.e + b.e;
#if ORACLE_MUTANT == MUT_NORMALISED_EXP
    /* exponent of the exact product's leading bit */
    p.g = floor_log2_u64((uint64_t)p.P) - 6 + p.g;
#endif
    return p;
}

/* ------------------------------------------------------------------------ */
/* Exact chain state: (-1)^neg * mag * 2^q; mag == 0 means +0. */
typedef struct {
    int neg;
    int64_t mag;
    int q;
} exact_val;

static const exact_val EXACT_PLUS_ZERO = {0, 0, 0};

/* floor(m * 2^sh) for m >= 0; callers keep m << sh below 2^62. */
static int64_t scale_floor(int64_t m, int sh)
{
    if (sh >= 0) return m << sh;
    if (-sh >= 63) return 0;
    return m >> (-sh);
}

/*
 * One block step, step(c, products) (user guide section 1; FAQ first answer;
 * validation page, scope table row "Hopper preset" and the H100 claims table
 * row on 32-product blocks and 13 fraction bits):
 *
 *  1. E is the largest alignment exponent among the nonzero products, and,
 *     when the incoming accumulator c is nonzero, its exponent ("c enters in
 *     the block's alignment"): floor(log2|c|), or binary32's emin -126 for a
 *     subnormal c.  Reading: the pages fix emin for subnormal FP8 inputs
 *     only; a binary32 c is taken the same way (an incoming c below 2^-126
 *     only arises from a caller's accumulator input).  With nothing nonzero
 *     the block gives +0.
 *  2. The quantum is 2^q with q = E - F: every term keeps F fraction bits
 *     relative to 2^E.
 *  3. Each term, and c, is cut to that quantum toward zero, on the
 *     magnitude with the sign kept apart (claims table, truncation row).
 *  4. The terms are added exactly.  A sum that is exactly zero gives +0
 *     (scope table row "Ada instruction model": zero block results, exact
 *     or after truncation, are positive zero).
 *  5. The sum is cut toward zero to 1+F significant bits (claims table,
 *     truncation row: the block sum keeps 13 fraction bits; the carry case).
 */
static exact_val block_step(exact_val c, const product *p, int n, int F)
{
    int have = 0, E = 0;
    for (int i = 0; i < n; i++) {
        if (p[i].cls != CLS_FINITE) continue;
        if (!have || p[i].g > E) E = p[i].g;
        have = 1;
    }
#if ORACLE_MUTANT != MUT_C_NOT_IN_MAX
    if (c.mag != 0) {
        int ec = c.q + floor_log2_u64((uint64_t)c.mag);
#if ORACLE_MUTANT != MUT_C_OWN_EXPONENT
        if (ec < -126) ec = -126;
#endif
        if (!have || ec > E) E = ec;
        have = 1;
    }
#else
    if (!have && c.mag != 0) {
        E = c.q + floor_log2_u64((uint64_t)c.mag);
        have = 1;
    }
#endif
    if (!have) return EXACT_PLUS_ZERO;

    const int q = E - F;
    int64_t T = 0;
    for (int i = 0; i < n; i++) {
        if (p[i].cls != CLS_FINITE) continue;
        /* |term| = P * 2^(g-6), measured in units of 2^q */
        int64_t t = scale_floor(p[i].P, p[i].g - 6 - q);
#if ORACLE_MUTANT == MUT_FLOOR_NOT_TRUNC
        if (p[i].s) {
            /* floor(-x) = -ceil(x) */
            int sh = p[i].g - 6 - q;
            int64_t exact_num = p[i].P;
            int inexact = (sh < 0) && ((-sh >= 63) ? (exact_num != 0)
                                                     : ((exact_num & (((int64_t)1 << -sh) - 1)) != 0));
            t += inexact;
        }
#endif
        T += p[i].s ? -t : t;
    }
    if (c.mag != 0) {
#if ORACLE_MUTANT == MUT_C_NOT_IN_MAX
        /* c taken at the block's quantum even when it does not fit */
        int sh = c.q - q;
        int64_t tc = (sh > 40) ? ((int64_t)1 << 60) : scale_floor(c.mag, sh);
#else
        int64_t tc = scale_floor(c.mag, c.q - q);
#endif
        T += c.neg ? -tc : tc;
    }
    if (T == 0) {
#if ORACLE_MUTANT == MUT_NEG_ZERO_BLOCK
        exact_val z = {0, 0, 0};
        for (int i = 0; i < n; i++)
            if (p[i].cls == CLS_FINITE) { z.neg = p[i].s; break; }
        return z;
#else
        return EXACT_PLUS_ZERO;
#endif
    }
    exact_val r;
    r.neg = T < 0;
    uint64_t mag = (uint64_t)(T < 0 ? -T : T);
#if ORACLE_MUTANT != MUT_NO_BLOCKSUM_TRUNC
    int L = floor_log2_u64(mag);
    if (L > F) mag = (mag >> (L - F)) << (L - F);
#endif
    r.mag = (int64_t)mag;
    r.q = q;
    return r;
}

/* ------------------------------------------------------------------------ */
/* Operand access. */
typedef struct {
    const uint8_t *x; int xfmt; int64_t ldx;
    const uint8_t *w; int wfmt; int64_t ldw;
    int64_t M, N, K;
} operands;

static uint8_t x_at(const operands *o, int64_t m, int64_t k) { return o->x[m * o->ldx + k]; }
static uint8_t w_at(const operands *o, int64_t n, int64_t k)
{
#if ORACLE_MUTANT == MUT_TRANSPOSED_W
    return o->w[k * o->ldw + n];
#else
    return o->w[n * o->ldw + k];
#endif
}

static int effective_B(const oracle_profile *pf)
{
#if ORACLE_MUTANT == MUT_B16
    (void)pf;
    return 16;
#else
    return pf->B;
#endif
}

static int effective_F(const oracle_profile *pf)
{
#if ORACLE_MUTANT == MUT_F12
    (void)pf;
    return 12;
#elif ORACLE_MUTANT == MUT_F14
    (void)pf;
    return 14;
#else
    return pf->F;
#endif
}

#define MAX_B 1024

/*
 * The ordered k-list of one split.  Round-robin: k-tiles of width W, tile
 * first, first + stride, ..., ntiles of them, each clipped to K; position p
 * of the sequence is k = (first + (p / W) * stride) * W + p % W (only the last
 * tile of a sequence can be short: it is the last tile of K).  Contiguous:
 * stride 0 marks the plain range [first, first + len).
 */
typedef struct {
    int64_t first, stride, ntiles, W;
    int64_t len;  /* number of k in the sequence */
} kseq;

static kseq kseq_range(int64_t k0, int64_t k1)
{
    kseq q = {k0, 0, 1, 1, k1 > k0 ? k1 - k0 : 0};
    return q;
}

static int64_t kseq_at(const kseq *q, int64_t pos)
{
    if (q->stride == 0) return q->first + pos;  /* contiguous range */
    return (q->first + (pos / q->W) * q->stride) * q->W + pos % q->W;
}

/*
 * chain(kappa): c <- +0, then c <- step(c, group) for each consecutive group
 * of B positions of the sequence in [p0, p1).  The last group may be short,
 * which is the same as padding with zero products (zeros are excluded from
 * the maximum).  Reading: blocks start at the start of each split's sequence
 * or chunk.
 */
static exact_val chain_exact(const operands *o, int64_t m, int64_t n, const kseq *ks, int64_t p0,
                             int64_t p1, const oracle_profile *pf, exact_val c)
{
    const int B = effective_B(pf), F = effective_F(pf);
    product buf[MAX_B];
    for (int64_t pb = p0; pb < p1; pb += B) {
        int cnt = 0;
        for (int64_t pos = pb; pos < p1 && pos < pb + B; pos++) {
            const int64_t k = kseq_at(ks, pos);
            buf[cnt++] = make_product(decode_fp8(x_at(o, m, k), o->xfmt),
                                      decode_fp8(w_at(o, n, k), o->wfmt));
        }
        c = block_step(c, buf, cnt, F);
    }
    return c;
}

/* (-1)^neg * mag * 2^q as binary32.  Exact whenever mag has at most 24
 * significant bits and the value is in the normal range, which holds for every
 * chain value with F <= 23. */
static float exact_to_f32(exact_val v)
{
    if (v.mag == 0) return v.neg ? -0.0f : 0.0f;  /* the oracle itself only makes +0 */
    float f = ldexpf((float)v.mag, v.q);
    return v.neg ? -f : f;
}

/*
 * Slow accumulation (validation page, H100 claims table, slow-accumulation
 * row: a new chain starts at every 128th position and the chunk results are
 * summed first to last; scope table row "Slow accumulation": per split when
 * split).
 * Reading: the adder is binary32 round-to-nearest-even and the running sum
 * starts at +0; chunks start at the start of the (split) range.
 */
static float slow_range(const operands *o, int64_t m, int64_t n, const kseq *ks, const oracle_profile *pf)
{
#if ORACLE_MUTANT == MUT_CHUNK64
    const int64_t Q = 64;
#else
    const int64_t Q = pf->Q;
#endif
#if ORACLE_MUTANT == MUT_SLOW_NO_RESTART
    (void)Q;
    return exact_to_f32(chain_exact(o, m, n, ks, 0, ks->len, pf, EXACT_PLUS_ZERO));
#else
    float a = 0.0f;
    for (int64_t cp = 0; cp < ks->len; cp += Q) {
        int64_t ce = (cp + Q < ks->len) ? cp + Q : ks->len;
        float r = exact_to_f32(chain_exact(o, m, n, ks, cp, ce, pf, EXACT_PLUS_ZERO));
        a = a + r;
    }
    return a;
#endif
}

/*
 * Split-K on the H100 PCIe profiles (validation page, scope table row
 * "Split-K on the H100 PCIe"; H100 claims table): contiguous runs of 128-wide
 * k-tiles, partial sums added serially; a split can hold no k-tile.
 * Reading: nt = ceil(K/W) tiles, tps = ceil(nt/S) tiles per split, split s
 * covers [s*tps*W, min((s+1)*tps*W, K)); an empty split gives +0.
 *
 * Split-K on the RTX 4060 profiles (limitations page, corrections table;
 * validation page, scope table row "Split-K" and claims table): 64-wide
 * k-tiles are dealt to the splits in turn, so split s owns tiles s, s+S,
 * s+2S, ... in that order, and its chain (and, for slow accumulation, its
 * chunking) runs along that sequence.
 */
static kseq split_seq(int64_t K, int S, const oracle_profile *pf, int s)
{
    int64_t W = pf->W;
    int layout = pf->layout;
#if ORACLE_MUTANT == MUT_RR_AS_CONTIGUOUS
    layout = LAYOUT_CONTIGUOUS;
#endif
#if ORACLE_MUTANT == MUT_RR_TILE_DOUBLED
    if (layout == LAYOUT_ROUND_ROBIN) W *= 2;
#endif
    int64_t nt = (K + W - 1) / W;
    if (layout == LAYOUT_ROUND_ROBIN) {
        kseq q = {s, S, 0, W, 0};
        q.ntiles = (s < nt) ? (nt - s + S - 1) / S : 0;
        if (q.ntiles > 0) {
            int64_t last = s + (q.ntiles - 1) * (int64_t)S;
            int64_t last_end = (last + 1) * W < K ? (last + 1) * W : K;
            q.len = (q.ntiles - 1) * W + (last_end - last * W);
        }
        return q;
    }
#if ORACLE_MUTANT == MUT_SPLIT_BALANCED
    int64_t base = nt / S, rem = nt % S;
    int64_t t0 = s * base + (s < rem ? s : rem);
    int64_t t1 = t0 + base + (s < rem ? 1 : 0);
    int64_t k0 = t0 * W;
    int64_t k1 = t1 * W < K ? t1 * W : K;
#else
    int64_t tps = (nt + S - 1) / S;
    int64_t k0 = (int64_t)s * tps * W;
    int64_t e = (int64_t)(s + 1) * tps * W;
    int64_t k1 = e < K ? e : K;
#endif
    if (k0 > K) k0 = K;
    return kseq_range(k0, k1);
}

/*
 * Combination of the S partials.  Serial (both platforms): acc = p0, then
 * acc = RN32(acc + p_s) for s = 1..S-1.  Pairwise (RTX 4060; the pages pin
 * only S = 3, as (p2 + p0) + p1).  Reading: a stride-halving tree over
 * P = the next power of two >= S: for h = P/2, P/4, ..., 1 and every i < h
 * with i + h < S, p_i = RN32(p_i + p_{i+h}); the result is p_0.  For S = 3
 * this is (p0 + p2) + p1.
 */
static float combine_partials(float *p, int S, const oracle_profile *pf)
{
    if (pf->combine == COMBINE_PAIRWISE) {
#if ORACLE_MUTANT == MUT_PAIRWISE_ADJACENT
        for (int width = 1; width < S; width *= 2)
            for (int i = 0; i + width < S; i += 2 * width) p[i] = p[i] + p[i + width];
        return p[0];
#else
        int P = 1;
        while (P < S) P *= 2;
        for (int h = P / 2; h >= 1; h /= 2)
            for (int i = 0; i < h; i++)
                if (i + h < S) p[i] = p[i] + p[i + h];
        return p[0];
#endif
    }
#if ORACLE_MUTANT == MUT_REVERSED_COMBINE
    float acc = p[S - 1];
    for (int s = S - 2; s >= 0; s--) acc = acc + p[s];
#else
    float acc = p[0];
    for (int s = 1; s < S; s++) acc = acc + p[s];
#endif
    return acc;
}

static float finite_accumulator(const operands *o, int64_t m, int64_t n, int fast, int S,
                                const oracle_profile *pf)
{
    float p[4096];
    for (int s = 0; s < S; s++) {
        kseq ks = split_seq(o->K, S, pf, s);
        if (ks.len <= 0) { p[s] = 0.0f; continue; }
        p[s] = fast ? exact_to_f32(chain_exact(o, m, n, &ks, 0, ks.len, pf, EXACT_PLUS_ZERO))
                    : slow_range(o, m, n, &ks, pf);
    }
    return combine_partials(p, S, pf);
}

/*
 * Non-finite inputs, decided per output from the whole rows x[m,:], w[n,:]
 * (limitations page, corrections table; validation page claims table on IEEE
 * specials): output (m, n) is the canonical NaN as soon as x's row m or w's
 * row n holds a NaN code, at any k.
 * Reading (E5M2 infinities; the pages record them but state no rule): a k
 * with Inf times zero, or infinite products of both signs, give NaN;
 * otherwise any infinite product gives that signed infinity.  This is the
 * IEEE outcome of adding the products in any order, and it is the same
 * whether taken over the whole row or per split / chunk and then added.
 * Returns CLS_NAN, CLS_INF (with *neg) or CLS_FINITE.
 */
static int special_class(const operands *o, int64_t m, int64_t n, int *neg)
{
    int nan = 0, pos_inf = 0, neg_inf = 0;
    for (int64_t k = 0; k < o->K; k++) {
        fp8_val a = decode_fp8(x_at(o, m, k), o->xfmt);
        fp8_val b = decode_fp8(w_at(o, n, k), o->wfmt);
        if (a.cls == CLS_NAN || b.cls == CLS_NAN) { nan = 1; continue; }
        if (a.cls == CLS_INF || b.cls == CLS_INF) {
#if ORACLE_MUTANT != MUT_INF_TIMES_ZERO
            if (a.cls == CLS_ZERO || b.cls == CLS_ZERO) { nan = 1; continue; }
#endif
#if ORACLE_MUTANT == MUT_INF_FIRST_SIGN
            if (pos_inf || neg_inf) continue;
#endif
            if (a.s ^ b.s) neg_inf = 1; else pos_inf = 1;
        }
    }
    if (nan || (pos_inf && neg_inf)) return CLS_NAN;
    if (pos_inf || neg_inf) { *neg = neg_inf; return CLS_INF; }
    return CLS_FINITE;
}

/* ------------------------------------------------------------------------ */
/* IEEE round-to-nearest-even of an exact value to a binary format with p
 * significand bits and exponent range [emin, emax], subnormals kept
 * (limitations page: flushing subnormals to zero is refused, since it
 * alters their arithmetic).  The argument must be exact in double, which every caller
 * guarantees (products of two binary32 values, binary32 values).
 * Returns the rounded value (+-inf on overflow), with the sign of v. */
static double round_to_format(double v, int p, int emin, int emax)
{
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    double a = fabs(v);
    int e;
    frexp(a, &e);
    e -= 1;                       /* a in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;       /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, e - (p - 1));
    double scaled = a / quantum;  /* exact: division by a power of two */
    double fl = floor(scaled);
    double rem = scaled - fl;     /* exact */
    double r;
    if (rem > 0.5) r = fl + 1.0;
    else if (rem < 0.5) r = fl;
    else r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double res = r * quantum;
    if (res >= ldexp(1.0, emax + 1)) res = INFINITY;
    return v < 0 ? -res : res;
}

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float f32_from(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

#if ORACLE_MUTANT == MUT_CANON_NAN
#define CANON_NAN_F32 0x7FC00000u
#define CANON_NAN_16 0x7FC0u
#else
/* Reading: the pages say NaN outputs are canonical without printing the bit
 * pattern; 0x7FFFFFFF (binary32) and 0x7FFF (bf16, fp16) is the canonical
 * NaN of NVIDIA's public PTX documentation.  Parity of this choice with
 * hardware is unpinned. */
#define CANON_NAN_F32 0x7FFFFFFFu
#define CANON_NAN_16 0x7FFFu
#endif
/* Reading: the FP8 NaN output is 0x7F for both formats (all exponent and
 * mantissa bits set; a NaN in e4m3fn and in e5m2).  Parity unpinned. */
#define CANON_NAN_8 0x7Fu

/* binary32 product RN32(a*b) of two binary32 values (IEEE multiplication). */
static float mul_f32(float a, float b)
{
    if (isnan(a) || isnan(b)) return NAN;
    if ((isinf(a) && b == 0.0f) || (isinf(b) && a == 0.0f)) return NAN;
    int neg = signbit(a) ^ signbit(b);
    if (isinf(a) || isinf(b)) return neg ? -INFINITY : INFINITY;
    double exact = (double)a * (double)b; /* 24x24 bits: exact in double */
    if (exact == 0.0) return neg ? -0.0f : 0.0f;
    return (float)round_to_format(exact, 24, -126, 127);
}

/*
 * Epilogue, first rounding (limitations page, corrections table: one fused
 * multiply-add of acc and alpha with +0 as the addend, rounded once;
 * validation page, scope table row "Epilogue": alpha is the binary32 product
 * of the two scales):
 * y32 = RN32(acc * alpha + (+0)).  An exactly zero product gives +0 (the
 * sum -0 + +0 is +0 under round to nearest); a nonzero product that rounds
 * to zero keeps its sign; overflow gives infinity.
 */
static float epilogue_f32(float acc, float alpha)
{
    if (isnan(acc) || isnan(alpha)) return NAN;
    if ((isinf(acc) && alpha == 0.0f) || (isinf(alpha) && acc == 0.0f)) return NAN;
    int neg = signbit(acc) ^ signbit(alpha);
    if (isinf(acc) || isinf(alpha)) return neg ? -INFINITY : INFINITY;
    double exact = (double)acc * (double)alpha;
    if (exact == 0.0) {
#if ORACLE_MUTANT == MUT_MUL_NOT_FMA
        return neg ? -0.0f : 0.0f;
#else
        return 0.0f;
#endif
    }
    return (float)round_to_format(exact, 24, -126, 127);
}

/* Second rounding: RNE of the binary32 value to the output format
 * (validation page, claims table, double-rounding row: bf16 and fp16
 * outputs are rounded from the binary32 result, not from the exact value). */
static uint32_t encode_output(float y32, int out_dtype)
{
    if (out_dtype == OUT_FP32) {
        if (isnan(y32)) return CANON_NAN_F32;
        return f32_bits(y32);
    }
    if (isnan(y32)) return CANON_NAN_16;
    if (out_dtype == OUT_BF16) {
        double r = round_to_format((double)y32, 8, -126, 127);
        /* r is exactly representable in bf16, hence in binary32; bf16 is the
         * top half of the binary32 pattern */
        return f32_bits((float)r) >> 16;
    }
    /* binary16 */
    double r = round_to_format((double)y32, 11, -14, 15);
    uint32_t sign = signbit(r) ? 0x8000u : 0u;
    double a = fabs(r);
    if (isinf(a)) return sign | 0x7C00u;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    e -= 1;
    if (e < -14) return sign | (uint32_t)(a / ldexp(1.0, -24)); /* subnormal */
    uint32_t frac = (uint32_t)(a / ldexp(1.0, e - 10)) - 1024u;
    return sign | ((uint32_t)(e + 15) << 10) | frac;
}

#if ORACLE_MUTANT == MUT_SINGLE_ROUNDING
static uint32_t encode_single_rounded(float acc, float alpha, int out_dtype)
{
    double exact = (double)acc * (double)alpha;
    if (out_dtype == OUT_FP32 || isnan(exact) || isinf(exact) || exact == 0.0)
        return encode_output(epilogue_f32(acc, alpha), out_dtype);
    if (out_dtype == OUT_BF16)
        return f32_bits((float)round_to_format(exact, 8, -126, 127)) >> 16;
    return encode_output((float)round_to_format(exact, 11, -14, 15), out_dtype);
}
#endif

/*
 * FP8 outputs (validation page, scope table row "Epilogue" and claims table,
 * FP8-output rows: scale_result enters through its own binary32
 * multiplication, and the result saturates at the format's largest value):
 *   y' = RN32(y32 * scale_result), a plain IEEE binary32 multiplication;
 *   |y'| is clamped to the format's largest finite value (448 for e4m3fn,
 *   57344 for e5m2), infinities included;
 *   the result is rounded to nearest even in the format, subnormals kept,
 *   the sign of a zero kept.
 * Reading: clamping before the rounding equals rounding with saturation,
 * because the largest finite value is representable.
 */
static uint32_t encode_fp8(float y, int out_dtype)
{
    const int e4 = out_dtype == OUT_E4M3FN;
    const int p = e4 ? 4 : 3, emin = e4 ? -6 : -14, bias = e4 ? 7 : 15, mb = p - 1;
    const double maxv = e4 ? 448.0 : 57344.0;
    if (isnan(y)) return CANON_NAN_8;
    uint32_t sign = signbit(y) ? 0x80u : 0u;
    double a = fabs((double)y);
#if ORACLE_MUTANT == MUT_FP8_NO_SATURATION
    if (a > maxv) return e4 ? (sign | 0x7Fu) : (sign | 0x7Cu);
#endif
    if (a > maxv) a = maxv;
    double r = round_to_format(a, p, emin, e4 ? 8 : 15);
    if (r == 0.0) return sign;
    int e;
    frexp(r, &e);
    e -= 1;
    if (e < emin) return sign | (uint32_t)(r / ldexp(1.0, emin - mb));
    return sign | ((uint32_t)(e + bias) << mb) | ((uint32_t)(r / ldexp(1.0, e - mb)) - (1u << mb));
}

/* ------------------------------------------------------------------------ */
/* Exported entry points. */

#define API __attribute__((visibility("default")))

/* The accumulator before the epilogue for output (m, n): the per-split
 * chains (fast) or chunked sums (slow), combined; non-finite inputs decided
 * first.  Returns the binary32 bit pattern (NaN canonical). */
static uint32_t acc_bits_at(const operands *o, int64_t m, int64_t n, int fast, int S,
                            const oracle_profile *pf)
{
    int neg = 0;
    int cls = special_class(o, m, n, &neg);
    if (cls == CLS_NAN) return CANON_NAN_F32;
    if (cls == CLS_INF) return neg ? 0xFF800000u : 0x7F800000u;
    return f32_bits(finite_accumulator(o, m, n, fast, S, pf));
}

static uint32_t out_bits_from_acc(uint32_t acc_bits, float alpha, float scale_result, int out_dtype)
{
    if (out_dtype == OUT_E4M3FN || out_dtype == OUT_E5M2) {
#if ORACLE_MUTANT == MUT_SR_FOLDED
        return encode_fp8(epilogue_f32(f32_from(acc_bits), mul_f32(alpha, scale_result)), out_dtype);
#else
        return encode_fp8(mul_f32(epilogue_f32(f32_from(acc_bits), alpha), scale_result), out_dtype);
#endif
    }
#if ORACLE_MUTANT == MUT_SINGLE_ROUNDING
    return encode_single_rounded(f32_from(acc_bits), alpha, out_dtype);
#else
    return encode_output(epilogue_f32(f32_from(acc_bits), alpha), out_dtype);
#endif
}

API int oracle_mutant_id(void) { return ORACLE_MUTANT; }

API int oracle_decode(uint8_t code, int fmt, int *cls, int *s, int *e, int *M)
{
    fp8_val v = decode_fp8(code, fmt);
    *cls = v.cls; *s = v.s; *e = v.e; *M = v.M;
    return 0;
}

API uint32_t oracle_mul_f32(uint32_t a, uint32_t b) { return f32_bits(mul_f32(f32_from(a), f32_from(b))); }

API uint32_t oracle_add_f32(uint32_t a, uint32_t b)
{
    float r = f32_from(a) + f32_from(b);
    return isnan(r) ? CANON_NAN_F32 : f32_bits(r);
}

API uint32_t oracle_epilogue_f32(uint32_t acc, uint32_t alpha)
{
    float y = epilogue_f32(f32_from(acc), f32_from(alpha));
    return isnan(y) ? CANON_NAN_F32 : f32_bits(y);
}

/* The last rounding alone: y32 (for FP8 outputs: y32 * scale_result) to the
 * output format. */
API uint32_t oracle_encode_output(uint32_t y32, int out_dtype)
{
    if (out_dtype == OUT_E4M3FN || out_dtype == OUT_E5M2) return encode_fp8(f32_from(y32), out_dtype);
    return encode_output(f32_from(y32), out_dtype);
}

/* Full epilogue: alpha = RN32(sx*sw), then y = out(RN32(acc*alpha)); FP8
 * outputs multiply by scale_result (sr) in between. */
API uint32_t oracle_output_from_acc(uint32_t acc_bits, uint32_t sx, uint32_t sw, uint32_t sr, int out_dtype)
{
    float alpha = mul_f32(f32_from(sx), f32_from(sw));
    return out_bits_from_acc(acc_bits, alpha, f32_from(sr), out_dtype);
}

/* The exact chain of [k0, k1) for one output, starting from +0 (no specials,
 * no split, no chunking).  Valid for any F up to 48. */
API int oracle_chain_exact(const uint8_t *x, int xfmt, int64_t ldx, const uint8_t *w, int wfmt,
                           int64_t ldw, int64_t m, int64_t n, int64_t k0, int64_t k1, int B, int F,
                           int *neg, int64_t *mag, int *q)
{
    if (B < 1 || B > MAX_B || F < 1 || F > 48) return -1;
    operands o = {x, xfmt, ldx, w, wfmt, ldw, 0, 0, k1};
    oracle_profile pf = {B, F, 128, 128, LAYOUT_CONTIGUOUS, COMBINE_SERIAL};
    kseq ks = kseq_range(k0, k1);
    exact_val r = chain_exact(&o, m, n, &ks, 0, ks.len, &pf, EXACT_PLUS_ZERO);
    *neg = r.neg; *mag = r.mag; *q = r.q;
    return 0;
}

/* One block step on explicit products: g[i], P[i], s[i] (P = 0 marks a zero
 * product), incoming c = (-1)^c_neg * c_mag * 2^c_q. */
API int oracle_block_step(const int *g, const int *P, const int *s, int n, int F, int c_neg,
                          int64_t c_mag, int c_q, int *neg, int64_t *mag, int *q)
{
    if (n < 0 || n > MAX_B) return -1;
    product buf[MAX_B];
    for (int i = 0; i < n; i++) {
        buf[i].cls = P[i] ? CLS_FINITE : CLS_ZERO;
        buf[i].g = g[i]; buf[i].P = P[i]; buf[i].s = s[i];
    }
    exact_val c = {c_neg, c_mag, c_q};
    exact_val r = block_step(c, buf, n, F);
    *neg = r.neg; *mag = r.mag; *q = r.q;
    return 0;
}

/*
 * The fast chain of one output started from an incoming binary32
 * accumulator c_in instead of +0 (the accumulator-only path: validation page,
 * claims table, a c passing through blocks without products, over all 2^32
 * binary32 patterns).  Readings, the pages printing no rule: with K = 0 there
 * is no block and c_in is returned unchanged (a NaN as the canonical NaN); a
 * NaN c_in gives NaN; an infinite c_in stays that infinity unless the
 * products hold a NaN code, an infinity times zero or the opposite infinity,
 * which give NaN; a finite c_in with infinite products gives the products'
 * result; -0 enters as +0.
 */
static uint32_t acc_bits_with_c(const operands *o, int64_t m, int64_t n, uint32_t c_in, const oracle_profile *pf)
{
    const uint32_t ce = (c_in >> 23) & 0xFFu, cm = c_in & 0x7FFFFFu;
    if (ce == 0xFFu && cm) return CANON_NAN_F32;
    if (o->K == 0) return c_in;
    int neg = 0;
    int cls = special_class(o, m, n, &neg);
    if (ce == 0xFFu) {
        if (cls == CLS_NAN) return CANON_NAN_F32;
#if ORACLE_MUTANT != MUT_C_INF_ABSORBS
        if (cls == CLS_INF && neg != (int)(c_in >> 31)) return CANON_NAN_F32;
#endif
        return c_in;
    }
    if (cls == CLS_NAN) return CANON_NAN_F32;
    if (cls == CLS_INF) return neg ? 0xFF800000u : 0x7F800000u;
    exact_val c = EXACT_PLUS_ZERO;
    if (ce || cm) {
        c.neg = (int)(c_in >> 31);
        c.mag = ce ? (int64_t)(cm | 0x800000u) : (int64_t)cm;
        c.q = ce ? (int)ce - 150 : -149;
    }
    kseq ks = kseq_range(0, o->K);
    return f32_bits(exact_to_f32(chain_exact(o, m, n, &ks, 0, ks.len, pf, c)));
}

/* Fast accumulation, one split, from incoming accumulators c_in [M, N]
 * (binary32 bit patterns, row stride N) into acc_out [M, N]. */
API int oracle_accumulate_c(const uint8_t *x, int xfmt, int64_t ldx, const uint8_t *w, int wfmt, int64_t ldw,
                            int64_t M, int64_t N, int64_t K, const uint32_t *c_in, int B, int F,
                            uint32_t *acc_out)
{
    if (B < 1 || B > MAX_B || F < 1 || F > 23) return -1;
    if ((xfmt != FMT_E4M3FN && xfmt != FMT_E5M2) || (wfmt != FMT_E4M3FN && wfmt != FMT_E5M2)) return -1;
    operands o = {x, xfmt, ldx, w, wfmt, ldw, M, N, K};
    oracle_profile pf = {B, F, 128, 128, LAYOUT_CONTIGUOUS, COMBINE_SERIAL};
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) acc_out[m * N + n] = acc_bits_with_c(&o, m, n, c_in[m * N + n], &pf);
    return 0;
}

static int check_args(int B, int F, int S, int Q, int W, int layout, int combine, int xfmt, int wfmt,
                      int out_dtype)
{
    if (out_dtype < OUT_BF16 || out_dtype > OUT_E5M2) return -1;
    if (B < 1 || B > MAX_B || F < 1 || F > 23) return -1;
    if (S < 1 || S > 4096 || Q < 1 || W < 1) return -1;
    if ((layout != LAYOUT_CONTIGUOUS && layout != LAYOUT_ROUND_ROBIN) ||
        (combine != COMBINE_SERIAL && combine != COMBINE_PAIRWISE)) return -1;
    if ((xfmt != FMT_E4M3FN && xfmt != FMT_E5M2) || (wfmt != FMT_E4M3FN && wfmt != FMT_E5M2)) return -1;
    return 0;
}

/* Accumulator and output at a list of (m, n) points. */
API int oracle_points(const uint8_t *x, int xfmt, int64_t ldx, const uint8_t *w, int wfmt, int64_t ldw,
                      int64_t K, int64_t npts, const int64_t *ms, const int64_t *ns, uint32_t sx,
                      uint32_t sw, uint32_t sr, int out_dtype, int fast, int S, int B, int F, int Q, int W,
                      int layout, int combine, uint32_t *acc_out, uint32_t *y_out)
{
    if (check_args(B, F, S, Q, W, layout, combine, xfmt, wfmt, out_dtype)) return -1;
    operands o = {x, xfmt, ldx, w, wfmt, ldw, 0, 0, K};
    oracle_profile pf = {B, F, Q, W, layout, combine};
    float alpha = mul_f32(f32_from(sx), f32_from(sw));
    for (int64_t i = 0; i < npts; i++) {
        uint32_t a = acc_bits_at(&o, ms[i], ns[i], fast, S, &pf);
        if (acc_out) acc_out[i] = a;
        if (y_out) y_out[i] = out_bits_from_acc(a, alpha, f32_from(sr), out_dtype);
    }
    return 0;
}

typedef struct {
    const operands *o;
    const oracle_profile *pf;
    float alpha, scale_result;
    int out_dtype, fast, S;
    uint32_t *acc_out, *y_out;
    int64_t row_begin, row_end;
} job;

static void *run_rows(void *arg)
{
    job *j = (job *)arg;
    for (int64_t m = j->row_begin; m < j->row_end; m++)
        for (int64_t n = 0; n < j->o->N; n++) {
            uint32_t a = acc_bits_at(j->o, m, n, j->fast, j->S, j->pf);
            if (j->acc_out) j->acc_out[m * j->o->N + n] = a;
            if (j->y_out) j->y_out[m * j->o->N + n] = out_bits_from_acc(a, j->alpha, j->scale_result, j->out_dtype);
        }
    return NULL;
}

/* The whole [M, N] result, rows spread over nthreads host threads.
 * acc_out and y_out are dense [M, N] arrays of bit patterns (either may be
 * NULL).  y_out holds 16-bit patterns in the low half for bf16/fp16 and
 * 8-bit patterns in the low byte for FP8 outputs. */
API int oracle_scaled_mm(const uint8_t *x, int xfmt, int64_t ldx, const uint8_t *w, int wfmt,
                         int64_t ldw, int64_t M, int64_t N, int64_t K, uint32_t sx, uint32_t sw,
                         uint32_t sr, int out_dtype, int fast, int S, int B, int F, int Q, int W, int layout,
                         int combine, uint32_t *acc_out, uint32_t *y_out, int nthreads)
{
    if (check_args(B, F, S, Q, W, layout, combine, xfmt, wfmt, out_dtype)) return -1;
    if (M < 0 || N < 0 || K < 0) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    operands o = {x, xfmt, ldx, w, wfmt, ldw, M, N, K};
    oracle_profile pf = {B, F, Q, W, layout, combine};
    float alpha = mul_f32(f32_from(sx), f32_from(sw));
    pthread_t th[256];
    job jobs[256];
    int nt = (int)((M < nthreads) ? (M > 0 ? M : 1) : nthreads);
    int64_t per = (M + nt - 1) / nt;
    for (int t = 0; t < nt; t++) {
        jobs[t].o = &o; jobs[t].pf = &pf; jobs[t].alpha = alpha; jobs[t].scale_result = f32_from(sr);
        jobs[t].out_dtype = out_dtype; jobs[t].fast = fast; jobs[t].S = S;
        jobs[t].acc_out = acc_out; jobs[t].y_out = y_out;
        jobs[t].row_begin = t * per < M ? t * per : M;
        jobs[t].row_end = (t + 1) * per < M ? (t + 1) * per : M;
    }
    if (nt == 1) { run_rows(&jobs[0]); return 0; }
    for (int t = 0; t < nt; t++) pthread_create(&th[t], NULL, run_rows, &jobs[t]);
    for (int t = 0; t < nt; t++) pthread_join(th[t], NULL);
    return 0;
}
