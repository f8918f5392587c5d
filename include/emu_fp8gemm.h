/*
 * emu_fp8gemm.h -- C ABI of the MI355X (gfx950) bit-exact emulated FP8 GEMM.
 *
 * Computes y = (x @ w.T) * scale_x * scale_w with the arithmetic that the
 * mmaemu v0.1 documentation describes for its default "hopper" profile
 * (user guide section 1 and section 3 "A first GEMM"; validation page,
 * scope table rows "Hopper preset", "Slow accumulation", "Split-K on the
 * H100 PCIe" and "Epilogue"; limitations page, corrections table), and for
 * its RTX 4060 profiles, which differ only in block width and split layout
 * (see emu_profile below):
 *
 *  - E4M3/E5M2 products are added in blocks of 32 (hopper) consecutive products; each
 *    block, together with the incoming accumulator, is aligned to the block's
 *    largest exponent (field exponents, subnormals at emin), every term is cut
 *    toward zero to 13 fraction bits, and the block sum is cut toward zero to
 *    14 significant bits; a zero block result is +0.
 *  - fast_accum != 0 chains the blocks along K; fast_accum == 0 starts a new
 *    chain at every 128th position of K and sums the chunk results, first
 *    chunk first, with binary32 round-to-nearest-even additions.
 *  - split_S > 1 splits K into runs of consecutive 128-wide k-tiles,
 *    ceil(ceil(K/128)/S) tiles per split (trailing splits may be empty and
 *    give +0), and adds the partials serially, p0 + p1 + ... in binary32.
 *  - the epilogue is alpha = RN32(scale_x * scale_w), y32 = RN32(acc*alpha+(+0))
 *    (an exactly zero product gives +0), then round-to-nearest-even to the
 *    output type; subnormals are kept everywhere.  FP8 outputs first take
 *    y' = RN32(y32 * scale_result), a plain binary32 multiplication, then
 *    saturate: |y'| at or above the format's largest finite value (448 for
 *    e4m3fn, 57344 for e5m2), infinities included, becomes that value
 *    (validation page, scope table row "Epilogue" and claims table).
 *  - an output (m, n) whose x row m or w row n holds a NaN code anywhere is
 *    the canonical NaN (0x7FFFFFFF for fp32, 0x7FFF for bf16/fp16, 0x7F for
 *    FP8; the bit patterns are a reading: the pages say "canonical" only).
 *    E5M2 infinities follow IEEE: Inf*0 or infinite products of both signs
 *    give NaN, otherwise the signed infinity.
 *
 * Layouts (all pointers are device pointers owned by the caller):
 *   x   [M, K] row-major FP8 codes, leading dimension ldx (bytes >= K);
 *   w   [N, K] row-major FP8 codes, leading dimension ldw (this is torch's
 *       mat2 = w.t(), a [K, N] column-major matrix);
 *   out [M, N] row-major, leading dimension ldo (elements >= N);
 *   scale_x, scale_w (and scale_result): one binary32 value each, read on
 *       the device.
 *
 * Ordering and ownership: every call only enqueues kernels on `stream` and
 * returns; it never synchronises and never allocates device memory.  The
 * caller keeps all buffers alive until the stream has run the work.  `out`
 * is fully overwritten and never read.  Results are deterministic: no
 * atomics take part in the arithmetic.  The library keeps no mutable state
 * between calls other than the thread-local error text.
 *
 * Errors: arguments are checked on the host before anything is enqueued; a
 * non-OK status means nothing was written.  emu_last_error_message() gives
 * a thread-local explanation of the last non-OK status.
 */
#ifndef EMU_FP8GEMM_H
#define EMU_FP8GEMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EMU_ABI_VERSION 5

#if defined(EMU_BUILDING_LIBRARY)
#define EMU_API __attribute__((visibility("default")))
#else
#define EMU_API
#endif

typedef enum {
    EMU_OK = 0,
    EMU_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad leading dimension, unknown enum, split_S < 1,
                                plan options out of range */
    EMU_ERR_REJECTED = 2,    /* a call torch 2.7.1 / cuBLASLt would reject (limitations page, features table;
                                validation page, claims table): e5m2 x e5m2, e4m3fn x e4m3fn -> e5m2,
                                K or N not a multiple of 16, x / w / out not 16-byte aligned,
                                ldx or ldw not a multiple of 16 */
    EMU_ERR_UNSUPPORTED = 3, /* a feature outside this library: split_S above 65535, M or N above 2^31-1,
                                scale_result with a non-FP8 output */
    EMU_ERR_WORKSPACE = 4,   /* workspace smaller than the required part of emu_workspace_bytes(...) */
    EMU_ERR_DEVICE = 5       /* a HIP launch or runtime error */
} emu_status;

typedef enum { EMU_FP8_E4M3FN = 0, EMU_FP8_E5M2 = 1 } emu_fp8_format;

/* Output types.  FP8 outputs (e4m3fn, e5m2) are one byte per element, with
 * scale_result and saturation; e4m3fn x e4m3fn inputs cannot produce e5m2
 * (rejected, as cuBLASLt does on both reference platforms). */
typedef enum {
    EMU_OUT_BF16 = 0,
    EMU_OUT_FP16 = 1,
    EMU_OUT_FP32 = 2,
    EMU_OUT_E4M3FN = 3,
    EMU_OUT_E5M2 = 4
} emu_out_dtype;

/* The arithmetic profile (user guide section 4: profiles name a reference
 * platform; hopper is the default).
 *   EMU_PROFILE_HOPPER: the H100 PCIe -- 32-product blocks; split_S > 1 cuts
 *     K into runs of consecutive 128-wide k-tiles (ceil layout), partials
 *     added serially.
 *   EMU_PROFILE_ADA_SERIAL / EMU_PROFILE_ADA_PAIRWISE: the RTX 4060 --
 *     16-product blocks (validation page, scope table row "Ada instruction
 *     model"); split_S > 1 deals 64-wide k-tiles to the splits in turn
 *     (tile t to split t mod S), each split chains (and, for slow
 *     accumulation, restarts every 128) along its own tiles in order, and
 *     the partials are added serially or by the pairwise tree (limitations
 *     page, corrections table; validation page, claims table: for S = 3
 *     pairwise is (p2 + p0) + p1).  The pairwise tree for other S is a
 *     reading: p_i += p_{i+h} for h = P/2, P/4, ..., 1 (P the next power of
 *     two >= S) wherever i + h < S; the result is p_0.
 * The block step, the 13 retained fraction bits, c in the alignment, slow
 * accumulation and the epilogue are the same for all profiles. */
typedef enum {
    EMU_PROFILE_HOPPER = 0,
    EMU_PROFILE_ADA_SERIAL = 1,
    EMU_PROFILE_ADA_PAIRWISE = 2
} emu_profile;

/* Tile configurations of the main kernel (output rows x columns per
 * workgroup; results never depend on the configuration). */
#define EMU_TILE_AUTO (-1)
#define EMU_TILE_COUNT 13

/*
 * Plan options, for testing and tuning; a NULL pointer means every field at
 * its automatic value.  Results do not depend on them.
 *   tile:  EMU_TILE_AUTO, or 0 .. EMU_TILE_COUNT-1 to force the main
 *          kernel's tile configuration: 64x128, 64x64, 32x64, 32x32 output
 *          tiles with one lane per output; 16x16 with 2 or 4 lanes per
 *          output; 64x64 and 64x128 with the block exponent maxima on the
 *          matrix cores; 16x8 with 4 lanes per output; 16x64 with
 *          matrix-core maxima in one wave; 32x32 staging 4 K-blocks per
 *          barrier, with VALU or matrix-core maxima; 32x16 with
 *          matrix-core maxima staging 5 K-blocks per barrier.
 *   defer: the deferred-infinity plan described at emu_workspace_bytes:
 *          -1 automatic (from 2^36 multiply-adds), 0 never, 1 at every size
 *          the plan allows.  Changes emu_workspace_bytes.
 * Any other value returns EMU_ERR_INVALID_ARG (emu_workspace_bytes: 0).
 */
typedef struct {
    int tile;
    int defer;
} emu_plan_options;

/*
 * y = (x @ w.T) * scale_x * scale_w (torch._scaled_mm semantics with
 * tensor-wise scales; user guide section 3).
 *
 * scale_result: NULL, or (FP8 outputs only) a device pointer to one binary32
 * value; NULL means no scale_result (the same bits as 1.0).  A non-NULL
 * scale_result with a bf16 / fp16 / fp32 output returns EMU_ERR_UNSUPPORTED.
 *
 * M >= 0 (any value), N >= 0 and K >= 0 multiples of 16.  M = 0 or N = 0
 * returns EMU_OK without enqueuing anything; K = 0 writes +0 everywhere.
 * workspace: device memory of emu_workspace_bytes(M, N, K, split_S,
 * fast_accum, profile, plan) bytes (may be NULL when that is 0), 4-byte
 * aligned; its contents on entry do not matter and on return are
 * unspecified (the combination may work in place).  Only the split partials and
 * stored chunk results are required (a smaller workspace returns
 * EMU_ERR_WORKSPACE); without the optional infinity lists at its end the
 * call is still bit-exact, only slower on large inputs whose e5m2 rows hold
 * infinities.  stream: the HIP stream to enqueue on (NULL = the default
 * stream).  plan: NULL, or plan options (above).
 */
EMU_API emu_status emu_scaled_mm(const uint8_t *x, emu_fp8_format x_fmt, int64_t ldx,
                                 const uint8_t *w, emu_fp8_format w_fmt, int64_t ldw,
                                 int64_t M, int64_t N, int64_t K,
                                 const float *scale_x, const float *scale_w, const float *scale_result,
                                 void *out, emu_out_dtype out_dtype, int64_t ldo,
                                 int fast_accum, int split_S, emu_profile profile,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream,
                                 const emu_plan_options *plan);

/*
 * The binary32 accumulator before the epilogue: acc [M, N] row-major with
 * leading dimension ldacc (mmaemu's accumulate(x, w, use_fast_accum), user
 * guide section 3).  NaN results are 0x7FFFFFFF.  Same rules for the
 * operands, workspace, stream and plan as emu_scaled_mm.
 */
EMU_API emu_status emu_accumulate(const uint8_t *x, emu_fp8_format x_fmt, int64_t ldx,
                                  const uint8_t *w, emu_fp8_format w_fmt, int64_t ldw,
                                  int64_t M, int64_t N, int64_t K,
                                  float *acc, int64_t ldacc,
                                  int fast_accum, int split_S, emu_profile profile,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream,
                                  const emu_plan_options *plan);

/*
 * Fast accumulation from incoming accumulators: acc[m, n] is the fast chain
 * of output (m, n) (split_S = 1) started from c_in[m, n] instead of +0, so
 * that c_in takes part in the first block's alignment exactly as the chain's
 * own accumulator does in later blocks -- the path that the mmaemu
 * validation page (claims table) records for every binary32 c with blocks
 * without products.  Feeding the accumulator of the first K1 columns (K1 a
 * multiple of the block width: 32 hopper, 16 ada) back as c_in for the
 * remaining columns gives the accumulator of all K columns.
 * Readings where the pages print no rule: a subnormal c_in is aligned at
 * binary32's emin (-126), as subnormal FP8 inputs are at theirs; K = 0
 * returns c_in unchanged (a NaN as 0x7FFFFFFF); a NaN c_in gives NaN; an
 * infinite c_in stays, unless the products hold a NaN code, an infinity
 * times zero or the opposite infinity (then NaN); -0 enters as +0.
 * c_in [M, N] row-major with leading dimension ldc, acc [M, N] with ldacc
 * (elements; device memory, 4-byte aligned); acc may be c_in itself (each
 * element is read before its output is written).  No workspace.  Operand
 * rules and errors as emu_accumulate; plan.defer is not used.
 */
EMU_API emu_status emu_accumulate_c(const uint8_t *x, emu_fp8_format x_fmt, int64_t ldx,
                                    const uint8_t *w, emu_fp8_format w_fmt, int64_t ldw,
                                    int64_t M, int64_t N, int64_t K,
                                    const float *c_in, int64_t ldc, float *acc, int64_t ldacc,
                                    emu_profile profile, hipStream_t stream, const emu_plan_options *plan);

/* Device workspace in bytes for emu_scaled_mm and emu_accumulate with these
 * arguments (0 for invalid sizes or plan options).  Required: split partials
 * (split_S * M * N * 4 when split_S > 1), or the results of groups of 128-K
 * chunks when slow accumulation over a small output grid stores them.
 * Optional, at the end: on problems of M * N * K >= 2^36 with K <= 64496
 * that store no chunk results, the infinity lists, 65 * 4 bytes per row of
 * the larger of M and N (e5m2 operands only use them): a pass over the e5m2
 * operand lists where each row holds infinities, the main kernel skips the
 * outputs those rows make non-finite, and a fix-up kernel resolves them from
 * the lists.  Depends on the plan only, never on the data or formats. */
EMU_API size_t emu_workspace_bytes(int64_t M, int64_t N, int64_t K, int split_S, int fast_accum,
                                   emu_profile profile, const emu_plan_options *plan);

/* Bytes of the device scratch that emu_scaled_mm_noalloc uses per GPU. */
#define EMU_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * For callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * emu_scaled_mm without a workspace argument.  Its split partials, stored
 * slow-mode chunk results and infinity lists live in a fixed array of
 * EMU_NOALLOC_SCRATCH_BYTES (64 MiB) in the library's device memory, one
 * copy per GPU, held until the process ends; the call allocates nothing (the
 * array's address is looked up once per device, on the first call with that
 * device current).  Arguments, results and errors are those of
 * emu_scaled_mm, on the current device, which must be the stream's.  Plans
 * whose required part does not fit the scratch: slow accumulation stores
 * its chunk results only when they fit (the results are the same either
 * way); split partials beyond it, split_S * M * N * 4 bytes above
 * EMU_NOALLOC_SCRATCH_BYTES, return EMU_ERR_WORKSPACE before anything is
 * enqueued.  Every call on one GPU shares that GPU's scratch: calls that may
 * run at the same time on one GPU (other streams, other threads) race and
 * must be ordered by the caller; the scratch needs no clearing between
 * calls.
 */
EMU_API emu_status emu_scaled_mm_noalloc(const uint8_t *x, emu_fp8_format x_fmt, int64_t ldx,
                                         const uint8_t *w, emu_fp8_format w_fmt, int64_t ldw,
                                         int64_t M, int64_t N, int64_t K,
                                         const float *scale_x, const float *scale_w, const float *scale_result,
                                         void *out, emu_out_dtype out_dtype, int64_t ldo,
                                         int fast_accum, int split_S, emu_profile profile,
                                         hipStream_t stream, const emu_plan_options *plan);

/* Static description of a status code. */
EMU_API const char *emu_status_string(emu_status status);

/* Thread-local detail text of the last non-OK status returned on this thread
 * (empty string if none).  The pointer stays valid until the next call on
 * the same thread. */
EMU_API const char *emu_last_error_message(void);

/* EMU_ABI_VERSION of the built library. */
EMU_API int emu_abi_version(void);

/*
 * Host builds of the library's own IEEE rounding routines, the same source
 * its kernels use, exported so that CPU tests can check them without a GPU.
 * All arguments and results are bit patterns.
 *   emu_host_mul_f32:      RN32(a * b), IEEE binary32 multiplication.
 *   emu_host_epilogue_f32: RN32(acc * alpha + (+0)); NaN results 0x7FFFFFFF.
 *   emu_host_f32_to_bf16 / emu_host_f32_to_f16: round to nearest even,
 *       subnormals kept, overflow to infinity, NaN -> 0x7FFF.
 *   emu_host_f32_to_e4m3fn / emu_host_f32_to_e5m2: round to nearest even,
 *       subnormals kept, saturation to +-448 / +-57344 (infinities
 *       included), NaN -> 0x7F.
 */
EMU_API uint32_t emu_host_mul_f32(uint32_t a, uint32_t b);
EMU_API uint32_t emu_host_epilogue_f32(uint32_t acc, uint32_t alpha);
EMU_API uint16_t emu_host_f32_to_bf16(uint32_t f);
EMU_API uint16_t emu_host_f32_to_f16(uint32_t f);
EMU_API uint8_t emu_host_f32_to_e4m3fn(uint32_t f);
EMU_API uint8_t emu_host_f32_to_e5m2(uint32_t f);

#ifdef __cplusplus
}
#endif

#endif /* EMU_FP8GEMM_H */
