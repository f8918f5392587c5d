// emu_internal.h -- launch plan shared by the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/emu_fp8gemm.h"

namespace emu {

// What the main kernel writes for each output.
enum OutKind : int {
    OUT_ACC_F32 = 0,  // binary32 accumulator (NaN canonical); also split partials
    OUT_BF16 = 1,     // epilogue, bf16
    OUT_F16 = 2,      // epilogue, binary16
    OUT_F32 = 3,      // epilogue, binary32
    OUT_E4M3 = 4,     // epilogue, times scale_result, e4m3fn with saturation
    OUT_E5M2 = 5,     // epilogue, times scale_result, e5m2 with saturation
};

struct MainParams {
    const uint8_t *x;      // [M, K] codes, row stride ldx bytes
    const uint8_t *w;      // [N, K] codes, row stride ldw bytes
    int64_t ldx, ldw;
    int M, N;              // rows of this launch (M may be a slice)
    int64_t K;
    // Split layout: K is cut into k-tiles of width 2^tile_shift.  Contiguous
    // (round_robin = 0): split z owns tiles [z*tps, (z+1)*tps).  Round-robin:
    // split z owns tiles z, z+S, z+2S, ...  Each split's chain (and slow
    // chunking) runs along its tiles in increasing order.
    int tile_shift;
    int round_robin;
    int64_t tps;
    int S;
    int fast;              // 1: one chain per split; 0: restart every 128 along the split
    // Slow mode with chunk results stored (chunked = 1): grid z is
    // S * chunk_groups; workgroup z takes split z / chunk_groups and the
    // chunks_per_group 128-chunks of group z % chunk_groups of that split's
    // k-list, and writes each chunk's chain result to out as partial
    // (split * cps + chunk) (+0 for chunks past the k-list), to be added in
    // order by the combine kernel.  Otherwise chunk_groups = 1, chunked = 0.
    int chunked;
    int chunk_groups;
    int chunks_per_group;
    int cps;               // chunks per split in the partial layout
    int out_kind;          // OutKind
    void *out;             // OUT_ACC_F32 / epilogue destination, [M, N] with row stride ldo elements
    int64_t ldo;
    int64_t split_stride;  // elements between consecutive splits' partials in `out` (S > 1)
    const float *scale_x, *scale_w;
    const float *scale_result;  // FP8 outputs only; null means 1
    // Incoming accumulators (fast accumulation, S = 1): chain (m, n) starts
    // from c_in[m * ldc + n] instead of +0.
    const float *c_in;
    int64_t ldc;
    // 1: outputs whose rows hold infinities (and no NaN) are left as the
    // chain computed them; the infinity fix-up kernel overwrites them.
    int defer_specials;
};

// Deferred infinities.  Operand A is the e5m2 one (the only format with
// infinities; the other, B, is e4m3fn).  The row kernel writes, for each A
// row, info[a] = the number of infinity codes in it, or 0 when there is none
// or the row holds a NaN code (the main kernel resolves NaN rows itself), and
// the positions k | sign << 31 of the first kDeferCap of them, in any order,
// to pos[a * kDeferCap + i].  The fix-up kernel overwrites every output whose
// A row has info != 0 and whose B row holds no NaN code with the specials
// rule's result, read from those lists and the B row (staged in LDS), or
// from the whole A row where a list overflowed.
constexpr int kDeferCap = 64;
constexpr int64_t kDeferLdsBytes = 63 * 1024;  // staged B rows per fix-up workgroup, at most

struct DeferParams {
    const uint8_t *a, *b;  // A and B rows, strides lda, ldb bytes
    int64_t lda, ldb;
    int ra, rb;            // A and B rows
    int64_t K;
    int a_is_w;            // 1: output (m, n) = (B row, A row); 0: (A row, B row)
    uint32_t *info;        // [ra]
    uint32_t *pos;         // [ra * kDeferCap]
    int b_rows;            // B rows staged per fix-up workgroup (1..16, row stride K + 16 bytes)
    int a_rows;            // A rows per fix-up workgroup
    int out_kind;          // OUT_ACC_F32 or an epilogue kind
    void *out;             // [M, N], row stride ldo elements
    int64_t ldo;
    const float *scale_x, *scale_w;
    const float *scale_result;
};

struct CombineParams {
    float *part;           // [S * cps, M, N] partials, dense (the pairwise tree over more than 16 splits runs in place)
    int S, M, N;
    int cps;               // partials per split: 1, or the slow-mode chunk results to add in order first
    int pairwise;          // 0: serial p0 + p1 + ...; 1: stride-halving pairwise tree
    int out_kind;          // OUT_ACC_F32 or an epilogue kind
    void *out;
    int64_t ldo;
    const float *scale_x, *scale_w;
    const float *scale_result;
};

// Tile configurations of the main kernel: rows x cols per workgroup; per
// thread 4x8, 4x4, 2x4, 2x2 outputs, or one output chain shared by 2 or 4
// lanes (G2, G4; these stage 8 K-blocks per barrier); MX: block exponent
// maxima on the matrix cores (16x64: one wave, for few rows).  The 32x32
// tile stages 2 K-blocks per barrier, and 4 in its S4 form (78 KB of LDS:
// two workgroups per CU, for grids that leave the GPU at most that full).
enum TileConfig : int {
    TILE_64x128 = 0,
    TILE_64x64 = 1,
    TILE_32x64 = 2,
    TILE_32x32 = 3,
    TILE_16x16_G2 = 4,
    TILE_16x16_G4 = 5,
    TILE_64x64_MX = 6,
    TILE_64x128_MX = 7,
    TILE_16x8_G4 = 8,
    TILE_16x64_MX = 9,
    TILE_32x32_S4 = 10,
    TILE_32x32_MX_S4 = 11,
    TILE_32x16_MX_S5 = 12,
    TILE_COUNT = 13
};

struct TileShape {
    int bm, bn, threads;
};
TileShape tile_shape(int cfg);

// Enqueue one main-kernel launch over grid (ceil(N/bn), ceil(M/bm), S) with
// blocks of `block` products (32 or 16).
hipError_t launch_main(int cfg, int block, int xfmt, int wfmt, const MainParams &p, int S, hipStream_t stream);

// One instantiation of the main kernel (block width BLK, x / w formats XF, WF:
// 0 = e4m3fn, 1 = e5m2), defined in emu_main_kernel.h and instantiated by
// emu_variant.hip.
template <int BLK, int XF, int WF>
hipError_t launch_variant(int cfg, const MainParams &p, int S, hipStream_t stream);
template <int BLK, int XF, int WF>
hipError_t launch_variant_cin(int cfg, const MainParams &p, hipStream_t stream);
// The main kernel from incoming accumulators (grid z = 1).
hipError_t launch_main_cin(int cfg, int block, int xfmt, int wfmt, const MainParams &p, hipStream_t stream);
hipError_t launch_combine(const CombineParams &p, hipStream_t stream);
// The infinity row kernel, then (after the main and combine kernels) the
// fix-up kernel.
hipError_t launch_inf_rows(const DeferParams &p, hipStream_t stream);
hipError_t launch_inf_fixup(const DeferParams &p, hipStream_t stream);

// emu_scaled_mm with a fixed device scratch of scratch_bytes in place of the
// caller's workspace: the same checks, a plan whose required part fits the
// scratch (slow-mode chunk results are stored only when they fit; split
// partials that do not fit return EMU_ERR_WORKSPACE), then scratch() for the
// current device's scratch address (nullptr and a message on failure), then
// the same launches.  No device memory is allocated.
emu_status scaled_mm_in_scratch(const uint8_t *x, emu_fp8_format x_fmt, int64_t ldx, const uint8_t *w,
                                emu_fp8_format w_fmt, int64_t ldw, int64_t M, int64_t N, int64_t K,
                                const float *scale_x, const float *scale_w, const float *scale_result, void *out,
                                emu_out_dtype out_dtype, int64_t ldo, int fast_accum, int split_S,
                                emu_profile profile, void *(*scratch)(size_t *bytes, std::string *err),
                                size_t scratch_bytes, hipStream_t stream, const emu_plan_options *plan);

}  // namespace emu
