// microbench.hip -- issue rates, on gfx950, of every VALU instruction that
// the main kernel's stage loop issues, and of the term loop's own mix.
//
// Each op kernel runs 8 independent chains of one instruction per lane, 32
// instructions per loop iteration, with 8 waves on every SIMD (2,048
// workgroups of 256 threads on 256 CUs).  The term-mix kernel runs, per
// chain and iteration, the term loop's sequence for one pair of products:
// two truncating FMAs, one byte permute, one sign-pair bitop and one 16-bit
// dot product (5 instructions, 2 multiply-adds).  The host times one launch
// with HIP events after an untimed one, which gives instructions per second
// over the whole chip.  Measurement code only: the GEMM library does not use
// it.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int CHAINS = 8;
constexpr int PER_ITER = 4 * CHAINS;  // instructions per loop iteration (op kernels)

// One instruction per op, in the form the main kernel issues it.  Ops on
// 64-bit operands use the pair b64 / a64.
#define MB_OPS(X)                                                                                                         \
    X(PK_ADD_U16, "v_pk_add_u16", "v_pk_add_u16 %[a], %[a], %[b]")                                                        \
    X(PK_MAXIMUM3_F16, "v_pk_maximum3_f16", "v_pk_maximum3_f16 %[a], %[a], %[b], %[b]")                                   \
    X(DOT2_I32_I16, "v_dot2_i32_i16", "v_dot2_i32_i16 %[a], %[b], %[b], %[a]")                                            \
    X(DOT2C_I32_I16, "v_dot2c_i32_i16", "v_dot2c_i32_i16 %[a], %[b], %[b]")                                               \
    X(FMA_F32, "v_fma_f32", "v_fma_f32 %[a], |%[b]|, |%[b]|, %[a]")                                                       \
    X(FMA_MIX_F32, "v_fma_mix_f32", "v_fma_mix_f32 %[a], |%[b]|, |%[b]|, %[a] op_sel_hi:[1,1,0]")                           \
    X(CVT_SCALEF32_PK_F16_FP8, "v_cvt_scalef32_pk_f16_fp8", "v_cvt_scalef32_pk_f16_fp8 %[a], %[b], %[sel]")                 \
    X(PERM_B32, "v_perm_b32", "v_perm_b32 %[a], %[b], %[a], %[sel]")                                                      \
    X(BITOP3_B32, "v_bitop3_b32", "v_bitop3_b32 %[a], %[a], %[b], %[sel] bitop3:0xbe")                                    \
    X(LSHRREV_B32, "v_lshrrev_b32", "v_lshrrev_b32 %[a], %[b], %[a]")                                                     \
    X(ADD3_U32, "v_add3_u32", "v_add3_u32 %[a], %[a], %[b], %[b]")                                                        \
    X(XAD_U32, "v_xad_u32", "v_xad_u32 %[a], %[a], %[b], %[b]")                                                           \
    X(MAX_U32, "v_max_u32", "v_max_u32 %[a], %[a], %[b]")                                                                 \
    X(MOV_DPP_QUAD, "v_mov_b32_dpp quad_perm", "v_mov_b32_dpp %[a], %[a] quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf") \
    X(CVT_F32_I32, "v_cvt_f32_i32", "v_cvt_f32_i32 %[a], %[a]")                                                           \
    X(ADD_U32, "v_add_u32", "v_add_u32 %[a], %[a], %[b]")                                                                 \
    X(MOV_B32, "v_mov_b32", "v_mov_b32 %[a], %[b]")                                                                       \
    X(AND_B32, "v_and_b32", "v_and_b32 %[a], %[a], %[b]")                                                                 \
    X(OR_B32, "v_or_b32", "v_or_b32 %[a], %[a], %[b]")                                                                    \
    X(OR3_B32, "v_or3_b32", "v_or3_b32 %[a], %[a], %[b], %[b]")                                                           \
    X(LSHLREV_B32, "v_lshlrev_b32", "v_lshlrev_b32 %[a], %[b], %[a]")                                                     \
    X(LSHL_ADD_U32, "v_lshl_add_u32", "v_lshl_add_u32 %[a], %[a], 23, %[b]")                                              \
    X(BFE_U32, "v_bfe_u32", "v_bfe_u32 %[a], %[a], 23, 8")                                                                \
    X(MAX3_U32, "v_max3_u32", "v_max3_u32 %[a], %[a], %[b], %[b]")                                                        \
    X(MED3_I32, "v_med3_i32", "v_med3_i32 %[a], %[a], -1, 1")                                                             \
    X(MAD_I32_I16, "v_mad_i32_i16", "v_mad_i32_i16 %[a], %[a], %[b], %[a]")                                               \
    X(MUL_F32, "v_mul_f32", "v_mul_f32 %[a], %[a], %[b]")                                                                 \
    X(SUB_F32, "v_sub_f32", "v_sub_f32 %[a], %[a], %[b]")                                                                 \
    X(MUL_LO_U32, "v_mul_lo_u32", "v_mul_lo_u32 %[a], %[a], %[b]")                                                        \
    X(CNDMASK_B32, "v_cndmask_b32", "v_cndmask_b32 %[a], %[a], %[b], vcc")                                                \
    X(CMP_EQ_U32, "v_cmp_eq_u32", "v_cmp_eq_u32 vcc, %[a], %[b]")                                                         \
    X(PK_MAX_U16, "v_pk_max_u16", "v_pk_max_u16 %[a], %[a], %[b]")                                                        \
    X(PK_MIN_U16, "v_pk_min_u16", "v_pk_min_u16 %[a], %[a], %[b]")                                                        \
    X(PK_MUL_LO_U16, "v_pk_mul_lo_u16", "v_pk_mul_lo_u16 %[a], %[a], %[b]")                                               \
    X(PK_MAD_U16, "v_pk_mad_u16", "v_pk_mad_u16 %[a], %[a], %[b], %[b]")                                                  \
    X(PK_LSHRREV_B16, "v_pk_lshrrev_b16", "v_pk_lshrrev_b16 %[a], 3, %[a] op_sel_hi:[0,1]")                               \
    X(PK_LSHLREV_B16, "v_pk_lshlrev_b16", "v_pk_lshlrev_b16 %[a], 9, %[a] op_sel_hi:[0,1]")                               \
    X(CVT_PK_F32_FP8, "v_cvt_pk_f32_fp8", "v_cvt_pk_f32_fp8 %[a64], %[b]")                                                \
    X(CVT_PK_F32_BF8, "v_cvt_pk_f32_bf8", "v_cvt_pk_f32_bf8 %[a64], %[b]")                                                \
    X(LSHL_ADD_U64, "v_lshl_add_u64", "v_lshl_add_u64 %[a64], %[a64], 0, %[b64]")                                         \
    X(MAD_U64_U32, "v_mad_u64_u32", "v_mad_u64_u32 %[a64], vcc, %[a], %[b], %[a64]")

enum Op : int {
#define MB_ENUM(id, name, text) OP_##id,
    MB_OPS(MB_ENUM)
#undef MB_ENUM
    OP_COUNT
};

const char *const kNames[OP_COUNT] = {
#define MB_NAME(id, name, text) name,
    MB_OPS(MB_NAME)
#undef MB_NAME
};

// a: this chain's 32-bit register; b: a per-lane value; sel: a permute
// selector / constant; a64: this chain's 64-bit pair, b64 a per-lane one,
// for the ops with 64-bit results.  Only a and a64 are written, so the 8
// chains of a lane are independent.
template <int OP>
__device__ __forceinline__ void op(uint32_t &a, const uint32_t b, const uint32_t sel, uint64_t &a64, const uint64_t b64)
{
#define MB_CASE(id, name, text)                                                                          \
    if constexpr (OP == OP_##id)                                                                         \
        asm volatile(text : [a] "+v"(a), [a64] "+v"(a64) : [b] "v"(b), [sel] "s"(sel), [b64] "v"(b64) : "vcc");
    MB_OPS(MB_CASE)
#undef MB_CASE
}

template <int OP>
__global__ __launch_bounds__(256) void issue_kernel(uint32_t *sink, int iters)
{
    uint32_t b = threadIdx.x * 2654435761u + 12345u;
    uint32_t sel = 0x05040100u;
    uint32_t a[CHAINS];
    uint64_t a64[CHAINS];
    uint64_t b64 = (uint64_t)b * 0x9E3779B97F4A7C15ull;
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) {
        a[j] = b ^ (j * 0x9E3779B9u);
        a64[j] = b64 + j;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < CHAINS; ++j) op<OP>(a[j], b, sel, a64[j], b64);
    }
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) x ^= a[j] ^ (uint32_t)a64[j] ^ (uint32_t)(a64[j] >> 32);
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    sink[gid] = x;
}

// The term loop's mix for one pair of products, per chain: two RTZ-style FMAs
// against the binade constant, the byte permute packing their low halves,
// the sign-pair bitop and the 16-bit dot product into the chain's sum.
__global__ __launch_bounds__(256) void term_mix_kernel(uint32_t *sink, int iters)
{
    const uint32_t b = threadIdx.x * 2654435761u + 12345u;
    const uint32_t C = 0x4B400000u;
    float av[CHAINS], bv[CHAINS];
    uint32_t sa[CHAINS], acc[CHAINS];
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) {
        av[j] = (float)((b >> j) & 15u);
        bv[j] = (float)((b >> (j + 4)) & 15u);
        sa[j] = (b & 0x80008000u) ? 0xFFFF0000u : 0x0000FFFFu;
        acc[j] = j;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < CHAINS; ++j) {
                uint32_t r0, r1, p, s;
                asm volatile(
                    "v_fma_f32 %0, |%6|, |%7|, %8\n\t"
                    "v_fma_f32 %1, |%7|, |%6|, %8\n\t"
                    "v_perm_b32 %2, %1, %0, %9\n\t"
                    "v_bitop3_b32 %3, %5, %10, %11 bitop3:0xbe\n\t"
                    "v_dot2c_i32_i16 %4, %2, %3"
                    : "=&v"(r0), "=&v"(r1), "=&v"(p), "=&v"(s), "+v"(acc[j])
                    : "v"(sa[j]), "v"(av[j]), "v"(bv[j]), "v"(C), "s"(0x05040100u), "v"(b), "s"(0x00010001u));
            }
    }
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) x ^= acc[j];
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    sink[gid] = x;
}

// The same mix with both operands of the pair of products as binary16 halves
// of one register each (v_fma_mix_f32 with the low, then the high halves).
__global__ __launch_bounds__(256) void term_mix16_kernel(uint32_t *sink, int iters)
{
    const uint32_t b = threadIdx.x * 2654435761u + 12345u;
    const uint32_t C = 0x4B400000u;
    uint32_t av[CHAINS], bv[CHAINS];
    uint32_t sa[CHAINS], acc[CHAINS];
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) {
        av[j] = (((b >> j) & 15u) << 10) | (((b >> (j + 8)) & 15u) << 26);
        bv[j] = (((b >> (j + 4)) & 15u) << 10) | (((b >> (j + 12)) & 15u) << 26);
        sa[j] = (b & 0x80008000u) ? 0xFFFF0000u : 0x0000FFFFu;
        acc[j] = j;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < CHAINS; ++j) {
                uint32_t r0, r1, p, s;
                asm volatile(
                    "v_fma_mix_f32 %0, |%6|, |%7|, %8 op_sel_hi:[1,1,0]\n\t"
                    "v_fma_mix_f32 %1, |%6|, |%7|, %8 op_sel:[1,1,0] op_sel_hi:[1,1,0]\n\t"
                    "v_perm_b32 %2, %1, %0, %9\n\t"
                    "v_bitop3_b32 %3, %5, %10, %11 bitop3:0xbe\n\t"
                    "v_dot2c_i32_i16 %4, %2, %3"
                    : "=&v"(r0), "=&v"(r1), "=&v"(p), "=&v"(s), "+v"(acc[j])
                    : "v"(sa[j]), "v"(av[j]), "v"(bv[j]), "v"(C), "s"(0x05040100u), "v"(b), "s"(0x00010001u));
            }
    }
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) x ^= acc[j];
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    sink[gid] = x;
}

template <int OP>
hipError_t launch(uint32_t *sink, int iters, int blocks)
{
    hipLaunchKernelGGL(issue_kernel<OP>, dim3(blocks), dim3(256), 0, 0, sink, iters);
    return hipGetLastError();
}

hipError_t launch_op(int opi, uint32_t *sink, int iters, int blocks)
{
    switch (opi) {
#define MB_LAUNCH(id, name, text)                                                                        \
    case OP_##id: return launch<OP_##id>(sink, iters, blocks);
        MB_OPS(MB_LAUNCH)
#undef MB_LAUNCH
    case OP_COUNT:
        hipLaunchKernelGGL(term_mix_kernel, dim3(blocks), dim3(256), 0, 0, sink, iters);
        return hipGetLastError();
    case OP_COUNT + 1:
        hipLaunchKernelGGL(term_mix16_kernel, dim3(blocks), dim3(256), 0, 0, sink, iters);
        return hipGetLastError();
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" {

// Ops 0 .. mb_op_count()-1 are single instructions (32 per loop iteration);
// ops mb_op_count() and mb_op_count()+1 are the term mix with binary32 and
// with binary16 operands (4 * 8 groups of 5 instructions per loop iteration).
__attribute__((visibility("default"))) int mb_op_count(void) { return OP_COUNT; }

__attribute__((visibility("default"))) const char *mb_op_name(int op)
{
    if (op == OP_COUNT) return "term mix: 2 v_fma_f32 + v_perm_b32 + v_bitop3_b32 + v_dot2c_i32_i16";
    if (op == OP_COUNT + 1) return "term mix16: 2 v_fma_mix_f32 + v_perm_b32 + v_bitop3_b32 + v_dot2c_i32_i16";
    return (op >= 0 && op < OP_COUNT) ? kNames[op] : "";
}

// Runs op `op` over `blocks` workgroups of 256 threads, `iters` loop
// iterations per wave, after one untimed launch.  Output: elapsed
// milliseconds of the timed launch (HIP events).  Returns 0, or a hipError_t.
__attribute__((visibility("default"))) int mb_issue_rate(int op, int iters, int blocks, double *ms)
{
    if (op < 0 || op > OP_COUNT + 1 || iters < 1 || blocks < 1) return (int)hipErrorInvalidValue;
    const int64_t threads = (int64_t)blocks * 256;
    uint32_t *sink = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t err = hipMalloc(&sink, threads * sizeof(uint32_t));
    if (err == hipSuccess) err = hipEventCreate(&e0);
    if (err == hipSuccess) err = hipEventCreate(&e1);
    if (err == hipSuccess) err = launch_op(op, sink, iters, blocks);  // warm-up
    if (err == hipSuccess) err = hipEventRecord(e0, 0);
    if (err == hipSuccess) err = launch_op(op, sink, iters, blocks);
    if (err == hipSuccess) err = hipEventRecord(e1, 0);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float f = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&f, e0, e1);
    if (err == hipSuccess) *ms = f;
    if (e0) hipEventDestroy(e0);
    if (e1) hipEventDestroy(e1);
    if (sink) hipFree(sink);
    return (int)err;
}

}  // extern "C"
