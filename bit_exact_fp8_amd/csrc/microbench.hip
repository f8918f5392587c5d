// microbench.hip -- issue-rate microbenchmark of the main kernel's VALU
// instruction mix on gfx950, and the sustained shader clock.
//
// Each op kernel runs 8 independent chains of one instruction per lane, 32
// instructions per loop iteration, with 8 waves on every SIMD (2,048
// workgroups of 256 threads on 256 CUs).  The host times the launch with HIP
// events, which gives lane operations per second over the whole chip; the
// sustained clock comes from the GRBM_GUI_ACTIVE counter of the same
// launches (rocprofv3).  Measurement code only: the GEMM library does not
// use it.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int CHAINS = 8;
constexpr int PER_ITER = 4 * CHAINS;  // instructions per loop iteration

enum Op : int {
    OP_PK_ADD_U16,
    OP_PK_MAXIMUM3_F16,
    OP_DOT2_I32_I16,
    OP_DOT2C_I32_I16,
    OP_FMA_F32,
    OP_PERM_B32,
    OP_BITOP3_B32,
    OP_LSHRREV_B32,
    OP_ADD3_U32,
    OP_XAD_U32,
    OP_MAX_U32,
    OP_MOV_DPP_QUAD,
    OP_CVT_F32_I32,
    OP_COUNT
};

const char *const kNames[OP_COUNT] = {
    "v_pk_add_u16",     "v_pk_maximum3_f16", "v_dot2_i32_i16", "v_dot2c_i32_i16", "v_fma_f32",
    "v_perm_b32",       "v_bitop3_b32",      "v_lshrrev_b32",  "v_add3_u32",      "v_xad_u32",
    "v_max_u32",        "v_mov_b32_dpp quad_perm", "v_cvt_f32_i32"};

template <int OP>
__device__ __forceinline__ void op(uint32_t &a, uint32_t b, uint32_t sel)
{
    if constexpr (OP == OP_PK_ADD_U16) asm volatile("v_pk_add_u16 %0, %0, %1" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_PK_MAXIMUM3_F16) asm volatile("v_pk_maximum3_f16 %0, %0, %1, %1" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_DOT2_I32_I16) asm volatile("v_dot2_i32_i16 %0, %1, %1, %0" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_DOT2C_I32_I16) asm volatile("v_dot2c_i32_i16 %0, %1, %1" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_FMA_F32) asm volatile("v_fma_f32 %0, |%1|, |%1|, %0" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_PERM_B32) asm volatile("v_perm_b32 %0, %1, %0, %2" : "+v"(a) : "v"(b), "s"(sel));
    if constexpr (OP == OP_BITOP3_B32) asm volatile("v_bitop3_b32 %0, %0, %1, %1 bitop3:0x6c" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_LSHRREV_B32) asm volatile("v_lshrrev_b32 %0, %1, %0" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_ADD3_U32) asm volatile("v_add3_u32 %0, %0, %1, %1" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_XAD_U32) asm volatile("v_xad_u32 %0, %0, %1, %1" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_MAX_U32) asm volatile("v_max_u32 %0, %0, %1" : "+v"(a) : "v"(b));
    if constexpr (OP == OP_MOV_DPP_QUAD)
        asm volatile("v_mov_b32_dpp %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "+v"(a));
    if constexpr (OP == OP_CVT_F32_I32) asm volatile("v_cvt_f32_i32 %0, %0" : "+v"(a));
}

template <int OP>
__global__ __launch_bounds__(256) void issue_kernel(uint32_t *sink, int iters)
{
    const uint32_t b = threadIdx.x * 2654435761u + 12345u;
    const uint32_t sel = 0x05040100u;
    uint32_t a[CHAINS];
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) a[j] = b ^ (j * 0x9E3779B9u);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < CHAINS; ++j) op<OP>(a[j], b, sel);
    }
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) x ^= a[j];
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
    case OP_PK_ADD_U16: return launch<OP_PK_ADD_U16>(sink, iters, blocks);
    case OP_PK_MAXIMUM3_F16: return launch<OP_PK_MAXIMUM3_F16>(sink, iters, blocks);
    case OP_DOT2_I32_I16: return launch<OP_DOT2_I32_I16>(sink, iters, blocks);
    case OP_DOT2C_I32_I16: return launch<OP_DOT2C_I32_I16>(sink, iters, blocks);
    case OP_FMA_F32: return launch<OP_FMA_F32>(sink, iters, blocks);
    case OP_PERM_B32: return launch<OP_PERM_B32>(sink, iters, blocks);
    case OP_BITOP3_B32: return launch<OP_BITOP3_B32>(sink, iters, blocks);
    case OP_LSHRREV_B32: return launch<OP_LSHRREV_B32>(sink, iters, blocks);
    case OP_ADD3_U32: return launch<OP_ADD3_U32>(sink, iters, blocks);
    case OP_XAD_U32: return launch<OP_XAD_U32>(sink, iters, blocks);
    case OP_MAX_U32: return launch<OP_MAX_U32>(sink, iters, blocks);
    case OP_MOV_DPP_QUAD: return launch<OP_MOV_DPP_QUAD>(sink, iters, blocks);
    case OP_CVT_F32_I32: return launch<OP_CVT_F32_I32>(sink, iters, blocks);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int mb_op_count(void) { return OP_COUNT; }

__attribute__((visibility("default"))) const char *mb_op_name(int op)
{
    return (op >= 0 && op < OP_COUNT) ? kNames[op] : "";
}

// Runs op `op` over `blocks` workgroups of 256 threads, `iters` loop
// iterations (32 instructions each) per wave, after one untimed launch.
// Output: elapsed milliseconds of the timed launch (HIP events).  Returns 0,
// or a hipError_t.
__attribute__((visibility("default"))) int mb_issue_rate(int op, int iters, int blocks, double *ms)
{
    if (op < 0 || op >= OP_COUNT || iters < 1 || blocks < 1) return (int)hipErrorInvalidValue;
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
