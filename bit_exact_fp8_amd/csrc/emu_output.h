// emu_output.h -- the epilogue and store of one output, shared by the main
// and the combine kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "emu_internal.h"
#include "fp_round.h"

namespace emu {

// Binary32 bits of scale_result (1.0 when there is none).
__device__ __forceinline__ uint32_t scale_result_bits(const float *sr)
{
    return sr ? __float_as_uint(*sr) : 0x3F800000u;
}

// out[idx] for accumulator acc: alpha = RN32(sx * sw) (limitations page,
// corrections table: y32 is one fused multiply-add of acc and alpha with a
// +0 addend, rounded once; validation page, claims table: bf16 / fp16
// rounded from the binary32 value, FP8
// outputs take scale_result as a separate binary32 multiplication and
// saturate).  RN32(y32 * 1) = y32, so sr = 1.0 stands for no scale_result.
__device__ __forceinline__ void store_epilogue(int out_kind, void *out, int64_t idx, uint32_t acc,
                                               uint32_t alpha, uint32_t sr)
{
    if (out_kind == OUT_ACC_F32) {
        reinterpret_cast<uint32_t *>(out)[idx] = canon_f32(acc);
        return;
    }
    const uint32_t y = epilogue_f32(acc, alpha);
    switch (out_kind) {
    case OUT_BF16: reinterpret_cast<uint16_t *>(out)[idx] = f32_to_bf16(y); break;
    case OUT_F16: reinterpret_cast<uint16_t *>(out)[idx] = f32_to_f16(y); break;
    case OUT_F32: reinterpret_cast<uint32_t *>(out)[idx] = canon_f32(y); break;
    case OUT_E4M3: reinterpret_cast<uint8_t *>(out)[idx] = f32_to_fp8_sat<true>(mul_f32(y, sr)); break;
    default: reinterpret_cast<uint8_t *>(out)[idx] = f32_to_fp8_sat<false>(mul_f32(y, sr)); break;
    }
}

}  // namespace emu
