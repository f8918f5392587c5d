// emu_noalloc.hip -- emu_scaled_mm_noalloc: emu_scaled_mm for callers that
// cannot allocate device memory (code under stream capture, tight serving
// loops, harnesses that forbid hipMalloc).  The split partials, stored
// slow-mode chunk results and infinity lists that emu_scaled_mm keeps in the
// caller's workspace live here in a fixed array in the code object's device
// memory, one copy per GPU, held until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/emu_fp8gemm.h"
#include "emu_internal.h"

namespace {

// The scratch: EMU_NOALLOC_SCRATCH_BYTES per device.  Every call on one GPU
// uses that GPU's copy; no kernel reads a scratch byte that the same call has
// not written first, so nothing in it needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[EMU_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Per device: the scratch address that hipGetSymbolAddress gives with that
// device current (the array's name is only a host-side stand-in), looked up
// once, on the first call with the device current.
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_slots[kMaxDevices];

void *scratch_of_current_device(size_t *bytes, std::string *err)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = std::string("hipGetDevice: ") + hipGetErrorString(e);
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = "device index beyond the scratch table";
        return nullptr;
    }
    ScratchSlot &slot = g_slots[dev];
    std::call_once(slot.once, [&slot] {
        void *p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        slot.ptr = slot.err == hipSuccess ? p : nullptr;
    });
    if (slot.err != hipSuccess || !slot.ptr) {
        *err = std::string("hipGetSymbolAddress of the scratch: ") + hipGetErrorString(slot.err);
        return nullptr;
    }
    *bytes = EMU_NOALLOC_SCRATCH_BYTES;
    return slot.ptr;
}

}  // namespace

extern "C" {

emu_status emu_scaled_mm_noalloc(const uint8_t *x, emu_fp8_format x_fmt, int64_t ldx, const uint8_t *w,
                                 emu_fp8_format w_fmt, int64_t ldw, int64_t M, int64_t N, int64_t K,
                                 const float *scale_x, const float *scale_w, const float *scale_result, void *out,
                                 emu_out_dtype out_dtype, int64_t ldo, int fast_accum, int split_S,
                                 emu_profile profile, hipStream_t stream, const emu_plan_options *plan)
{
    return emu::scaled_mm_in_scratch(x, x_fmt, ldx, w, w_fmt, ldw, M, N, K, scale_x, scale_w, scale_result, out,
                                     out_dtype, ldo, fast_accum, split_S, profile, scratch_of_current_device,
                                     EMU_NOALLOC_SCRATCH_BYTES, stream, plan);
}

}  // extern "C"
