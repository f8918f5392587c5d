// emu_variant.hip -- one instantiation of the main kernel: block width
// EMU_VARIANT_BLK (32 or 16) and x / w formats EMU_VARIANT_XF, EMU_VARIANT_WF
// (0 = e4m3fn, 1 = e5m2), all tile configurations.  The build compiles this
// file once per variant, in parallel.
#include "emu_main_kernel.h"

#if !defined(EMU_VARIANT_BLK) || !defined(EMU_VARIANT_XF) || !defined(EMU_VARIANT_WF)
#error "define EMU_VARIANT_BLK, EMU_VARIANT_XF and EMU_VARIANT_WF"
#endif

namespace emu {
template hipError_t launch_variant<EMU_VARIANT_BLK, EMU_VARIANT_XF, EMU_VARIANT_WF>(int, const MainParams &, int,
                                                                                     hipStream_t);
}  // namespace emu
