// emu_cin_variant.hip -- fast accumulation from incoming accumulators (the
// main kernel's ACC_FAST_CIN instantiations, every tile configuration) for
// one block width EMU_VARIANT_BLK and format pair EMU_VARIANT_XF,
// EMU_VARIANT_WF.  A translation unit of its own, so that these kernels
// cannot change the code of the other main-kernel instantiations.
#include "emu_main_kernel.h"

#if !defined(EMU_VARIANT_BLK) || !defined(EMU_VARIANT_XF) || !defined(EMU_VARIANT_WF)
#error "define EMU_VARIANT_BLK, EMU_VARIANT_XF and EMU_VARIANT_WF"
#endif

namespace emu {
template hipError_t launch_variant_cin<EMU_VARIANT_BLK, EMU_VARIANT_XF, EMU_VARIANT_WF>(int, const MainParams &,
                                                                                         hipStream_t);
}  // namespace emu
