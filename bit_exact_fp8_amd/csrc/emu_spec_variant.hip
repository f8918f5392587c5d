// emu_spec_variant.hip -- the exponent-speculation kernels (guess, block
// words, walk) of one block width EMU_VARIANT_BLK and format pair
// EMU_VARIANT_XF, EMU_VARIANT_WF.  A translation unit of their own: compiled
// together with the other main-kernel instantiations they changed those
// kernels' register assignment (and speed) through module-wide decisions.
#include "emu_main_kernel.h"

#if !defined(EMU_VARIANT_BLK) || !defined(EMU_VARIANT_XF) || !defined(EMU_VARIANT_WF)
#error "define EMU_VARIANT_BLK, EMU_VARIANT_XF and EMU_VARIANT_WF"
#endif

namespace emu {
template hipError_t launch_variant_spec<EMU_VARIANT_BLK, EMU_VARIANT_XF, EMU_VARIANT_WF>(int, int, const MainParams &,
                                                                                          int, hipStream_t);
}  // namespace emu
