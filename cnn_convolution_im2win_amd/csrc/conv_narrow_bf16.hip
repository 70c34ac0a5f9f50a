// conv_narrow_bf16.hip -- bf16 instantiations of the few-channel in-LDS kernel
// (conv_narrow_impl.hpp), one per reduction-step count and output type.
#include "conv_narrow_impl.hpp"

namespace ciw {

hipError_t launch_conv_narrow_bf16(const Geom& g, ciw_dtype out, const void* x, const void* w,
                                 const void* bias, void* y, const Epi& epi, hipStream_t st) {
    NarrowPlan pl;
    if (!narrow_plan(g, elem_bytes(out), epi, 256, pl)) return hipErrorInvalidValue;
    return out == CIW_F32 ? launch_narrow_t<bf16_t, float>(pl, x, w, bias, y, st)
                          : launch_narrow_t<bf16_t, bf16_t>(pl, x, w, bias, y, st);
}

}  // namespace ciw
