// conv_narrow.hip -- entry points of the in-LDS contraction for fp16/bf16
// layers with few input channels and an even horizontal stride
// (conv_narrow_impl.hpp): eligibility and dispatch by input and output type.
#include "conv_narrow_impl.hpp"

namespace ciw {

bool narrow_supported(const Geom& g, ciw_dtype out, const Epi& epi) {
    NarrowPlan pl;
    return narrow_plan(g, elem_bytes(out), epi, 256, pl);   // eligibility does not depend on the CU count
}

hipError_t launch_conv_narrow(const Geom& g, ciw_dtype in, ciw_dtype out, const void* x, const void* w,
                              const void* bias, void* y, const Epi& epi, hipStream_t st) {
    NarrowPlan pl;
    if (!narrow_plan(g, elem_bytes(out), epi, 256, pl)) return hipErrorInvalidValue;
    if (g.N == 0) return hipSuccess;
    if (in == CIW_F16)
        return out == CIW_F32 ? launch_narrow_t<half_t, float>(pl, x, w, bias, y, st)
                              : launch_narrow_t<half_t, half_t>(pl, x, w, bias, y, st);
    return out == CIW_F32 ? launch_narrow_t<bf16_t, float>(pl, x, w, bias, y, st)
                          : launch_narrow_t<bf16_t, bf16_t>(pl, x, w, bias, y, st);
}

}  // namespace ciw
