// conv_implicit_f16.hip -- the in-LDS window contraction for f16 inputs
// (outputs of the input type or fp32); kernels from conv_implicit_impl.hpp.
#include "conv_implicit_impl.hpp"

namespace ciw {

hipError_t launch_conv_implicit_f16(const Geom& g, ciw_dtype out, const void* x,
                                    const void* aperm, const void* bias, void* y, const Epi& epi,
                                    hipStream_t st) {
    MfImpPlan pl;
    if (!mf_imp_plan(g, elem_bytes(out), epi, device_cus(), pl)) return hipErrorInvalidValue;
    return out == CIW_F32 ? launch_imp_t<half_t, float>(pl, x, aperm, bias, y, st)
                          : launch_imp_t<half_t, half_t>(pl, x, aperm, bias, y, st);
}

}  // namespace ciw
