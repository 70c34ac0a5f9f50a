// conv_band_f16.hip -- the band kernel for f16 inputs (outputs of the input
// type or fp32); kernels from conv_band_impl.hpp.
#include "conv_band_impl.hpp"

namespace ciw {

hipError_t launch_conv_band_f16(const Geom& g, ciw_dtype out, const void* x, const void* w,
                                const void* bias, void* y, const Epi& epi, hipStream_t st) {
    BandPlan pl;
    if (!band_plan(g, elem_bytes(out), epi, device_cus(), pl)) return hipErrorInvalidValue;
    return out == CIW_F32 ? launch_band_t<half_t, float>(pl, x, w, bias, y, st)
                          : launch_band_t<half_t, half_t>(pl, x, w, bias, y, st);
}

}  // namespace ciw
