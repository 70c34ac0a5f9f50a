// conv_narrow.hip -- entry points of the in-LDS contraction for fp16/bf16
// layers with few input channels and an even horizontal stride
// (conv_narrow_impl.hpp): eligibility and dispatch by input type to the
// per-type files.
#include "conv_narrow_impl.hpp"

namespace ciw {

hipError_t launch_conv_narrow_f16(const Geom& g, ciw_dtype out, const void* x, const void* w,
                                  const void* bias, void* y, const Epi& epi, hipStream_t st);
hipError_t launch_conv_narrow_bf16(const Geom& g, ciw_dtype out, const void* x, const void* w,
                                   const void* bias, void* y, const Epi& epi, hipStream_t st);

bool narrow_supported(const Geom& g, ciw_dtype out, const Epi& epi) {
    NarrowPlan pl;
    return narrow_plan(g, elem_bytes(out), epi, 256, pl);   // eligibility does not depend on the CU count
}

hipError_t launch_conv_narrow(const Geom& g, ciw_dtype in, ciw_dtype out, const void* x, const void* w,
                              const void* bias, void* y, const Epi& epi, hipStream_t st) {
    if (!narrow_supported(g, out, epi)) return hipErrorInvalidValue;
    if (g.N == 0) return hipSuccess;
    return in == CIW_F16 ? launch_conv_narrow_f16(g, out, x, w, bias, y, epi, st)
                         : launch_conv_narrow_bf16(g, out, x, w, bias, y, epi, st);
}

}  // namespace ciw
