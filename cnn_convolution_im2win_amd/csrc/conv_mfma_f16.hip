// conv_mfma_f16.hip -- the matrix-core contraction for f16 inputs
// (outputs of the input type or fp32); kernels from conv_mfma_impl.hpp.
#include "conv_mfma_impl.hpp"

namespace ciw {

hipError_t launch_conv_mfma_f16(const Geom& g, ciw_dtype out, const void* xw, const void* w,
                                 const void* aperm, const void* bias, void* y, int n_images,
                                 bool generic, const Epi& epi, hipStream_t st) {
#if CIW_ROWS_ABLATION_ONLY
    if (out == CIW_F32) return hipErrorNotSupported;
    return launch_t<half_t, half_t>(g, xw, w, aperm, bias, y, n_images, generic, epi, st);
#else
    return out == CIW_F32 ? launch_t<half_t, float>(g, xw, w, aperm, bias, y, n_images, generic, epi, st)
                          : launch_t<half_t, half_t>(g, xw, w, aperm, bias, y, n_images, generic, epi, st);
#endif
}

}  // namespace ciw
