// conv_implicit.hip -- entry points of the fp16/bf16 contractions that build
// their window rows in LDS from x: the band kernel (conv_band_impl.hpp: 3x3
// filters, no pool; no workspace) where it runs the layer, otherwise the
// row-band kernel of conv_implicit_impl.hpp (workspace: the re-laid-out
// filter, written by a kernel before the contraction), otherwise the
// few-channel kernel of conv_narrow_impl.hpp (no workspace).  Eligibility,
// workspace and dispatch by input type to the per-type files.
#include "conv_band_impl.hpp"

// CIW_BAND_OFF: always take the row-band kernel (the ablation builds of that
// kernel set it, so they measure the kernel their switches change); 0 in the
// library
#ifndef CIW_BAND_OFF
#define CIW_BAND_OFF 0
#endif

namespace ciw {

hipError_t launch_conv_implicit_f16(const Geom& g, ciw_dtype out, const void* x,
                                    const void* aperm, const void* bias, void* y, const Epi& epi,
                                    hipStream_t st);
hipError_t launch_conv_implicit_bf16(const Geom& g, ciw_dtype out, const void* x,
                                     const void* aperm, const void* bias, void* y, const Epi& epi,
                                     hipStream_t st);
hipError_t launch_conv_band_f16(const Geom& g, ciw_dtype out, const void* x, const void* w,
                                const void* bias, void* y, const Epi& epi, hipStream_t st);
hipError_t launch_conv_band_bf16(const Geom& g, ciw_dtype out, const void* x, const void* w,
                                 const void* bias, void* y, const Epi& epi, hipStream_t st);

bool implicit_workspace(const Geom& g, ciw_dtype out, const Epi& epi, size_t* bytes) {
    BandPlan bp;
    if (!CIW_BAND_OFF && band_plan(g, elem_bytes(out), epi, 256, bp)) {   // eligibility does not depend on the CU count
        *bytes = 0;
        return true;
    }
    MfImpPlan pl;
    if (mf_imp_plan(g, elem_bytes(out), epi, 256, pl)) {
        *bytes = (size_t)2 * pl.steps * 512 * sizeof(uint16_t);
        return true;
    }
    if (!narrow_supported(g, out, epi)) return false;
    *bytes = 0;
    return true;
}

hipError_t launch_conv_implicit(const Geom& g, ciw_dtype in, ciw_dtype out, const void* x,
                                const void* w, const void* bias, void* y, void* ws,
                                const Epi& epi, hipStream_t st) {
    BandPlan bp;
    if (!CIW_BAND_OFF && band_plan(g, elem_bytes(out), epi, 256, bp)) {
        if (g.N == 0) return hipSuccess;
        return in == CIW_F16 ? launch_conv_band_f16(g, out, x, w, bias, y, epi, st)
                             : launch_conv_band_bf16(g, out, x, w, bias, y, epi, st);
    }
    MfImpPlan pl;
    if (!mf_imp_plan(g, elem_bytes(out), epi, 256, pl))
        return launch_conv_narrow(g, in, out, x, w, bias, y, epi, st);
    ImpPermArgs p;
    p.C = g.C; p.K = g.K; p.R = g.R; p.S = g.S; p.CB = pl.CB; p.steps = pl.steps;
    p.total = (uint32_t)(2 * pl.steps * 512);
    hipLaunchKernelGGL(mfma_implicit_filter_kernel, dim3((p.total + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, st, (const uint16_t*)w, (uint16_t*)ws, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (g.N == 0) return hipSuccess;
    return in == CIW_F16 ? launch_conv_implicit_f16(g, out, x, ws, bias, y, epi, st)
                         : launch_conv_implicit_bf16(g, out, x, ws, bias, y, epi, st);
}

}  // namespace ciw
