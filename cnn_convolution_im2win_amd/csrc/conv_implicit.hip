// conv_implicit.hip -- entry points of the fp16/bf16 contraction that builds
// its window rows in LDS from x (kernels and plan in conv_implicit_impl.hpp):
// eligibility, workspace (the re-laid-out filter), the filter re-layout and
// dispatch by input type to the per-type files.
#include "conv_implicit_impl.hpp"

namespace ciw {

hipError_t launch_conv_implicit_f16(const Geom& g, ciw_dtype out, const void* x,
                                    const void* aperm, const void* bias, void* y, const Epi& epi,
                                    hipStream_t st);
hipError_t launch_conv_implicit_bf16(const Geom& g, ciw_dtype out, const void* x,
                                     const void* aperm, const void* bias, void* y, const Epi& epi,
                                     hipStream_t st);

size_t implicit_workspace_bytes(const Geom& g, ciw_dtype out, const Epi& epi) {
    MfImpPlan pl;
    if (!mf_imp_plan(g, elem_bytes(out), epi, 256, pl)) return 0;
    return (size_t)2 * pl.steps * 512 * sizeof(uint16_t);
}

hipError_t launch_conv_implicit(const Geom& g, ciw_dtype in, ciw_dtype out, const void* x,
                                const void* w, const void* bias, void* y, void* ws,
                                const Epi& epi, hipStream_t st) {
    MfImpPlan pl;
    if (!mf_imp_plan(g, elem_bytes(out), epi, 256, pl)) return hipErrorInvalidValue;
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
