// conv_mfma.hip -- entry points of the fp16/bf16 matrix-core contraction:
// workspace size and launch of the filter re-layout, and dispatch by input
// type to the per-type files (kernels and plan in conv_mfma_impl.hpp).
#include "conv_mfma_impl.hpp"

namespace ciw {

hipError_t launch_conv_mfma_f16(const Geom& g, ciw_dtype out, const void* xw, const void* w,
                                const void* aperm, const void* bias, void* y, int n_images,
                                bool generic, const Epi& epi, hipStream_t st);
hipError_t launch_conv_mfma_bf16(const Geom& g, ciw_dtype out, const void* xw, const void* w,
                                 const void* aperm, const void* bias, void* y, int n_images,
                                 bool generic, const Epi& epi, hipStream_t st);

size_t mfma_prep_bytes(const Geom& g) {
    MfRowPlan pl;
    // the plan with 4-byte outputs needs the most LDS; size for any output type
    if (!mf_row_plan(g, 2, pl) && !mf_row_plan(g, 4, pl)) return 0;
    return (size_t)pl.a.nph * 64 * pl.steps * 16 * sizeof(uint16_t);
}

hipError_t launch_mfma_prep(const Geom& g, ciw_dtype out, const void* w, void* aperm,
                            hipStream_t st) {
    MfRowPlan pl;
    if (!mf_row_plan(g, elem_bytes(out), pl)) return hipSuccess;   // generic kernel: no prep
    if (CIW_ABLATE_ROWS_NO_INDEX) return hipSuccess;                // the kernel gathers itself
    PermArgs p;
    p.C = g.C; p.K = g.K; p.R = g.R; p.S = g.S;
    p.D = pl.a.D; p.T = pl.a.T; p.steps = pl.steps;
    p.fdSteps = make_fastdiv(pl.steps);
    p.fdC = make_fastdiv(g.C);
    p.fdR = make_fastdiv(g.R);
    p.total = (uint32_t)(pl.a.nph * 2 * pl.steps * 512);
    hipLaunchKernelGGL(mfma_filter_perm_kernel, dim3((p.total + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, st, (const uint16_t*)w, (uint16_t*)aperm, p);
    return hipGetLastError();
}

hipError_t launch_conv_mfma(const Geom& g, ciw_dtype in, ciw_dtype out, const void* xw,
                            const void* w, const void* aperm, const void* bias, void* y,
                            int n_images, bool generic, const Epi& epi, hipStream_t st) {
    return in == CIW_F16
               ? launch_conv_mfma_f16(g, out, xw, w, aperm, bias, y, n_images, generic, epi, st)
               : launch_conv_mfma_bf16(g, out, xw, w, aperm, bias, y, n_images, generic, epi, st);
}

}  // namespace ciw
