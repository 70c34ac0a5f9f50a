// conv_dw.hip -- depthwise (groups = C) windowed dot product (gfx950).
//
// Each channel has its own R x S filter; output (n, c, h, w) is the dot
// product of the CHW window row (n, c, h) at columns w*stride_w + q*dil_w
// (R contiguous values each) with that filter, plus the bias, accumulated in
// fp32.  Nine multiply-adds per output against 4 bytes in and 4 bytes out:
// the kernel is bound by HBM bandwidth, not arithmetic ("Diagonalwise
// Refactorization: An Efficient Training Method for Depthwise Convolutions"
// reports the same imbalance for depthwise layers).
#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

constexpr int kThreads = 256;

struct DwArgs {
    int C, R, S, P, Q, sw, dw, pitch;
    FastDiv fdQ, fdP, fdC;
    int64_t total;
};

template <typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads) void conv_dw_generic_kernel(
    const TIn* __restrict__ xw, const TIn* __restrict__ w, const TIn* __restrict__ bias,
    TOut* __restrict__ y, DwArgs a) {
    int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= a.total) return;
    uint32_t t = (uint32_t)idx;
    uint32_t t1 = fdiv(t, a.fdQ);
    int wo = t - t1 * a.Q;
    uint32_t t2 = fdiv(t1, a.fdP);
    int h = t1 - t2 * a.P;
    uint32_t n = fdiv(t2, a.fdC);
    int c = t2 - n * a.C;
    const TIn* row = xw + (((size_t)n * a.C + c) * a.P + h) * a.pitch + (size_t)wo * a.sw * a.R;
    const TIn* f = w + (size_t)c * a.R * a.S;
    float acc = 0.f;
    for (int q = 0; q < a.S; ++q)
        for (int r = 0; r < a.R; ++r)
            acc = fmaf(to_f32(row[q * a.dw * a.R + r]), to_f32(f[r * a.S + q]), acc);
    if (bias) acc += to_f32(bias[c]);
    y[idx] = from_f32<TOut>(acc);
}

template <typename TIn, typename TOut>
hipError_t launch_t(const Geom& g, const void* xw, const void* w, const void* bias, void* y,
                    int n_images, hipStream_t st) {
    DwArgs a;
    a.C = g.C; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
    a.sw = g.sw; a.dw = g.dw; a.pitch = g.pitchA;
    a.fdQ = make_fastdiv(g.Q);
    a.fdP = make_fastdiv(g.P);
    a.fdC = make_fastdiv(g.C);
    a.total = (int64_t)n_images * g.C * g.P * g.Q;
    if (a.total == 0) return hipSuccess;
    if (a.total >= (1ll << 31)) return hipErrorInvalidValue;
    uint32_t blocks = (uint32_t)((a.total + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((conv_dw_generic_kernel<TIn, TOut>), dim3(blocks), dim3(kThreads), 0, st,
                       (const TIn*)xw, (const TIn*)w, (const TIn*)bias, (TOut*)y, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_dw(const Geom& g, ciw_dtype in, ciw_dtype out, const void* xw,
                          const void* w, const void* bias, void* y, int n_images,
                          bool generic, hipStream_t st) {
    (void)generic;
    if (in == CIW_F32) return launch_t<float, float>(g, xw, w, bias, y, n_images, st);
    if (in == CIW_F16)
        return out == CIW_F32 ? launch_t<half_t, float>(g, xw, w, bias, y, n_images, st)
                              : launch_t<half_t, half_t>(g, xw, w, bias, y, n_images, st);
    return out == CIW_F32 ? launch_t<bf16_t, float>(g, xw, w, bias, y, n_images, st)
                          : launch_t<bf16_t, bf16_t>(g, xw, w, bias, y, n_images, st);
}

}  // namespace ciw
