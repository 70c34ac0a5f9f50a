// conv_fp32.hip -- fp32 windowed dot product on the vector ALUs (gfx950).
//
// The im2win convolution ("Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support ...", §III-C; fp32 on the non-matrix cores,
// §III-F): every output is the dot product of its window -- for each filter
// column q the R contiguous elements of the CHW window row at column
// w*stride_w + q*dil_w -- with the filter read height before width; the bias
// is added after the sum.  Accumulation is fp32.
//
// When one image's outputs are too few to fill the chip (a 13x13 layer with
// N = 1 has 169 pixels), the channel sum is split into slices whose partial
// sums a second kernel adds in slice order, so results do not depend on
// scheduling.
#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

constexpr int kThreads = 256;
constexpr int kTK = 4;   // output channels per thread (generic kernel)

struct Fp32Args {
    int C, K, R, S, P, Q, sw, dw, pitch;
    int n_images, splits, c_per_split, kgroups;
    FastDiv fdPQ, fdKg, fdQ, fdSplit;
    int64_t total;   // threads doing work
};

// Generic: one thread computes kTK consecutive output channels of one pixel.
__global__ __launch_bounds__(kThreads) void conv_fp32_generic_kernel(
    const float* __restrict__ xw, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ out, Fp32Args a) {
    int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= a.total) return;
    const int PQ = a.P * a.Q;
    uint32_t t = (uint32_t)idx;
    uint32_t t1 = fdiv(t, a.fdPQ);
    int pix = t - t1 * PQ;
    uint32_t t2 = fdiv(t1, a.fdKg);
    int kg = t1 - t2 * a.kgroups;
    uint32_t n = fdiv(t2, a.fdSplit);
    int sidx = t2 - n * a.splits;
    int h = fdiv(pix, a.fdQ);
    int wo = pix - h * a.Q;

    const int k0 = kg * kTK;
    const int c_begin = sidx * a.c_per_split;
    const int c_end = min(a.C, c_begin + a.c_per_split);
    const int RS = a.R * a.S;
    float acc[kTK];
#pragma unroll
    for (int i = 0; i < kTK; ++i) acc[i] = 0.f;

    for (int c = c_begin; c < c_end; ++c) {
        const float* row = xw + (((size_t)n * a.C + c) * a.P + h) * a.pitch +
                           (size_t)wo * a.sw * a.R;
        for (int q = 0; q < a.S; ++q) {
            const float* col = row + q * a.dw * a.R;
            for (int r = 0; r < a.R; ++r) {
                float v = col[r];
#pragma unroll
                for (int i = 0; i < kTK; ++i) {
                    int k = min(k0 + i, a.K - 1);
                    acc[i] = fmaf(v, w[((size_t)k * a.C + c) * RS + r * a.S + q], acc[i]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kTK; ++i) {
        int k = k0 + i;
        if (k >= a.K) break;
        if (a.splits == 1) {
            float v = acc[i];
            if (bias) v += bias[k];
            out[(((size_t)n * a.K + k) * PQ) + pix] = v;
        } else {
            out[((((size_t)sidx * a.n_images + n) * a.K + k) * PQ) + pix] = acc[i];
        }
    }
}

// y = bias + sum over slices, in slice order.
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(const float* __restrict__ part,
                                                                const float* __restrict__ bias,
                                                                float* __restrict__ y,
                                                                int64_t per_split, int splits,
                                                                int PQ, int K) {
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= per_split) return;
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += part[(size_t)s * per_split + i];
    if (bias) v += bias[(i / PQ) % K];
    y[i] = v;
}

}  // namespace

int fp32_splits(const Geom& g, int n_images) {
    // aim for >= 128K threads of work; keep >= 16 channels per slice
    int64_t base = (int64_t)n_images * ((g.K + kTK - 1) / kTK) * g.P * g.Q;
    int64_t want = (131072 + base - 1) / base;
    int64_t maxs = g.C / 16;
    int64_t s = want < maxs ? want : maxs;
    return s < 1 ? 1 : (int)s;
}

hipError_t launch_conv_fp32(const Geom& g, const float* xw, const float* w, const float* bias,
                            float* y, int n_images, float* partials, int splits, bool generic,
                            hipStream_t st) {
    (void)generic;
    Fp32Args a;
    a.C = g.C; a.K = g.K; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
    a.sw = g.sw; a.dw = g.dw; a.pitch = g.pitchA;
    a.n_images = n_images;
    a.splits = splits;
    a.c_per_split = (g.C + splits - 1) / splits;
    a.kgroups = (g.K + kTK - 1) / kTK;
    a.fdPQ = make_fastdiv(g.P * g.Q);
    a.fdKg = make_fastdiv(a.kgroups);
    a.fdQ = make_fastdiv(g.Q);
    a.fdSplit = make_fastdiv(splits);
    a.total = (int64_t)n_images * splits * a.kgroups * g.P * g.Q;
    if (a.total == 0) return hipSuccess;
    if (a.total >= (1ll << 31)) return hipErrorInvalidValue;
    uint32_t blocks = (uint32_t)((a.total + kThreads - 1) / kThreads);
    float* dst = splits == 1 ? y : partials;
    hipLaunchKernelGGL(conv_fp32_generic_kernel, dim3(blocks), dim3(kThreads), 0, st, xw, w,
                       bias, dst, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    int64_t per_split = (int64_t)n_images * g.K * g.P * g.Q;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((uint32_t)((per_split + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, partials, bias, y, per_split, splits, g.P * g.Q,
                       g.K);
    return hipGetLastError();
}

}  // namespace ciw
