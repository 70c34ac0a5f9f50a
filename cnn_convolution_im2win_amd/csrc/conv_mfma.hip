// conv_mfma.hip -- fp16/bf16 windowed contraction on the gfx950 matrix cores.
//
// The im2win paper ("Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support ...", §III-D) maps the output to a matrix product
// with M = output channels and N = images x output rows x output columns,
// reducing over the window.  With the HWC window layout the window of output
// (n, h, w) is, for each filter column q, the R*C contiguous elements at
// column w*stride_w + q*dil_w of row (n, h); with dil_w = 1 the whole window
// (S*R*C elements) is one contiguous run.  The reduction index is
// t = (q*R + r)*C + c and the filter operand is F[k][c][r][q] ("height before
// width", §III-C).  Products are exact in fp32 and accumulate in fp32
// (§III-F); the bias is added in fp32 and the result rounded once.
#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMB = 64;       // output channels per workgroup
constexpr int kNB = 64;       // pixels per workgroup
constexpr int kKB = 32;       // reduction step (one 16x16x32 MFMA)
constexpr int kLdsRow = 40;   // 32 + 8 halves: rows 80 B apart

struct MfmaArgs {
    int C, K, R, S, P, Q, sw, dw, pitch;
    int T, RC, npix;
    FastDiv fdRC, fdC, fdPQ, fdQ;
};

template <typename TIn>
__device__ __forceinline__ f32x4 mfma16x16x32(const uint16_t* a, const uint16_t* b, f32x4 acc);

template <>
__device__ __forceinline__ f32x4 mfma16x16x32<half_t>(const uint16_t* a, const uint16_t* b,
                                                      f32x4 acc) {
    f16x8 va = *reinterpret_cast<const f16x8*>(a);
    f16x8 vb = *reinterpret_cast<const f16x8*>(b);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(va, vb, acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mfma16x16x32<bf16_t>(const uint16_t* a, const uint16_t* b,
                                                      f32x4 acc) {
    bf16x8 va = *reinterpret_cast<const bf16x8*>(a);
    bf16x8 vb = *reinterpret_cast<const bf16x8*>(b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, vb, acc, 0, 0, 0);
}

// Generic tile kernel: 64 output channels x 64 pixels per workgroup, four
// waves each owning a 32x32 quadrant (2x2 MFMA tiles).  Operands go through
// LDS one 32-wide reduction step at a time.
template <typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads) void conv_mfma_generic_kernel(
    const uint16_t* __restrict__ xw, const uint16_t* __restrict__ w,
    const TIn* __restrict__ bias, TOut* __restrict__ y, MfmaArgs a) {
    __shared__ __align__(16) uint16_t As[kMB * kLdsRow];
    __shared__ __align__(16) uint16_t Bs[kNB * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int k0 = blockIdx.y * kMB;
    const int p0 = blockIdx.x * kNB;

    // loader role: row (filter or pixel) and 8-element slot of the step
    const int lrow = tid >> 2;
    const int lslot = (tid & 3) * 8;
    const int kload = k0 + lrow;
    const int pload = p0 + lrow;
    // per-thread window base of its pixel (index precomputation)
    int64_t bbase = -1;
    if (pload < a.npix) {
        uint32_t n = fdiv(pload, a.fdPQ);
        int pix = pload - n * (a.P * a.Q);
        int h = fdiv(pix, a.fdQ);
        int wo = pix - h * a.Q;
        bbase = ((int64_t)n * a.P + h) * a.pitch + (int64_t)wo * a.sw * a.RC;
    }

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wm = wave >> 1, wn = wave & 1;
    for (int t0 = 0; t0 < a.T; t0 += kKB) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int t = t0 + lslot + i;
            uint16_t av = 0, bv = 0;
            if (t < a.T) {
                uint32_t q = fdiv(t, a.fdRC);
                int rc = t - q * a.RC;
                uint32_t r = fdiv(rc, a.fdC);
                int c = rc - r * a.C;
                if (kload < a.K) av = w[(((int64_t)kload * a.C + c) * a.R + r) * a.S + q];
                if (bbase >= 0) bv = xw[bbase + (int64_t)q * a.dw * a.RC + rc];
            }
            As[lrow * kLdsRow + lslot + i] = av;
            Bs[lrow * kLdsRow + lslot + i] = bv;
        }
        __syncthreads();
        const int kq = (lane >> 4) * 8;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                acc[mi][ni] = mfma16x16x32<TIn>(
                    &As[(wm * 32 + mi * 16 + (lane & 15)) * kLdsRow + kq],
                    &Bs[(wn * 32 + ni * 16 + (lane & 15)) * kLdsRow + kq], acc[mi][ni]);
        __syncthreads();
    }

    // epilogue: lane holds D[4*(lane/16) + i][lane % 16] of each 16x16 tile
    const int PQ = a.P * a.Q;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        int p = p0 + wn * 32 + ni * 16 + (lane & 15);
        if (p >= a.npix) continue;
        uint32_t n = fdiv(p, a.fdPQ);
        int pix = p - n * PQ;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int k = k0 + wm * 32 + mi * 16 + (lane >> 4) * 4 + i;
                if (k >= a.K) continue;
                float v = acc[mi][ni][i];
                if (bias) v += to_f32(bias[k]);
                y[((int64_t)n * a.K + k) * PQ + pix] = from_f32<TOut>(v);
            }
    }
}

template <typename TIn, typename TOut>
hipError_t launch_t(const Geom& g, const void* xw, const void* w, const void* bias, void* y,
                    int n_images, hipStream_t st) {
    MfmaArgs a;
    a.C = g.C; a.K = g.K; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
    a.sw = g.sw; a.dw = g.dw; a.pitch = g.pitchB;
    a.RC = g.R * g.C;
    a.T = g.S * a.RC;
    a.npix = n_images * g.P * g.Q;
    a.fdRC = make_fastdiv(a.RC);
    a.fdC = make_fastdiv(g.C);
    a.fdPQ = make_fastdiv(g.P * g.Q);
    a.fdQ = make_fastdiv(g.Q);
    dim3 grid((a.npix + kNB - 1) / kNB, (g.K + kMB - 1) / kMB);
    if (a.npix == 0) return hipSuccess;
    hipLaunchKernelGGL((conv_mfma_generic_kernel<TIn, TOut>), grid, dim3(kThreads), 0, st,
                       (const uint16_t*)xw, (const uint16_t*)w, (const TIn*)bias, (TOut*)y, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_mfma(const Geom& g, ciw_dtype in, ciw_dtype out, const void* xw,
                            const void* w, const void* bias, void* y, int n_images,
                            bool generic, hipStream_t st) {
    (void)generic;
    if (in == CIW_F16)
        return out == CIW_F32 ? launch_t<half_t, float>(g, xw, w, bias, y, n_images, st)
                              : launch_t<half_t, half_t>(g, xw, w, bias, y, n_images, st);
    return out == CIW_F32 ? launch_t<bf16_t, float>(g, xw, w, bias, y, n_images, st)
                          : launch_t<bf16_t, bf16_t>(g, xw, w, bias, y, n_images, st);
}

}  // namespace ciw
