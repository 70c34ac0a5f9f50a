// internal.hpp -- shared declarations of the im2win library (host + device).
//
// Geometry, kernel argument blocks and the launchers each kernel file
// exports.  Nothing here is part of the C ABI (include/conv_im2win.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "conv_im2win.h"

namespace ciw {

// Unsigned division by a divisor fixed at launch time, as a multiply-high and
// a shift (Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication", 1994, the round-up variant).  Valid for n < 2^31.
// The host precomputes (m, s) once per launch -- the "index precomputation"
// of the im2win paper §III-E1 -- so kernels never issue an integer divide.
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f{d, 0u, 0u};
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.s = s;
    f.m = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1ull);
    return f;
}

__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t hi = __umulhi(n, f.m);
#else
    uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
#endif
    return (hi + n) >> f.s;
}

// Resolved convolution geometry (all extents fit in int32; checked on entry).
struct Geom {
    int N, C, H, W, K, R, S, P, Q;
    int sh, sw, ph, pw, dh, dw, G;
    int Wwin;          // columns of the padded input one output row touches
    int elem;          // bytes per input element
    int lenA, pitchA;  // CHW window row: Wwin*R elements, pitch (16-byte multiple)
    int lenB, pitchB;  // HWC window row: Wwin*R*C elements, pitch
};

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Epilogue fused into the contraction kernels (CIW_FLAG_RELU,
// CIW_FLAG_MAXPOOL2): after the bias, ReLU = max(v, 0), then the max over
// each non-overlapping 2x2 region; the output is then P/2 x Q/2 (floor).
// Maxima are IEEE maxNum (fmaxf).
struct Epi {
    bool relu = false;
    bool pool = false;
};

inline int out_rows(const Geom& g, const Epi& e) { return e.pool ? g.P / 2 : g.P; }
inline int out_cols(const Geom& g, const Epi& e) { return e.pool ? g.Q / 2 : g.Q; }

inline int elem_bytes(ciw_dtype t) { return t == CIW_F32 ? 4 : 2; }

// Allow `fn` more than the default 64 KB of dynamic LDS per workgroup on the
// current device.  The attribute persists for the process, so each
// (device, kernel) pair is raised once and later launches, graph captures
// included, skip the call: the only state the library keeps between calls.
hipError_t allow_dynamic_lds(const void* fn, size_t bytes);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the error of the launch.  Pointers are already
// offset to the chunk; n_images is the chunk's image count.  y has
// out_rows x out_cols outputs per (image, channel).

hipError_t launch_transform(const Geom& g, ciw_dtype dt, ciw_win_layout lay, const void* x,
                            void* xw, int n_images, hipStream_t st);

// fp32 dense contraction over a CHW window tensor.  splits > 1 sums the
// channels in `splits` slices into `partials` ([splits][n][K][P][Q] fp32)
// and a second kernel reduces them in slice order (deterministic).
// Kernel choice for the fp32 contraction: automatic (the matrix cores when
// their plan has at least 4 channel slices), or forced.
enum Fp32Kernel { FP32_AUTO = 0, FP32_MATRIX = 1, FP32_VECTOR = 2 };
int fp32_splits(const Geom& g, int n_images);
hipError_t launch_conv_fp32(const Geom& g, const float* xw, const float* w, const float* bias,
                            float* y, int n_images, float* partials, int splits, bool generic,
                            Fp32Kernel kernel, const Epi& epi, hipStream_t st);

// fp32 dense contraction over a CHW window tensor on the matrix cores (3x3
// and 1x1 filters, output rows of at most 192 pixels, no pooling).
// fp32_mfma_splits is its channel-slice count (partials [splits][n][K][P*Q]
// in the workspace), 0 for layers it does not run; launch_conv_fp32 takes it
// by the Fp32Kernel choice when it runs the layer in at most max_splits
// slices.
int fp32_mfma_splits(const Geom& g, int n_images);
hipError_t launch_conv_fp32_mfma(const Geom& g, const float* xw, const float* w, const float* bias,
                                 float* y, int n_images, float* partials, int max_splits,
                                 const Epi& epi, hipStream_t st);

// fp32 dense contraction on the matrix cores with the whole channel sum in
// one workgroup (16 output channels x 48 pixels; 3x3 and 1x1 filters, C a
// multiple of 4, no pooling): no partial sums, one kernel, no workspace.
// Over a CHW window tensor xw, or with imp in its in-LDS form over x.
// fp32_m16_tasks is its workgroup count, 0 for layers it does not run.
int fp32_m16_tasks(const Geom& g, int n_images, bool imp);
hipError_t launch_conv_fp32_m16(const Geom& g, const float* xw, const float* w, const float* bias,
                                float* y, int n_images, const Epi& epi, bool imp, hipStream_t st);

// fp16/bf16 dense contraction over an HWC window tensor on the matrix cores.
// The row kernel multiplies a re-laid-out copy of the filter (`aperm`,
// mfma_prep_bytes(g) bytes, written by launch_mfma_prep once per call);
// mfma_prep_bytes is 0 when the layer takes the generic kernel.
size_t mfma_prep_bytes(const Geom& g);
hipError_t launch_mfma_prep(const Geom& g, ciw_dtype out, const void* w, void* aperm,
                            hipStream_t st);
hipError_t launch_conv_mfma(const Geom& g, ciw_dtype in, ciw_dtype out, const void* xw,
                            const void* w, const void* aperm, const void* bias, void* y,
                            int n_images, bool generic, const Epi& epi, hipStream_t st);

// fp16/bf16 dense contraction that builds its window rows in LDS from x
// (no window tensor in memory).  implicit_workspace is false for layers no
// such kernel runs; otherwise *bytes is the workspace: 0 for the band
// kernel (3x3, no pool) and for the few-channel kernel below, else the
// re-laid-out filter of the row-band kernel, which launch_conv_implicit
// writes before the contraction.
bool implicit_workspace(const Geom& g, ciw_dtype out, const Epi& epi, size_t* bytes);
// fp32 dense in-LDS form of the matrix-core contraction (no pool): the
// zero-padded input rows of each pixel block staged in LDS straight from x.
// Its workspace holds only the channel slices' partial sums (0 bytes when
// the channel sum is not split); false for layers it does not run.
bool fp32_implicit_workspace(const Geom& g, const Epi& epi, size_t* bytes);
hipError_t launch_conv_fp32_implicit(const Geom& g, const float* x, const float* w, const float* bias,
                                     float* y, float* partials, const Epi& epi, hipStream_t st);
hipError_t launch_conv_implicit(const Geom& g, ciw_dtype in, ciw_dtype out, const void* x,
                                const void* w, const void* bias, void* y, void* ws,
                                const Epi& epi, hipStream_t st);
// fp16/bf16 dense in-LDS form for layers with few input channels and an
// even horizontal stride (C R <= 22, stride_w even, dil_w 1, no pool: the
// 3-channel 7x7 stride-2 stem).  No workspace; implicit_workspace and
// launch_conv_implicit take it for the layers the two kernels above do not
// run.
bool narrow_supported(const Geom& g, ciw_dtype out, const Epi& epi);
hipError_t launch_conv_narrow(const Geom& g, ciw_dtype in, ciw_dtype out, const void* x, const void* w,
                              const void* bias, void* y, const Epi& epi, hipStream_t st);

// Depthwise convolution with the windows built in LDS from x (no window
// tensor, no workspace); dw_implicit_supported is false when a padded
// input plane does not fit the kernel's LDS budget.
bool dw_implicit_supported(const Geom& g, const Epi& epi);
hipError_t launch_conv_dw_implicit(const Geom& g, ciw_dtype in, ciw_dtype out, const void* x,
                                   const void* w, const void* bias, void* y, const Epi& epi,
                                   hipStream_t st);

// Depthwise contraction over a CHW window tensor.
hipError_t launch_conv_dw(const Geom& g, ciw_dtype in, ciw_dtype out, const void* xw,
                          const void* w, const void* bias, void* y, int n_images,
                          bool generic, const Epi& epi, hipStream_t st);

}  // namespace ciw
