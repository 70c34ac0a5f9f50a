// conv_dw.hip -- depthwise (groups = C) windowed dot product (gfx950).
//
// Each channel has its own R x S filter; output (n, c, h, w) is the dot
// product of the CHW window row (n, c, h) at columns w*stride_w + q*dil_w
// (R contiguous values each) with that filter, plus the bias, accumulated in
// fp32.  Nine multiply-adds per output against a few bytes in and 4 bytes
// out: the kernel is bound by HBM bandwidth, not arithmetic ("Diagonalwise
// Refactorization: An Efficient Training Method for Depthwise Convolutions"
// reports the same imbalance for depthwise layers).
//
// Block kernel (common filter sizes).  Window rows (n, c, h) are stored one
// after another and so are output rows, so a run of consecutive rows is one
// contiguous stretch of the window tensor and one of the output.  A
// workgroup copies its stretch of window rows into LDS with 16-byte loads
// that run along memory (each byte of the window tensor crosses HBM once),
// stages the filters of the few channels it spans, and then computes its
// outputs in memory order, so the stores are contiguous too.
//
// Generic kernel: any shape; one thread per output.
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

// ----------------------------------------------------------- block kernel
struct DwBlockArgs {
    int C, P, Q, pitch, sw, dw;
    int rows_per_block;      // window rows (= output rows) per workgroup
    uint32_t rows;           // total rows of the chunk: n_images * C * P
    FastDiv fdQ, fdP, fdC;
};

constexpr int kDwLdsBytes = 16384;

template <typename TIn, typename TOut, int R, int S>
__global__ __launch_bounds__(kThreads) void conv_dw_block_kernel(
    const TIn* __restrict__ xw, const TIn* __restrict__ w, const TIn* __restrict__ bias,
    TOut* __restrict__ y, DwBlockArgs a) {
    constexpr int V = 16 / sizeof(TIn);
    constexpr int T = R * S;
    constexpr int kMaxCh = 64;                          // channels one block may span
    __shared__ __align__(16) TIn tile[kDwLdsBytes / sizeof(TIn)];
    __shared__ float filt[kMaxCh * T + kMaxCh];

    const uint32_t r0 = blockIdx.x * (uint32_t)a.rows_per_block;
    const int nrows = min((uint32_t)a.rows_per_block, a.rows - r0);

    // 1. the block's window rows are one contiguous run: copy it with
    //    16-byte loads, consecutive threads on consecutive 16 bytes
    const int nvec = nrows * a.pitch / V;
    const uint4* src = reinterpret_cast<const uint4*>(xw + (size_t)r0 * a.pitch);
    uint4* dstv = reinterpret_cast<uint4*>(tile);
    for (int i = threadIdx.x; i < nvec; i += kThreads) dstv[i] = src[i];

    // 2. filters and biases of the channels the block spans
    const uint32_t nc_first = fdiv(r0, a.fdP);
    const uint32_t nc_last = fdiv(r0 + nrows - 1, a.fdP);
    const int nch = nc_last - nc_first + 1;             // <= kMaxCh (host-checked)
    for (int i = threadIdx.x; i < nch * T; i += kThreads) {
        const uint32_t ncx = nc_first + i / T;
        const int c = ncx - fdiv(ncx, a.fdC) * a.C;
        filt[i] = to_f32(w[(size_t)c * T + i % T]);
    }
    for (int i = threadIdx.x; i < nch; i += kThreads) {
        const uint32_t ncx = nc_first + i;
        const int c = ncx - fdiv(ncx, a.fdC) * a.C;
        filt[kMaxCh * T + i] = bias ? to_f32(bias[c]) : 0.f;
    }
    __syncthreads();

    // 3. outputs of the block, contiguous in y: consecutive threads take
    //    consecutive outputs (adjacent columns read window elements R*SW
    //    apart, an odd stride for odd R and SW: no bank conflicts)
    const int nout = nrows * a.Q;
    TOut* yb = y + (size_t)r0 * a.Q;
    for (int o = threadIdx.x; o < nout; o += kThreads) {
        const uint32_t rl = fdiv(o, a.fdQ);
        const int wo = o - rl * a.Q;
        const int cl = fdiv(r0 + rl, a.fdP) - nc_first;
        const TIn* row = tile + rl * a.pitch + wo * a.sw * R;
        const float* f = filt + cl * T;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < S; ++q)
#pragma unroll
            for (int r = 0; r < R; ++r) acc = fmaf(to_f32(row[q * a.dw * R + r]), f[r * S + q], acc);
        yb[o] = from_f32<TOut>(acc + filt[kMaxCh * T + cl]);
    }
}

template <typename TIn, typename TOut, int R, int S>
hipError_t launch_block(const Geom& g, const void* xw, const void* w, const void* bias, void* y,
                        int n_images, hipStream_t st) {
    DwBlockArgs a;
    a.C = g.C; a.P = g.P; a.Q = g.Q; a.pitch = g.pitchA; a.sw = g.sw; a.dw = g.dw;
    const int64_t rows = (int64_t)n_images * g.C * g.P;
    if (rows >= (1ll << 31)) return hipErrorInvalidValue;
    a.rows = (uint32_t)rows;
    const int64_t row_bytes = (int64_t)g.pitchA * sizeof(TIn);
    int rpb = (int)(kDwLdsBytes / row_bytes);
    // a block spans at most rpb/P + 2 channels; keep that within 64
    const int max_rows_for_ch = (64 - 2) * g.P;
    if (rpb > max_rows_for_ch) rpb = max_rows_for_ch;
    a.rows_per_block = rpb;
    a.fdQ = make_fastdiv(g.Q);
    a.fdP = make_fastdiv(g.P);
    a.fdC = make_fastdiv(g.C);
    const int64_t blocks = (rows + rpb - 1) / rpb;
    hipLaunchKernelGGL((conv_dw_block_kernel<TIn, TOut, R, S>), dim3((uint32_t)blocks),
                       dim3(kThreads), 0, st, (const TIn*)xw, (const TIn*)w, (const TIn*)bias,
                       (TOut*)y, a);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_generic(const Geom& g, const void* xw, const void* w, const void* bias, void* y,
                          int n_images, hipStream_t st) {
    DwArgs a;
    a.C = g.C; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
    a.sw = g.sw; a.dw = g.dw; a.pitch = g.pitchA;
    a.fdQ = make_fastdiv(g.Q);
    a.fdP = make_fastdiv(g.P);
    a.fdC = make_fastdiv(g.C);
    a.total = (int64_t)n_images * g.C * g.P * g.Q;
    if (a.total >= (1ll << 31)) return hipErrorInvalidValue;
    uint32_t blocks = (uint32_t)((a.total + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((conv_dw_generic_kernel<TIn, TOut>), dim3(blocks), dim3(kThreads), 0, st,
                       (const TIn*)xw, (const TIn*)w, (const TIn*)bias, (TOut*)y, a);
    return hipGetLastError();
}

// Block-kernel shapes (taps unrolled); rows that do not fit the LDS tile
// go to the generic kernel.
template <typename TIn, typename TOut>
hipError_t launch_t(const Geom& g, const void* xw, const void* w, const void* bias, void* y,
                    int n_images, bool generic, hipStream_t st) {
    if (n_images == 0) return hipSuccess;
    const bool fits = (int64_t)g.pitchA * (int64_t)sizeof(TIn) <= kDwLdsBytes;
    if (!generic && fits) {
        if (g.R == 3 && g.S == 3) return launch_block<TIn, TOut, 3, 3>(g, xw, w, bias, y, n_images, st);
        if (g.R == 5 && g.S == 5) return launch_block<TIn, TOut, 5, 5>(g, xw, w, bias, y, n_images, st);
        if (g.R == 7 && g.S == 7) return launch_block<TIn, TOut, 7, 7>(g, xw, w, bias, y, n_images, st);
        if (g.R == 1 && g.S == 1) return launch_block<TIn, TOut, 1, 1>(g, xw, w, bias, y, n_images, st);
    }
    return launch_generic<TIn, TOut>(g, xw, w, bias, y, n_images, st);
}

}  // namespace

hipError_t launch_conv_dw(const Geom& g, ciw_dtype in, ciw_dtype out, const void* xw,
                          const void* w, const void* bias, void* y, int n_images,
                          bool generic, hipStream_t st) {
    if (in == CIW_F32) return launch_t<float, float>(g, xw, w, bias, y, n_images, generic, st);
    if (in == CIW_F16)
        return out == CIW_F32
                   ? launch_t<half_t, float>(g, xw, w, bias, y, n_images, generic, st)
                   : launch_t<half_t, half_t>(g, xw, w, bias, y, n_images, generic, st);
    return out == CIW_F32 ? launch_t<bf16_t, float>(g, xw, w, bias, y, n_images, generic, st)
                          : launch_t<bf16_t, bf16_t>(g, xw, w, bias, y, n_images, generic, st);
}

}  // namespace ciw
