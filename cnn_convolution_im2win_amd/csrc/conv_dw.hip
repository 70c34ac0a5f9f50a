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
//
// Fused epilogue: bias, optional ReLU, optional 2x2 max-pool; with the pool
// a thread computes the four outputs of its region and stores their max.
#include <algorithm>

#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

constexpr int kThreads = 256;

struct DwArgs {
    int C, R, S, P, Q, sw, dw, pitch;
    int relu, pool, Po, Qo;         // epilogue; output extent (P/2 x Q/2 with pool)
    FastDiv fdQo, fdPo, fdC;
    int64_t total;                  // outputs
};

// Bias, then the optional ReLU (maxNum against 0).
__device__ __forceinline__ float act(float v, float b, int relu) {
    v += b;
    return relu ? fmaxf(v, 0.f) : v;
}

template <typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads) void conv_dw_generic_kernel(
    const TIn* __restrict__ xw, const TIn* __restrict__ w, const TIn* __restrict__ bias,
    TOut* __restrict__ y, DwArgs a) {
    int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= a.total) return;
    uint32_t t = (uint32_t)idx;
    uint32_t t1 = fdiv(t, a.fdQo);
    const int wo2 = t - t1 * a.Qo;
    uint32_t nc = fdiv(t1, a.fdPo);
    const int h2 = t1 - nc * a.Po;
    const int c = nc - fdiv(nc, a.fdC) * a.C;
    const TIn* f = w + (size_t)c * a.R * a.S;
    const float b = bias ? to_f32(bias[c]) : 0.f;
    // one output, or the four of its 2x2 region with the pool
    const int side = a.pool ? 2 : 1;
    float m = 0.f;
    for (int dy = 0; dy < side; ++dy)
        for (int dx = 0; dx < side; ++dx) {
            const int h = h2 * side + dy, wo = wo2 * side + dx;
            const TIn* row = xw + ((size_t)nc * a.P + h) * a.pitch + (size_t)wo * a.sw * a.R;
            float acc = 0.f;
            for (int q = 0; q < a.S; ++q)
                for (int r = 0; r < a.R; ++r)
                    acc = fmaf(to_f32(row[q * a.dw * a.R + r]), to_f32(f[r * a.S + q]), acc);
            const float v = act(acc, b, a.relu);
            m = (dy | dx) ? fmaxf(m, v) : v;
        }
    y[idx] = from_f32<TOut>(m);
}

// ----------------------------------------------------------- block kernel
// Work unit: one output row (n, c, h) -- one pooled row (n, c, j), which
// reads window rows 2j and 2j + 1, with the pool.
struct DwBlockArgs {
    int C, P, Q, pitch, sw, dw;
    int units_per_block;     // output rows per workgroup
    uint32_t units;          // output rows of the chunk: n_images * C * Po
    int relu, pool, Po, Qo;
    FastDiv fdQo, fdPo, fdC;
};

constexpr int kDwLdsBytes = 16384;
constexpr int kDwMaxCh = 64;                            // channels one block may span

template <typename TIn, typename TOut, int R, int S>
__global__ __launch_bounds__(kThreads) void conv_dw_block_kernel(
    const TIn* __restrict__ xw, const TIn* __restrict__ w, const TIn* __restrict__ bias,
    TOut* __restrict__ y, DwBlockArgs a) {
    constexpr int V = 16 / sizeof(TIn);
    constexpr int T = R * S;
    __shared__ __align__(16) TIn tile[kDwLdsBytes / sizeof(TIn)];
    __shared__ float filt[kDwMaxCh * T + kDwMaxCh];

    const uint32_t u0 = blockIdx.x * (uint32_t)a.units_per_block;
    const int nu = min((uint32_t)a.units_per_block, a.units - u0);
    // first window row of unit u: its own row, or row 2j of its plane
    auto first_row = [&](uint32_t u) -> uint32_t {
        if (!a.pool) return u;
        const uint32_t nc = fdiv(u, a.fdPo);
        return nc * a.P + 2 * (u - nc * a.Po);
    };
    const uint32_t r_lo = first_row(u0);
    const int nrows = first_row(u0 + nu - 1) + (a.pool ? 2 : 1) - r_lo;   // <= LDS rows (host-checked)

    // 1. the block's window rows are one contiguous run: copy it with
    //    16-byte loads, consecutive threads on consecutive 16 bytes
    const int nvec = nrows * a.pitch / V;
    const uint4* src = reinterpret_cast<const uint4*>(xw + (size_t)r_lo * a.pitch);
    uint4* dstv = reinterpret_cast<uint4*>(tile);
    for (int i = threadIdx.x; i < nvec; i += kThreads) dstv[i] = src[i];

    // 2. filters and biases of the channels the block spans
    const uint32_t nc_first = fdiv(u0, a.fdPo);
    const uint32_t nc_last = fdiv(u0 + nu - 1, a.fdPo);
    const int nch = nc_last - nc_first + 1;             // <= kDwMaxCh (host-checked)
    for (int i = threadIdx.x; i < nch * T; i += kThreads) {
        const uint32_t ncx = nc_first + i / T;
        const int c = ncx - fdiv(ncx, a.fdC) * a.C;
        filt[i] = to_f32(w[(size_t)c * T + i % T]);
    }
    for (int i = threadIdx.x; i < nch; i += kThreads) {
        const uint32_t ncx = nc_first + i;
        const int c = ncx - fdiv(ncx, a.fdC) * a.C;
        filt[kDwMaxCh * T + i] = bias ? to_f32(bias[c]) : 0.f;
    }
    __syncthreads();

    // 3. outputs of the block, contiguous in y: consecutive threads take
    //    consecutive outputs (adjacent columns read window elements R*SW
    //    apart, an odd stride for odd R and SW: no bank conflicts).  With
    //    the pool, four neighbouring lanes take the four pixels of one
    //    output's region (the work per lane stays one pixel) and two lane
    //    exchanges give the max; a region's lanes are always active together
    //    (256 is a multiple of 4).
    const int nout = nu * a.Qo;
    const int sub_bits = a.pool ? 2 : 0;
    TOut* yb = y + (size_t)u0 * a.Qo;
    for (int t = threadIdx.x; t < (nout << sub_bits); t += kThreads) {
        const int o = t >> sub_bits;
        const int d = t & ((1 << sub_bits) - 1);   // pixel of the region: row d / 2, column d % 2
        const uint32_t ul = fdiv(o, a.fdQo);
        const int wo2 = o - ul * a.Qo;
        const uint32_t u = u0 + ul;
        const int cl = fdiv(u, a.fdPo) - nc_first;
        const int trow = first_row(u) - r_lo + (d >> 1);
        const int wo = a.pool ? 2 * wo2 + (d & 1) : wo2;
        const float* f = filt + cl * T;
        const TIn* row = tile + trow * a.pitch + wo * a.sw * R;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < S; ++q)
#pragma unroll
            for (int r = 0; r < R; ++r) acc = fmaf(to_f32(row[q * a.dw * R + r]), f[r * S + q], acc);
        float v = act(acc, filt[kDwMaxCh * T + cl], a.relu);
        if (a.pool) {
            v = fmaxf(v, __shfl_xor(v, 1));
            v = fmaxf(v, __shfl_xor(v, 2));
            if (d == 0) yb[o] = from_f32<TOut>(v);
        } else {
            yb[o] = from_f32<TOut>(v);
        }
    }
}

// Output rows per workgroup such that the window rows they read fit the
// LDS tile and span at most kDwMaxCh channels; 0 if not even one fits.
int dw_units_per_block(const Geom& g, const Epi& epi, int64_t row_bytes) {
    const int64_t rpb = kDwLdsBytes / row_bytes;        // window rows the tile holds
    if (!epi.pool) {
        const int64_t cap = (int64_t)(kDwMaxCh - 2) * g.P;   // spans <= cap/P + 2 channels
        return (int)std::min(rpb, cap);
    }
    // pooled rows u .. u + n - 1 read 2n window rows, plus the skipped last
    // row of every plane they cross when P is odd (at most (n + Po - 2) / Po)
    const int Po = g.P / 2;
    for (int64_t n = std::min<int64_t>(rpb / 2, (int64_t)(kDwMaxCh - 2) * Po); n >= 1; --n) {
        const int64_t crossings = (n + Po - 2) / Po;
        if (2 * n + (g.P & 1) * crossings <= rpb) return (int)n;
    }
    return 0;
}

template <typename TIn, typename TOut, int R, int S>
hipError_t launch_block(const Geom& g, const Epi& epi, int upb, const void* xw, const void* w,
                        const void* bias, void* y, int n_images, hipStream_t st) {
    DwBlockArgs a;
    a.C = g.C; a.P = g.P; a.Q = g.Q; a.pitch = g.pitchA; a.sw = g.sw; a.dw = g.dw;
    a.relu = epi.relu;
    a.pool = epi.pool;
    a.Po = out_rows(g, epi);
    a.Qo = out_cols(g, epi);
    const int64_t units = (int64_t)n_images * g.C * a.Po;
    if (units >= (1ll << 31)) return hipErrorInvalidValue;
    a.units = (uint32_t)units;
    a.units_per_block = upb;
    a.fdQo = make_fastdiv(a.Qo);
    a.fdPo = make_fastdiv(a.Po);
    a.fdC = make_fastdiv(g.C);
    const int64_t blocks = (units + upb - 1) / upb;
    hipLaunchKernelGGL((conv_dw_block_kernel<TIn, TOut, R, S>), dim3((uint32_t)blocks),
                       dim3(kThreads), 0, st, (const TIn*)xw, (const TIn*)w, (const TIn*)bias,
                       (TOut*)y, a);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_generic(const Geom& g, const Epi& epi, const void* xw, const void* w,
                          const void* bias, void* y, int n_images, hipStream_t st) {
    DwArgs a;
    a.C = g.C; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
    a.sw = g.sw; a.dw = g.dw; a.pitch = g.pitchA;
    a.relu = epi.relu;
    a.pool = epi.pool;
    a.Po = out_rows(g, epi);
    a.Qo = out_cols(g, epi);
    a.fdQo = make_fastdiv(a.Qo);
    a.fdPo = make_fastdiv(a.Po);
    a.fdC = make_fastdiv(g.C);
    a.total = (int64_t)n_images * g.C * a.Po * a.Qo;
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
                    int n_images, bool generic, const Epi& epi, hipStream_t st) {
    if (n_images == 0) return hipSuccess;
    const int upb = dw_units_per_block(g, epi, (int64_t)g.pitchA * (int64_t)sizeof(TIn));
    if (!generic && upb > 0) {
#define CIW_DW(RR, SS)                                                                         \
        if (g.R == RR && g.S == SS)                                                            \
            return launch_block<TIn, TOut, RR, SS>(g, epi, upb, xw, w, bias, y, n_images, st);
        CIW_DW(3, 3) CIW_DW(5, 5) CIW_DW(7, 7) CIW_DW(1, 1)
#undef CIW_DW
    }
    return launch_generic<TIn, TOut>(g, epi, xw, w, bias, y, n_images, st);
}

}  // namespace

hipError_t launch_conv_dw(const Geom& g, ciw_dtype in, ciw_dtype out, const void* xw,
                          const void* w, const void* bias, void* y, int n_images,
                          bool generic, const Epi& epi, hipStream_t st) {
    if (in == CIW_F32) return launch_t<float, float>(g, xw, w, bias, y, n_images, generic, epi, st);
    if (in == CIW_F16)
        return out == CIW_F32
                   ? launch_t<half_t, float>(g, xw, w, bias, y, n_images, generic, epi, st)
                   : launch_t<half_t, half_t>(g, xw, w, bias, y, n_images, generic, epi, st);
    return out == CIW_F32 ? launch_t<bf16_t, float>(g, xw, w, bias, y, n_images, generic, epi, st)
                          : launch_t<bf16_t, bf16_t>(g, xw, w, bias, y, n_images, generic, epi, st);
}

}  // namespace ciw
