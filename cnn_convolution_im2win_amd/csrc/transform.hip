// transform.hip -- the im2win repack (window tensor) kernels for gfx950.
//
// The im2win paper ("Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support on GPU CUDA and Tensor Cores", §III-B/§III-C)
// repacks the input once so that the inputs of one output row sit in one
// contiguous row, column after column, the R values of a column adjacent
// (height before width); §III-D uses the NHWC order, channels innermost, on
// the matrix units.  Both layouts are produced here with zero padding
// materialised and each row's tail (up to its 16-byte pitch) zeroed, so the
// contraction kernels never test bounds.
//
// Both kernels stage a zero-padded input tile in LDS with reads that are
// contiguous along the input width, then write the window rows with stores
// that are contiguous along the window row: HBM sees one pass over x and one
// pass over the window tensor.
#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsBytes = 32768;

// ---------------------------------------------------------------- CHW layout
// One workgroup: image n, channel c, output rows [h0, h0+TH), window columns
// [x0, x0+TX).  LDS holds the input rows those output rows read, with the
// padding columns and rows already zero.
struct ChwArgs {
    int C, H, W, P;
    int sh, ph, pw, dh, R;
    int Wwin, len, pitch;
    int TH, TX, rows_in;        // tile extents (rows_in = (TH-1)*sh + (R-1)*dh + 1)
    int h_tiles, x_tiles;
    FastDiv fdR, fdHt, fdXt;
};

template <typename T, bool kWholeRow>
__global__ __launch_bounds__(kThreads) void im2win_chw_kernel(const T* __restrict__ x,
                                                              T* __restrict__ xw, ChwArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T* tile = reinterpret_cast<T*>(smem_raw);

    uint32_t bid = blockIdx.x;
    uint32_t xt = bid - fdiv(bid, a.fdXt) * a.x_tiles;
    bid = fdiv(bid, a.fdXt);
    uint32_t ht = bid - fdiv(bid, a.fdHt) * a.h_tiles;
    uint32_t nc = fdiv(bid, a.fdHt);           // n*C + c

    const int h0 = ht * a.TH;
    const int th = min(a.TH, a.P - h0);
    const int x0 = xt * a.TX;
    const int tx = min(a.TX, a.Wwin - x0);
    const int ih0 = h0 * a.sh - a.ph;
    const int rows_in = (th - 1) * a.sh + (a.R - 1) * a.dh + 1;
    const T* xp = x + (size_t)nc * a.H * a.W;

    // load: padded input rows ih0 .. ih0+rows_in-1, columns x0-pw .. x0-pw+tx-1
    for (int i = threadIdx.x; i < rows_in * a.TX; i += kThreads) {
        int ri = i / a.TX;
        int xi = i - ri * a.TX;
        int ih = ih0 + ri;
        int iw = x0 + xi - a.pw;
        T v = T(0);
        if (xi < tx && ih >= 0 && ih < a.H && iw >= 0 && iw < a.W) v = xp[ih * a.W + iw];
        tile[i] = v;
    }
    __syncthreads();

    T* out = xw + ((size_t)nc * a.P + h0) * a.pitch;
    if (kWholeRow) {
        // the tile covers whole rows: write rows h0..h0+th-1 (contiguous,
        // pitch included) as 16-byte vectors
        constexpr int VEC = 16 / sizeof(T);
        const int vec_per_row = a.pitch / VEC;
        const int total = th * vec_per_row;
        for (int v = threadIdx.x; v < total; v += kThreads) {
            int hr = v / vec_per_row;
            int e0 = (v - hr * vec_per_row) * VEC;
            const T* trow = tile + hr * a.sh * a.TX;
            union {
                uint4 u;
                T e[VEC];
            } pack;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                int e = e0 + i;
                T val = T(0);
                if (e < a.len) {
                    int xc = fdiv(e, a.fdR);
                    int r = e - xc * a.R;
                    val = trow[r * a.dh * a.TX + xc];
                }
                pack.e[i] = val;
            }
            reinterpret_cast<uint4*>(out + (size_t)hr * a.pitch)[e0 / VEC] = pack.u;
        }
    } else {
        // column-tiled: elements [x0*R, (x0+tx)*R) of each row, plus the
        // zero tail when this is the last column tile
        const bool last = (x0 + tx == a.Wwin);
        const int span = tx * a.R + (last ? a.pitch - a.len : 0);
        for (int i = threadIdx.x; i < th * span; i += kThreads) {
            int hr = i / span;
            int e = i - hr * span;
            T val = T(0);
            if (e < tx * a.R) {
                int xc = fdiv(e, a.fdR);
                int r = e - xc * a.R;
                val = tile[(hr * a.sh + r * a.dh) * a.TX + xc];
            }
            out[(size_t)hr * a.pitch + x0 * a.R + e] = val;
        }
    }
}

// ---------------------------------------------------------------- HWC layout
// One workgroup: image n, output row h, window columns [x0, x0+TX), channels
// [c0, c0+TC).  LDS tile[(cl*R + r)*TX + xi] = padded x[n][c0+cl][h*sh-ph+r*dh][x0+xi-pw].
struct HwcArgs {
    int C, H, W, P;
    int sh, ph, pw, dh, R;
    int Wwin, len, pitch;
    int TX, TC, x_tiles, c_tiles;
    FastDiv fdC, fdR, fdTC, fdXt, fdCt, fdP;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void im2win_hwc_kernel(const T* __restrict__ x,
                                                              T* __restrict__ xw, HwcArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T* tile = reinterpret_cast<T*>(smem_raw);

    uint32_t bid = blockIdx.x;
    uint32_t ct = bid - fdiv(bid, a.fdCt) * a.c_tiles;
    bid = fdiv(bid, a.fdCt);
    uint32_t xt = bid - fdiv(bid, a.fdXt) * a.x_tiles;
    bid = fdiv(bid, a.fdXt);
    uint32_t h = bid - fdiv(bid, a.fdP) * a.P;
    uint32_t n = fdiv(bid, a.fdP);

    const int c0 = ct * a.TC;
    const int tc = min(a.TC, a.C - c0);
    const int x0 = xt * a.TX;
    const int tx = min(a.TX, a.Wwin - x0);
    const int ih0 = (int)h * a.sh - a.ph;

    // load, contiguous along the input width
    const int per_c = a.R * a.TX;
    for (int i = threadIdx.x; i < tc * per_c; i += kThreads) {
        int cl = i / per_c;
        int rem = i - cl * per_c;
        int r = rem / a.TX;
        int xi = rem - r * a.TX;
        int ih = ih0 + r * a.dh;
        int iw = x0 + xi - a.pw;
        T v = T(0);
        if (xi < tx && ih >= 0 && ih < a.H && iw >= 0 && iw < a.W)
            v = x[(((size_t)n * a.C + c0 + cl) * a.H + ih) * a.W + iw];
        tile[i] = v;
    }
    __syncthreads();

    T* out = xw + ((size_t)n * a.P + h) * a.pitch;
    if (tc == a.C) {
        // all channels: the elements of columns [x0, x0+tx) are one contiguous run
        const int run = tx * a.R * a.C;
        const int base = x0 * a.R * a.C;
        for (int t = threadIdx.x; t < run; t += kThreads) {
            uint32_t t2 = fdiv(t, a.fdC);
            int cl = t - t2 * a.C;
            uint32_t xi = fdiv(t2, a.fdR);
            int r = t2 - xi * a.R;
            out[base + t] = tile[(cl * a.R + r) * a.TX + xi];
        }
    } else {
        // channel-tiled: runs of tc channels at stride C (the last channel
        // tile may be narrower than TC)
        const int run = tx * a.R * a.TC;
        for (int t = threadIdx.x; t < run; t += kThreads) {
            uint32_t t2 = fdiv(t, a.fdTC);
            int cl = t - t2 * a.TC;
            if (cl >= tc) continue;
            uint32_t xi = fdiv(t2, a.fdR);
            int r = t2 - xi * a.R;
            out[((x0 + xi) * a.R + r) * a.C + c0 + cl] = tile[(cl * a.R + r) * a.TX + xi];
        }
    }
    // zero tail, written once per row
    if (ct == 0 && x0 + tx == a.Wwin) {
        for (int e = a.len + threadIdx.x; e < a.pitch; e += kThreads) out[e] = T(0);
    }
}

template <typename T>
hipError_t launch_chw(const Geom& g, const void* x, void* xw, int n_images, hipStream_t st) {
    ChwArgs a;
    a.C = g.C; a.H = g.H; a.W = g.W; a.P = g.P;
    a.sh = g.sh; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh; a.R = g.R;
    a.Wwin = g.Wwin; a.len = g.lenA; a.pitch = g.pitchA;
    const int esz = sizeof(T);
    const int budget = kLdsBytes / esz;
    // widest column tile first, then as many output rows as fit
    int TX = g.Wwin;
    int rows1 = (g.R - 1) * g.dh + 1;
    if ((int64_t)rows1 * TX > budget) TX = budget / rows1;   // column tiling
    if (TX < 1) return hipErrorInvalidValue;                  // filter taller than the tile
    int TH = 1;
    if (TX == g.Wwin) {
        while (TH < g.P && (int64_t)((TH) * g.sh + (g.R - 1) * g.dh + 1) * TX <= budget &&
               TH < 64)
            ++TH;
    }
    a.TH = TH;
    a.TX = TX;
    a.rows_in = (TH - 1) * g.sh + (g.R - 1) * g.dh + 1;
    a.h_tiles = (g.P + TH - 1) / TH;
    a.x_tiles = (g.Wwin + TX - 1) / TX;
    a.fdR = make_fastdiv(g.R);
    a.fdHt = make_fastdiv(a.h_tiles);
    a.fdXt = make_fastdiv(a.x_tiles);
    int64_t blocks = (int64_t)n_images * g.C * a.h_tiles * a.x_tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks >= (1ll << 31)) return hipErrorInvalidValue;
    size_t lds = (size_t)a.rows_in * TX * esz;
    if (a.x_tiles == 1)
        hipLaunchKernelGGL((im2win_chw_kernel<T, true>), dim3((uint32_t)blocks), dim3(kThreads),
                           lds, st, (const T*)x, (T*)xw, a);
    else
        hipLaunchKernelGGL((im2win_chw_kernel<T, false>), dim3((uint32_t)blocks), dim3(kThreads),
                           lds, st, (const T*)x, (T*)xw, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_hwc(const Geom& g, const void* x, void* xw, int n_images, hipStream_t st) {
    HwcArgs a;
    a.C = g.C; a.H = g.H; a.W = g.W; a.P = g.P;
    a.sh = g.sh; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh; a.R = g.R;
    a.Wwin = g.Wwin; a.len = g.lenB; a.pitch = g.pitchB;
    const int esz = sizeof(T);
    const int budget = kLdsBytes / esz;
    int TX = g.Wwin;
    int TC = g.C;
    if ((int64_t)TC * g.R * TX > budget) {
        TC = budget / (g.R * TX);
        if (TC < 1) {
            TC = 1;
            TX = budget / g.R;
        }
    }
    if (TX < 1) return hipErrorInvalidValue;
    a.TX = TX;
    a.TC = TC;
    a.x_tiles = (g.Wwin + TX - 1) / TX;
    a.c_tiles = (g.C + TC - 1) / TC;
    a.fdC = make_fastdiv(g.C);
    a.fdR = make_fastdiv(g.R);
    a.fdTC = make_fastdiv(TC);
    a.fdXt = make_fastdiv(a.x_tiles);
    a.fdCt = make_fastdiv(a.c_tiles);
    a.fdP = make_fastdiv(g.P);
    int64_t blocks = (int64_t)n_images * g.P * a.x_tiles * a.c_tiles;
    if (blocks <= 0) return hipSuccess;
    if (blocks >= (1ll << 31)) return hipErrorInvalidValue;
    size_t lds = (size_t)TC * g.R * TX * esz;
    hipLaunchKernelGGL((im2win_hwc_kernel<T>), dim3((uint32_t)blocks), dim3(kThreads), lds, st,
                       (const T*)x, (T*)xw, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_transform(const Geom& g, ciw_dtype dt, ciw_win_layout lay, const void* x,
                            void* xw, int n_images, hipStream_t st) {
    // the repack copies element bit patterns (as unsigned integers of the
    // element's width), so fp16 and bf16 share a kernel
    if (lay == CIW_WIN_CHW)
        return dt == CIW_F32 ? launch_chw<uint32_t>(g, x, xw, n_images, st)
                             : launch_chw<uint16_t>(g, x, xw, n_images, st);
    return dt == CIW_F32 ? launch_hwc<uint32_t>(g, x, xw, n_images, st)
                         : launch_hwc<uint16_t>(g, x, xw, n_images, st);
}

}  // namespace ciw
