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

// ------------------------------------------------- CHW layout, whole planes
// One workgroup: `ppb` consecutive input planes (n, c), which are one
// contiguous run of x, and their window rows, one contiguous run of the
// window tensor.  Each plane is staged in LDS as the zero-padded tile of the
// padded-input rows and columns its windows touch; the window rows are then
// written with 16-byte stores in memory order.
struct PlaneArgs {
    int H, W, P, sh, ph, pw, dh, R;
    int Wwin, len, pitch, Hp;      // Hp: padded input rows the windows touch
    int planes, ppb, vec_in;
    FastDiv fdHW, fdW, fdPP, fdPitch, fdR;
};

constexpr int kPlaneLds = 16384;

template <typename T>
__global__ __launch_bounds__(kThreads) void im2win_chw_planes_kernel(const T* __restrict__ x,
                                                                     T* __restrict__ xw,
                                                                     PlaneArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T* tile = reinterpret_cast<T*>(smem_raw);
    constexpr int V = 16 / sizeof(T);
    const int tid = threadIdx.x;
    const int p0 = blockIdx.x * a.ppb;
    const int np = min(a.ppb, a.planes - p0);
    const int tsz = a.Hp * a.Wwin;
    const int HW = a.H * a.W;

    for (int i = tid; i < np * tsz; i += kThreads) tile[i] = T(0);
    __syncthreads();

    // input element (plane, ih, iw) -> padded tile position (ih + ph, iw + pw)
    auto put = [&](int e, T v) {
        const uint32_t pl = fdiv(e, a.fdHW);
        const int rem = e - pl * HW;
        const uint32_t ih = fdiv(rem, a.fdW);
        const int iw = rem - ih * a.W;
        const int tr = ih + a.ph, tc = iw + a.pw;
        if (tr < a.Hp && tc < a.Wwin) tile[pl * tsz + tr * a.Wwin + tc] = v;
    };
    const T* src = x + (size_t)p0 * HW;
    const int nin = np * HW;
    if (a.vec_in) {   // HW % V == 0: the planes start on 16-byte boundaries
        for (int v = tid; v < nin / V; v += kThreads) {
            union {
                uint4 u;
                T e[V];
            } pk;
            pk.u = reinterpret_cast<const uint4*>(src)[v];
#pragma unroll
            for (int i = 0; i < V; ++i) put(v * V + i, pk.e[i]);
        }
    } else {
        for (int e = tid; e < nin; e += kThreads) put(e, src[e]);
    }
    __syncthreads();

    // window rows of the block: np * P rows of `pitch` elements; element j
    // of row (plane, h) is column x = j / R, filter row r = j % R, i.e. the
    // padded input at (h*sh + r*dh, x); zero in the pitch tail
    T* dst = xw + (size_t)p0 * a.P * a.pitch;
    const int nvec = np * a.P * a.pitch / V;
    for (int v = tid; v < nvec; v += kThreads) {
        const int e0 = v * V;
        const uint32_t rowi = fdiv(e0, a.fdPitch);
        const int j0 = e0 - rowi * a.pitch;
        const uint32_t pl = fdiv(rowi, a.fdPP);
        const int h = rowi - pl * a.P;
        const T* tp = tile + pl * tsz + h * a.sh * a.Wwin;
        uint32_t xx = fdiv(j0, a.fdR);
        int r = j0 - xx * a.R;
        union {
            uint4 u;
            T e[V];
        } pk;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            pk.e[i] = (j0 + i < a.len) ? tp[r * a.dh * a.Wwin + xx] : T(0);
            if (++r == a.R) {
                r = 0;
                ++xx;
            }
        }
        reinterpret_cast<uint4*>(dst)[v] = pk.u;
    }
}

template <typename T>
bool launch_chw_planes(const Geom& g, const void* x, void* xw, int n_images, hipStream_t st,
                       hipError_t* err) {
    PlaneArgs a;
    a.H = g.H; a.W = g.W; a.P = g.P; a.sh = g.sh; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh; a.R = g.R;
    a.Wwin = g.Wwin; a.len = g.lenA; a.pitch = g.pitchA;
    // input rows a plane's windows span, in 64 bits (a huge vertical stride
    // is legal); the plane must fit LDS
    const int64_t hp = (int64_t)(g.P - 1) * g.sh + (int64_t)(g.R - 1) * g.dh + 1;
    const int64_t tile_bytes = hp * a.Wwin * (int64_t)sizeof(T);
    if (hp > kPlaneLds || tile_bytes > kPlaneLds) return false;
    a.Hp = (int)hp;
    const int64_t planes = (int64_t)n_images * g.C;
    if (planes >= (1ll << 31) || planes * g.H * g.W >= (1ll << 31)) return false;
    a.planes = (int)planes;
    int ppb = (int)(kPlaneLds / tile_bytes);
    // keep at least ~1024 workgroups when there are enough planes
    const int64_t cap = (planes + 1023) / 1024;
    if (ppb > cap) ppb = (int)cap;
    if (ppb < 1) ppb = 1;
    a.ppb = ppb;
    a.vec_in = ((int64_t)g.H * g.W) % (16 / (int)sizeof(T)) == 0 ? 1 : 0;
    a.fdHW = make_fastdiv(g.H * g.W);
    a.fdW = make_fastdiv(g.W);
    a.fdPP = make_fastdiv(g.P);
    a.fdPitch = make_fastdiv(g.pitchA);
    a.fdR = make_fastdiv(g.R);
    const int64_t blocks = (planes + ppb - 1) / ppb;
    hipLaunchKernelGGL((im2win_chw_planes_kernel<T>), dim3((uint32_t)blocks), dim3(kThreads),
                       (size_t)ppb * tile_bytes, st, (const T*)x, (T*)xw, a);
    *err = hipGetLastError();
    return true;
}

// ------------------------------------------------- HWC layout, whole rows
// One workgroup: one window row (n, h) with all channels.  LDS holds the
// row in output order, [x][r][c], with each column x padded so that
// 16-byte accesses of neighbouring columns fall on different banks.  Loads
// run along input rows (consecutive lanes, consecutive x) and gather a
// vector of channels per lane (or one channel when C is not a multiple of
// the vector width); the row then leaves with 16-byte stores.  Consecutive
// rows h of an image
// read overlapping input rows, so they are kept on one XCD (its L2).
struct HwcRowArgs {
    int C, H, W, P, sh, ph, pw, dh, R;
    int Wwin, len, pitch;
    int xs;                        // LDS column stride (elements)
    int rows, vec_w;               // vec_w: input rows are whole 16-byte vectors
    FastDiv fdP, fdCv, fdRC, fdWwin, fdWv, fdR;
    uint32_t xcd_per, xcd_rem;
};

// CV channels per load item: the 16-byte vector width when C is a multiple
// of it, else 1 (then the LDS row is exactly the output row, xs = R*C, and
// its tail up to a whole vector is zeroed).
template <typename T, int CV>
__global__ __launch_bounds__(kThreads) void im2win_hwc_rows_kernel(const T* __restrict__ x,
                                                                   T* __restrict__ xw,
                                                                   HwcRowArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T* tile = reinterpret_cast<T*>(smem_raw);
    constexpr int V = 16 / sizeof(T);
    const int tid = threadIdx.x;
    const uint32_t bid = blockIdx.x;
    const uint32_t xcd = bid & 7u, slot = bid >> 3;
    const uint32_t row = xcd < a.xcd_rem ? xcd * (a.xcd_per + 1) + slot
                                         : a.xcd_rem * (a.xcd_per + 1) + (xcd - a.xcd_rem) * a.xcd_per + slot;
    const uint32_t n = fdiv(row, a.fdP);
    const int h = row - n * a.P;
    const int HW = a.H * a.W;
    const int cv = a.C / CV;                // channel groups of CV
    if (CV == 1 && a.vec_w) {
        // input rows are whole 16-byte vectors: zero the LDS row, then each
        // item moves 16 bytes of one input row (channel c, filter row r)
        const int len_v = (a.len + V - 1) / V * V;
        for (int i = tid; i < len_v / V; i += kThreads)
            reinterpret_cast<uint4*>(tile)[i] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        const int wv = a.W / V;
        const int vitems = a.C * a.R * wv;
        // up to kBatch items per thread: all their loads are in flight before
        // the first is scattered into LDS
        constexpr int kBatch = 4;
        for (int base = tid; base < vitems; base += kBatch * kThreads) {
            union {
                uint4 u;
                T e[V];
            } pk[kBatch];
            int dst[kBatch], col0[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int it = base + u * kThreads;
                dst[u] = -1;
                col0[u] = 0;
                pk[u].u = make_uint4(0u, 0u, 0u, 0u);
                if (it < vitems) {
                    const uint32_t q = fdiv(it, a.fdWv);
                    const int jv = it - q * wv;
                    const uint32_t c = fdiv(q, a.fdR);
                    const int r = q - c * a.R;
                    const int ih = h * a.sh - a.ph + r * a.dh;
                    if (ih >= 0 && ih < a.H) {
                        pk[u].u = reinterpret_cast<const uint4*>(
                            x + (((size_t)n * a.C + c) * a.H + ih) * a.W)[jv];
                        col0[u] = jv * V + a.pw;
                        dst[u] = col0[u] * a.xs + r * a.C + c;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (dst[u] < 0) continue;
#pragma unroll
                for (int i = 0; i < V; ++i)
                    if (col0[u] + i < a.Wwin) tile[dst[u] + i * a.xs] = pk[u].e[i];
            }
        }
        __syncthreads();
    } else if (CV == 1) {
        const int len_v = (a.len + V - 1) / V * V;
        for (int i = a.len + tid; i < len_v; i += kThreads) tile[i] = T(0);
    }

    // load: item (column xx, channel group gq, filter row r), xx fastest so
    // that consecutive lanes read consecutive input columns
    const int items = (CV == 1 && a.vec_w) ? 0 : a.Wwin * a.R * cv;
    for (int it = tid; it < items; it += kThreads) {
        const uint32_t q = fdiv(it, a.fdWwin);
        const int xx = it - q * a.Wwin;
        const uint32_t r = fdiv(q, a.fdCv);
        const int gq = q - r * cv;
        const int ih = h * a.sh - a.ph + r * a.dh;
        const int iw = xx - a.pw;
        const bool inside = ih >= 0 && ih < a.H && iw >= 0 && iw < a.W;
        const T* sp = x + ((size_t)n * a.C + gq * CV) * HW + ih * a.W + iw;
        if (CV == 1) {
            tile[xx * a.xs + r * a.C + gq] = inside ? sp[0] : T(0);
        } else {
            union {
                uint4 u;
                T e[V];
            } pk;
            pk.u = make_uint4(0u, 0u, 0u, 0u);
            if (inside) {
#pragma unroll
                for (int i = 0; i < V; ++i) pk.e[i] = sp[(size_t)i * HW];
            }
            *reinterpret_cast<uint4*>(tile + xx * a.xs + r * a.C + gq * V) = pk.u;
        }
    }
    __syncthreads();

    // store: the row's `pitch` elements as 16-byte vectors (zero past len)
    T* dst = xw + (size_t)row * a.pitch;
    const int rc = a.R * a.C;
    for (int v = tid; v < a.pitch / V; v += kThreads) {
        const int e0 = v * V;
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (e0 < a.len) {
            const uint32_t xx = fdiv(e0, a.fdRC);
            u = *reinterpret_cast<const uint4*>(tile + xx * a.xs + (e0 - xx * rc));
        }
        reinterpret_cast<uint4*>(dst)[v] = u;
    }
}

template <typename T>
bool launch_hwc_rows(const Geom& g, const void* x, void* xw, int n_images, hipStream_t st,
                     hipError_t* err) {
    constexpr int V = 16 / sizeof(T);
    const bool vec = g.C % V == 0;
    HwcRowArgs a;
    a.C = g.C; a.H = g.H; a.W = g.W; a.P = g.P; a.sh = g.sh; a.ph = g.ph; a.pw = g.pw;
    a.dh = g.dh; a.R = g.R;
    a.Wwin = g.Wwin; a.len = g.lenB; a.pitch = g.pitchB;
    // column stride: R*C plus a pad that makes it 4 mod 8 dwords, so the
    // 16-byte writes of 8 consecutive columns hit distinct bank groups
    const int rc = g.R * g.C;
    int xs = rc;
    for (int pad = 0; vec && pad < 8 * V; pad += V) {
        const int words = (rc + pad) * (int)sizeof(T) / 4;
        if (words % 8 == 4) {
            xs = rc + pad;
            break;
        }
    }
    a.xs = xs;
    const int64_t lds = ((int64_t)g.Wwin * xs + V) * sizeof(T);
    if (lds > 32768) return false;
    const int64_t rows = (int64_t)n_images * g.P;
    if (rows >= (1ll << 31)) return false;
    a.rows = (int)rows;
    a.fdP = make_fastdiv(g.P);
    a.fdCv = make_fastdiv(vec ? g.C / V : g.C);
    a.fdRC = make_fastdiv(rc);
    a.fdWwin = make_fastdiv(g.Wwin);
    a.vec_w = (g.W % V == 0) ? 1 : 0;
    a.fdWv = make_fastdiv(g.W / V > 0 ? g.W / V : 1);
    a.fdR = make_fastdiv(g.R);
    a.xcd_per = (uint32_t)(rows / 8);
    a.xcd_rem = (uint32_t)(rows % 8);
    if (vec)
        hipLaunchKernelGGL((im2win_hwc_rows_kernel<T, V>), dim3((uint32_t)rows), dim3(kThreads),
                           (size_t)lds, st, (const T*)x, (T*)xw, a);
    else
        hipLaunchKernelGGL((im2win_hwc_rows_kernel<T, 1>), dim3((uint32_t)rows), dim3(kThreads),
                           (size_t)lds, st, (const T*)x, (T*)xw, a);
    *err = hipGetLastError();
    return true;
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
    if (n_images == 0) return hipSuccess;
    hipError_t e = hipSuccess;
    if (lay == CIW_WIN_CHW) {
        if (dt == CIW_F32 ? launch_chw_planes<uint32_t>(g, x, xw, n_images, st, &e)
                          : launch_chw_planes<uint16_t>(g, x, xw, n_images, st, &e))
            return e;
        return dt == CIW_F32 ? launch_chw<uint32_t>(g, x, xw, n_images, st)
                             : launch_chw<uint16_t>(g, x, xw, n_images, st);
    }
    if (dt == CIW_F32 ? launch_hwc_rows<uint32_t>(g, x, xw, n_images, st, &e)
                      : launch_hwc_rows<uint16_t>(g, x, xw, n_images, st, &e))
        return e;
    return dt == CIW_F32 ? launch_hwc<uint32_t>(g, x, xw, n_images, st)
                         : launch_hwc<uint16_t>(g, x, xw, n_images, st);
}

}  // namespace ciw
