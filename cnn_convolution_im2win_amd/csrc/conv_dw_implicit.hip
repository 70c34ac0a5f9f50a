// conv_dw_implicit.hip -- depthwise convolution (groups = C = K) with the
// windows built in LDS from x: no window tensor in memory.
//
// Depthwise work is a per-channel windowed dot product ("Diagonalwise
// Refactorization", abstract: one filter per input channel), with about one
// multiply-add per byte moved, so the HBM traffic decides its time.  The
// materialised path writes the window tensor (about R/stride_h times x) and
// reads it back; here a workgroup copies a run of whole input planes
// (n, c), which are contiguous in NCHW, into LDS with zero padding around
// each plane, so every window of the im2win paper (§III-C: for output
// (h, w), the R x S inputs at rows h*stride_h + r*dil_h, columns
// w*stride_w + q*dil_w of the padded plane) is read from LDS, and x and y
// each cross HBM once.  Loads and stores are consecutive across lanes.
// The epilogue is the library's: bias in fp32, optional ReLU (maxNum
// against 0) and 2x2 max-pool, one rounding to the output type.
#include <algorithm>

#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

constexpr int kDThreads = 256;
constexpr int kDwLdsBytes = 48 * 1024;   // staged planes per workgroup: at most this

struct DwImpArgs {
    int C, H, W, P, Q, R, S;
    int sh, sw, ph, pw, dh, dw;
    int Hp, Wp;          // padded plane extent in LDS
    int planes;          // total planes N * C
    int per;             // planes per workgroup
    int Po, Qo;          // output extent (pooled or not)
    int relu, pool;
    int strip;           // 3x3 strip form (planes padded to whole strips)
    int pairs;           // strip form, no pool: a lane takes two adjacent columns (Qo even)
    int dQ, dH, dW;      // 256 input elements as planes, rows and columns (dH < H, dW < W)
    int vec4;            // H * W a multiple of 4 and W >= 4: fp32 input staged with 16-byte loads
    FastDiv fdHW, fdW, fdPQo, fdQo;
    FastDiv fdStrip;     // strip items per plane: Qo * ceil(P / kSH), Qo / 2 * ceil(P / kSH) with
                         // pairs, or Qo * ceil(Po / kPS) with the pool
    FastDiv fdQh;        // Qo / 2
};

// KR x KS: the filter extent when fixed at compile time (0: run time).
// Every LDS access has consecutive lanes on consecutive words (no bank
// conflicts): the planes are zeroed with consecutive 16-byte stores, then x
// is copied element by element (consecutive lanes, consecutive elements:
// coalesced), and lane i of a pass computes output o0 + i.
// Two adjacent outputs, each rounded once to the output type, as one store
// (p is aligned to two elements).
template <typename T>
__device__ __forceinline__ void store_pair(T* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)f32_bits<T>(a) | ((uint32_t)f32_bits<T>(b) << 16);
}

template <>
__device__ __forceinline__ void store_pair<float>(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

constexpr int kSH = 7;   // outputs per lane down a column (strip form)
constexpr int kPS = 4;   // pooled outputs per lane down a column (strip form with the pool)

template <typename TIn, typename TOut, int KR, int KS, bool STRIP>
__global__ __launch_bounds__(kDThreads) void conv_dw_implicit_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ w, const TIn* __restrict__ bias,
    TOut* __restrict__ y, DwImpArgs a) {
    extern __shared__ __align__(16) float pl[];   // [per][Hp][Wp], per * R * S taps, per biases
    const int tid = threadIdx.x;
    const int p0 = blockIdx.x * a.per;             // first plane (n * C + c)
    const int np = min(a.per, a.planes - p0);
    const int R = KR ? KR : a.R, S = KS ? KS : a.S;
    const int HW = a.H * a.W, HpWp = a.Hp * a.Wp, RS = R * S;
    float* wl = pl + a.per * HpWp;
    float* bl = wl + a.per * RS;

    // x's elements go to registers first (consecutive elements on
    // consecutive lanes: coalesced), so the zeroing and the filter staging
    // run while they are in flight
    const TIn* xs = x + (size_t)p0 * HW;
    const int total = np * HW;
    constexpr int kU = 16;
    float v[kU];
    // fp32 planes whose area is a multiple of 4 come in 16-byte loads:
    // e0 then counts float4s, and float4 e0 + u * kDThreads lands in
    // v[4u .. 4u + 3]
    const bool vec4 = sizeof(TIn) == 4 && a.vec4;
    auto load = [&](int e0) {
        if (vec4) {
            const float4* xs4 = reinterpret_cast<const float4*>(xs);
#pragma unroll
            for (int u = 0; u < kU / 4; ++u) {
                const int e4 = e0 + u * kDThreads;
                const float4 t = 4 * e4 < total ? xs4[e4] : make_float4(0.f, 0.f, 0.f, 0.f);
                v[4 * u] = t.x;
                v[4 * u + 1] = t.y;
                v[4 * u + 2] = t.z;
                v[4 * u + 3] = t.w;
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int e = e0 + u * kDThreads;
            v[u] = e < total ? to_f32(xs[e]) : 0.f;
        }
    };
    load(tid);
    // zero the planes (padding included; a.per * HpWp is a multiple of 4)
    for (int e = tid; 4 * e < np * HpWp; e += kDThreads)
        reinterpret_cast<float4*>(pl)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int e = tid; e < np * RS; e += kDThreads) {
        const int c = (p0 + e / RS) % a.C;
        wl[e] = to_f32(w[(size_t)c * RS + e % RS]);
    }
    for (int e = tid; e < np; e += kDThreads) bl[e] = bias ? to_f32(bias[(p0 + e) % a.C]) : 0.f;
    __syncthreads();
    if (vec4) {
        // four elements of one plane a float4 (the area is a multiple of 4),
        // the last ones on the next row when the row ends inside it
        const int total4 = total / 4;
        for (int e0 = tid; e0 < total4; e0 += (kU / 4) * kDThreads) {
            if (e0 != tid) load(e0);
#pragma unroll
            for (int u = 0; u < kU / 4; ++u) {
                const int e4 = e0 + u * kDThreads;
                if (e4 < total4) {
                    const int el = 4 * e4;
                    const uint32_t q = fdiv((uint32_t)el, a.fdHW);
                    const int r = el - (int)q * HW;
                    const int hh = (int)fdiv((uint32_t)r, a.fdW);
                    const int ww = r - hh * a.W;
                    float* row = pl + q * HpWp + (hh + a.ph) * a.Wp + a.pw;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = ww + j;
                        row[c < a.W ? c : c - a.W + a.Wp] = v[4 * u + j];
                    }
                }
            }
        }
    }
    // the planes' interiors: a thread's elements are kDThreads apart, so
    // its LDS position is split into (plane, row, column) once and then
    // stepped by (dQ, dH, dW) with the carries
    const int step = a.dQ * HpWp + a.dH * a.Wp + a.dW;
    for (int e0 = tid; !vec4 && e0 < total; e0 += kU * kDThreads) {
        if (e0 != tid) load(e0);
        const uint32_t q0 = fdiv((uint32_t)e0, a.fdHW);
        const int r0 = e0 - (int)q0 * HW;
        int hh = (int)fdiv((uint32_t)r0, a.fdW);
        int ww = r0 - hh * a.W;
        int off = (int)q0 * HpWp + (hh + a.ph) * a.Wp + ww + a.pw;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (e0 + u * kDThreads < total) pl[off] = v[u];
            ww += a.dW;
            hh += a.dH;
            off += step;
            if (ww >= a.W) {            // next row
                ww -= a.W;
                ++hh;
                off += a.Wp - a.W;
            }
            if (hh >= a.H) {            // next plane
                hh -= a.H;
                off += HpWp - a.H * a.Wp;
            }
        }
    }
    __syncthreads();

    const int PQo = a.Po * a.Qo;
    TOut* ys = y + (size_t)p0 * PQo;
    if (STRIP && a.pool) {
        // 3x3, stride 1, dilation 1 with the 2x2 pool: a lane computes kPS
        // pooled outputs down one pooled column, the 2 kPS x 2 convolution
        // outputs under them from the (2 kPS + 2) x 4 inputs and the 9 taps
        // read once (the plane's zero rows reach the last strip's end)
        const int nps = (a.Po + kPS - 1) / kPS;
        const int per_plane = a.Qo * nps;
        for (int it = tid; it < np * per_plane; it += kDThreads) {
            const uint32_t q = fdiv((uint32_t)it, a.fdStrip);
            const int r = it - (int)q * per_plane;
            const uint32_t st = fdiv((uint32_t)r, a.fdQo);
            const int ow = r - (int)st * a.Qo;
            const int oi0 = (int)st * kPS;
            const float* src = pl + q * HpWp + 2 * oi0 * a.Wp + 2 * ow;
            const float* wt = wl + q * 9;
            float wr[9];
#pragma unroll
            for (int t = 0; t < 9; ++t) wr[t] = wt[t];
            float in[2 * kPS + 2][4];
#pragma unroll
            for (int rr = 0; rr < 2 * kPS + 2; ++rr)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) in[rr][cc] = src[rr * a.Wp + cc];
            const float b = bl[q];
            TOut* yo = ys + (size_t)q * PQo + (size_t)oi0 * a.Qo + ow;
#pragma unroll
            for (int i = 0; i < kPS; ++i) {
                if (oi0 + i < a.Po) {
                    float m = 0.f;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const int dr = 2 * i + (d >> 1), dc = d & 1;
                        float acc = 0.f;
#pragma unroll
                        for (int rr = 0; rr < 3; ++rr)
#pragma unroll
                            for (int cc = 0; cc < 3; ++cc)
                                acc = fmaf(in[dr + rr][dc + cc], wr[rr * 3 + cc], acc);
                        float v = acc + b;
                        if (a.relu) v = fmaxf(v, 0.f);
                        m = d == 0 ? v : fmaxf(m, v);
                    }
                    yo[i * a.Qo] = from_f32<TOut>(m);
                }
            }
        }
        return;
    }
    if (STRIP && a.pairs) {
        // 3x3, stride 1, dilation 1, no pool, Qo even: a lane computes kSH
        // outputs down two adjacent columns 2 cp, 2 cp + 1.  Their inputs are
        // the plane's columns 2 cp .. 2 cp + 3 (LDS columns; the interior
        // starts at pad_w), an 8-byte-aligned run (Wp and the plane area are
        // even): two 8-byte reads a row, and each output row leaves as one
        // 2-element store (Qo and P * Qo even).
        const int nstrip = (a.P + kSH - 1) / kSH;
        const int qh = a.Qo >> 1;
        const int per_plane = qh * nstrip;
        for (int it = tid; it < np * per_plane; it += kDThreads) {
            const uint32_t q = fdiv((uint32_t)it, a.fdStrip);
            const int r = it - (int)q * per_plane;
            const uint32_t st = fdiv((uint32_t)r, a.fdQh);
            const int cp = r - (int)st * qh;
            const int oh0 = (int)st * kSH;
            const float* src = pl + q * HpWp + oh0 * a.Wp + 2 * cp;
            const float* wt = wl + q * 9;
            float wr[9];
#pragma unroll
            for (int t = 0; t < 9; ++t) wr[t] = wt[t];
            const float b = bl[q];
            float in[kSH + 2][4];
#pragma unroll
            for (int rr = 0; rr < kSH + 2; ++rr) {
                const float2 lo = *reinterpret_cast<const float2*>(src + rr * a.Wp);
                const float2 hi = *reinterpret_cast<const float2*>(src + rr * a.Wp + 2);
                in[rr][0] = lo.x; in[rr][1] = lo.y; in[rr][2] = hi.x; in[rr][3] = hi.y;
            }
            TOut* yo = ys + (size_t)q * PQo + (size_t)oh0 * a.Qo + 2 * cp;
#pragma unroll
            for (int i = 0; i < kSH; ++i) {
                if (oh0 + i < a.P) {
                    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
                    for (int rr = 0; rr < 3; ++rr)
#pragma unroll
                        for (int cc = 0; cc < 3; ++cc) {
                            acc0 = fmaf(in[i + rr][cc], wr[rr * 3 + cc], acc0);
                            acc1 = fmaf(in[i + rr][cc + 1], wr[rr * 3 + cc], acc1);
                        }
                    float v0 = acc0 + b, v1 = acc1 + b;   // bias, then ReLU (maxNum against 0)
                    if (a.relu) {
                        v0 = fmaxf(v0, 0.f);
                        v1 = fmaxf(v1, 0.f);
                    }
                    store_pair(yo + i * a.Qo, v0, v1);
                }
            }
        }
        return;
    }
    if (STRIP) {
        // 3x3, stride 1, dilation 1, no pool: a lane computes kSH outputs
        // down one column (consecutive lanes: consecutive columns), reading
        // the (kSH + 2) x 3 inputs and the 9 taps once (the plane's zero
        // rows reach the last strip's end)
        const int nstrip = (a.P + kSH - 1) / kSH;
        const int per_plane = a.Qo * nstrip;
        for (int it = tid; it < np * per_plane; it += kDThreads) {
            const uint32_t q = fdiv((uint32_t)it, a.fdStrip);
            const int r = it - (int)q * per_plane;
            const uint32_t st = fdiv((uint32_t)r, a.fdQo);
            const int ow = r - (int)st * a.Qo;
            const int oh0 = (int)st * kSH;
            const float* src = pl + q * HpWp + oh0 * a.Wp + ow;
            const float* wt = wl + q * 9;
            float wr[9];
#pragma unroll
            for (int t = 0; t < 9; ++t) wr[t] = wt[t];
            float in[kSH + 2][3];
#pragma unroll
            for (int rr = 0; rr < kSH + 2; ++rr)
#pragma unroll
                for (int cc = 0; cc < 3; ++cc)
                    in[rr][cc] = src[rr * a.Wp + cc];
            const float b = bl[q];
            TOut* yo = ys + (size_t)q * PQo + (size_t)oh0 * a.Qo + ow;
#pragma unroll
            for (int i = 0; i < kSH; ++i) {
                if (oh0 + i < a.P) {
                    float acc = 0.f;
#pragma unroll
                    for (int rr = 0; rr < 3; ++rr)
#pragma unroll
                        for (int cc = 0; cc < 3; ++cc) acc = fmaf(in[i + rr][cc], wr[rr * 3 + cc], acc);
                    const float v = acc + b;
                    yo[i * a.Qo] = from_f32<TOut>(a.relu ? fmaxf(v, 0.f) : v);
                }
            }
        }
        return;
    }
    // outputs: consecutive elements of y on consecutive lanes
    for (int o = tid; o < np * PQo; o += kDThreads) {
        const uint32_t q = fdiv((uint32_t)o, a.fdPQo);
        const int r = o - (int)q * PQo;
        const uint32_t oh = fdiv((uint32_t)r, a.fdQo);
        const int ow = r - (int)oh * a.Qo;
        const float b = bl[q];
        const float* src = pl + q * HpWp;
        const float* wt = wl + q * RS;
        auto conv_at = [&](int h, int ww) {
            float acc = 0.f;
            const float* s0 = src + h * a.sh * a.Wp + ww * a.sw;
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
                for (int qq = 0; qq < S; ++qq)
                    acc = fmaf(s0[rr * a.dh * a.Wp + qq * a.dw], wt[rr * S + qq], acc);
            const float v = acc + b;
            return a.relu ? fmaxf(v, 0.f) : v;   // bias, then ReLU (maxNum against 0)
        };
        float v;
        if (a.pool) {
            const int h = 2 * (int)oh, ww = 2 * ow;
            v = fmaxf(fmaxf(conv_at(h, ww), conv_at(h, ww + 1)),
                      fmaxf(conv_at(h + 1, ww), conv_at(h + 1, ww + 1)));
        } else {
            v = conv_at((int)oh, ow);
        }
        ys[o] = from_f32<TOut>(v);
    }
}

bool dw_imp_plan(const Geom& g, const Epi& epi, int n_images, DwImpArgs& a, size_t& lds, int64_t& grid) {
    a.C = g.C; a.H = g.H; a.W = g.W; a.P = g.P; a.Q = g.Q; a.R = g.R; a.S = g.S;
    a.sh = g.sh; a.sw = g.sw; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh; a.dw = g.dw;
    a.Wp = g.W + 2 * g.pw;
    // LDS plane area a multiple of 4 words (the zeroing writes 16 bytes)
    auto plane_of = [&](int hp) {
        while (((int64_t)hp * a.Wp) % 4) ++hp;
        return hp;
    };
    auto bytes_of = [&](int hp) { return ((int64_t)hp * a.Wp + (int64_t)g.R * g.S + 1) * 4; };
    a.Hp = plane_of(g.H + 2 * g.ph);
    if (bytes_of(a.Hp) > kDwLdsBytes) return false;
    // the strip form reads kSH + 2 rows from each strip's first row: pad the
    // plane with zero rows to the last strip's end, when that still fits
    // (with the pool: 2 kPS + 2 rows from each pooled strip's first row)
    const int nstrip = epi.pool ? (g.P / 2 + kPS - 1) / kPS : (g.P + kSH - 1) / kSH;
    const int strip_rows = epi.pool ? 2 * kPS : kSH;
    a.strip = g.R == 3 && g.S == 3 && g.sh == 1 && g.sw == 1 && g.dh == 1 && g.dw == 1;
    if (a.strip) {
        const int hs = plane_of(std::max(a.Hp, nstrip * strip_rows + 2));
        if (bytes_of(hs) <= kDwLdsBytes) a.Hp = hs;
        else a.strip = 0;
    }
    // two columns a lane: Qo even (then Wp = Qo + 2 and P * Qo are even too)
    a.pairs = a.strip && !epi.pool && g.Q % 2 == 0 && a.Wp % 2 == 0 ? 1 : 0;
    const int64_t plane_bytes = bytes_of(a.Hp);
    const int64_t planes = (int64_t)n_images * g.C;
    if (planes * std::max<int64_t>((int64_t)g.H * g.W, (int64_t)g.P * g.Q) >= ((int64_t)1 << 31)) return false;
    a.planes = (int)planes;
    // as many planes as fit, up to about 16 input elements per thread, and
    // at least about 1024 workgroups
    int per = (int)std::min<int64_t>(kDwLdsBytes / plane_bytes, std::max<int64_t>(1, 16 * kDThreads / ((int64_t)g.H * g.W)));
    per = std::max(1, std::min<int>(per, (int)std::max<int64_t>(1, planes / 1024)));
    if (a.strip) {
        // every thread the same number of strips where that costs less
        // time per plane: 20 planes of 28 strips take 3 passes of 256
        // threads (2.2 on average), 18 planes take 2
        const int spp = (epi.pool || a.pairs ? g.Q / 2 : g.Q) * nstrip;
        const int it = (per * spp + kDThreads - 1) / kDThreads;
        const int per2 = (it - 1) * kDThreads / spp;
        if (it > 1 && per2 >= 1 && (int64_t)(it - 1) * per < (int64_t)it * per2) per = per2;
    }
    a.per = per;
    a.relu = epi.relu;
    a.pool = epi.pool;
    a.Po = out_rows(g, epi);
    a.Qo = out_cols(g, epi);
    {
        const int HW = g.H * g.W;
        a.dQ = kDThreads / HW;
        a.dH = (kDThreads % HW) / g.W;
        a.dW = (kDThreads % HW) % g.W;
        a.vec4 = (HW % 4 == 0 && g.W >= 4) ? 1 : 0;
    }
    a.fdHW = make_fastdiv((uint32_t)(g.H * g.W));
    a.fdW = make_fastdiv((uint32_t)g.W);
    a.fdPQo = make_fastdiv((uint32_t)(a.Po * a.Qo));
    a.fdQo = make_fastdiv((uint32_t)a.Qo);
    a.fdStrip = make_fastdiv((uint32_t)((a.pairs ? a.Qo / 2 : a.Qo) * nstrip));
    a.fdQh = make_fastdiv((uint32_t)std::max(a.Qo / 2, 1));
    lds = (size_t)per * plane_bytes;
    grid = (planes + per - 1) / per;
    return true;
}

template <typename TIn, typename TOut>
hipError_t launch_dwi(const Geom& g, const void* x, const void* w, const void* bias, void* y,
                      const Epi& epi, hipStream_t st) {
    DwImpArgs a;
    size_t lds = 0;
    int64_t grid = 0;
    if (!dw_imp_plan(g, epi, g.N, a, lds, grid)) return hipErrorInvalidValue;
    if ((uintptr_t)y % (2 * sizeof(TOut)) != 0) {   // pair stores need y aligned to two elements
        if (a.pairs) {
            a.pairs = 0;
            a.fdStrip = make_fastdiv((uint32_t)(a.Qo * ((a.P + kSH - 1) / kSH)));
        }
    }
    const bool r3 = g.R == 3 && g.S == 3;
    void (*kfn)(const TIn*, const TIn*, const TIn*, TOut*, DwImpArgs) =
        a.strip ? conv_dw_implicit_kernel<TIn, TOut, 3, 3, true>
              : r3 ? conv_dw_implicit_kernel<TIn, TOut, 3, 3, false>
                   : conv_dw_implicit_kernel<TIn, TOut, 0, 0, false>;
    hipLaunchKernelGGL(kfn, dim3((uint32_t)grid), dim3(kDThreads), lds, st,
                       (const TIn*)x, (const TIn*)w, (const TIn*)bias, (TOut*)y, a);
    return hipGetLastError();
}

}  // namespace

bool dw_implicit_supported(const Geom& g, const Epi& epi) {
    DwImpArgs a;
    size_t lds = 0;
    int64_t grid = 0;
    return dw_imp_plan(g, epi, std::max(g.N, 1), a, lds, grid);
}

hipError_t launch_conv_dw_implicit(const Geom& g, ciw_dtype in, ciw_dtype out, const void* x,
                                   const void* w, const void* bias, void* y, const Epi& epi,
                                   hipStream_t st) {
    if (g.N == 0) return hipSuccess;
    if (in == CIW_F32) return launch_dwi<float, float>(g, x, w, bias, y, epi, st);
    if (in == CIW_F16)
        return out == CIW_F32 ? launch_dwi<half_t, float>(g, x, w, bias, y, epi, st)
                              : launch_dwi<half_t, half_t>(g, x, w, bias, y, epi, st);
    return out == CIW_F32 ? launch_dwi<bf16_t, float>(g, x, w, bias, y, epi, st)
                          : launch_dwi<bf16_t, bf16_t>(g, x, w, bias, y, epi, st);
}

}  // namespace ciw
