// conv_fp32_mfma.hip -- fp32 dense windowed contraction on the gfx950
// matrix cores (v_mfma_f32_32x32x2_f32), over the CHW window tensor.
//
// The im2win paper runs fp32 on CUDA cores (§III-F).  On this GPU the fp32
// matrix instruction has twice the throughput of the plain vector FMA, and
// the contraction is a dense product: output channels x output pixels,
// reduced over (channel, filter row, filter column).  The window of output
// (n, h, w) in the CHW window tensor is, per channel c, the elements
// xw[n][c][h][(w*stride_w + q*dil_w)*R + r] (§III-C: the R values of a
// column adjacent, columns in order).
//
// A workgroup (8 waves) owns 32 output channels, a block of up to 192
// output pixels (whole output rows of one image) and a slice of up to 64
// input channels, which it streams through LDS in chunks of 16 channels
// (filter rows and window rows, double-buffered).  Wave t owns pixel tiles
// 3 (t & 1) .. 3 (t & 1) + 2 and reduces quarter t >> 1 of each chunk's
// channels.  One MFMA step takes two reduction entries (lane / 32 picks
// one): a channel pair at one filter tap.  The four quarters' sums are added
// through LDS in quarter order; with several slices the slice sums go to a
// partial buffer [slice][n][K][P*Q] that a second kernel adds in slice
// order, then the bias and ReLU.  Every sum is in a fixed order: results
// are deterministic.  (32 channels per workgroup rather than 64 keeps the
// filter read once while halving the slices, and with them the partial
// sums written and read back.)
#include <algorithm>

#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

constexpr int kMThreads = 512;   // 8 waves
constexpr int kMaxPix = 192;     // pixels per block: 6 tiles of 32
constexpr int kMT = 32;          // output channels per workgroup
constexpr int kTC = 64;          // input channels per slice (at most)
constexpr int kCh = 16;          // channels per LDS chunk (two pairs per quarter)
constexpr int kMaxB = 6;         // window float4 loads per thread per chunk
constexpr int kMaxBI = 10;       // in-LDS form: input elements per thread per chunk

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct F32MArgs {
    int C, K, P, Q, pitch, sw, dw;
    int HB;          // output rows per pixel block
    int pblocks;     // pixel blocks per image
    int mblocks;     // 32-channel blocks
    int splits, TC;  // channel slices, channels per slice (even)
    int AS;          // LDS row stride of the staged filter (floats)
    int BS;          // LDS stride between staged channels of the window (floats)
    int ntask, nimg;
    int relu;
    // in-LDS form: the block's input rows staged from x, zero-padded
    int H, W, sh, ph, pw, dh;
    int Hr, Wpl;     // staged rows and columns per channel
    int nBI;         // staged elements per chunk (kCh * Hr * Wpl)
};

// IMP: the in-LDS form.  xw is then x itself, and a chunk stages, per
// channel, the zero-padded input rows h0 * stride_h - pad_h .. of its pixel
// block ([Hr][Wpl] with Wpl the padded columns the windows touch) instead of
// the block's window rows; the window of output (h, w) at tap (r, q) is the
// staged element (h * stride_h + r * dil_h, w * stride_w + q * dil_w).  The
// window tensor is never written.
template <int R, int S, bool IMP>
__global__ __launch_bounds__(kMThreads, 1) void conv_fp32_mfma_kernel(
    const float* __restrict__ xw, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ out, F32MArgs a) {
    constexpr int RS = R * S;
    extern __shared__ __align__(16) float smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qt = wave >> 1;         // quarter of each chunk's channels
    const int pg = wave & 1;          // pixel tiles 3 pg .. 3 pg + 2
    const int j = lane & 31;          // A row (channel) / B column (pixel) of the lane
    const int kk = lane >> 5;         // reduction entry of the pair

    // task = (slice, image, pixel block, channel block), channel block
    // fastest; with the grid a multiple of 8 consecutive tasks share an XCD
    // (dispatch is round-robin over 8), so the channel blocks reading one
    // slice's window rows meet in one L2
    int task = blockIdx.x;
    if ((a.ntask & 7) == 0) task = (int)(blockIdx.x & 7) * (a.ntask >> 3) + (int)(blockIdx.x >> 3);
    const int mb = task % a.mblocks;
    int rest = task / a.mblocks;
    const int pb = rest % a.pblocks;
    rest /= a.pblocks;
    const int n_img = rest % a.nimg;
    const int sl = rest / a.nimg;
    const int k0 = mb * kMT;
    const int h0 = pb * a.HB;
    const int rows = min(a.HB, a.P - h0);
    const int npx = rows * a.Q;
    const int c0 = sl * a.TC;
    const int tc = min(a.TC, a.C - c0);          // channels present in this slice

    // ---- the slice in chunks of kCh channels, double-buffered in LDS: the
    // global loads of chunk ch + 1 are in flight (in registers) while chunk
    // ch multiplies, then land in the other buffer.  A chunk holds the
    // filter rows k0 .. k0 + 31 over its channels cc .. cc + kCh - 1,
    // entries (c - cc) * RS + r * S + q of the KCRS filter ([32][AS], zero
    // past K and C), and the window rows h0 .. h0 + rows - 1 of its
    // channels ([kCh][BS]).  Consecutive lanes load consecutive floats of
    // a filter row and write consecutive LDS banks.
    const int chunk_floats = kMT * a.AS + kCh * a.BS;
    const int nch = (tc + kCh - 1) / kCh;
    constexpr int T = kCh * RS;                  // filter entries per chunk row
    constexpr int kAL = (kMT * T + kMThreads - 1) / kMThreads;  // filter loads per thread
    const int run4 = rows * a.pitch / 4;         // float4 per channel (pitch is a multiple of 4)
    const int nB4 = kCh * run4;
    const int kBL = (nB4 + kMThreads - 1) / kMThreads;          // window loads per thread (<= kMaxB)
    // in-LDS form: a thread's staged elements are the same positions in
    // every chunk (only the channel base moves), so each one's source offset
    // within its channel's plane (-1: zero padding), channel and LDS offset
    // are worked out once
    int bi_src[IMP ? kMaxBI : 1], bi_cl[IMP ? kMaxBI : 1], bi_dst[IMP ? kMaxBI : 1];
    if constexpr (IMP) {
        const int per_ch = a.Hr * a.Wpl;
#pragma unroll
        for (int u = 0; u < kMaxBI; ++u) {
            const int e = tid + u * kMThreads;
            const int cl = e / per_ch, rr = e - cl * per_ch;
            const int y = rr / a.Wpl, xx = rr - y * a.Wpl;
            const int iy = h0 * a.sh - a.ph + y, ix = xx - a.pw;
            bi_cl[u] = e < a.nBI ? cl : kCh;             // kCh: nothing to stage
            bi_src[u] = (iy >= 0 && iy < a.H && ix >= 0 && ix < a.W) ? iy * a.W + ix : -1;
            bi_dst[u] = cl * a.BS + y * a.Wpl + xx;
        }
    }
    struct Fetched {
        float ra[kAL];
        float4 rb[IMP ? 1 : kMaxB];
        float rbi[IMP ? kMaxBI : 1];
    };
    auto fetch = [&](Fetched& f, int ch) {
        float (&ra)[kAL] = f.ra;
        auto& rb = f.rb;
        const int cc = c0 + ch * kCh;            // first channel of the chunk
        const int nc = min(kCh, c0 + tc - cc);   // channels present
#pragma unroll
        for (int u = 0; u < kAL; ++u) {
            const int e = tid + u * kMThreads;
            const int row = e / T, t = e - row * T;
            ra[u] = 0.f;
            if (e < kMT * T && k0 + row < a.K && t < nc * RS)
                ra[u] = w[((size_t)(k0 + row) * a.C + cc) * RS + t];
        }
        if constexpr (IMP) {
            const float* xc = xw + ((size_t)n_img * a.C + cc) * ((size_t)a.H * a.W);
#pragma unroll
            for (int u = 0; u < kMaxBI; ++u) {
                f.rbi[u] = 0.f;
                if (bi_cl[u] < nc && bi_src[u] >= 0)
                    f.rbi[u] = xc[(size_t)bi_cl[u] * a.H * a.W + bi_src[u]];
            }
            return;
        } else {
#pragma unroll
            for (int u = 0; u < kMaxB; ++u) {
                const int e = tid + u * kMThreads;
                const int cl = e / run4, o = (e - cl * run4) * 4;
                rb[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (u < kBL && e < nB4 && cl < nc)
                    rb[u] = *reinterpret_cast<const float4*>(
                        xw + (((size_t)n_img * a.C + cc + cl) * a.P + h0) * a.pitch + o);
            }
        }
    };
    auto stash = [&](const Fetched& f, int buf) {
        const float (&ra)[kAL] = f.ra;
        const auto& rb = f.rb;
        float* As = smem + buf * chunk_floats;
        float* Bs = As + kMT * a.AS;
#pragma unroll
        for (int u = 0; u < kAL; ++u) {
            const int e = tid + u * kMThreads;
            const int row = e / T, t = e - row * T;
            if (e < kMT * T) As[row * a.AS + t] = ra[u];
        }
        if constexpr (IMP) {
#pragma unroll
            for (int u = 0; u < kMaxBI; ++u)
                if (bi_cl[u] < kCh) Bs[bi_dst[u]] = f.rbi[u];
        } else {
#pragma unroll
            for (int u = 0; u < kMaxB; ++u) {
                const int e = tid + u * kMThreads;
                const int cl = e / run4, o = (e - cl * run4) * 4;
                if (u < kBL && e < nB4) *reinterpret_cast<float4*>(Bs + cl * a.BS + o) = rb[u];
            }
        }
    };

    int pxoff[3];
#pragma unroll
    for (int t3 = 0; t3 < 3; ++t3) {
        // pixels past the block read its last pixel (never stored)
        const int px = min((3 * pg + t3) * 32 + j, npx - 1);
        const int hh = px / a.Q, ww = px - hh * a.Q;
        pxoff[t3] = IMP ? hh * a.sh * a.Wpl + ww * a.sw : hh * a.pitch + ww * a.sw * R;
    }
    int toff[RS];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < S; ++q) toff[r * S + q] = IMP ? r * a.dh * a.Wpl + q * a.dw : q * a.dw * R + r;
    f32x16 acc[3];
#pragma unroll
    for (int t3 = 0; t3 < 3; ++t3)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t3][v] = 0.f;

    // One chunk: the quarter's channel pairs (kCh / 8 of them), each the
    // lane's filter taps and, per pixel tile, its window taps; the second
    // pair's operands are read while the first pair multiplies.
    struct Ops {
        float av[RS];
        float bv[3][RS];
    };
    auto multiply = [&](int buf) {
        const float* As = smem + buf * chunk_floats;
        const float* Bs = As + kMT * a.AS;
        const float* arow = As + j * a.AS + kk * RS;
        const float* bch = Bs + kk * a.BS;
        auto load = [&](Ops& o, int cp) {
            const int cl = qt * (kCh / 4) + 2 * cp;     // lane's channel: cl + kk
            const float* ap = arow + cl * RS;
            const float* bp = bch + cl * a.BS;
#pragma unroll
            for (int t = 0; t < RS; ++t) o.av[t] = ap[t];
#pragma unroll
            for (int t3 = 0; t3 < 3; ++t3)
#pragma unroll
                for (int t = 0; t < RS; ++t) o.bv[t3][t] = bp[pxoff[t3] + toff[t]];
        };
        auto mul = [&](const Ops& o) {
#pragma unroll
            for (int t = 0; t < RS; ++t)
#pragma unroll
                for (int t3 = 0; t3 < 3; ++t3)
                    acc[t3] = __builtin_amdgcn_mfma_f32_32x32x2f32(o.av[t], o.bv[t3][t], acc[t3], 0, 0, 0);
        };
        Ops o0, o1;
        load(o0, 0);
        load(o1, 1);
        mul(o0);
        mul(o1);
    };

    // chunk ch + 1's loads are in flight while chunk ch multiplies
    Fetched f;
    fetch(f, 0);
    stash(f, 0);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        if (ch + 1 < nch) fetch(f, ch + 1);
        multiply(ch & 1);
        if (ch + 1 < nch) stash(f, (ch + 1) & 1);
        __syncthreads();
    }

    // ---- the four quarters' sums (through LDS; the chunk buffers are no
    // longer read after the loop's last barrier).  Wave (pg, qt) finishes
    // entries 4 qt .. 4 qt + 3 of each of its tiles' 16: it hands the other
    // 12 to the waves of the other quarters with the same tiles, and adds
    // the four quarters' values of its own entries in quarter order.
    // red[dst quarter][pg][src quarter][t3][4][64]
    float* red = smem;
    auto slot = [&](int dq, int sq) { return red + (((dq * 2 + pg) * 4 + sq) * 3) * 4 * 64; };
#pragma unroll
    for (int dq = 0; dq < 4; ++dq) {
        if (dq == qt) continue;
        float* to = slot(dq, qt);
#pragma unroll
        for (int t3 = 0; t3 < 3; ++t3)
#pragma unroll
            for (int e = 0; e < 4; ++e) to[(t3 * 4 + e) * 64 + lane] = acc[t3][4 * dq + e];
    }
    __syncthreads();
    // lane holds D[i][j] for channel i = 8 (v / 4) + 4 kk + v % 4 of the
    // tile, pixel j of the tile
    const int PQ = a.P * a.Q;
    const bool final_out = a.splits == 1;
    float* base = out + ((size_t)(final_out ? 0 : sl) * a.nimg + n_img) * a.K * PQ + (size_t)h0 * a.Q;
#pragma unroll
    for (int t3 = 0; t3 < 3; ++t3) {
        const int px = (3 * pg + t3) * 32 + j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = k0 + 8 * qt + 4 * kk + e;
            // the wave's own value of entry vv (qt is uniform: a branch, no
            // indexed register access)
            const float mine = qt == 0 ? acc[t3][e] : qt == 1 ? acc[t3][4 + e]
                             : qt == 2 ? acc[t3][8 + e] : acc[t3][12 + e];
            float s = 0.f;
#pragma unroll
            for (int sq = 0; sq < 4; ++sq)
                s += sq == qt ? mine : slot(qt, sq)[(t3 * 4 + e) * 64 + lane];
            if (px < npx && k < a.K) {
                if (final_out) {
                    s += bias ? bias[k] : 0.f;
                    if (a.relu) s = fmaxf(s, 0.f);
                }
                base[(size_t)k * PQ + px] = s;
            }
        }
    }
}

// y[i] = bias[k] + sum over slices s (in order) of part[s][i], i = (n*K + k)*PQ + pix.
// One output per thread (consecutive threads, consecutive outputs: every
// slice's loads are coalesced), the slices' loads issued kRedMax at a time
// before their in-order sum.
constexpr int kRedMax = 16;
__global__ __launch_bounds__(256) void split_reduce_nkp_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, float* __restrict__ y,
    uint32_t per_split, int splits, int PQ, int K, int relu) {
    const uint32_t t = blockIdx.x * 256 + threadIdx.x;
    if (t >= per_split) return;
    float acc = 0.f;
    for (int s0 = 0; s0 < splits; s0 += kRedMax) {
        float v[kRedMax];
#pragma unroll
        for (int s = 0; s < kRedMax; ++s)
            if (s0 + s < splits) v[s] = part[(size_t)(s0 + s) * per_split + t];
#pragma unroll
        for (int s = 0; s < kRedMax; ++s)
            if (s0 + s < splits) acc += v[s];
    }
    const int k = (int)((t / (uint32_t)PQ) % (uint32_t)K);
    const float v = acc + (bias ? bias[k] : 0.f);
    y[t] = relu ? fmaxf(v, 0.f) : v;
}

struct F32MPlan {
    F32MArgs a;
    size_t lds;
};

// Layers this kernel runs: fp32, 3x3 or 1x1 filters, an output row of at
// most 192 pixels, and the staged slice within 160 KB of LDS.  imp: the
// in-LDS form (a chunk's zero-padded input rows at most kMaxBI elements a
// thread).
bool f32m_plan(const Geom& g, int n_images, F32MPlan& pl, bool imp = false) {
    if (!((g.R == 3 && g.S == 3) || (g.R == 1 && g.S == 1))) return false;
    if (g.Q > kMaxPix || g.C < 2) return false;
    F32MArgs& a = pl.a;
    a.C = g.C; a.K = g.K; a.P = g.P; a.Q = g.Q; a.pitch = g.pitchA; a.sw = g.sw; a.dw = g.dw;
    a.HB = std::min(g.P, kMaxPix / g.Q);
    a.pblocks = (g.P + a.HB - 1) / a.HB;
    a.mblocks = (g.K + kMT - 1) / kMT;
    const int RS = g.R * g.S;
    // slices: about one workgroup per CU in total, each slice whole chunks
    // of kCh channels, at most kTC
    const int64_t others = (int64_t)n_images * a.pblocks * a.mblocks;
    int want = (int)std::max<int64_t>(1, (256 + others - 1) / others);
    int tc = (g.C + want - 1) / want;
    tc = (tc + kCh - 1) / kCh * kCh;             // whole chunks
    tc = std::min(tc, kTC);
    a.TC = tc;
    a.splits = (g.C + tc - 1) / tc;
    a.AS = kCh * RS + 1;                         // odd stride: lanes of a fragment in distinct banks
    a.H = g.H; a.W = g.W; a.sh = g.sh; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh;
    if (imp) {
        // the input rows a pixel block's windows span, and the padded columns
        const int64_t hr = (int64_t)(a.HB - 1) * g.sh + (int64_t)(g.R - 1) * g.dh + 1;
        const int64_t per_ch = hr * g.Wwin;
        if (kCh * per_ch > (int64_t)kMaxBI * kMThreads) return false;
        a.Hr = (int)hr;
        a.Wpl = g.Wwin;
        a.BS = (int)per_ch + 4;
        a.nBI = (int)(kCh * per_ch);
    } else {
        a.Hr = a.Wpl = a.nBI = 0;
        a.BS = a.HB * g.pitchA + 4;
        // window float4 loads per thread per chunk
        if ((kCh * (a.HB * g.pitchA / 4) + kMThreads - 1) / kMThreads > kMaxB) return false;
    }
    const int64_t ntask = others * a.splits;
    if (ntask >= (1ll << 31)) return false;
    a.ntask = (int)ntask;
    a.nimg = n_images;
    const size_t staged = (size_t)2 * ((size_t)kMT * a.AS + (size_t)kCh * a.BS) * 4;
    const size_t red = (size_t)4 * 2 * 4 * 3 * 4 * 64 * 4;   // [4][2][4][3][4][64] floats
    pl.lds = std::max(staged, red);
    return pl.lds <= 160 * 1024;
}

// The contraction kernel (window rows from xw, or the in-LDS form from x),
// then the slice reduction when the channel sum is split.
hipError_t launch_f32m(const Geom& g, const F32MPlan& pl, const float* src, const float* w,
                       const float* bias, float* y, int n_images, float* partials, const Epi& epi,
                       hipStream_t st, bool imp) {
    void (*kfn)(const float*, const float*, const float*, float*, F32MArgs) =
        imp ? (g.R == 3 ? conv_fp32_mfma_kernel<3, 3, true> : conv_fp32_mfma_kernel<1, 1, true>)
            : (g.R == 3 ? conv_fp32_mfma_kernel<3, 3, false> : conv_fp32_mfma_kernel<1, 1, false>);
    if (pl.lds > 65536 && allow_dynamic_lds(reinterpret_cast<const void*>(kfn), pl.lds) != hipSuccess)
        return hipErrorInvalidValue;
    float* dst = pl.a.splits == 1 ? y : partials;
    hipLaunchKernelGGL(kfn, dim3((uint32_t)pl.a.ntask), dim3(kMThreads), pl.lds, st, src, w, bias, dst, pl.a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.a.splits == 1) return e;
    const int64_t per_split = (int64_t)n_images * g.K * g.P * g.Q;
    hipLaunchKernelGGL(split_reduce_nkp_kernel, dim3((uint32_t)((per_split + 255) / 256)), dim3(256), 0,
                       st, partials, bias, y, (uint32_t)per_split, pl.a.splits, g.P * g.Q, g.K,
                       (int)epi.relu);
    return hipGetLastError();
}

}  // namespace

int fp32_mfma_splits(const Geom& g, int n_images) {
    F32MPlan pl;
    return f32m_plan(g, n_images, pl) ? pl.a.splits : 0;
}

hipError_t launch_conv_fp32_mfma(const Geom& g, const float* xw, const float* w, const float* bias,
                                 float* y, int n_images, float* partials, int max_splits,
                                 const Epi& epi, hipStream_t st) {
    F32MPlan pl;
    if (n_images == 0) return hipSuccess;
    if (epi.pool || !f32m_plan(g, n_images, pl) || pl.a.splits > max_splits) return hipErrorNotSupported;
    pl.a.relu = epi.relu;
    return launch_f32m(g, pl, xw, w, bias, y, n_images, partials, epi, st, false);
}

bool fp32_implicit_workspace(const Geom& g, const Epi& epi, size_t* bytes) {
    if (!epi.pool && fp32_m16_tasks(g, std::max(g.N, 1), true) > 0) {   // the whole-sum kernel: no workspace
        *bytes = 0;
        return true;
    }
    F32MPlan pl;
    if (epi.pool || !f32m_plan(g, std::max(g.N, 1), pl, true)) return false;
    const int64_t per_split = (int64_t)std::max(g.N, 1) * g.K * g.P * g.Q;
    *bytes = pl.a.splits > 1 ? (size_t)pl.a.splits * (size_t)per_split * sizeof(float) : 0;
    return true;
}

hipError_t launch_conv_fp32_implicit(const Geom& g, const float* x, const float* w, const float* bias,
                                     float* y, float* partials, const Epi& epi, hipStream_t st) {
    F32MPlan pl;
    if (g.N == 0) return hipSuccess;
    if (!epi.pool && fp32_m16_tasks(g, g.N, true) > 0)
        return launch_conv_fp32_m16(g, x, w, bias, y, g.N, epi, true, st);
    if (epi.pool || !f32m_plan(g, g.N, pl, true)) return hipErrorNotSupported;
    pl.a.relu = epi.relu;
    return launch_f32m(g, pl, x, w, bias, y, g.N, partials, epi, st, true);
}

}  // namespace ciw
