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
// A workgroup (8 waves) owns 64 output channels, a block of up to 192
// output pixels (whole output rows of one image) and a slice of TC input
// channels, which it streams through LDS in chunks of 8 channels (filter
// rows and window rows, double-buffered).  Waves 0-3 reduce the first half
// of each chunk, waves 4-7 the second; within a half, wave t owns channel tile t & 1 (32
// channels) and pixel tiles 3 (t >> 1) .. 3 (t >> 1) + 2.  One MFMA step
// takes two reduction entries (lane / 32 picks one): a channel pair at one
// filter tap.  The two halves' sums are added through LDS, first half
// first; with several slices the slice sums go to a partial
// buffer [slice][n][K][P*Q] that a second kernel adds in slice order, then
// the bias and ReLU.  Every sum is in a fixed order: results are
// deterministic.
#include <algorithm>

#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

constexpr int kMThreads = 512;   // 8 waves
constexpr int kMaxPix = 192;     // pixels per block: 6 tiles of 32
constexpr int kTC = 32;          // input channels per slice (at most)
constexpr int kCh = 8;           // channels per LDS chunk (two pairs per half)
constexpr int kMaxB = 3;         // window float4 loads per thread per chunk

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct F32MArgs {
    int C, K, P, Q, pitch, sw, dw;
    int HB;          // output rows per pixel block
    int pblocks;     // pixel blocks per image
    int mblocks;     // 64-channel blocks
    int splits, TC;  // channel slices, channels per slice (even)
    int AS;          // LDS row stride of the staged filter (floats)
    int BS;          // LDS stride between staged channels of the window (floats)
    int ntask, nimg;
    int relu;
};

template <int R, int S>
__global__ __launch_bounds__(kMThreads, 1) void conv_fp32_mfma_kernel(
    const float* __restrict__ xw, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ out, F32MArgs a) {
    constexpr int RS = R * S;
    extern __shared__ __align__(16) float smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2;
    const int ct = wave & 1;          // channel tile
    const int pg = (wave >> 1) & 1;   // pixel tiles 3 pg .. 3 pg + 2
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
    const int k0 = mb * 64;
    const int h0 = pb * a.HB;
    const int rows = min(a.HB, a.P - h0);
    const int npx = rows * a.Q;
    const int c0 = sl * a.TC;
    const int tc = min(a.TC, a.C - c0);          // channels present in this slice

    // ---- the slice in chunks of kCh channels, double-buffered in LDS: the
    // global loads of chunk ch + 1 are in flight (in registers) while chunk
    // ch multiplies, then land in the other buffer.  A chunk holds the
    // filter rows k0 .. k0 + 63 over its channels cc .. cc + kCh - 1,
    // entries (c - cc) * RS + r * S + q of the KCRS filter ([64][AS], zero
    // past K and C), and the window rows h0 .. h0 + rows - 1 of its
    // channels ([kCh][BS]).  Consecutive lanes load consecutive floats of
    // a filter row and write consecutive LDS banks.
    const int chunk_floats = 64 * a.AS + kCh * a.BS;
    const int nch = (tc + kCh - 1) / kCh;
    constexpr int T = kCh * RS;                  // filter entries per chunk row
    constexpr int kAL = (64 * T + kMThreads - 1) / kMThreads;   // filter loads per thread
    const int run4 = rows * a.pitch / 4;         // float4 per channel (pitch is a multiple of 4)
    const int nB4 = kCh * run4;
    const int kBL = (nB4 + kMThreads - 1) / kMThreads;          // window loads per thread (<= kMaxB)
    struct Fetched {
        float ra[kAL];
        float4 rb[kMaxB];
    };
    auto fetch = [&](Fetched& f, int ch) {
        float (&ra)[kAL] = f.ra;
        float4 (&rb)[kMaxB] = f.rb;
        const int cc = c0 + ch * kCh;            // first channel of the chunk
        const int nc = min(kCh, c0 + tc - cc);   // channels present
#pragma unroll
        for (int u = 0; u < kAL; ++u) {
            const int e = tid + u * kMThreads;
            const int row = e / T, t = e - row * T;
            ra[u] = 0.f;
            if (e < 64 * T && k0 + row < a.K && t < nc * RS)
                ra[u] = w[((size_t)(k0 + row) * a.C + cc) * RS + t];
        }
#pragma unroll
        for (int u = 0; u < kMaxB; ++u) {
            const int e = tid + u * kMThreads;
            const int cl = e / run4, o = (e - cl * run4) * 4;
            rb[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (u < kBL && e < nB4 && cl < nc)
                rb[u] = *reinterpret_cast<const float4*>(
                    xw + (((size_t)n_img * a.C + cc + cl) * a.P + h0) * a.pitch + o);
        }
    };
    auto stash = [&](const Fetched& f, int buf) {
        const float (&ra)[kAL] = f.ra;
        const float4 (&rb)[kMaxB] = f.rb;
        float* As = smem + buf * chunk_floats;
        float* Bs = As + 64 * a.AS;
#pragma unroll
        for (int u = 0; u < kAL; ++u) {
            const int e = tid + u * kMThreads;
            const int row = e / T, t = e - row * T;
            if (e < 64 * T) As[row * a.AS + t] = ra[u];
        }
#pragma unroll
        for (int u = 0; u < kMaxB; ++u) {
            const int e = tid + u * kMThreads;
            const int cl = e / run4, o = (e - cl * run4) * 4;
            if (u < kBL && e < nB4) *reinterpret_cast<float4*>(Bs + cl * a.BS + o) = rb[u];
        }
    };

    int pxoff[3];
#pragma unroll
    for (int t3 = 0; t3 < 3; ++t3) {
        // pixels past the block read its last pixel (never stored)
        const int px = min((3 * pg + t3) * 32 + j, npx - 1);
        const int hh = px / a.Q, ww = px - hh * a.Q;
        pxoff[t3] = hh * a.pitch + ww * a.sw * R;
    }
    int toff[RS];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < S; ++q) toff[r * S + q] = q * a.dw * R + r;
    f32x16 acc[3];
#pragma unroll
    for (int t3 = 0; t3 < 3; ++t3)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t3][v] = 0.f;

    // One chunk: the half's channel pairs (kCh / 4 of them), each the
    // lane's filter taps and, per pixel tile, its window taps; the second
    // pair's operands are read while the first pair multiplies.
    struct Ops {
        float av[RS];
        float bv[3][RS];
    };
    auto multiply = [&](int buf) {
        const float* As = smem + buf * chunk_floats;
        const float* Bs = As + 64 * a.AS;
        const float* arow = As + (ct * 32 + j) * a.AS + kk * RS;
        const float* bch = Bs + kk * a.BS;
        auto load = [&](Ops& o, int cp) {
            const int cl = half * (kCh / 2) + 2 * cp;   // lane's channel: cl + kk
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

    // ---- the two halves' sums (through LDS; the chunk buffers are no
    // longer read after the loop's last barrier).
    // Each half finishes 8 of a lane's 16 entries per tile (half h the
    // entries 8 h .. 8 h + 7): it hands the other 8 to the wave of the
    // other half with the same tiles, which adds them after its own (first
    // half first, the sum's fixed order).
    float* red = smem;                           // [2 halves][4 waves][3][8][64]
    const int tg = wave & 3;
    const int mine = half * 8, theirs = 8 - half * 8;
    float* to_other = red + ((1 - half) * 4 + tg) * 3 * 8 * 64;
    const float* from_other = red + (half * 4 + tg) * 3 * 8 * 64;
#pragma unroll
    for (int t3 = 0; t3 < 3; ++t3)
#pragma unroll
        for (int v = 0; v < 8; ++v) to_other[(t3 * 8 + v) * 64 + lane] = acc[t3][theirs + v];
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
        for (int v = 0; v < 8; ++v) {
            const int vv = mine + v;
            const int k = k0 + ct * 32 + 8 * (vv >> 2) + 4 * kk + (vv & 3);
            const float o = from_other[(t3 * 8 + v) * 64 + lane];
            float s = half == 0 ? acc[t3][vv] + o : o + acc[t3][vv];
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
// VEC (a slice holds a multiple of 4 outputs, so every slice starts 16-byte
// aligned): four consecutive outputs per thread with 16-byte loads and
// stores, every slice's loads issued before the sums, which then run in
// slice order.  Otherwise one output per thread.
constexpr int kRedMax = 32;   // slices a thread holds in registers at once
template <bool VEC>
__global__ __launch_bounds__(256) void split_reduce_nkp_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, float* __restrict__ y,
    uint32_t per_split, int splits, int PQ, int K, int relu) {
    const uint32_t t = blockIdx.x * 256 + threadIdx.x;
    if (!VEC) {
        if (t >= per_split) return;
        float v = 0.f;
        for (int s = 0; s < splits; ++s) v += part[(size_t)s * per_split + t];
        const int k = (int)((t / (uint32_t)PQ) % (uint32_t)K);
        v += bias ? bias[k] : 0.f;
        y[t] = relu ? fmaxf(v, 0.f) : v;
        return;
    }
    if (4 * t >= per_split) return;
    const float4* p4 = reinterpret_cast<const float4*>(part) + t;
    const uint32_t stride4 = per_split / 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < splits; s0 += kRedMax) {
        float4 v[kRedMax];
#pragma unroll
        for (int s = 0; s < kRedMax; ++s)
            if (s0 + s < splits) v[s] = p4[(size_t)(s0 + s) * stride4];
#pragma unroll
        for (int s = 0; s < kRedMax; ++s)
            if (s0 + s < splits) {
                acc.x += v[s].x; acc.y += v[s].y; acc.z += v[s].z; acc.w += v[s].w;
            }
    }
    float* a = &acc.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int k = (int)(((4 * t + e) / (uint32_t)PQ) % (uint32_t)K);
        const float v = a[e] + (bias ? bias[k] : 0.f);
        a[e] = relu ? fmaxf(v, 0.f) : v;
    }
    reinterpret_cast<float4*>(y)[t] = acc;
}

struct F32MPlan {
    F32MArgs a;
    size_t lds;
};

// Layers this kernel runs: fp32, 3x3 or 1x1 filters, an output row of at
// most 192 pixels, and the staged slice within 160 KB of LDS.
bool f32m_plan(const Geom& g, int n_images, F32MPlan& pl) {
    if (!((g.R == 3 && g.S == 3) || (g.R == 1 && g.S == 1))) return false;
    if (g.Q > kMaxPix || g.C < 2) return false;
    F32MArgs& a = pl.a;
    a.C = g.C; a.K = g.K; a.P = g.P; a.Q = g.Q; a.pitch = g.pitchA; a.sw = g.sw; a.dw = g.dw;
    a.HB = std::min(g.P, kMaxPix / g.Q);
    a.pblocks = (g.P + a.HB - 1) / a.HB;
    a.mblocks = (g.K + 63) / 64;
    const int RS = g.R * g.S;
    // slices: about one workgroup per CU in total, each slice an even
    // channel count of at most kTC (a multiple of 4: two halves of pairs)
    const int64_t others = (int64_t)n_images * a.pblocks * a.mblocks;
    int want = (int)std::max<int64_t>(1, (256 + others - 1) / others);
    int tc = (g.C + want - 1) / want;
    tc = (tc + kCh - 1) / kCh * kCh;             // whole chunks
    tc = std::min(tc, kTC);
    a.TC = tc;
    a.splits = (g.C + tc - 1) / tc;
    a.AS = kCh * RS + 1;                         // odd stride: lanes of a fragment in distinct banks
    a.BS = a.HB * g.pitchA + 4;
    // window float4 loads per thread per chunk
    if ((kCh * (a.HB * g.pitchA / 4) + kMThreads - 1) / kMThreads > kMaxB) return false;
    const int64_t ntask = others * a.splits;
    if (ntask >= (1ll << 31)) return false;
    a.ntask = (int)ntask;
    a.nimg = n_images;
    const size_t staged = (size_t)2 * ((size_t)64 * a.AS + (size_t)kCh * a.BS) * 4;
    const size_t red = (size_t)2 * 4 * 3 * 8 * 64 * 4;
    pl.lds = std::max(staged, red);
    return pl.lds <= 160 * 1024;
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
    void (*kfn)(const float*, const float*, const float*, float*, F32MArgs) =
        g.R == 3 ? conv_fp32_mfma_kernel<3, 3> : conv_fp32_mfma_kernel<1, 1>;
    if (pl.lds > 65536 && allow_dynamic_lds(reinterpret_cast<const void*>(kfn), pl.lds) != hipSuccess)
        return hipErrorInvalidValue;
    float* dst = pl.a.splits == 1 ? y : partials;
    hipLaunchKernelGGL(kfn, dim3((uint32_t)pl.a.ntask), dim3(kMThreads), pl.lds, st, xw, w, bias, dst, pl.a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.a.splits == 1) return e;
    const int64_t per_split = (int64_t)n_images * g.K * g.P * g.Q;
    // float4 form: every slice starts 16-byte aligned (per_split % 4 == 0,
    // partials is) and so must y, which is offset by the chunk's first
    // image and need not be
    const bool vec = per_split % 4 == 0 && ((uintptr_t)y & 15u) == 0;
    const int64_t threads = vec ? per_split / 4 : per_split;
    hipLaunchKernelGGL(vec ? split_reduce_nkp_kernel<true> : split_reduce_nkp_kernel<false>,
                       dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0,
                       st, partials, bias, y, (uint32_t)per_split, pl.a.splits, g.P * g.Q, g.K,
                       (int)epi.relu);
    return hipGetLastError();
}

}  // namespace ciw
