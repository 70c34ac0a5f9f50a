// conv_fp32.hip -- fp32 windowed dot product on the vector ALUs (gfx950).
//
// The im2win convolution ("Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support ...", §III-C; fp32 on the non-matrix cores,
// §III-F): every output is the dot product of its window -- for each filter
// column q the R contiguous elements of the CHW window row at column
// w*stride_w + q*dil_w -- with the filter read height before width; the bias
// is added after the sum.  Accumulation is fp32.
//
// Fast kernel (small filters, dil_w = 1).  The 64 lanes of a wave are 64
// output channels; each lane accumulates TN consecutive output columns of
// one output row.  For one input channel the window-row segment those TN
// columns read is the same for every lane, so it is loaded once per wave
// into scalar registers and every multiply-add takes it as its scalar
// operand; the lane's own R*S filter taps sit in vector registers.  Per
// input channel a lane therefore issues TN*R*S multiply-adds against R*S
// vector loads -- the reuse of overlapping windows that the paper credits
// to the cache (§III-C) happens here in registers.
//
// The channel sum is split two ways so that small layers (one 13x13 image)
// still fill 256 compute units: the four waves of a workgroup take
// interleaved channels and add their sums in LDS, and `splits` workgroups
// take disjoint channel slices whose partial sums a second kernel adds in
// slice order.  Both orders are fixed, so results do not depend on
// scheduling.
//
// Generic kernel: any filter size, stride and dilation; one thread computes
// kTK output channels of one pixel.
//
// Fused epilogue (bias, optional ReLU, optional 2x2 max-pool).  The max is
// not linear, so it is taken where the whole channel sum is known: in the
// fast kernel's registers (a row group is the two rows of a pooled row, a
// column tile an even run of columns), in the generic kernel's thread
// (which computes the four outputs of its region), or in the split
// reduction, which reads the four pixels' partial sums.
#include <algorithm>
#include <cmath>

#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

constexpr int kThreads = 256;
constexpr int kTK = 4;          // output channels per thread (generic kernel)
constexpr int kWaves = 4;       // waves per workgroup (fast kernel)

// ------------------------------------------------------------ generic kernel
struct Fp32Args {
    int C, K, R, S, P, Q, sw, dw, pitch;
    int n_images, splits, c_per_split, kgroups;
    int relu, pool, Po, Qo;          // epilogue; output extent
    FastDiv fdPQo, fdKg, fdQo, fdSplit;
    int64_t total;   // threads doing work
};

// Bias, then the optional ReLU (maxNum against 0).
__device__ __forceinline__ float act(float v, float b, int relu) {
    v += b;
    return relu ? fmaxf(v, 0.f) : v;
}

__global__ __launch_bounds__(kThreads) void conv_fp32_generic_kernel(
    const float* __restrict__ xw, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ out, Fp32Args a) {
    int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= a.total) return;
    const int PQ = a.P * a.Q;
    const int PQo = a.Po * a.Qo;
    uint32_t t = (uint32_t)idx;
    uint32_t t1 = fdiv(t, a.fdPQo);
    const int opix = t - t1 * PQo;               // output pixel
    uint32_t t2 = fdiv(t1, a.fdKg);
    int kg = t1 - t2 * a.kgroups;
    uint32_t n = fdiv(t2, a.fdSplit);
    int sidx = t2 - n * a.splits;
    const int h2 = fdiv(opix, a.fdQo);
    const int w2 = opix - h2 * a.Qo;

    const int k0 = kg * kTK;
    const int c_begin = sidx * a.c_per_split;
    const int c_end = min(a.C, c_begin + a.c_per_split);
    const int RS = a.R * a.S;
    // one pixel, or the four of the output's 2x2 region with the pool
    const int side = a.pool ? 2 : 1;
    float m[kTK];
    for (int sub = 0; sub < side * side; ++sub) {
        const int h = h2 * side + (sub >> 1);
        const int wo = w2 * side + (sub & 1);
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
            const int k = min(k0 + i, a.K - 1);
            if (a.splits == 1) {
                const float v = act(acc[i], bias ? bias[k] : 0.f, a.relu);
                m[i] = sub ? fmaxf(m[i], v) : v;
            } else if (k0 + i < a.K) {
                out[((((size_t)sidx * a.n_images + n) * PQ) + h * a.Q + wo) * a.K + k] = acc[i];
            }
        }
    }
    if (a.splits == 1) {
#pragma unroll
        for (int i = 0; i < kTK; ++i)
            if (k0 + i < a.K) out[(((size_t)n * a.K + k0 + i) * PQo) + opix] = m[i];
    }
}

// --------------------------------------------------------------- fast kernel
// Output rows per wave (fast kernel).  Two balance the row groups of
// small images (13 rows split 2,2,...,1 rather than 4,3,3,3) and leave
// registers for more resident waves; measured faster than 3 or 4 on the
// 13x13 and 32x32 layers even though each filter tap then serves 2 rows.
constexpr int kRW = 2;
static_assert(kRW >= 2, "a pooled row group holds the two rows of its region");

struct KlArgs {
    int C, K, P, Q, pitch;
    int Qc;                        // columns computed: Q, or 2 (Q / 2) with the pool
    int Po, Qo;                    // output extent
    int col_tiles, kblocks, splits, c_per_split, row_groups;
    FastDiv fdN, fdKb, fdTiles, fdRg;
    int n_images;
    uint32_t xcd_per, xcd_rem;   // blocks / 8 and blocks % 8
};

// Window-row elements the TN output columns of one tile read: columns
// w0*SW .. (w0+TN-1)*SW + S-1 of the padded input, R values each.
template <int R, int S, int SW, int TN>
struct KlShape {
    static constexpr int kLen = ((TN - 1) * SW + S) * R;
    static constexpr int kTaps = R * S;
};

// One workgroup: 64 output channels (one per lane) x up to kRW output rows
// x TN output columns, over one slice of input channels that its four
// waves share out (wave w takes every fourth channel).  A lane loads its
// R*S filter taps of a channel once and applies them to all its rows, so
// the filter stream is read once per row group rather than once per row.
template <int R, int S, int SW, int TN, bool RELU, bool POOL>
__global__ __launch_bounds__(kThreads) void conv_fp32_klanes_kernel(
    const float* __restrict__ xw, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ out, KlArgs a) {
    using Sh = KlShape<R, S, SW, TN>;
    constexpr int L = Sh::kLen;
    constexpr int T = Sh::kTaps;
    __shared__ float red[(kWaves - 1) * TN * 64];

    // Workgroups are dispatched round-robin over the 8 XCDs (bid % 8), each
    // with its own L2.  Renumber so that each XCD gets a contiguous range
    // of logical indices, and order the logical index (row group fastest,
    // then column tile, image, k block, channel slice) so the workgroups
    // that read one filter slice sit on one XCD and share its L2.
    const uint32_t bid = blockIdx.x;
    const uint32_t xcd = bid & 7u, slot = bid >> 3;
    const uint32_t lid = xcd < a.xcd_rem ? xcd * (a.xcd_per + 1) + slot
                                         : a.xcd_rem * (a.xcd_per + 1) + (xcd - a.xcd_rem) * a.xcd_per + slot;
    uint32_t t1 = fdiv(lid, a.fdRg);
    const int rg = lid - t1 * a.row_groups;
    uint32_t t2 = fdiv(t1, a.fdTiles);
    const int tile = t1 - t2 * a.col_tiles;
    uint32_t t3 = fdiv(t2, a.fdN);
    const uint32_t n = t2 - t3 * a.n_images;
    uint32_t sidx = fdiv(t3, a.fdKb);
    const int kb = t3 - sidx * a.kblocks;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int k = kb * 64 + lane;
    const int kk = min(k, a.K - 1);

    // rows [h0, h0 + nrows): the P rows split evenly over the row groups;
    // with the pool, row group j is rows 2j and 2j + 1
    const int h0 = POOL ? 2 * rg : rg * a.P / a.row_groups;
    const int nrows = POOL ? 2 : (rg + 1) * a.P / a.row_groups - h0;   // 1 .. kRW

    // the last tile is shifted left so it ends at column Qc (its leading
    // columns repeat the previous tile's and are not stored); with the pool
    // TN and Qc are even, so tiles start on even columns
    const int w_store = tile * TN;
    const int w0 = min(w_store, a.Qc - TN);

    const int c_begin = sidx * a.c_per_split;
    const int c_end = min(a.C, c_begin + a.c_per_split);

    float acc[kRW][TN];
#pragma unroll
    for (int rr = 0; rr < kRW; ++rr)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[rr][t] = 0.f;

    // window row (n, c, h) starts at this element offset; uniform per wave
    const int row_step = a.P * a.pitch;
    int xoff = ((n * a.C + c_begin + wave) * a.P + h0) * a.pitch + w0 * SW * R;
    xoff = __builtin_amdgcn_readfirstlane(xoff);
    const float* wk = w + (size_t)kk * a.C * T;

    for (int c = c_begin + wave; c < c_end; c += kWaves) {
        float f[T];
#pragma unroll
        for (int j = 0; j < T; ++j) f[j] = wk[c * T + j];
#pragma unroll
        for (int rr = 0; rr < kRW; ++rr) {
            if (rr < nrows) {
                float xv[L];
#pragma unroll
                for (int e = 0; e < L; ++e) xv[e] = xw[xoff + rr * a.pitch + e];
#pragma unroll
                for (int q = 0; q < S; ++q)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float fv = f[r * S + q];
#pragma unroll
                        for (int t = 0; t < TN; ++t)
                            acc[rr][t] = fmaf(xv[(t * SW + q) * R + r], fv, acc[rr][t]);
                    }
            }
        }
        xoff += kWaves * row_step;
    }

    // add the four waves' sums in wave order, one output row at a time
    const int PQ = a.P * a.Q;
#pragma unroll
    for (int rr = 0; rr < kRW; ++rr) {
        if (rr >= nrows) break;
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < TN; ++t) red[((wave - 1) * TN + t) * 64 + lane] = acc[rr][t];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < kWaves - 1; ++i)
#pragma unroll
                for (int t = 0; t < TN; ++t) acc[rr][t] += red[(i * TN + t) * 64 + lane];
            const int h = h0 + rr;
            if (k < a.K) {
                if (a.splits == 1) {
                    if (!POOL) {
                        const float b = bias ? bias[k] : 0.f;
                        float* yp = out + ((size_t)n * a.K + k) * PQ + h * a.Q + w0;
#pragma unroll
                        for (int t = 0; t < TN; ++t)
                            if (w0 + t >= w_store) yp[t] = act(acc[rr][t], b, RELU);
                    }
                } else {
                    // partial sums [slice][n][h][w][k]: output channels
                    // innermost, so the 64 lanes store one contiguous run
                    float* pp = out + ((((size_t)sidx * a.n_images + n) * a.P + h) * a.Q + w0) * a.K + k;
#pragma unroll
                    for (int t = 0; t < TN; ++t)
                        if (w0 + t >= w_store) pp[(size_t)t * a.K] = acc[rr][t];
                }
            }
        }
        __syncthreads();
    }
    // pooled row rg: wave 0 holds both rows' full sums; columns 2t, 2t + 1
    // of the tile form output column (w0 / 2) + t
    if (POOL && a.splits == 1 && wave == 0 && k < a.K) {
        const float b = bias ? bias[k] : 0.f;
        float* yp = out + ((size_t)n * a.K + k) * a.Po * a.Qo + rg * a.Qo + w0 / 2;
#pragma unroll
        for (int t = 0; t < TN / 2; ++t)
            if (w0 + 2 * t >= w_store)
                yp[t] = fmaxf(fmaxf(act(acc[0][2 * t], b, RELU), act(acc[0][2 * t + 1], b, RELU)),
                              fmaxf(act(acc[1][2 * t], b, RELU), act(acc[1][2 * t + 1], b, RELU)));
    }
}

// y[n][k][pix] = bias[k] + sum over slices s (in order) of part[s][n][pix][k].
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, float* __restrict__ y,
    uint32_t per_split, int splits, int PQ, int K, int relu, FastDiv fdK, FastDiv fdPQ) {
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= per_split) return;
    float v = 0.f;
    int s = 0;
    for (; s + 4 <= splits; s += 4) {
        float p0 = part[(size_t)s * per_split + i];
        float p1 = part[(size_t)(s + 1) * per_split + i];
        float p2 = part[(size_t)(s + 2) * per_split + i];
        float p3 = part[(size_t)(s + 3) * per_split + i];
        v += p0;
        v += p1;
        v += p2;
        v += p3;
    }
    for (; s < splits; ++s) v += part[(size_t)s * per_split + i];
    const uint32_t t = fdiv(i, fdK);
    const int k = i - t * K;
    const uint32_t n = fdiv(t, fdPQ);
    const int pix = t - n * PQ;
    y[((size_t)n * K + k) * PQ + pix] = act(v, bias ? bias[k] : 0.f, relu);
}

// Pooled form.  One workgroup per (image n, region (j, i), 64 channels): wave
// d adds, in slice order, the partial sums of pixel (2j + d / 2, 2i + d % 2)
// for its 64 channels (64 consecutive floats per slice: coalesced), then
// bias and ReLU; the region's max goes through LDS.
__global__ __launch_bounds__(kThreads) void split_reduce_pool_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, float* __restrict__ y,
    uint32_t per_split, int splits, int P, int Q, int Po, int Qo, int K, int kblocks, int relu,
    FastDiv fdKb, FastDiv fdQo, FastDiv fdPo) {
    __shared__ float red[3][64];
    const uint32_t bid = blockIdx.x;
    const uint32_t t1 = fdiv(bid, fdKb);
    const int kb = bid - t1 * kblocks;
    const uint32_t t2 = fdiv(t1, fdQo);
    const int i2 = t1 - t2 * Qo;
    const uint32_t n = fdiv(t2, fdPo);
    const int j = t2 - n * Po;
    const int lane = threadIdx.x & 63;
    const int d = threadIdx.x >> 6;
    const int k = kb * 64 + lane;
    const int kk = min(k, K - 1);
    const int pix = (2 * j + (d >> 1)) * Q + 2 * i2 + (d & 1);
    const float* pp = part + ((size_t)n * P * Q + pix) * K + kk;
    float v = 0.f;
    int s = 0;
    for (; s + 4 <= splits; s += 4) {
        const float p0 = pp[(size_t)s * per_split];
        const float p1 = pp[(size_t)(s + 1) * per_split];
        const float p2 = pp[(size_t)(s + 2) * per_split];
        const float p3 = pp[(size_t)(s + 3) * per_split];
        v += p0;
        v += p1;
        v += p2;
        v += p3;
    }
    for (; s < splits; ++s) v += pp[(size_t)s * per_split];
    v = act(v, bias ? bias[kk] : 0.f, relu);
    if (d > 0) red[d - 1][lane] = v;
    __syncthreads();
    if (d == 0 && k < K) {
        v = fmaxf(fmaxf(v, red[0][lane]), fmaxf(red[1][lane], red[2][lane]));
        y[((size_t)n * K + k) * Po * Qo + j * Qo + i2] = v;
    }
}

// ------------------------------------------------------------------ planning
typedef void (*KlKernel)(const float*, const float*, const float*, float*, KlArgs);

// One variant per shape, compiled for each epilogue (index relu + 2 pool).
struct KlVariant {
    int R, S, SW, TN;
    KlKernel fn[4];
};

#define CIW_KL(R, S, SW, TN)                                                                   \
    {R, S, SW, TN, {conv_fp32_klanes_kernel<R, S, SW, TN, false, false>,                     \
                    conv_fp32_klanes_kernel<R, S, SW, TN, true, false>,                      \
                    conv_fp32_klanes_kernel<R, S, SW, TN, false, true>,                      \
                    conv_fp32_klanes_kernel<R, S, SW, TN, true, true>}}
// Column-tile widths per filter shape: the scalar window segment
// ((TN-1)*SW + S)*R stays at or below 60 registers.
// The even widths 12 and 6 serve pooled layers, whose computed width 2 (Q / 2)
// is even (12 for the 13-wide layers).
const KlVariant kKlVariants[] = {
    CIW_KL(1, 1, 1, 16), CIW_KL(1, 1, 1, 14), CIW_KL(1, 1, 1, 13), CIW_KL(1, 1, 1, 12),
    CIW_KL(1, 1, 1, 8), CIW_KL(1, 1, 1, 7), CIW_KL(1, 1, 1, 6),
    CIW_KL(1, 1, 2, 16), CIW_KL(1, 1, 2, 14), CIW_KL(1, 1, 2, 13), CIW_KL(1, 1, 2, 12),
    CIW_KL(1, 1, 2, 8), CIW_KL(1, 1, 2, 7), CIW_KL(1, 1, 2, 6),
    CIW_KL(3, 3, 1, 16), CIW_KL(3, 3, 1, 14), CIW_KL(3, 3, 1, 13), CIW_KL(3, 3, 1, 12),
    CIW_KL(3, 3, 1, 8), CIW_KL(3, 3, 1, 7), CIW_KL(3, 3, 1, 6),
    CIW_KL(3, 3, 2, 8), CIW_KL(3, 3, 2, 7), CIW_KL(3, 3, 2, 6), CIW_KL(3, 3, 2, 4),
    CIW_KL(5, 5, 1, 8), CIW_KL(5, 5, 1, 7), CIW_KL(5, 5, 1, 6), CIW_KL(5, 5, 1, 4),
};
#undef CIW_KL

struct Fp32Plan {
    const KlVariant* kl;   // null: generic kernel
    int col_tiles, kblocks, row_groups;
    int splits;            // channel slices across workgroups (partial-sum passes)
    int c_per_split;
};

// The fast kernel's variant for this shape: the tile width that wastes the
// fewest recomputed columns (ties: the widest).  Pooled layers need an even
// width, so that tiles cover whole 2x2 regions.
const KlVariant* pick_variant(const Geom& g, bool even) {
    if (g.dw != 1) return nullptr;
    const KlVariant* best = nullptr;
    int64_t best_cols = 0;
    for (const KlVariant& v : kKlVariants) {
        if (v.R != g.R || v.S != g.S || v.SW != g.sw || v.TN > g.Q) continue;
        if (even && (v.TN & 1)) continue;
        int64_t cols = (int64_t)((g.Q + v.TN - 1) / v.TN) * v.TN;
        if (!best || cols < best_cols || (cols == best_cols && v.TN > best->TN)) {
            best = &v;
            best_cols = cols;
        }
    }
    return best;
}

int generic_splits(const Geom& g, int n_images) {
    // aim for >= 128K threads of work; keep >= 16 channels per slice
    int64_t base = (int64_t)n_images * ((g.K + kTK - 1) / kTK) * g.P * g.Q;
    int64_t want = (131072 + base - 1) / base;
    int64_t maxs = g.C / 16;
    int64_t s = want < maxs ? want : maxs;
    return s < 1 ? 1 : (int)s;
}

// Channel-slice count for the fast kernel from a small cost model, in
// cycles of one SIMD: each workgroup puts one wave on each SIMD of its CU,
// at most 8 waves are resident per SIMD, and a wave spends about 4*TN*R*S
// cycles of multiply-adds per stage plus a fixed latency that other
// resident waves hide; every extra slice adds one pass over the partial
// sums.  Smallest cost wins (ties: fewer slices).
int fast_splits(const Geom& g, const KlVariant& v, int n_images, int col_tiles, int kblocks,
                int row_groups) {
    const double units = (double)n_images * row_groups * col_tiles * kblocks;
    const double stage_cycles = 4.0 * v.TN * v.R * v.S * ((double)g.P / row_groups);
    const double latency = 2500.0;
    const double outputs = (double)n_images * g.K * g.P * g.Q;
    const int smax = g.C / kWaves > 1 ? g.C / kWaves : 1;
    int best = 1;
    double best_cost = 0.0;
    for (int s = 1; s <= smax; ++s) {
        const int cps = (g.C + s - 1) / s;
        if (s > 1 && (g.C + cps - 1) / cps != s) continue;   // not a distinct slicing
        const double wgs_per_cu = std::ceil(units * s / 256.0);
        const double stages = std::ceil(cps / (double)kWaves);
        double cost = 0.0;
        for (double left = wgs_per_cu; left > 0; left -= 8) {
            const double w = left < 8 ? left : 8;
            cost += stages * std::max(w * stage_cycles, stage_cycles + latency);
        }
        if (s > 1) cost += 2000.0 + s * outputs * 4.0 / 2000.0;   // second pass
        if (s == 1 || cost < best_cost) {
            best = s;
            best_cost = cost;
        }
    }
    return best;
}

// The fast kernel works on the pixels that reach an output: all of them, or
// with the pool the 2 (P / 2) x 2 (Q / 2) that the regions cover.
Geom computed_region(const Geom& g, const Epi& epi) {
    Geom c = g;
    if (epi.pool) {
        c.P = 2 * (g.P / 2);
        c.Q = 2 * (g.Q / 2);
    }
    return c;
}

Fp32Plan plan(const Geom& g, int n_images, bool generic, const Epi& epi) {
    Fp32Plan p{};
    const Geom gc = computed_region(g, epi);
    p.kl = generic ? nullptr : pick_variant(gc, epi.pool);
    if (!p.kl) {
        p.splits = generic_splits(g, n_images);
        p.c_per_split = (g.C + p.splits - 1) / p.splits;
        return p;
    }
    p.col_tiles = (gc.Q + p.kl->TN - 1) / p.kl->TN;
    p.kblocks = (g.K + 63) / 64;
    p.row_groups = epi.pool ? gc.P / 2 : (g.P + kRW - 1) / kRW;
    const int s = fast_splits(gc, *p.kl, n_images, p.col_tiles, p.kblocks, p.row_groups);
    p.c_per_split = (g.C + s - 1) / s;
    p.splits = (g.C + p.c_per_split - 1) / p.c_per_split;
    return p;
}

}  // namespace

int fp32_splits(const Geom& g, int n_images) {
    // partial-sum slices the workspace must hold: the larger of the two
    // kernels' plans, so either may run in a workspace sized by this
    // (without the epilogue: a pooled plan that wants more slices than fit
    // is cut down to this count at launch)
    int a = plan(g, n_images, false, Epi{}).splits;
    int b = plan(g, n_images, true, Epi{}).splits;
    int m = fp32_mfma_splits(g, n_images);
    return std::max(std::max(a, b), m);
}

hipError_t launch_conv_fp32(const Geom& g, const float* xw, const float* w, const float* bias,
                            float* y, int n_images, float* partials, int max_splits,
                            bool generic, Fp32Kernel kernel, const Epi& epi, hipStream_t st) {
    if (n_images == 0) return hipSuccess;
    // the matrix-core kernel when it runs the layer (not with the pool, the
    // single-pass request or the generic-kernel request): forced, or by
    // default when its channel sum splits into at least 4 slices (below
    // that the layer is too small to fill the GPU through it, and the
    // vector kernel was measured faster)
    if (kernel != FP32_VECTOR && !generic && !epi.pool && fp32_m16_tasks(g, n_images, false) > 0)
        return launch_conv_fp32_m16(g, xw, w, bias, y, n_images, epi, false, st);
    if (kernel != FP32_VECTOR && !generic && !epi.pool && max_splits > 1) {
        const int ms = fp32_mfma_splits(g, n_images);
        if (ms > 0 && ms <= max_splits && (kernel == FP32_MATRIX || ms >= 4))
            return launch_conv_fp32_mfma(g, xw, w, bias, y, n_images, partials, max_splits, epi, st);
    }
    Fp32Plan p = plan(g, n_images, generic, epi);
    const int Po = out_rows(g, epi), Qo = out_cols(g, epi);
    if (max_splits <= 1) {   // single pass requested
        p.splits = 1;
        p.c_per_split = g.C;
    }
    if (p.splits > max_splits) {   // a smaller last chunk wants more slices than fit
        p.c_per_split = (g.C + max_splits - 1) / max_splits;
        p.splits = (g.C + p.c_per_split - 1) / p.c_per_split;
    }
    float* dst = p.splits == 1 ? y : partials;
    if (p.kl) {
        KlArgs a;
        a.C = g.C; a.K = g.K; a.P = g.P; a.Q = g.Q; a.pitch = g.pitchA;
        a.Qc = epi.pool ? 2 * Qo : g.Q;
        a.Po = Po;
        a.Qo = Qo;
        a.col_tiles = p.col_tiles;
        a.kblocks = p.kblocks;
        a.splits = p.splits;
        a.c_per_split = p.c_per_split;
        a.row_groups = p.row_groups;
        a.fdN = make_fastdiv(n_images);
        a.fdKb = make_fastdiv(p.kblocks);
        a.fdTiles = make_fastdiv(p.col_tiles);
        a.fdRg = make_fastdiv(p.row_groups);
        a.n_images = n_images;
        int64_t blocks = (int64_t)n_images * p.row_groups * p.col_tiles * p.kblocks * p.splits;
        if (blocks >= (1ll << 31)) return hipErrorInvalidValue;
        a.xcd_per = (uint32_t)(blocks / 8);
        a.xcd_rem = (uint32_t)(blocks % 8);
        hipLaunchKernelGGL(p.kl->fn[(epi.relu ? 1 : 0) + (epi.pool ? 2 : 0)], dim3((uint32_t)blocks), dim3(kThreads), 0, st, xw, w, bias,
                           dst, a);
    } else {
        Fp32Args a;
        a.C = g.C; a.K = g.K; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
        a.sw = g.sw; a.dw = g.dw; a.pitch = g.pitchA;
        a.n_images = n_images;
        a.splits = p.splits;
        a.c_per_split = p.c_per_split;
        a.kgroups = (g.K + kTK - 1) / kTK;
        a.relu = epi.relu;
        a.pool = epi.pool;
        a.Po = Po;
        a.Qo = Qo;
        a.fdPQo = make_fastdiv(Po * Qo);
        a.fdKg = make_fastdiv(a.kgroups);
        a.fdQo = make_fastdiv(Qo);
        a.fdSplit = make_fastdiv(p.splits);
        a.total = (int64_t)n_images * p.splits * a.kgroups * Po * Qo;
        if (a.total >= (1ll << 31)) return hipErrorInvalidValue;
        uint32_t blocks = (uint32_t)((a.total + kThreads - 1) / kThreads);
        hipLaunchKernelGGL(conv_fp32_generic_kernel, dim3(blocks), dim3(kThreads), 0, st, xw, w,
                           bias, dst, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t per_split = (int64_t)n_images * g.K * g.P * g.Q;
    if (epi.pool) {
        const int kblocks = (g.K + 63) / 64;
        const int64_t blocks = (int64_t)n_images * Po * Qo * kblocks;
        if (blocks >= (1ll << 31)) return hipErrorInvalidValue;
        hipLaunchKernelGGL(split_reduce_pool_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, st,
                           partials, bias, y, (uint32_t)per_split, p.splits, g.P, g.Q, Po, Qo,
                           g.K, kblocks, (int)epi.relu, make_fastdiv(kblocks), make_fastdiv(Qo),
                           make_fastdiv(Po));
    } else {
        hipLaunchKernelGGL(split_reduce_kernel, dim3((uint32_t)((per_split + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, st, partials, bias, y, (uint32_t)per_split, p.splits,
                           g.P * g.Q, g.K, (int)epi.relu, make_fastdiv(g.K), make_fastdiv(g.P * g.Q));
    }
    return hipGetLastError();
}

}  // namespace ciw
