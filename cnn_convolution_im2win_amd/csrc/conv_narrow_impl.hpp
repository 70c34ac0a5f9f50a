// conv_narrow_impl.hpp -- fp16/bf16 dense contraction for layers with few
// input channels and an even horizontal stride (the 3-channel 7x7 stride-2
// stem), with the windows built in LDS from x: kernel, plan and launcher.
//
// The im2win paper ("Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support on GPU CUDA and Tensor Cores") lays its window
// tensor out channel innermost for the tensor cores (§III-D), so that one
// matrix step covers many channels of one tap.  With three channels that
// order leaves most of a 16-entry step empty.  Here the reduction is ordered
// (channel c, filter row r, filter column s), the order of the NCHW input
// itself:
//   - for one (c, r) pair, output column w reads the S consecutive input
//     columns w*stride_w - pad_w .. + S - 1 of input row h*stride_h - pad_h +
//     r*dil_h: one strip of a row of x.  A lane's 8 entries of a
//     v_mfma_f32_32x32x16 step are one such strip, plus d leading and
//     8 - d - S trailing columns that belong to other windows.  A mask
//     clears those, so they count as zeros whatever they hold; the filter's
//     entries there are zero as well.  A step covers two (c, r) pairs (the
//     lane halves), so the stem's 147 taps take 11 steps;
//   - the workgroup keeps a ring of NR zero-padded input rows in LDS.  Each
//     slot holds the C channel rows, [channel][column], and a row of zeros
//     that the unused pairs of the last step read.  With an even stride the
//     strip of every output column starts on a 4-byte boundary, so a
//     fragment is two 8-byte LDS reads (ds_read2_b32);
//   - a band of output rows of one image is computed SR rows per step.  A
//     step's pixels are cut into blocks of 32 consecutive outputs (a block
//     may span two output rows), and each block is one wave's task: KS steps
//     of window fragment (first operand) x filter fragment of 32 output
//     channels (second operand), both 32-channel halves, with fp32
//     accumulators seeded with the bias;
//   - a step's new input rows are loaded into registers one step ahead.
//     Each wave writes its share into the ring between its last task's
//     multiplies and its stores, so the loads have a whole step to arrive.
//     Every input element crosses HBM once per band, and no window tensor
//     is written;
//   - the filter (K x C x R x S, at most 22.5 KB) is copied into LDS once
//     per workgroup, and every lane builds its fragments from there.  No
//     workspace, no separate kernel;
//   - stores go through a per-wave LDS tile, so one store instruction
//     writes whole 64-byte runs of output rows.
// The sum is the convolution's sum in another order, accumulated in fp32
// with the bias first, rounded once at the store.
#pragma once

#include "conv_mfma_impl.hpp"

namespace ciw {
namespace {

constexpr int kNarrowThreads = 256;   // four waves; two workgroups per CU
constexpr int kNarrowMaxIt = 3;       // row-copy items per thread per step
constexpr int kNarrowMaxIt0 = 8;      // ... for the first step's rows
constexpr int kNarrowMaxFilt = 8;     // 16-byte filter chunks per thread
constexpr int kNarrowLds = 80 * 1024; // LDS per workgroup (two per CU)

struct NarrowArgs {
    int C, K, H, W, P, Q;
    int R, S, sh, sw, ph, pw, dh;
    int CR;                  // (channel, filter row) pairs: C * R
    int span;                // input rows one output row reads: (R - 1) dil_h + 1
    int L;                   // LDS column of input column 0 (a multiple of 4)
    int col0;                // LDS column of output column 0's first fragment entry: L - pad_w - d
    uint32_t m[4];           // fragment word masks: entry e kept iff d <= e < d + S
    int RB;                  // bytes of one channel row of a slot (a multiple of 16)
    int slot_bytes;          // (C + 1) RB: the channel rows and a zero row
    int NR;                  // ring slots (at most 255)
    int SR;                  // output rows per step
    int wv;                  // 16-byte vectors of an input row: W / 8
    int nl, nr;              // 8-byte zero stores of a channel row's left / right padding
    int band, nbands, ntask;
    int relu, staged, vec;
    int filt_off, tile_off;  // LDS byte offsets of the staged filter and the per-wave output tiles
    int filt_elems;          // K C R S
    uint32_t plane_x, plane_y;
    FastDiv fdQ, fdNR, fdRow, fdWv;   // divisors Q, NR, C * W / 8, W / 8
};

// fp32 outputs: four adjacent values as one 16-byte store.
template <typename TOut>
__device__ __forceinline__ void narrow_store4(char* p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2<TOut>(a0, a1), pack2<TOut>(a2, a3));
}

template <>
__device__ __forceinline__ void narrow_store4<float>(char* p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<float4*>(p) = make_float4(a0, a1, a2, a3);
}

template <typename TIn, typename TOut, int KS>
__global__ __launch_bounds__(kNarrowThreads, 2) void conv_mfma_narrow_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const TIn* __restrict__ bias, TOut* __restrict__ y, NarrowArgs a) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;         // which (c, r) pair of a step
    const int ml = lane & 31;        // fragment pixel (window) / output channel (filter)

    // band = (image, first output row); with the grid a multiple of 8 the
    // bands of one image land on one XCD (workgroups are dispatched
    // round-robin over the 8 XCDs), so the halo rows of two bands meet in
    // its L2
    int task = blockIdx.x;
    if ((a.ntask & 7) == 0) task = (int)(blockIdx.x & 7) * (a.ntask >> 3) + (int)(blockIdx.x >> 3);
    const int n = task / a.nbands;
    const int h0 = (task - n * a.nbands) * a.band;
    const int rows = min(a.band, a.P - h0);
    // step t covers band output rows [orow(t), orow(t + 1)) and needs band
    // input rows below rb(t); band input row j is x row h0 stride_h - pad_h + j
    const int nsteps = (rows + a.SR - 1) / a.SR;
    auto orow = [&](int t) { return min(t * a.SR, rows); };
    auto rb = [&](int t) { return (orow(t + 1) - 1) * a.sh + a.span; };
    const int xr0 = h0 * a.sh - a.ph;
    const char* ximg = reinterpret_cast<const char*>(x + (size_t)n * a.C * a.plane_x);
    char* yband = reinterpret_cast<char*>(y + (size_t)n * a.K * a.plane_y + (size_t)h0 * a.Q);

    // ---- row copies.  Item it of band input rows [j0, j1): columns
    // 8 v .. 8 v + 7 of channel c of row j, one 16-byte load, written at ring
    // slot j % NR, channel row c, columns L + 8 v ..; rows outside the input
    // are written as zeros (no load).
    auto load_item = [&](int j0, int j1, int it, int& dst) -> uint4 {
        dst = -1;
        if (it >= (j1 - j0) * a.C * a.wv) return make_uint4(0u, 0u, 0u, 0u);
        const int jr = (int)fdiv((uint32_t)it, a.fdRow);
        const int rem = it - jr * a.C * a.wv;
        const int c = (int)fdiv((uint32_t)rem, a.fdWv);
        const int vv = rem - c * a.wv;
        const uint32_t j = (uint32_t)(j0 + jr);
        const int slot = (int)(j - fdiv(j, a.fdNR) * a.NR);
        dst = slot * a.slot_bytes + c * a.RB + (a.L + 8 * vv) * 2;
        const int xrow = xr0 + (int)j;
        if (xrow < 0 || xrow >= a.H) return make_uint4(0u, 0u, 0u, 0u);
        return *reinterpret_cast<const uint4*>(
            ximg + 2u * ((uint32_t)c * a.plane_x + (uint32_t)(xrow * a.W + 8 * vv)));
    };
    auto store_item = [&](const uint4& v, int dst) {
        if (dst < 0) return;
        // 8-byte aligned (L is a multiple of 4 columns)
        *reinterpret_cast<uint2*>(lds + dst) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(lds + dst + 8) = make_uint2(v.z, v.w);
    };

    // ---- prologue: filter and first step's rows requested together; the
    // padding columns and zero rows (which no copy writes) zeroed meanwhile
    {
        const int nfc = (a.filt_elems * 2) >> 4;   // whole 16-byte filter chunks
        uint4 fv[kNarrowMaxFilt];
#pragma unroll
        for (int k = 0; k < kNarrowMaxFilt; ++k) {
            const int it = tid + k * kNarrowThreads;
            fv[k] = it < nfc ? reinterpret_cast<const uint4*>(w)[it] : make_uint4(0u, 0u, 0u, 0u);
        }
        uint4 pv[kNarrowMaxIt0];
        int pd[kNarrowMaxIt0];
        const int r0 = rb(0);
#pragma unroll
        for (int k = 0; k < kNarrowMaxIt0; ++k) pv[k] = load_item(0, r0, tid + k * kNarrowThreads, pd[k]);
        // zeros: per slot, each channel row's nl + nr padding words, then the zero row
        const int per_c = a.nl + a.nr;
        const int units = a.C * per_c + a.RB / 8;
        for (int it = tid; it < a.NR * units; it += kNarrowThreads) {
            const int slot = it / units;
            const int u = it - slot * units;
            int off = slot * a.slot_bytes;
            if (u < a.C * per_c) {
                const int c = u / per_c, k = u - c * per_c;
                off += c * a.RB + (k < a.nl ? 8 * k : 2 * (a.L + a.W) + 8 * (k - a.nl));
            } else {
                off += a.C * a.RB + 8 * (u - a.C * per_c);
            }
            *reinterpret_cast<uint2*>(lds + off) = make_uint2(0u, 0u);
        }
        for (int e = nfc * 8 + tid; e < a.filt_elems; e += kNarrowThreads)
            *reinterpret_cast<uint16_t*>(lds + a.filt_off + 2 * e) = w[e];
#pragma unroll
        for (int k = 0; k < kNarrowMaxFilt; ++k) {
            const int it = tid + k * kNarrowThreads;
            if (it < nfc) *reinterpret_cast<uint4*>(lds + a.filt_off + 16 * it) = fv[k];
        }
#pragma unroll
        for (int k = 0; k < kNarrowMaxIt0; ++k) store_item(pv[k], pd[k]);
    }
    __syncthreads();   // filter, first rows and zeros are in LDS

    // filter fragments: lane holds F[k][c][r][e - d] for e = 0..7, k = 32 ct + ml,
    // (c, r) pair u = 2 ks + g; zero outside the filter
    const int d = a.L - a.pw - a.col0;
    uint4 F[2][KS];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int k = 32 * ct + ml;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int u = 2 * ks + g;
            const bool ok = k < a.K && u < a.CR;
            const uint16_t* fr = reinterpret_cast<const uint16_t*>(lds + a.filt_off) + (ok ? (k * a.CR + u) * a.S : 0);
            auto el = [&](int e) -> uint32_t {
                const int s = e - d;
                return (ok && s >= 0 && s < a.S) ? (uint32_t)fr[s] : 0u;
            };
            F[ct][ks] = make_uint4(el(0) | (el(1) << 16), el(2) | (el(3) << 16), el(4) | (el(5) << 16),
                                   el(6) | (el(7) << 16));
        }
    }
    // pair offsets: (byte offset of channel row c in a slot) << 8 | r dil_h;
    // pairs past C R read the slot's zero row
    uint32_t pu[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int u = 2 * ks + g;
        const int c = u < a.CR ? u / a.R : a.C;
        const int r = u < a.CR ? u - c * a.R : 0;
        pu[ks] = ((uint32_t)(c * a.RB) << 8) | (uint32_t)(r * a.dh);
    }
    float bk[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
        bk[ct] = (bias != nullptr && 32 * ct + ml < a.K) ? to_f32(bias[32 * ct + ml]) : 0.f;

    // the second step's rows
    uint4 lv[kNarrowMaxIt];
    int ldst[kNarrowMaxIt];
#pragma unroll
    for (int k = 0; k < kNarrowMaxIt; ++k) {
        ldst[k] = -1;
        if (nsteps > 1) lv[k] = load_item(rb(0), rb(1), tid + k * kNarrowThreads, ldst[k]);
    }

    const uint32_t NRu = (uint32_t)a.NR;
    // ---- steps
    for (int t = 0; t < nsteps; ++t) {
        if (t > 0) __syncthreads();   // rows of step t are in the ring
        const int o0 = orow(t);
        const int npx = (orow(t + 1) - o0) * a.Q;   // pixels of the step
        const int nblk = (npx + 31) >> 5;
        const int pix0 = o0 * a.Q;                  // band pixel of the first
        // the next step's rows (loaded one step ago) into slots no wave reads
        // in this step, then the loads for the step after
        auto move_rows = [&]() {
            if (t + 1 < nsteps) {
#pragma unroll
                for (int k = 0; k < kNarrowMaxIt; ++k) store_item(lv[k], ldst[k]);
            }
            if (t + 2 < nsteps) {
#pragma unroll
                for (int k = 0; k < kNarrowMaxIt; ++k) lv[k] = load_item(rb(t + 1), rb(t + 2), tid + k * kNarrowThreads, ldst[k]);
            }
        };
        for (int b = wave; b < nblk; b += 4) {
            // the lane's window pixel (past the step's end: its last pixel,
            // read but never stored)
            const uint32_t pb = (uint32_t)(pix0 + min(32 * b + ml, npx - 1));
            const int i = (int)fdiv(pb, a.fdQ);              // band output row
            const int q = (int)pb - i * a.Q;                 // output column
            const uint32_t jb = (uint32_t)(i * a.sh);        // band input row of filter row 0
            const uint32_t s0 = jb - fdiv(jb, a.fdNR) * NRu; // its slot
            const uint32_t colb = (uint32_t)(q * a.sw + a.col0) * 2u;
            auto frag = [&](int ks) -> uint4 {
                uint32_t s = s0 + (pu[ks] & 255u);
                s = min(s, s - NRu);                          // s mod NR (both terms below NR)
                const uint32_t* p = reinterpret_cast<const uint32_t*>(lds + (s * (uint32_t)a.slot_bytes + (pu[ks] >> 8) + colb));
                return make_uint4(p[0] & a.m[0], p[1] & a.m[1], p[2] & a.m[2], p[3] & a.m[3]);
            };
            f32x16 acc0, acc1;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                acc0[e] = bk[0];
                acc1[e] = bk[1];
            }
            constexpr int PF = 3;   // window fragments read ahead
            uint4 bq[PF];
#pragma unroll
            for (int s = 0; s < PF && s < KS; ++s) bq[s] = frag(s);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint4 bv = bq[s % PF];
                if (s + PF < KS) bq[s % PF] = frag(s + PF);
                acc0 = mfma32<TIn>(bv, F[0][s], acc0);
                acc1 = mfma32<TIn>(bv, F[1][s], acc1);
            }
            if (a.relu) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    acc0[e] = fmaxf(acc0[e], 0.f);
                    acc1[e] = fmaxf(acc1[e], 0.f);
                }
            }
            if (b + 4 >= nblk) move_rows();
            // lane holds channel 32 ct + ml at block pixels 8 jq + 4 g + 0..3
            constexpr int EB = (int)sizeof(TOut);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const f32x16& acc = ct == 0 ? acc0 : acc1;
                if (32 * ct >= a.K) break;
                if (a.staged) {
                    // Through the wave's LDS tile, RPR channels at a time: the
                    // lanes of those channels write their 16 pixels, then
                    // every lane reads 16 bytes of one channel's 32-pixel run
                    // and stores them, so one store instruction writes whole
                    // 64-byte runs of RPR channels.  (LDS operations of one
                    // wave complete in order: no barrier.)
                    constexpr int RPR = 1024 / (32 * EB);      // channels per round
                    constexpr int OSTR = 32 * EB + 16;         // tile row stride (bytes)
                    constexpr int LPR = 64 / RPR;              // lanes per channel run
                    unsigned char* tile = lds + a.tile_off + wave * RPR * OSTR;
#pragma unroll
                    for (int rd = 0; rd < 32 / RPR; ++rd) {
                        if (ml / RPR == rd) {
                            unsigned char* row = tile + (ml % RPR) * OSTR + 4 * g * EB;
#pragma unroll
                            for (int jq = 0; jq < 4; ++jq)
                                narrow_store4<TOut>(reinterpret_cast<char*>(row + 8 * jq * EB), acc[4 * jq],
                                                    acc[4 * jq + 1], acc[4 * jq + 2], acc[4 * jq + 3]);
                        }
                        const int rr = lane / LPR, seg = lane % LPR;
                        const uint4 v = *reinterpret_cast<const uint4*>(tile + rr * OSTR + 16 * seg);
                        const int kk = 32 * ct + rd * RPR + rr;
                        const int p = 32 * b + seg * (16 / EB);    // pixel of the step
                        if (kk < a.K && p < npx)
                            *reinterpret_cast<uint4*>(yband + (uint32_t)EB * ((uint32_t)kk * a.plane_y +
                                                                            (uint32_t)(pix0 + p))) = v;
                    }
                } else {
                    const int k = 32 * ct + ml;
                    if (k < a.K) {
                        // byte offset of the lane's channel at the step's first pixel
                        const uint32_t yoff = (uint32_t)EB * ((uint32_t)k * a.plane_y + (uint32_t)pix0);
#pragma unroll
                        for (int jq = 0; jq < 4; ++jq) {
                            const int p = 32 * b + 8 * jq + 4 * g;   // pixel of the step
                            if (a.vec) {
                                if (p < npx)
                                    narrow_store4<TOut>(yband + (yoff + (uint32_t)EB * (uint32_t)p), acc[4 * jq],
                                                        acc[4 * jq + 1], acc[4 * jq + 2], acc[4 * jq + 3]);
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (p + e < npx)
                                        *reinterpret_cast<TOut*>(yband + (yoff + (uint32_t)EB * (uint32_t)(p + e))) =
                                            from_f32<TOut>(acc[4 * jq + e]);
                            }
                        }
                    }
                }
            }
        }
        if (wave >= nblk) move_rows();   // a wave with no task this step
    }
}

struct NarrowPlan {
    NarrowArgs a;
    int KS;                  // reduction steps of the instantiation: 6 or 11
    size_t lds_bytes;
};

// Which layers the kernel runs, and its launch plan.  Requirements:
// fp16/bf16 input and groups == 1 (checked by the caller), C R <= 22
// (filter fragments of both 32-channel halves stay in registers), K <= 64,
// an even stride_w with dil_w == 1 (strips start on 4-byte boundaries),
// S + d <= 8 where d = (L - pad_w) mod 2 and L = pad_w rounded up to a
// multiple of 4 (the strip and its leading column fit 8 entries), W a
// multiple of 8 (16-byte row copies), no pool, 32-bit offsets within an
// image, and a ring of at least one output row per step in 80 KB of LDS.
inline bool narrow_plan(const Geom& g, int out_bytes, const Epi& epi, int cus, NarrowPlan& pl) {
    if (epi.pool || g.dw != 1 || g.sw % 2 != 0 || g.K > 64 || g.W % 8 != 0) return false;
    const int CR = g.C * g.R;
    if (CR > 22) return false;
    const int L = (g.pw + 3) / 4 * 4;
    const int d = (L - g.pw) & 1;
    if (g.S + d > 8) return false;
    if ((int64_t)g.C * g.H * g.W >= ((int64_t)1 << 31)) return false;
    if ((int64_t)g.K * g.P * g.Q * out_bytes >= ((int64_t)1 << 32)) return false;   // byte offsets in an image of y
    NarrowArgs& a = pl.a;
    a.C = g.C; a.K = g.K; a.H = g.H; a.W = g.W; a.P = g.P; a.Q = g.Q;
    a.R = g.R; a.S = g.S; a.sh = g.sh; a.sw = g.sw; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh;
    a.CR = CR;
    a.span = (g.R - 1) * g.dh + 1;
    a.L = L;
    a.col0 = L - g.pw - d;
    for (int i = 0; i < 4; ++i) {
        auto keep = [&](int e) { return e >= d && e < d + g.S; };
        a.m[i] = (keep(2 * i) ? 0xffffu : 0u) | (keep(2 * i + 1) ? 0xffff0000u : 0u);
    }
    // columns a slot row needs: the input's (from L) and every fragment's 8
    const int64_t cols = std::max<int64_t>((int64_t)L + g.W, (int64_t)(g.Q - 1) * g.sw + a.col0 + 8);
    const int64_t RB = round_up(cols, 8) * 2;
    const int64_t slot_bytes = (int64_t)(g.C + 1) * RB;
    if (slot_bytes * a.span > kNarrowLds) return false;
    a.RB = (int)RB;
    a.slot_bytes = (int)slot_bytes;
    a.wv = g.W / 8;
    a.nl = L / 4;
    a.nr = (int)((RB / 2 - L - g.W) / 4);
    a.filt_elems = g.K * CR * g.S;
    const int64_t filt_bytes = round_up((int64_t)a.filt_elems * 2, 16);
    if (filt_bytes / 16 > (int64_t)kNarrowMaxFilt * kNarrowThreads) return false;
    const int eb = out_bytes;
    const int64_t tiles = (int64_t)4 * (1024 / (32 * eb)) * (32 * eb + 16);
    // bands: about two workgroups per CU over the batch, whole rows each
    const int64_t N = std::max(g.N, 1);
    const int64_t nb = std::max<int64_t>(1, std::min<int64_t>(g.P, (2 * cus + N - 1) / N));
    a.band = (int)((g.P + nb - 1) / nb);
    a.nbands = (g.P + a.band - 1) / a.band;
    const int64_t ntask = (int64_t)g.N * a.nbands;
    if (ntask >= ((int64_t)1 << 31)) return false;
    a.ntask = (int)ntask;
    // the most output rows per step whose new input rows are at most
    // kNarrowMaxIt copies per thread, whose first step's rows are at most
    // kNarrowMaxIt0, and whose ring fits
    const int64_t per_row = (int64_t)g.C * a.wv;
    a.SR = 0;
    for (int sr = std::min(a.band, 16); sr >= 1 && a.SR == 0; --sr) {
        const int64_t nr = (int64_t)(2 * sr - 1) * g.sh + a.span;
        const int64_t r0 = (int64_t)(sr - 1) * g.sh + a.span;
        const int64_t need = nr * slot_bytes + filt_bytes + tiles;
        if (nr <= 255 && need <= kNarrowLds && sr * g.sh * per_row <= kNarrowMaxIt * kNarrowThreads &&
            r0 * per_row <= kNarrowMaxIt0 * kNarrowThreads) {
            a.SR = sr;
            a.NR = (int)nr;
            pl.lds_bytes = (size_t)need;
        }
    }
    if (a.SR == 0) return false;
    a.filt_off = (int)((int64_t)a.NR * slot_bytes);
    a.tile_off = (int)(a.filt_off + filt_bytes);
    a.relu = epi.relu ? 1 : 0;
    a.staged = g.Q % (16 / eb) == 0 ? 1 : 0;
    a.vec = g.Q % 4 == 0 ? 1 : 0;
    a.plane_x = (uint32_t)((int64_t)g.H * g.W);
    a.plane_y = (uint32_t)((int64_t)g.P * g.Q);
    a.fdQ = make_fastdiv((uint32_t)g.Q);
    a.fdNR = make_fastdiv((uint32_t)a.NR);
    a.fdRow = make_fastdiv((uint32_t)per_row);
    a.fdWv = make_fastdiv((uint32_t)a.wv);
    pl.KS = (CR + 1) / 2 <= 6 ? 6 : 11;
    return true;
}

template <typename TIn, typename TOut, int KS>
hipError_t launch_narrow_one(const NarrowPlan& pl, const void* x, const void* w, const void* bias,
                             void* y, hipStream_t st) {
    void (*kfn)(const uint16_t*, const uint16_t*, const TIn*, TOut*, NarrowArgs) =
        conv_mfma_narrow_kernel<TIn, TOut, KS>;
    if (pl.lds_bytes > 65536 && allow_dynamic_lds(reinterpret_cast<const void*>(kfn), pl.lds_bytes) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kfn, dim3((uint32_t)pl.a.ntask), dim3(kNarrowThreads), pl.lds_bytes, st,
                       (const uint16_t*)x, (const uint16_t*)w, (const TIn*)bias, (TOut*)y, pl.a);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_narrow_t(const NarrowPlan& pl, const void* x, const void* w, const void* bias, void* y,
                           hipStream_t st) {
    return pl.KS == 6 ? launch_narrow_one<TIn, TOut, 6>(pl, x, w, bias, y, st)
                      : launch_narrow_one<TIn, TOut, 11>(pl, x, w, bias, y, st);
}

}  // namespace
}  // namespace ciw
