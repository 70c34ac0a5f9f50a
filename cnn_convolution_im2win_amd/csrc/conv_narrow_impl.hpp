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
//   - the workgroup keeps a ring of NR zero-padded input rows in LDS, each
//     slot the C channel rows of one input row, [channel][column].  The
//     first span - 1 slots are also written to span - 1 slots after the
//     ring, so the rows of one output row are consecutive slots from its
//     first, and a fragment's address is the block's base plus a per-lane
//     pair offset.  With an even stride the strip of every output column
//     starts on a 4-byte boundary, so a fragment is two 8-byte LDS reads
//     (ds_read2_b32).  With C R odd, the last step's second pair does not
//     exist; its lanes read pair (0, 0) and clear the fragment;
//   - a band of output rows of one image is computed SR rows per step.  A
//     step's pixels are cut into blocks of 32 consecutive outputs (a block
//     may span two output rows).  Each (block, 32-channel half) is one
//     wave's task: KS steps of window fragment (first operand) x filter
//     fragment (second operand), fp32 accumulators seeded with the bias.
//     Waves 0-3 take the first half and waves 4-7 the second, each wave
//     every fourth block.  A wave holds only its half's filter fragments,
//     which leaves room for four waves a SIMD;
//   - a step's new input rows are loaded into registers one step ahead.
//     Each wave writes its share into the ring between its last task's
//     multiplies and its stores, so the loads have a whole step to arrive.
//     Every input element crosses HBM once per band, and no window tensor
//     is written;
//   - the filter (K x C x R x S, at most 22.5 KB) is copied into LDS once
//     per workgroup.  A fragment's S taps are consecutive there, so every
//     lane reads each of its fragments as one 16-byte read, masked like a
//     window fragment.  No workspace, no separate kernel;
//   - stores go through a per-wave LDS tile of a block's 64 channels (in
//     the filter's region, once every lane has its fragments): one round of
//     tile writes, one of reads, then stores that write whole 64-byte runs
//     of output rows.
// The sum is the convolution's sum in another order, accumulated in fp32
// with the bias first, rounded once at the store.
#pragma once

#include "conv_mfma_impl.hpp"

namespace ciw {
namespace {

constexpr int kNarrowThreads = 256;   // four waves, two per SIMD with the other workgroup
constexpr int kNarrowMaxIt = 6;       // row-copy items per thread per step
constexpr int kNarrowMaxIt0 = 8;      // ... for the first step's rows
constexpr int kNarrowMaxFilt = 6;     // 16-byte filter chunks per thread
constexpr int kNarrowLds = 80 * 1024; // LDS per workgroup (two per CU)

struct NarrowArgs {
    int C, K, H, W, P, Q;
    int R, S, sh, sw, ph, pw, dh;
    int CR;                  // (channel, filter row) pairs: C * R
    int span;                // input rows one output row reads: (R - 1) dil_h + 1
    int L;                   // LDS column of input column 0 (a multiple of 4)
    int col0;                // LDS column of output column 0's first fragment entry: L - pad_w - d
    uint32_t m0, m3;         // masks of a fragment's first and last words: entry e kept
                             // iff d <= e < d + S (the middle words are always whole)
    int RB;                  // bytes of one channel row of a slot (a multiple of 16)
    int slot_bytes;          // C RB
    int NR;                  // ring slots; slots NR .. NR + span - 2 mirror slots 0 .. span - 2
    int ring_bytes;          // NR slot_bytes
    int mirror_lim;          // (span - 1) slot_bytes: writes below it are made twice
    int SR;                  // output rows per step
    int wv;                  // 16-byte vectors of an input row: W / 8
    int nl, nr;              // 8-byte zero stores of a channel row's left / right padding
    int band, nbands, ntask;
    int relu, staged, vec;
    int filt_off;            // LDS byte offset of the staged filter; after the prologue,
                             // of the per-wave output tiles
    int filt_elems;          // K C R S
    uint32_t zero;           // 0
    uint32_t plane_x, plane_y;
    FastDiv fdQ, fdNR, fdRow, fdWv;   // divisors Q, NR, C * W / 8, W / 8
};

// 16 bytes read from a 2-byte boundary.
typedef uint4 __attribute__((aligned(2))) uint4_u2;

// Four adjacent outputs of one channel as one store (8 bytes of halves or
// 16 bytes of floats).
template <typename TOut>
__device__ __forceinline__ void narrow_store4(char* p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2<TOut>(a0, a1), pack2<TOut>(a2, a3));
}

template <>
__device__ __forceinline__ void narrow_store4<float>(char* p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<float4*>(p) = make_float4(a0, a1, a2, a3);
}

// KS = ceil(C R / 2) reduction steps.
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
    const int bfirst = wave;         // the wave's first block of a step (then every fourth)

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
        const bool in = it < (j1 - j0) * a.C * a.wv;
        const int iu = in ? it : 0;
        const int jr = (int)fdiv((uint32_t)iu, a.fdRow);
        const int rem = iu - jr * a.C * a.wv;
        const int c = (int)fdiv((uint32_t)rem, a.fdWv);
        const int vv = rem - c * a.wv;
        const uint32_t j = (uint32_t)(j0 + jr);
        const int slot = (int)(j - fdiv(j, a.fdNR) * a.NR);
        dst = in ? slot * a.slot_bytes + c * a.RB + (a.L + 8 * vv) * 2 : -1;
        const int xrow = xr0 + (int)j;
        const bool inside = xrow >= 0 && xrow < a.H;
        // every lane issues its load (from row 0 where the item is padding
        // or past the rows), so the number of loads in flight is fixed and
        // the waits for them can be counted.  Padding is cleared with a
        // zero the compiler cannot see (a.zero), so it cannot skip the load.
        const uint4 v = *reinterpret_cast<const uint4*>(
            ximg + 2u * ((uint32_t)c * a.plane_x + (uint32_t)((inside ? xrow : 0) * a.W + 8 * vv)));
        const uint32_t km = inside ? ~0u : a.zero;
        return make_uint4(v.x & km, v.y & km, v.z & km, v.w & km);
    };
    auto store_item = [&](const uint4& v, int dst) {
        if (dst < 0) return;
        // 8-byte aligned (L is a multiple of 4 columns)
        *reinterpret_cast<uint2*>(lds + dst) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(lds + dst + 8) = make_uint2(v.z, v.w);
        if (dst < a.mirror_lim) {   // and into the mirror slot
            *reinterpret_cast<uint2*>(lds + a.ring_bytes + dst) = make_uint2(v.x, v.y);
            *reinterpret_cast<uint2*>(lds + a.ring_bytes + dst + 8) = make_uint2(v.z, v.w);
        }
    };

    // ---- prologue.  The filter's loads are issued first, then the first
    // step's rows: the filter can be staged and every lane's fragments built
    // while the rows are still arriving.  The padding columns (which no
    // copy writes) are zeroed meanwhile.
    const int nfc = (a.filt_elems * 2) >> 4;   // whole 16-byte filter chunks
    uint4 pv[kNarrowMaxIt0];
    int pd[kNarrowMaxIt0];
    {
        uint4 fv[kNarrowMaxFilt];
#pragma unroll
        for (int k = 0; k < kNarrowMaxFilt; ++k) {
            const int it = tid + k * kNarrowThreads;
            fv[k] = reinterpret_cast<const uint4*>(w)[it < nfc ? it : 0];
        }
        const int r0 = rb(0);
#pragma unroll
        for (int k = 0; k < kNarrowMaxIt0; ++k) pv[k] = load_item(0, r0, tid + k * kNarrowThreads, pd[k]);
        // the filter's chunks are needed here: waiting for them (and, the
        // loads returning in order, for nothing issued later) before the
        // zeroing below; left to itself the compiler would load each chunk
        // where it is stored and wait for every row as well
#pragma unroll
        for (int k = 0; k < kNarrowMaxFilt; ++k) asm volatile("" : "+v"(fv[k].x), "+v"(fv[k].y), "+v"(fv[k].z), "+v"(fv[k].w));
        // zeros: per slot (mirrors included), each channel row's nl + nr padding words
        const int per_c = a.nl + a.nr;
        const int units = a.C * per_c;
        const int nslots = a.NR + a.span - 1;
        for (int it = tid; it < nslots * units; it += kNarrowThreads) {
            const int slot = it / units;
            const int u = it - slot * units;
            const int c = u / per_c, k = u - c * per_c;
            *reinterpret_cast<uint2*>(lds + slot * a.slot_bytes + c * a.RB +
                                      (k < a.nl ? 8 * k : 2 * (a.L + a.W) + 8 * (k - a.nl))) = make_uint2(0u, 0u);
        }
        // the filter 16 bytes into its region
        for (int e = nfc * 8 + tid; e < a.filt_elems; e += kNarrowThreads)
            *reinterpret_cast<uint16_t*>(lds + a.filt_off + 16 + 2 * e) = w[e];
#pragma unroll
        for (int k = 0; k < kNarrowMaxFilt; ++k) {
            const int it = tid + k * kNarrowThreads;
            if (it < nfc) *reinterpret_cast<uint4*>(lds + a.filt_off + 16 + 16 * it) = fv[k];
        }
    }
    __syncthreads();   // the filter and the padding zeros are in LDS

    // filter fragments of both 32-channel halves: lane holds F[k][c][r][e - d]
    // for e = 0..7, k = 32 ct + ml, (c, r) pair u = 2 ks + g; zero outside
    // the filter.  Entries d .. d + S - 1 are the S taps of (k, c, r),
    // consecutive in KCRS order: the fragment is the 8 elements from
    // (k C R + u) S - d, read as aligned words, shifted into place and
    // masked like a window fragment.
    const int d = a.L - a.pw - a.col0;
    const uint32_t* fw = reinterpret_cast<const uint32_t*>(lds + a.filt_off);
    uint4 F[2][KS];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const int k = 32 * ct + ml;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int u = 2 * ks + g;
            const bool ok = k < a.K && u < a.CR;
            // half-word index of entry 0 in the staged region (the filter
            // starts 16 bytes in, so entry 0 of (0, 0), one element before
            // it when d = 1, still lies inside)
            const int e0 = ok ? (k * a.CR + u) * a.S - d + 8 : 8;
            const uint32_t* p = fw + (e0 >> 1);
            const uint32_t sh = (uint32_t)(e0 & 1) * 16u;
            const uint32_t okm = ok ? ~0u : 0u;   // a mask, not a branch: the reads stay in flight together
            const uint32_t w0 = p[0], w1 = p[1], w2 = p[2], w3 = p[3], w4 = p[4];
            F[ct][ks] = make_uint4(__builtin_amdgcn_alignbit(w1, w0, sh) & a.m0 & okm,
                                   __builtin_amdgcn_alignbit(w2, w1, sh) & okm,
                                   __builtin_amdgcn_alignbit(w3, w2, sh) & okm,
                                   __builtin_amdgcn_alignbit(w4, w3, sh) & a.m3 & okm);
            // the fragment as a value of its own: otherwise the compiler
            // keeps the five words and rebuilds the fragment where it is used
            asm volatile("" : "+v"(F[ct][ks].x), "+v"(F[ct][ks].y), "+v"(F[ct][ks].z), "+v"(F[ct][ks].w));
        }
    }
    // pair offsets: byte offset of pair (c, r)'s row in the slot of a
    // block's filter row 0: r dil_h slots on (no wrap: the mirror slots
    // continue the ring), channel row c.  With C R odd the last step's
    // second pair does not exist: those lanes read pair (0, 0) and their
    // fragment is cleared (tailm).
    uint32_t pu[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int u = 2 * ks + g;
        const int c = u < a.CR ? u / a.R : 0;
        const int r = u < a.CR ? u - c * a.R : 0;
        pu[ks] = (uint32_t)(r * a.dh * a.slot_bytes + c * a.RB);
    }
    // the first step's rows (their loads had the fragments' time to arrive)
#pragma unroll
    for (int k = 0; k < kNarrowMaxIt0; ++k) store_item(pv[k], pd[k]);
    const uint32_t tailm = (2 * (KS - 1) + g < a.CR) ? ~0u : 0u;
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
    __syncthreads();   // the first rows are in the ring, and every lane has its
                       // filter fragments: the output tiles may take the region

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
                // the loads' addresses are computed here, where they are
                // used (hoisted to the step's start they would stay live
                // through its blocks)
                int tl = tid;
                asm volatile("" : "+v"(tl));
#pragma unroll
                for (int k = 0; k < kNarrowMaxIt; ++k)
                    lv[k] = load_item(rb(t + 1), rb(t + 2), tl + k * kNarrowThreads, ldst[k]);
            }
        };
        for (int b = bfirst; b < nblk; b += 4) {
            // the pair table and the bias are re-read from their registers
            // every block: hoisted out of the loop, the values derived from
            // them (two fields of each entry, a 16-register bias splat) would
            // not leave room for four waves a SIMD
            uint32_t pk[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                pk[ks] = pu[ks];
                asm volatile("" : "+v"(pk[ks]));
            }
            float bkb[2] = {bk[0], bk[1]};
            asm volatile("" : "+v"(bkb[0]), "+v"(bkb[1]));
            // the lane's window pixel (past the step's end: its last pixel,
            // read but never stored)
            const uint32_t pb = (uint32_t)(pix0 + min(32 * b + ml, npx - 1));
            const int i = (int)fdiv(pb, a.fdQ);              // band output row
            const int q = (int)pb - i * a.Q;                 // output column
            const uint32_t jb = (uint32_t)(i * a.sh);        // band input row of filter row 0
            const uint32_t s0 = jb - fdiv(jb, a.fdNR) * NRu; // its slot
            // byte offset of the lane's strip in filter row 0's slot, channel 0
            // (slot offsets are below 2^24)
            const uint32_t blk = __umul24(s0, (uint32_t)a.slot_bytes) + (uint32_t)(q * a.sw + a.col0) * 2u;
            auto frag = [&](int ks) -> uint4 {
                const uint32_t* p = reinterpret_cast<const uint32_t*>(lds + (blk + pk[ks]));
                if (ks == KS - 1)
                    return make_uint4(p[0] & a.m0 & tailm, p[1] & tailm, p[2] & tailm, p[3] & a.m3 & tailm);
                return make_uint4(p[0] & a.m0, p[1], p[2], p[3] & a.m3);
            };
            f32x16 acc2[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                acc2[0][e] = bkb[0];
                acc2[1][e] = bkb[1];
            }
            constexpr int PF = KS < 3 ? KS : 3;   // window fragments read ahead
            uint4 bq[PF];
#pragma unroll
            for (int s = 0; s < PF; ++s) bq[s] = frag(s);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint4 bv = bq[s % PF];
                if (s + PF < KS) bq[s % PF] = frag(s + PF);
                acc2[0] = mfma32<TIn>(bv, F[0][s], acc2[0]);
                acc2[1] = mfma32<TIn>(bv, F[1][s], acc2[1]);
            }
            if (a.relu) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    acc2[0][e] = fmaxf(acc2[0][e], 0.f);
                    acc2[1][e] = fmaxf(acc2[1][e], 0.f);
                }
            }
            if (b + 4 >= nblk) move_rows();
            // lane holds channel 32 ct + ml at block pixels 8 jq + 4 g + 0..3
            constexpr int EB = (int)sizeof(TOut);
            if (a.staged) {
                // Through the wave's LDS tile: every lane writes its 16
                // pixels, then reads 16-byte pieces of the tile's rows and
                // stores them, so one store instruction writes whole 64-byte
                // runs (128 with fp32 outputs) of 16 (8) channels.  (LDS
                // operations of one wave complete in order: no barrier.)
                constexpr int OSTR = 32 * EB + 16;         // tile row stride (bytes)
                constexpr int CPR = 2 * EB;                // 16-byte pieces per row
                constexpr int NRD = 64 * CPR / 64;         // pieces per lane
                unsigned char* tile = lds + a.filt_off + wave * 64 * OSTR;
                unsigned char* row = tile + ml * OSTR + 4 * g * EB;
#pragma unroll
                for (int jq = 0; jq < 4; ++jq)
                    narrow_store4<TOut>(reinterpret_cast<char*>(row + 8 * jq * EB), acc2[0][4 * jq],
                                        acc2[0][4 * jq + 1], acc2[0][4 * jq + 2], acc2[0][4 * jq + 3]);
                if (a.K > 32) {
#pragma unroll
                    for (int jq = 0; jq < 4; ++jq)
                        narrow_store4<TOut>(reinterpret_cast<char*>(row + 32 * OSTR + 8 * jq * EB), acc2[1][4 * jq],
                                            acc2[1][4 * jq + 1], acc2[1][4 * jq + 2], acc2[1][4 * jq + 3]);
                }
                uint4 v[NRD];
#pragma unroll
                for (int r = 0; r < NRD; ++r) {
                    const int piece = lane + 64 * r;
                    v[r] = *reinterpret_cast<const uint4*>(tile + (piece / CPR) * OSTR + 16 * (piece % CPR));
                }
#pragma unroll
                for (int r = 0; r < NRD; ++r) {
                    const int piece = lane + 64 * r;
                    const int kk = piece / CPR;                       // channel
                    const int p = 32 * b + (piece % CPR) * (16 / EB); // pixel of the step
                    if (kk < a.K && p < npx)
                        *reinterpret_cast<uint4*>(yband + (uint32_t)EB * ((uint32_t)kk * a.plane_y +
                                                                        (uint32_t)(pix0 + p))) = v[r];
                }
            } else {
                // straight from the registers: 4 adjacent outputs of one
                // channel a store, or single outputs when Q % 4 != 0
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const f32x16& acc = acc2[ct];
                    const int k = 32 * ct + ml;
                    if (k >= a.K) continue;
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
        if (bfirst >= nblk) move_rows();   // a wave with no task this step
    }
}

struct NarrowPlan {
    NarrowArgs a;
    int KS;                  // reduction steps: ceil(C R / 2)
    size_t lds_bytes;
};

// Which layers the kernel runs, and its launch plan.  Requirements:
// fp16/bf16 input and groups == 1 (checked by the caller), C R <= 22
// (a wave's filter fragments stay in registers), K <= 64, an even stride_w
// with dil_w == 1 (strips start on 4-byte boundaries), 6 <= S + d <= 8
// where d = (L - pad_w) mod 2 and L = pad_w rounded up to a multiple of 4
// (the strip and its leading column fit 8 entries, and only a fragment's
// first and last words hold entries of other windows), W a multiple of 8
// (16-byte row copies), no pool, 32-bit offsets within an image, and a ring
// of at least one output row per step in 80 KB of LDS.
inline bool narrow_plan(const Geom& g, int out_bytes, const Epi& epi, int cus, NarrowPlan& pl) {
    if (epi.pool || g.dw != 1 || g.sw % 2 != 0 || g.K > 64 || g.W % 8 != 0) return false;
    const int CR = g.C * g.R;
    if (CR > 22) return false;
    const int L = (g.pw + 3) / 4 * 4;
    const int d = (L - g.pw) & 1;
    if (g.S + d > 8 || g.S + d < 6) return false;
    if ((int64_t)g.C * g.H * g.W >= ((int64_t)1 << 31)) return false;
    if ((int64_t)g.K * g.P * g.Q * out_bytes >= ((int64_t)1 << 32)) return false;   // byte offsets in an image of y
    NarrowArgs& a = pl.a;
    a.C = g.C; a.K = g.K; a.H = g.H; a.W = g.W; a.P = g.P; a.Q = g.Q;
    a.R = g.R; a.S = g.S; a.sh = g.sh; a.sw = g.sw; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh;
    a.CR = CR;
    a.span = (g.R - 1) * g.dh + 1;
    a.L = L;
    a.col0 = L - g.pw - d;
    auto keep = [&](int e) { return e >= d && e < d + g.S; };
    a.m0 = (keep(0) ? 0xffffu : 0u) | (keep(1) ? 0xffff0000u : 0u);
    a.m3 = (keep(6) ? 0xffffu : 0u) | (keep(7) ? 0xffff0000u : 0u);
    // columns a slot row needs: the input's (from L) and every fragment's 8
    const int64_t cols = std::max<int64_t>((int64_t)L + g.W, (int64_t)(g.Q - 1) * g.sw + a.col0 + 8);
    const int64_t RB = round_up(cols, 8) * 2;
    const int64_t slot_bytes = (int64_t)g.C * RB;
    if (slot_bytes * (2 * a.span - 1) > kNarrowLds) return false;
    a.RB = (int)RB;
    a.slot_bytes = (int)slot_bytes;
    a.wv = g.W / 8;
    a.nl = L / 4;
    a.nr = (int)((RB / 2 - L - g.W) / 4);
    a.filt_elems = g.K * CR * g.S;
    a.zero = 0;
    if ((int64_t)a.filt_elems * 2 / 16 > (int64_t)kNarrowMaxFilt * kNarrowThreads) return false;
    // staged filter with 16 bytes below it and 16 above (read by the
    // fragments of the first and last (k, c, r) rows); then the per-wave
    // output tiles in the same region
    const int64_t filt_bytes = round_up((int64_t)a.filt_elems * 2, 16) + 32;
    const int eb = out_bytes;
    const int64_t tiles = (int64_t)(kNarrowThreads / 64) * 64 * (32 * eb + 16);
    const int64_t region = std::max(filt_bytes, tiles);
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
        const int64_t need = (nr + a.span - 1) * slot_bytes + region;   // ring and mirror slots
        if (need <= kNarrowLds && sr * g.sh * per_row <= kNarrowMaxIt * kNarrowThreads &&
            r0 * per_row <= kNarrowMaxIt0 * kNarrowThreads) {
            a.SR = sr;
            a.NR = (int)nr;
            pl.lds_bytes = (size_t)need;
        }
    }
    if (a.SR == 0) return false;
    a.ring_bytes = (int)((int64_t)a.NR * slot_bytes);
    a.mirror_lim = (int)((int64_t)(a.span - 1) * slot_bytes);
    a.filt_off = (int)((int64_t)(a.NR + a.span - 1) * slot_bytes);
    a.relu = epi.relu ? 1 : 0;
    a.staged = g.Q % (16 / eb) == 0 ? 1 : 0;
    a.vec = g.Q % 4 == 0 ? 1 : 0;
    a.plane_x = (uint32_t)((int64_t)g.H * g.W);
    a.plane_y = (uint32_t)((int64_t)g.P * g.Q);
    a.fdQ = make_fastdiv((uint32_t)g.Q);
    a.fdNR = make_fastdiv((uint32_t)a.NR);
    a.fdRow = make_fastdiv((uint32_t)per_row);
    a.fdWv = make_fastdiv((uint32_t)a.wv);
    pl.KS = (CR + 1) / 2;
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
    switch (pl.KS) {
#define CIW_NARROW_KS(k) \
    case k: return launch_narrow_one<TIn, TOut, k>(pl, x, w, bias, y, st);
        CIW_NARROW_KS(1) CIW_NARROW_KS(2) CIW_NARROW_KS(3) CIW_NARROW_KS(4) CIW_NARROW_KS(5)
        CIW_NARROW_KS(6) CIW_NARROW_KS(7) CIW_NARROW_KS(8) CIW_NARROW_KS(9) CIW_NARROW_KS(10)
        CIW_NARROW_KS(11)
#undef CIW_NARROW_KS
        default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace ciw
