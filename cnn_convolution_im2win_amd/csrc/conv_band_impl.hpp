// conv_band_impl.hpp -- fp16/bf16 im2win contraction for 3x3 filters with
// the window rows built in LDS, one persistent workgroup per band of output
// rows: kernel, plan and launcher templates.  Included by one file per input
// type.
//
// The im2win paper ("Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support on GPU CUDA and Tensor Cores") repacks the input
// into a window tensor whose row for an output row holds, column by column,
// the input rows it reads (§III-B, §III-C; channel innermost on tensor cores,
// §III-D), and contracts each output's window with the filter.  Here the
// window rows never reach memory:
//   - the workgroup keeps a ring of NR input rows in LDS, each stored
//     [column][channel] with zero padding columns (the row of the window
//     tensor with its filter-row index split over R ring slots);
//   - output rows are computed SR at a time ("steps").  A step's pixels are
//     cut into blocks of 32 consecutive pixels (a block may span two output
//     rows, so no MFMA column is wasted on row ends), and each (block,
//     32-channel half) is one task: 36 v_mfma_f32_32x32x16 multiplies of a
//     window fragment (32 pixels x 16 channels of one filter tap, one 16-byte
//     LDS read per lane) by a filter fragment held in registers;
//   - while a step multiplies, the input rows of the next step are already
//     in registers (loaded one step earlier); each wave transposes its share
//     into the ring between its last task's multiplies and stores, then
//     loads its share of the rows of the step after, so memory latency hides
//     behind a whole step of multiplies.  The first step is short, so that
//     multiplying starts after a few input rows have arrived;
//   - every input element is read from HBM once per band, and every output
//     once written: the window tensor's traffic (twice its size) is gone.
// The filter is re-laid out inside the kernel: in the prologue each wave
// reads one (output-channel half, 16-channel block) slice of the KCRS
// filter with consecutive 16-byte loads, passes it through its own LDS area
// so that each lane gets its channels' taps, permutes them in registers
// into MFMA fragment order and writes them to LDS, from where every wave
// takes its 36 fragments.  No workspace and no separate kernel are needed.
// The reduction is ordered (filter row, filter column, channel), a
// reordering of the paper's window order; the sum is the same sum in
// another order, accumulated in fp32, with the bias added in fp32 first
// and one rounding at the store.
#pragma once

#include "conv_implicit_impl.hpp"

namespace ciw {
namespace {

constexpr int kBandThreads = 512;   // eight waves, two per SIMD

struct BandArgs {
    int C, K, H, W, P, Q;
    int sw, ph, pw, dh, dw;
    int span;            // input rows one output row reads: 2 * dil_h + 1
    int SR0, SR, NR;     // output rows of the first step, of the others; ring slots (2 SR + span - 1)
    int CS;              // 16-byte chunks per ring column (C / 8 rounded up to odd)
    int wb;              // columns of a ring slot: max(pad_w + W, (Q - 1) stride_w + 2 dil_w + 1)
    int row_bytes;       // bytes of one ring slot: wb * CS * 16
    int wv;              // 8-column vectors of an input row: W / 8
    int band, nbands, ntask;
    int nkh;             // 32-channel output halves: 1 (K <= 32) or 2 (K <= 64)
    int relu, vec;       // ReLU; 4-pixel vector stores (Q % 4 == 0)
    int staged;          // stores go through the per-wave LDS tile: 16 bytes per lane,
                         // whole 64-byte channel runs (16 / element size divides Q)
    int ostage_off;      // LDS byte offset of the per-wave output tiles
    int filt_off;        // LDS byte offset of the prologue's filter staging (the
                         // filter's raw pieces lie below it, from offset 0)
    uint32_t plane_x;    // H * W
    uint32_t plane_y;    // P * Q
    FastDiv fdQ, fdNR;
};

// Four adjacent outputs of one channel as one store (8 bytes of halves or 16
// bytes of floats).
template <typename TOut>
__device__ __forceinline__ void store4(TOut* p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2<TOut>(a0, a1), pack2<TOut>(a2, a3));
}

template <>
__device__ __forceinline__ void store4<float>(float* p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<float4*>(p) = make_float4(a0, a1, a2, a3);
}

// DV (stride_w = dil_w = 1, Q even): each (filter row, 16-channel block)
// reads the fragments of filter columns 0 and 2 only; column 1's is taken
// from the neighbouring lanes of those (see below), a third fewer LDS reads.
template <typename TIn, typename TOut, int CB, bool DV>
__global__ __launch_bounds__(kBandThreads, 1) void conv_mfma_band_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const TIn* __restrict__ bias, TOut* __restrict__ y, BandArgs a) {
    constexpr int R = 3, S = 3, RS = R * S;
    constexpr int STEPS = RS * CB;   // MFMA steps of a task: one per (tap, 16 channels)
    constexpr int CG = 2 * CB;       // 8-channel groups
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;         // which 8 of a step's 16 channels
    const int ml = lane & 31;        // fragment pixel (window) / output channel (filter)
    // wave -> (output-channel half, first block); waves w and w + 4 share a
    // SIMD and take interleaved blocks of the same half
    const int kh = a.nkh == 2 ? (wave & 1) : 0;
    const int bfirst = a.nkh == 2 ? (wave >> 1) : wave;
    const int bstep = a.nkh == 2 ? 4 : 8;

    // band = (image, first output row); with the grid a multiple of 8 the
    // bands of one image land on one XCD (workgroups are dispatched round-robin
    // over the 8 XCDs), so the halo rows two bands share meet in its L2
    int task = blockIdx.x;
    if ((a.ntask & 7) == 0) task = (int)(blockIdx.x & 7) * (a.ntask >> 3) + (int)(blockIdx.x >> 3);
    const int n = task / a.nbands;
    const int h0 = (task - n * a.nbands) * a.band;
    const int rows = min(a.band, a.P - h0);
    // Steps: the first multiplies SR0 output rows, the others SR each (the
    // first is short so that computing starts after few input rows have
    // arrived).  Step t covers band output rows [orow(t), orow(t + 1)) and
    // needs band input rows below rb(t); band input row j is x row
    // h0 - pad_h + j.
    const int nsteps = rows <= a.SR0 ? 1 : 1 + (rows - a.SR0 + a.SR - 1) / a.SR;
    auto orow = [&](int t) { return t == 0 ? 0 : min(a.SR0 + (t - 1) * a.SR, rows); };
    auto rb = [&](int t) { return orow(t + 1) + a.span - 1; };
    // image base pointers are uniform (scalar registers); per-lane offsets
    // stay 32-bit (an image of x and of y has fewer than 2^31 elements)
    const char* ximg = reinterpret_cast<const char*>(x + (size_t)n * a.C * a.plane_x);
    char* yband = reinterpret_cast<char*>(y + (size_t)n * a.K * a.plane_y + (size_t)h0 * a.Q);

    // ---- input row transposes.  Item it of rows [j0, j1): 8 channels (group
    // gi) x 8 columns (vector xv) of band input row j.  Its 8 loads are the 8
    // channels' 16-byte column runs; its 8 writes are the 8 columns' 16-byte
    // channel runs, at ring slot j % NR, columns pad_w + 8 xv .. + 7, chunk gi.
    // Rows outside the input are zero (no loads).
    auto load_item = [&](uint4 (&v)[8], int& dst, int j0, int j1, int it) {
        dst = -1;
        if (it >= (j1 - j0) * CG * a.wv) return;
        const int gi = it % CG;
        const int rest = it / CG;
        const int xv = rest % a.wv;
        const int j = j0 + rest / a.wv;
        const int hin = h0 - a.ph + j;
        dst = (j % a.NR) * a.row_bytes + ((a.pw + 8 * xv) * a.CS + gi) * 16;
        if (hin >= 0 && hin < a.H) {
            uint32_t off = 2u * ((uint32_t)(8 * gi) * a.plane_x + (uint32_t)(hin * a.W + 8 * xv));
            // keep the address arithmetic here: hoisted out of the task loop,
            // eight 64-bit addresses would stay live across the multiplies
            asm volatile("" : "+v"(off));
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = *reinterpret_cast<const uint4*>(ximg + (off + 2u * (uint32_t)e * a.plane_x));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    // v[e] holds the 8 columns of channel 8 gi + e, two per dword; column c
    // is written as its 8 channels, one column at a time (few live registers)
    auto store_item = [&](const uint4 (&v)[8], int dst) {
        if (dst < 0) return;
        asm volatile("" : "+v"(dst));   // as above: no hoisted addresses
        auto dw = [&](int e, int d) -> uint32_t {
            return d == 0 ? v[e].x : d == 1 ? v[e].y : d == 2 ? v[e].z : v[e].w;
        };
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = dw(2 * q, c >> 1), hi = dw(2 * q + 1, c >> 1);
                o[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            *reinterpret_cast<uint4*>(lds + dst + c * a.CS * 16) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    };
    // Transposes write only the input's columns [pad_w, pad_w + W) of a slot,
    // so only the padding columns need zeros, once: no transpose writes them.
    auto zero_pads = [&](int s0, int s1) {
        const int npc = a.wb - a.W;                          // padding columns per slot
        const int total = (s1 - s0) * npc * a.CS;
        for (int it = tid; it < total; it += kBandThreads) {
            const int ch = it % a.CS;
            const int rest = it / a.CS;
            const int pc = rest % npc;
            const int col = pc < a.pw ? pc : a.W + pc;       // left pads, then right pads
            *reinterpret_cast<uint4*>(lds + (s0 + rest / npc) * a.row_bytes + (col * a.CS + ch) * 16) =
                make_uint4(0u, 0u, 0u, 0u);
        }
    };

    // ---- prologue.  Loads are issued in the order they are needed: the
    // filter slice; once it is in, the first step's rows (ring slots
    // [0, rb(0)); every CU asks for the same filter at the start, and rows
    // requested alongside it delay it); once those are in, the second
    // step's rows (kept in registers until the end of the first step).  The
    // filter is staged in LDS above the first step's slots and read into
    // registers while the rows arrive; only after every wave has read it
    // (the first step's barrier) may the other slots be touched.
    // Filter slice of wave (fkh, fcb): F[32 fkh + 0 .. 31][16 fcb + 0 .. 15]
    // [taps], 32 runs of 16 RS halves of KCRS (one an output channel, C RS
    // halves apart), PPR 16-byte pieces each.  Load i of lane L takes piece
    // 64 i + L of the slice (run (64 i + L) / PPR), so each load instruction
    // reads about 1 KB of consecutive bytes rather than 32 scattered runs;
    // the pieces go to the wave's own LDS area in that order (at the bottom
    // of LDS, below the fragment staging: ring slots that no wave writes
    // before the filter's barrier) and each lane reads back its RS pieces:
    // F[k][c0 .. c0 + 7][taps], k = 32 fkh + ml, c0 = 16 fcb + 8 g.
    constexpr int PPR = 2 * RS;
    const bool stager = wave < a.nkh * CB;
    const int fkh = stager ? wave % a.nkh : 0, fcb = stager ? wave / a.nkh : 0;
    uint32_t fq[4 * RS];   // the lane's pieces, as words
#pragma unroll
    for (int i = 0; i < 4 * RS; ++i) fq[i] = 0u;
    if (stager) {
#pragma unroll
        for (int i = 0; i < RS; ++i) {
            const int j = 64 * i + lane;
            const int run = j / PPR;
            const int k = min(32 * fkh + run, a.K - 1);   // channels past K: dropped below
            const uint4 u =
                *reinterpret_cast<const uint4*>(w + ((size_t)k * a.C + 16 * fcb) * RS + 8 * (j - run * PPR));
            fq[4 * i] = u.x; fq[4 * i + 1] = u.y; fq[4 * i + 2] = u.z; fq[4 * i + 3] = u.w;
        }
    }
    const int r0 = rb(0);
    uint4 pv[8];
    int pdst = -1;
    if (stager) {
        unsigned char* fraw = lds + wave * (32 * PPR * 16);
#pragma unroll
        for (int i = 0; i < RS; ++i)
            *reinterpret_cast<uint4*>(fraw + (64 * i + lane) * 16) =
                make_uint4(fq[4 * i], fq[4 * i + 1], fq[4 * i + 2], fq[4 * i + 3]);
        // (LDS operations of one wave complete in order: no barrier)
        uint32_t raw[4 * RS];
#pragma unroll
        for (int i = 0; i < RS; ++i) {
            const uint4 u = *reinterpret_cast<const uint4*>(fraw + (ml * PPR + RS * g + i) * 16);
            raw[4 * i] = u.x; raw[4 * i + 1] = u.y; raw[4 * i + 2] = u.z; raw[4 * i + 3] = u.w;
        }
        const uint32_t fkeep = 32 * fkh + ml < a.K ? 0xffffu : 0u;
        auto half_at = [&](int i) -> uint32_t { return (raw[i >> 1] >> (16 * (i & 1))) & fkeep; };
        // fragment of tap t: channels c0 + 2d, c0 + 2d + 1 in dword d
#pragma unroll
        for (int t = 0; t < RS; ++t) {
            uint32_t d[4];
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) d[dd] = half_at(2 * dd * RS + t) | (half_at((2 * dd + 1) * RS + t) << 16);
            *reinterpret_cast<uint4*>(lds + a.filt_off + ((fkh * STEPS + t * CB + fcb) * 64 + lane) * 16) =
                make_uint4(d[0], d[1], d[2], d[3]);
        }
    }
    load_item(pv, pdst, 0, r0, tid);
    __syncthreads();   // the staged filter is complete; the raw pieces are dead
    // the fragments are read while the first rows are still arriving
    uint4 F[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
        F[s] = *reinterpret_cast<const uint4*>(lds + a.filt_off + ((kh * STEPS + s) * 64 + lane) * 16);
    zero_pads(0, r0);
    const float bk = (bias != nullptr && 32 * kh + ml < a.K) ? to_f32(bias[32 * kh + ml]) : 0.f;
    store_item(pv, pdst);
    // the second step's rows: issued once the first step's have arrived (all
    // bands request their first rows at once; these would compete with them)
    uint4 lv[8];
    int ldst = -1;
    if (nsteps > 1) load_item(lv, ldst, r0, rb(1), tid);

    int coff[S];
#pragma unroll
    for (int q = 0; q < S; ++q) coff[q] = q * a.dw * a.CS * 16;

    // ---- steps
    for (int t = 0; t < nsteps; ++t) {
        __syncthreads();   // rows of step t are in the ring
        // every wave has read its filter fragments (before the first of these
        // barriers): the padding columns of the slots that held the staged
        // filter can be zeroed; the first step does not read those slots
        if (t == 0) zero_pads(r0, a.NR);
        const int o0 = orow(t);
        const int npx = (orow(t + 1) - o0) * a.Q;           // pixels of the step
        const int nblk = (npx + 31) >> 5;
        const int pix0 = o0 * a.Q;                          // band pixel of the first
        // the next step's rows, loaded one step ago, into the ring (slots no
        // wave reads in this step), then the loads for the step after.  A
        // wave does this between its last task's multiplies and its stores:
        // the wait for the loads then covers only stores of earlier tasks,
        // which have long completed.
        auto move_rows = [&]() {
            if (t + 1 < nsteps) store_item(lv, ldst);
            if (t + 2 < nsteps) load_item(lv, ldst, rb(t + 1), rb(t + 2), tid);
        };
        for (int b = bfirst; b < nblk; b += bstep) {
            // the lane's window pixel (past the step's end: its last pixel,
            // read but never stored)
            const uint32_t pb = (uint32_t)(pix0 + min(32 * b + ml, npx - 1));
            const int i = (int)fdiv(pb, a.fdQ);               // band output row
            const int wc = (int)pb - i * a.Q;                 // output column
            int base[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t j = (uint32_t)(i + r * a.dh);
                const int slot = (int)(j - fdiv(j, a.fdNR) * a.NR);
                base[r] = slot * a.row_bytes + (wc * a.sw * a.CS + g) * 16;
            }
            auto frag = [&](int s) {
                const int cb = s % CB, tq = s / CB;
                return *reinterpret_cast<const uint4*>(lds + base[tq / S] + coff[tq % S] + 32 * cb);
            };
            f32x16 acc;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = bk;   // the bias seeds the sum
            if constexpr (DV) {
                // With stride_w = dil_w = 1 the window column of filter
                // column 1 at pixel m is filter column 0's at pixel m + 1
                // and filter column 2's at pixel m - 1, whenever those
                // pixels are in m's output row.  So lane m takes column 1's
                // fragment from lane m + 1's column-0 fragment (a whole-wave
                // DPP shift), or, where m is the last pixel of its row or of
                // the lane's 32-lane half, from lane m - 1's column-2
                // fragment.  (With Q even neither neighbour is missing: a
                // block's first pixel never ends a row and its last never
                // starts one.)  The products and their order are those of
                // the reads the fragments replace.
                const bool next = ml != 31 && wc != a.Q - 1;
                auto from_next = [&](uint32_t v) {
                    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x130, 0xf, 0xf, true);
                };
                auto from_prev = [&](uint32_t v) {
                    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x138, 0xf, 0xf, true);
                };
                auto frag_rqc = [&](int r, int q, int cb) {
                    return *reinterpret_cast<const uint4*>(lds + base[r] + coff[q] + 32 * cb);
                };
                uint4 f0 = frag_rqc(0, 0, 0), f2 = frag_rqc(0, 2, 0);
#pragma unroll
                for (int r = 0; r < R; ++r) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        // both shifts run in every lane: a DPP move under a
                        // partial exec mask reads nothing from the lanes
                        // masked off, so the choice is made on the values
                        const uint4 sn = {from_next(f0.x), from_next(f0.y), from_next(f0.z), from_next(f0.w)};
                        const uint4 sp = {from_prev(f2.x), from_prev(f2.y), from_prev(f2.z), from_prev(f2.w)};
                        uint4 f1;
                        f1.x = next ? sn.x : sp.x;
                        f1.y = next ? sn.y : sp.y;
                        f1.z = next ? sn.z : sp.z;
                        f1.w = next ? sn.w : sp.w;
                        const int rn = cb + 1 < CB ? r : r + 1, cn = cb + 1 < CB ? cb + 1 : 0;
                        acc = mfma32<TIn>(f0, F[(r * S + 0) * CB + cb], acc);
                        const uint4 f0n = rn < R ? frag_rqc(rn, 0, cn) : f0;
                        acc = mfma32<TIn>(f1, F[(r * S + 1) * CB + cb], acc);
                        acc = mfma32<TIn>(f2, F[(r * S + 2) * CB + cb], acc);
                        const uint4 f2n = rn < R ? frag_rqc(rn, 2, cn) : f2;
                        f0 = f0n;
                        f2 = f2n;
                    }
                }
            } else {
                constexpr int PF = 3;   // window fragments read ahead
                uint4 bq[PF];
#pragma unroll
                for (int s = 0; s < PF; ++s) bq[s] = frag(s);
#pragma unroll
                for (int s = 0; s < STEPS; ++s) {
                    const uint4 bv = bq[s % PF];
                    if (s + PF < STEPS) bq[s % PF] = frag(s + PF);
                    acc = mfma32<TIn>(bv, F[s], acc);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
                for (int s = 0; s < STEPS; ++s) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (s + PF < STEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
            if (a.relu) {
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] = fmaxf(acc[e], 0.f);
            }
            // lane holds channel k at block pixels 8 jq + 4 g + 0..3, rounded
            // once to the output type
            const int k = 32 * kh + ml;
            constexpr int EB = (int)sizeof(TOut);
            uint32_t pk[16 / (4 / EB)];   // 8 words of two halves, or 16 floats
#pragma unroll
            for (int e = 0; e < 16 / (4 / EB); ++e) {
                if constexpr (EB == 2) pk[e] = pack2<TOut>(acc[2 * e], acc[2 * e + 1]);
                else pk[e] = __float_as_uint(acc[e]);
            }
            if (b + bstep >= nblk) move_rows();
            if (a.staged) {
                // Through the wave's LDS tile, RPR channels at a time: the
                // lanes of those channels write their 16 pixels, then every
                // lane reads 16 bytes of one channel's 32-pixel run and
                // stores them, so one store instruction writes whole 64-byte
                // runs of RPR channels.  (LDS operations of one wave complete
                // in order: no barrier.)
                constexpr int RPR = 1024 / (32 * EB);          // channels per round
                constexpr int OSTR = 32 * EB + 16;             // tile row stride (bytes)
                constexpr int LPR = 64 / RPR;                  // lanes per channel run
                unsigned char* tile = lds + a.ostage_off + wave * RPR * OSTR;
#pragma unroll
                for (int rd = 0; rd < 32 / RPR; ++rd) {
                    if (ml / RPR == rd) {
                        unsigned char* row = tile + (ml % RPR) * OSTR + 4 * g * EB;
#pragma unroll
                        for (int jq = 0; jq < 4; ++jq) {
                            if constexpr (EB == 2)
                                *reinterpret_cast<uint2*>(row + 8 * jq * EB) = make_uint2(pk[2 * jq], pk[2 * jq + 1]);
                            else
                                *reinterpret_cast<uint4*>(row + 8 * jq * EB) =
                                    make_uint4(pk[4 * jq], pk[4 * jq + 1], pk[4 * jq + 2], pk[4 * jq + 3]);
                        }
                    }
                    const int rr = lane / LPR, seg = lane % LPR;
                    const uint4 v = *reinterpret_cast<const uint4*>(tile + rr * OSTR + 16 * seg);
                    const int kk = 32 * kh + rd * RPR + rr;
                    const int p = 32 * b + seg * (16 / EB);    // pixel of the step
                    if (kk < a.K && p < npx)
                        store_stream(yband + (uint32_t)EB * ((uint32_t)kk * a.plane_y + (uint32_t)(pix0 + p)), v);
                }
            } else if (k < a.K) {
                // byte offset of the lane's channel at the step's first pixel
                const uint32_t yoff = (uint32_t)EB * ((uint32_t)k * a.plane_y + (uint32_t)pix0);
#pragma unroll
                for (int jq = 0; jq < 4; ++jq) {
                    const int p = 32 * b + 8 * jq + 4 * g;   // pixel of the step
                    if (a.vec) {
                        if (p < npx) {
                            if constexpr (EB == 2)
                                store_stream(yband + (yoff + 2u * (uint32_t)p), make_uint2(pk[2 * jq], pk[2 * jq + 1]));
                            else
                                store_stream(yband + (yoff + 4u * (uint32_t)p),
                                             make_uint4(pk[4 * jq], pk[4 * jq + 1], pk[4 * jq + 2], pk[4 * jq + 3]));
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (p + e < npx) {
                                if constexpr (EB == 2)
                                    store_stream(yband + (yoff + 2u * (uint32_t)(p + e)),
                                                 (uint16_t)(pk[2 * jq + (e >> 1)] >> (16 * (e & 1))));
                                else
                                    store_stream(yband + (yoff + 4u * (uint32_t)(p + e)), pk[4 * jq + e]);
                            }
                    }
                }
            }
        }
        if (bfirst >= nblk) move_rows();   // a wave with no task this step
    }
}

struct BandPlan {
    BandArgs a;
    int CB;
    size_t lds_bytes;
};

// Which layers the band kernel runs, and its launch plan.  Requirements:
// fp16/bf16 input (checked by the caller), groups == 1, a 3x3 filter,
// C a multiple of 16 and at most 64, K <= 64, W a multiple of 8 (16-byte
// row loads), stride_h == 1 (one new input row per output row), no pool,
// and a ring of at least one output row per step that fits LDS.  out_bytes
// is the output element size (the staged stores need room for their tiles).
inline bool band_plan(const Geom& g, int out_bytes, const Epi& epi, int cus, BandPlan& pl) {
    if (g.R != 3 || g.S != 3 || g.C % 16 != 0 || g.C > 64 || g.K > 64 || g.W % 8 != 0 || g.sh != 1 || epi.pool)
        return false;
    if ((int64_t)g.C * g.H * g.W >= ((int64_t)1 << 31)) return false;         // 32-bit offsets in an image
    if ((int64_t)g.K * g.P * g.Q * out_bytes >= ((int64_t)1 << 32)) return false;   // byte offsets in an image of y
    BandArgs& a = pl.a;
    a.C = g.C; a.K = g.K; a.H = g.H; a.W = g.W; a.P = g.P; a.Q = g.Q;
    a.sw = g.sw; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh; a.dw = g.dw;
    a.span = 2 * g.dh + 1;
    const int cg = g.C / 8;
    a.CS = cg | 1;
    const int wb = std::max(g.pw + g.W, (g.Q - 1) * g.sw + 2 * g.dw + 1);
    const int64_t row_bytes = (int64_t)wb * a.CS * 16;
    a.wb = wb;
    a.wv = g.W / 8;
    a.nkh = g.K > 32 ? 2 : 1;
    const int CB = g.C / 16;
    const int64_t filt_bytes = (int64_t)a.nkh * 9 * CB * 64 * 16;
    const int64_t raw_bytes = (int64_t)a.nkh * CB * 32 * 18 * 16;   // the stager waves' raw pieces
    const int64_t lds_max = 160 * 1024;
    // bands: one per CU in total where the batch allows, at least 8 rows each
    const int64_t N = std::max(g.N, 1);
    const int64_t nb = std::max<int64_t>(1, std::min<int64_t>(g.P, (cus + N - 1) / N));
    a.band = (int)std::max<int64_t>((g.P + nb - 1) / nb, std::min(g.P, 8));
    a.nbands = (g.P + a.band - 1) / a.band;
    const int64_t ntask = (int64_t)g.N * a.nbands;
    if (ntask >= ((int64_t)1 << 31)) return false;
    a.ntask = (int)ntask;
    // the most output rows per step such that the ring and the prologue's
    // filter staging fit LDS and a step's new rows are at most one transpose
    // item per thread; the first step about half as many (its rows arrive
    // before any multiply), its input rows also at most one item per thread
    const int64_t per_row = (int64_t)cg * a.wv;   // transpose items of one input row
    a.SR = 0;
    for (int sr = std::min(a.band, 16); sr >= 1 && a.SR == 0; --sr) {
        const int64_t nr = 2 * sr + a.span - 1;
        int sr0 = std::max(1, sr / 2);
        while (sr0 > 1 && (sr0 + a.span - 1) * per_row > kBandThreads) --sr0;
        const int64_t r0 = sr0 + a.span - 1;
        const int64_t lds = std::max(nr * row_bytes, std::max(r0 * row_bytes, raw_bytes) + filt_bytes);
        if (lds <= lds_max && sr * per_row <= kBandThreads && r0 * per_row <= kBandThreads) {
            a.SR = sr;
            a.SR0 = sr0;
            a.NR = (int)nr;
            pl.lds_bytes = (size_t)lds;
        }
    }
    if (a.SR == 0) return false;
    a.row_bytes = (int)row_bytes;
    a.filt_off = (int)std::max<int64_t>((a.SR0 + a.span - 1) * row_bytes, raw_bytes);
    a.relu = epi.relu ? 1 : 0;
    a.vec = g.Q % 4 == 0 ? 1 : 0;
    // per-wave output tiles (1 KB of outputs a round, rows padded by 16 B)
    // after the ring / filter staging, where they fit
    const int eb = out_bytes;
    const size_t tiles = (size_t)8 * (1024 / (32 * eb)) * (32 * eb + 16);
    a.staged = (g.Q % (16 / eb) == 0 && pl.lds_bytes + tiles <= (size_t)lds_max) ? 1 : 0;
    a.ostage_off = (int)pl.lds_bytes;
    if (a.staged) pl.lds_bytes += tiles;
    a.plane_x = (uint32_t)((int64_t)g.H * g.W);
    a.plane_y = (uint32_t)((int64_t)g.P * g.Q);
    a.fdQ = make_fastdiv((uint32_t)g.Q);
    a.fdNR = make_fastdiv((uint32_t)a.NR);
    pl.CB = CB;
    return true;
}

template <typename TIn, typename TOut, int CB>
hipError_t launch_band_one(const BandPlan& pl, const void* x, const void* w, const void* bias,
                           void* y, hipStream_t st) {
    // column-1 fragments from the neighbouring lanes where the geometry allows
    const bool dv = pl.a.sw == 1 && pl.a.dw == 1 && pl.a.Q % 2 == 0;
    void (*kfn)(const uint16_t*, const uint16_t*, const TIn*, TOut*, BandArgs) =
        dv ? conv_mfma_band_kernel<TIn, TOut, CB, true> : conv_mfma_band_kernel<TIn, TOut, CB, false>;
    if (pl.lds_bytes > 65536 && allow_dynamic_lds(reinterpret_cast<const void*>(kfn), pl.lds_bytes) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kfn, dim3((uint32_t)pl.a.ntask), dim3(kBandThreads), pl.lds_bytes, st,
                       (const uint16_t*)x, (const uint16_t*)w, (const TIn*)bias, (TOut*)y, pl.a);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_band_t(const BandPlan& pl, const void* x, const void* w, const void* bias, void* y,
                         hipStream_t st) {
    switch (pl.CB) {
        case 1: return launch_band_one<TIn, TOut, 1>(pl, x, w, bias, y, st);
        case 2: return launch_band_one<TIn, TOut, 2>(pl, x, w, bias, y, st);
        case 3: return launch_band_one<TIn, TOut, 3>(pl, x, w, bias, y, st);
        default: return launch_band_one<TIn, TOut, 4>(pl, x, w, bias, y, st);
    }
}

}  // namespace
}  // namespace ciw
