// conv_implicit_impl.hpp -- fp16/bf16 im2win contraction with the window
// rows built in LDS from x (no window tensor in HBM): kernel, plan and
// launcher templates.  Included by one file per input type.
//
// The im2win paper ("Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support ...") repacks the input once into a window tensor
// whose rows hold, for one output row, the R input rows it reads, channel
// innermost in the NHWC-based variant (§III-D).  Its memory discussion
// (§III-B, processing strategies in §IV-D1) is about the size of that
// tensor.  Here each workgroup builds the window rows of a band of output
// rows in LDS and never writes them to memory:
//   - input rows x[n][0..C)[h][0..W) are copied from global memory straight
//     into an LDS staging ring, pf rows ahead of their use;
//   - each staged row is transposed once (8 channels x 8 columns per item,
//     16-byte reads and writes) into a window-row buffer holding the padded
//     input row channel innermost, [column][channel]; padding columns are
//     zero, and rows outside the input are written as zeros;
//   - the window of output (h, w) is, for every filter tap (r, q), the C
//     channels at column w*stride_w + q*dil_w of buffer h + r*dil_h: the
//     window row of the paper with its (column, filter row) pairs kept in
//     R separate buffers.  One buffer serves the R output rows that read it,
//     so each input element crosses HBM once per band (the paper's point
//     that overlapping windows reuse inputs already in cache, §III-C);
//   - the reduction is ordered t = (r*S + q)*C + c, a reordering of the
//     paper's window order, so one 16-entry MFMA step is 16 channels of one
//     tap and a lane's 8 entries are one 16-byte LDS read.
// Matrix-core mapping as in the row kernel: a wave multiplies 32-pixel
// window fragments (first operand) by register-resident filter fragments of
// 32 output channels (second operand), v_mfma_f32_32x32x16, fp32
// accumulation, bias seeding the accumulators, one rounding at the store.
//
// Ablation switches (the im2win paper §IV-E ablates double buffering,
// asynchronous copies and its zig-zag order; build.py builds a copy of the
// library per switch), all 0 in the library:
//   CIW_ABLATE_NO_DOUBLE: input row u + 1 is copied at the step that needs
//     it and waited for at once (no copy ahead);
//   CIW_ABLATE_NO_ASYNC: rows go global memory -> registers -> LDS instead
//     of straight into LDS;
//   CIW_ABLATE_NO_XCD: bands in dispatch order (no XCD-aware placement).
#pragma once

#include "conv_mfma_impl.hpp"

#ifndef CIW_ABLATE_NO_DOUBLE
#define CIW_ABLATE_NO_DOUBLE 0
#endif
#ifndef CIW_ABLATE_NO_ASYNC
#define CIW_ABLATE_NO_ASYNC 0
#endif
#ifndef CIW_ABLATE_NO_XCD
#define CIW_ABLATE_NO_XCD 0
#endif

namespace ciw {
namespace {

struct MfImpArgs {
    int C, K, H, W, P, Q;
    int sw, ph, pw, dh, dw;
    int span;            // input rows one output row reads: (R - 1) * dil_h + 1
    int CS;              // 16-byte chunks per column of a window-row buffer (odd)
    int row_bytes;       // bytes of one window-row buffer
    int nt;              // window-row buffers: span + 1
    int stage_bytes;     // bytes of one staged input row
    int nstage, pf;      // staging buffers, input rows copied ahead (nstage = pf + 1)
    int nd;              // copy instructions per wave per input row
    int nchunks;         // 16-byte chunks of an input row over all channels: C * W / 8
    int cg, wv;          // channel groups of 8, column vectors of 8
    int nblk, nkh;       // 32-pixel blocks per output row, 32-channel halves (1 or 2)
    int ostride;         // output tile row stride (elements of TOut)
    int se, nq, nsv;     // elements per store (a power of two, at most 16 bytes),
                         // stores per channel row, stores per thread
    int band, nbands, ntask;  // output rows per workgroup, bands per image, workgroups
    int relu, pool;      // epilogue: ReLU; 2x2 max-pool (stride 2, floor)
    int Pc;              // output rows computed: P, or 2 * (P / 2) with the pool
    int qout, yplane;    // outputs per stored row and per channel plane of y
    uint32_t plane_bytes;     // H * W * 2: bytes between channel planes of x
    int off_stage, off_tile, off_bias;   // LDS regions (bytes)
};

constexpr int kImpMaxCopies = 4;   // copy instructions per wave per input row
constexpr int kImpMaxStores = 4;   // output stores per thread per output row

// Filter fragments in load order: aperm[kh][s][lane][e] = F[k][c][r][q] with
// k = 32 kh + lane % 32 and, for step s = (r*S + q)*CB + cb, channel
// c = 16 cb + 8 (lane / 32) + e; zero for k >= K.  One wave's load of a step
// is 1 KB of consecutive bytes.
struct ImpPermArgs {
    int C, K, R, S, CB, steps;
    uint32_t total;      // 2 * steps * 512
};

__global__ __launch_bounds__(kThreads) __attribute__((unused)) void mfma_implicit_filter_kernel(
    const uint16_t* __restrict__ w, uint16_t* __restrict__ aperm, ImpPermArgs p) {
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= p.total) return;
    const int e = i & 7;
    const int lane = (i >> 3) & 63;
    const int rest = (int)(i >> 9);        // kh * steps + s
    const int kh = rest / p.steps;
    const int s = rest - kh * p.steps;
    const int k = kh * 32 + (lane & 31);
    const int cb = s % p.CB;
    const int q = (s / p.CB) % p.S;
    const int r = s / (p.CB * p.S);
    const int c = 16 * cb + 8 * (lane >> 5) + e;
    uint16_t v = 0;
    if (k < p.K) v = w[(((size_t)k * p.C + c) * p.R + r) * p.S + q];
    aperm[i] = v;
}

// One item of the transpose: 8 channels (8 cg .. 8 cg + 7) x 8 columns.
// in[e] holds the 8 columns of channel 8 cg + e (two per dword); out[j]
// holds the 8 channels of column j.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
    auto dw = [&](int e, int d) -> uint32_t {
        return d == 0 ? in[e].x : d == 1 ? in[e].y : d == 2 ? in[e].z : in[e].w;
    };
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int d = j >> 1;
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t lo = dw(2 * p, d), hi = dw(2 * p + 1, d);
            o[p] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        out[j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Output stores of E elements of T (E * sizeof(T) in {2, 4, 8, 16} bytes).
template <int B> struct Word;
template <> struct Word<2> { using type = uint16_t; };
template <> struct Word<4> { using type = uint32_t; };
template <> struct Word<8> { using type = uint2; };
template <> struct Word<16> { using type = uint4; };

// E adjacent tile elements to y.
template <typename T, int E>
__device__ __forceinline__ void copy_out(T* dst, const T* src) {
    using U = typename Word<E * (int)sizeof(T)>::type;
    *reinterpret_cast<U*>(dst) = *reinterpret_cast<const U*>(src);
}

// Horizontal half of the 2x2 pool: 2E adjacent tile elements (whose rows
// already hold the vertical maximum) to E outputs, each the larger of a
// pair.  Both values of a pair are T values, so the maximum is exact.
template <typename T, int E>
__device__ __forceinline__ void pool_out(T* dst, const T* src) {
    if constexpr (sizeof(T) == 2) {
        // a 32-bit word holds one horizontal pair
        uint32_t w[E];
        if constexpr (E == 8) {
            const uint4 p = reinterpret_cast<const uint4*>(src)[0];
            const uint4 q = reinterpret_cast<const uint4*>(src)[1];
            w[0] = p.x; w[1] = p.y; w[2] = p.z; w[3] = p.w;
            w[4] = q.x; w[5] = q.y; w[6] = q.z; w[7] = q.w;
        } else if constexpr (E == 4) {
            const uint4 p = *reinterpret_cast<const uint4*>(src);
            w[0] = p.x; w[1] = p.y; w[2] = p.z; w[3] = p.w;
        } else if constexpr (E == 2) {
            const uint2 p = *reinterpret_cast<const uint2*>(src);
            w[0] = p.x; w[1] = p.y;
        } else {
            w[0] = *reinterpret_cast<const uint32_t*>(src);
        }
        uint32_t o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float lo = to_f32(__builtin_bit_cast(T, (uint16_t)(w[e] & 0xffffu)));
            const float hi = to_f32(__builtin_bit_cast(T, (uint16_t)(w[e] >> 16)));
            o[e] = f32_bits<T>(fmaxf(lo, hi));
        }
        if constexpr (E == 8) {
            *reinterpret_cast<uint4*>(dst) = make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16),
                                                        o[4] | (o[5] << 16), o[6] | (o[7] << 16));
        } else if constexpr (E == 4) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
        } else if constexpr (E == 2) {
            *reinterpret_cast<uint32_t*>(dst) = o[0] | (o[1] << 16);
        } else {
            *reinterpret_cast<uint16_t*>(dst) = (uint16_t)o[0];
        }
    } else {
        float v[2 * E];
        if constexpr (E == 4) {
            const float4 p = reinterpret_cast<const float4*>(src)[0];
            const float4 q = reinterpret_cast<const float4*>(src)[1];
            v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
            v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
        } else if constexpr (E == 2) {
            const float4 p = *reinterpret_cast<const float4*>(src);
            v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
        } else {
            const float2 p = *reinterpret_cast<const float2*>(src);
            v[0] = p.x; v[1] = p.y;
        }
        if constexpr (E == 4) {
            *reinterpret_cast<float4*>(dst) = make_float4(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]),
                                                          fmaxf(v[4], v[5]), fmaxf(v[6], v[7]));
        } else if constexpr (E == 2) {
            *reinterpret_cast<float2*>(dst) = make_float2(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        } else {
            *dst = fmaxf(v[0], v[1]);
        }
    }
}

// One output row's stores: nsv per thread at fixed tile / y offsets.
template <typename T, int E, bool POOL>
__device__ __forceinline__ void store_tile_row(T* yrow, const T* tl, const int* src, const int* dst,
                                               int nsv) {
#pragma unroll
    for (int j = 0; j < kImpMaxStores; ++j) {
        if (j < nsv) {
            if constexpr (POOL) pool_out<T, E>(yrow + dst[j], tl + src[j]);
            else copy_out<T, E>(yrow + dst[j], tl + src[j]);
        }
    }
}

template <typename TIn, typename TOut, int R, int S, int CB>
__global__ __launch_bounds__(kThreads, 2) void conv_mfma_implicit_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ aperm,
    const TIn* __restrict__ bias, TOut* __restrict__ y, MfImpArgs a) {
    constexpr int STEPS = R * S * CB;
    extern __shared__ __align__(16) uint16_t lds[];
    char* const lb = reinterpret_cast<char*>(lds);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = a.nkh == 2 ? (wave & 1) : 0;     // output channels [32 kh, 32 kh + 32)
    const int pb0 = a.nkh == 2 ? (wave >> 1) : wave;  // first pixel block
    const int npb = 4 / a.nkh;                      // waves per channel half
    const int g = lane >> 5;                        // which 8 of a step's 16 entries
    const int ml = lane & 31;                       // fragment pixel / channel

    // Task = (image, band of output rows).  With the grid a multiple of 8,
    // the workgroups of consecutive tasks are placed on one XCD (workgroups
    // are dispatched round-robin over the 8 XCDs), so the input rows that
    // neighbouring bands share meet in that XCD's L2.
    int task = blockIdx.x;
    if (!CIW_ABLATE_NO_XCD && (a.ntask & 7) == 0)
        task = (int)(blockIdx.x & 7) * (a.ntask >> 3) + (int)(blockIdx.x >> 3);
    const int n = task / a.nbands;
    const int h0 = (task - n * a.nbands) * a.band;
    const int rows = min(a.band, a.Pc - h0);   // even with the pool
    const int J = rows + a.span - 1;                // input rows of the band

    // ---- filter fragments of channel half kh, kept for the whole kernel
    uint4 F[STEPS];
    {
        const uint16_t* fp = aperm + ((size_t)kh * STEPS * 64 + lane) * 8;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) F[s] = *reinterpret_cast<const uint4*>(fp + 512 * s);
    }
    float* bias_l = reinterpret_cast<float*>(lb + a.off_bias);
    if (tid < 64) bias_l[tid] = (bias && tid < a.K) ? to_f32(bias[tid]) : 0.f;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) asm volatile("" ::"v"(F[s].x));
    wait_vm_lgkm(0);   // the counts below cover only row copies and output stores

    // ---- input rows: global -> LDS staging directly.  Staging position
    // p = (xv * 8 + e) * cg + gi holds columns 8 xv .. 8 xv + 7 of channel
    // 8 gi + e, so the transpose's reads are consecutive across lanes.  Every
    // wave issues exactly nd copies per row; copy j fills positions
    // [256 j, 256 j + 256), the last one moved back to end at the row's last
    // position (positions it shares with the one before get the same chunk).
    const uint32_t stage_lds =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(lb + a.off_stage);
    uint32_t src_off[kImpMaxCopies];
    int pos_base[kImpMaxCopies];
#pragma unroll
    for (int j = 0; j < kImpMaxCopies; ++j) {
        pos_base[j] = (j == a.nd - 1 && a.nd > 1) ? a.nchunks - kThreads : j * kThreads;
        const int p = min(pos_base[j] + tid, a.nchunks - 1);
        const int gi = p % a.cg;
        const int rest = p / a.cg;
        src_off[j] = (uint32_t)(8 * gi + (rest & 7)) * a.plane_bytes + 16u * (uint32_t)(rest >> 3);
    }
    const uint16_t* ximg = x + (size_t)n * a.C * a.H * a.W;
    auto copy_row = [&](int j) {
        // rows outside the input copy a valid row; the transpose writes zeros
        const int hin = min(max(h0 - a.ph + j, 0), a.H - 1);
        const uint16_t* src = ximg + (size_t)hin * a.W;
        const uint32_t dst0 = stage_lds + (uint32_t)((j % a.nstage) * a.stage_bytes) + 1024u * (uint32_t)wave;
#pragma unroll
        for (int jj = 0; jj < kImpMaxCopies; ++jj) {
            if (jj < a.nd) {
                if (CIW_ABLATE_NO_ASYNC) {
                    // through registers: lane tid's chunk lands at the
                    // position the direct copy would write
                    const uint4 v = *reinterpret_cast<const uint4*>(
                        reinterpret_cast<const char*>(src) + src_off[jj]);
                    *reinterpret_cast<uint4*>(lb + a.off_stage + (j % a.nstage) * a.stage_bytes +
                                              16 * (pos_base[jj] + tid)) = v;
                } else {
                    const uint32_t dst = __builtin_amdgcn_readfirstlane(dst0 + 16u * (uint32_t)pos_base[jj]);
                    // the row's address is uniform; readfirstlane keeps it in
                    // scalar registers, which the instruction's operand needs
                    // whatever the register allocation around it
                    const uint64_t sp = reinterpret_cast<uint64_t>(src);
                    const uint64_t su = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(sp >> 32)) << 32) |
                                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sp);
                    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
                                 :: "v"(src_off[jj]), "s"(dst), "s"(su) : "memory");
                }
            }
        }
    };

    // ---- staged row j -> window-row buffer j % nt, [column][channel].
    // Piece (jp, gi, xv): channels 8 gi .. 8 gi + 7 at columns 8 xv + 2 jp
    // and 8 xv + 2 jp + 1, one dword of each channel in, one 16-byte chunk
    // per column out; the pieces of a row are spread over every thread.
    auto transpose_row = [&](int j) {
        const int hin = h0 - a.ph + j;
        const bool inside = hin >= 0 && hin < a.H;
        char* trow = lb + (j % a.nt) * a.row_bytes;
        const char* srow = lb + a.off_stage + (j % a.nstage) * a.stage_bytes;
        for (int it = tid; it < 4 * a.cg * a.wv; it += kThreads) {
            const int jp = it & 3;
            const int rest = it >> 2;
            const int gi = rest % a.cg;
            const int xv = rest / a.cg;
            uint32_t v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = inside ? *reinterpret_cast<const uint32_t*>(srow + 16 * ((xv * 8 + e) * a.cg + gi) + 4 * jp)
                              : 0u;
            // column 2 jp: low halves; column 2 jp + 1: high halves
            const uint4 lo = make_uint4((v[0] & 0xffffu) | (v[1] << 16), (v[2] & 0xffffu) | (v[3] << 16),
                                        (v[4] & 0xffffu) | (v[5] << 16), (v[6] & 0xffffu) | (v[7] << 16));
            const uint4 hi = make_uint4((v[0] >> 16) | (v[1] & 0xffff0000u), (v[2] >> 16) | (v[3] & 0xffff0000u),
                                        (v[4] >> 16) | (v[5] & 0xffff0000u), (v[6] >> 16) | (v[7] & 0xffff0000u));
            char* dst = trow + 16 * ((a.pw + 8 * xv + 2 * jp) * a.CS + gi);
            *reinterpret_cast<uint4*>(dst) = lo;
            *reinterpret_cast<uint4*>(dst + 16 * a.CS) = hi;
        }
    };

    // ---- output stores: K rows of qout elements, se at a time, from the
    // tile; exactly nsv per thread (surplus threads repeat the last one),
    // positions fixed.  With the pool a stored row is the pair of output
    // rows 2m, 2m + 1, already merged in one tile (their vertical maximum),
    // and each stored element the larger of two adjacent tile elements.
    int st_src[kImpMaxStores], st_dst[kImpMaxStores];
#pragma unroll
    for (int j = 0; j < kImpMaxStores; ++j) {
        const int idx = min(tid + kThreads * j, a.K * a.nq - 1);
        const int k = idx / a.nq, v = idx - (idx / a.nq) * a.nq;
        st_src[j] = k * a.ostride + (v * a.se << a.pool);
        st_dst[j] = k * a.yplane + v * a.se;
    }
    TOut* const tile0 = reinterpret_cast<TOut*>(lb + a.off_tile);
    const int tile_elems = a.K * a.ostride;
    TOut* const yimg = y + (size_t)n * a.K * a.yplane;
    // output row i's tile: alternate rows, or alternate row pairs with the pool
    auto tile_of = [&](int i) { return tile0 + ((i >> a.pool) & 1) * tile_elems; };
    constexpr int kW16 = 16 / (int)sizeof(TOut), kW8 = 8 / (int)sizeof(TOut);
    constexpr int kW4 = 4 / (int)sizeof(TOut), kW2 = sizeof(TOut) == 2 ? 1 : kW4;
    auto store_row = [&](int i) {
        const TOut* tl = tile_of(i);
        TOut* yrow = yimg + (size_t)((h0 + i) >> a.pool) * a.qout;
        const int bytes = a.se * (int)sizeof(TOut);
        if (a.pool) {
            if (bytes == 16) store_tile_row<TOut, kW16, true>(yrow, tl, st_src, st_dst, a.nsv);
            else if (bytes == 8) store_tile_row<TOut, kW8, true>(yrow, tl, st_src, st_dst, a.nsv);
            else if (bytes == 4) store_tile_row<TOut, kW4, true>(yrow, tl, st_src, st_dst, a.nsv);
            else store_tile_row<TOut, kW2, true>(yrow, tl, st_src, st_dst, a.nsv);
        } else {
            if (bytes == 16) store_tile_row<TOut, kW16, false>(yrow, tl, st_src, st_dst, a.nsv);
            else if (bytes == 8) store_tile_row<TOut, kW8, false>(yrow, tl, st_src, st_dst, a.nsv);
            else if (bytes == 4) store_tile_row<TOut, kW4, false>(yrow, tl, st_src, st_dst, a.nsv);
            else store_tile_row<TOut, kW2, false>(yrow, tl, st_src, st_dst, a.nsv);
        }
    };
    // row i - 1 is stored at the step of row i: every row, or with the pool
    // the second row of each pair
    auto stores_at = [&](int i) { return i >= 1 && (!a.pool || ((i - 1) & 1)); };

    // prologue: copies of input rows 0 .. pf; zero every window-row buffer
    // (padding columns stay zero: the transpose writes only columns
    // pw .. pw + W - 1)
    for (int j = 0; j <= (CIW_ABLATE_NO_DOUBLE ? 0 : a.pf) && j < J; ++j) copy_row(j);
    for (int o = 16 * tid; o < a.nt * a.row_bytes; o += 16 * kThreads)
        *reinterpret_cast<uint4*>(lb + o) = make_uint4(0u, 0u, 0u, 0u);
    f32x16 bias_vec;

    // byte offsets of the filter columns q within a buffer
    int coff[S];
#pragma unroll
    for (int q = 0; q < S; ++q) coff[q] = q * a.dw * a.CS * 16;

    // Vector-memory operations this wave issues after the copy of row j:
    // copies of later rows and output stores, in issue order (the prologue
    // copies rows 0 .. pf; step v copies row v + pf + 1, then stores output
    // row v - span, if that step stores).  Waiting for at most that many
    // lets them stay in flight.
    auto dma_of = [&](int v) { return v + a.pf + 1 < J ? a.nd : 0; };
    auto st_of = [&](int v) { return stores_at(v - a.span + 1) ? a.nsv : 0; };
    auto later_ops = [&](int j) {
        int c = 0;
        if (j <= a.pf) {
            c = a.nd * (min(a.pf + 1, J) - 1 - j);
            for (int v = 0; v < j - 1; ++v) c += dma_of(v) + st_of(v);
        } else {
            c = st_of(j - a.pf - 1);
            for (int v = j - a.pf; v < j - 1; ++v) c += dma_of(v) + st_of(v);
        }
        return c;
    };

    // row 0 into its buffer, once every buffer is zeroed (and the bias
    // staged)
    wait_vm_lgkm(CIW_ABLATE_NO_DOUBLE ? 0 : later_ops(0));
    wg_barrier();
#pragma unroll
    for (int e = 0; e < 16; ++e) bias_vec[e] = bias_l[kh * 32 + ml];
    transpose_row(0);

    // Step u: row u + 1's copy has landed and every wave is done with step
    // u - 1 (wait, barrier); copy row u + pf + 1 into the staging buffer row
    // u used; store output row i - 1 from its tile; transpose row u + 1 into
    // the buffer output row i - 1 used; multiply output row i = u - span + 1
    // (rows i .. u, transposed in earlier steps) into the other tile.  One
    // barrier a step: transposes and multiplies of different waves overlap.
    for (int u = 0; u < J; ++u) {
        if (CIW_ABLATE_NO_DOUBLE) {
            // the row this step transposes, copied now and waited for
            if (u + 1 < J) copy_row(u + 1);
            wait_vm_lgkm(0);
        } else {
            wait_vm_lgkm(u + 1 < J ? later_ops(u + 1) : 0);
        }
        wg_barrier();
        if (!CIW_ABLATE_NO_DOUBLE && u + a.pf + 1 < J) copy_row(u + a.pf + 1);
        const int i = u - a.span + 1;
        if (stores_at(i)) store_row(i - 1);
        if (u + 1 < J) transpose_row(u + 1);
        if (i < 0) continue;

        int soff[R];
#pragma unroll
        for (int r = 0; r < R; ++r) soff[r] = ((i + r * a.dh) % a.nt) * a.row_bytes;
        TOut* tile = tile_of(i);
        for (int b = pb0; b < a.nblk; b += npb) {
            // pixels past the row end read the last pixel (never stored)
            const int wr = min(32 * b + ml, a.Q - 1);
            const char* base = lb + (wr * a.sw * a.CS + g) * 16;
            auto frag = [&](int s) {
                const int cb = s % CB, q = (s / CB) % S, r = s / (CB * S);
                return *reinterpret_cast<const uint4*>(base + soff[r] + coff[q] + 32 * cb);
            };
            f32x16 acc = bias_vec;
            uint4 bq[kPf];
#pragma unroll
            for (int s = 0; s < kPf && s < STEPS; ++s) bq[s] = frag(s);
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                const uint4 bv = bq[s % kPf];
                if (s + kPf < STEPS) bq[s % kPf] = frag(s + kPf);
                acc = mfma32<TIn>(bv, F[s], acc);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, kPf < STEPS ? kPf : STEPS, 0);
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (s + kPf < STEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            // lane holds channel k = 32 kh + ml at block pixels
            // 8 (i / 4) + 4 g + i % 4
            // ReLU as maxNum against 0.  fmaxf, not inline asm: a vector
            // instruction reading a fresh MFMA result needs wait states the
            // compiler inserts only for instructions it sees
            if (a.relu) {
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] = fmaxf(acc[e], 0.f);
            }
            const int k = kh * 32 + ml;
            if (k < a.K) {
                TOut* orow = tile + k * a.ostride + 32 * b + 4 * g;
                // the second row of a pooled pair: this lane wrote the same
                // tile elements for the first row in the previous step
                // (LDS operations of one wave complete in order)
                if (a.pool && (i & 1)) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 o = get4<TOut>(orow + 8 * q);
                        acc[4 * q] = fmaxf(acc[4 * q], o.x);
                        acc[4 * q + 1] = fmaxf(acc[4 * q + 1], o.y);
                        acc[4 * q + 2] = fmaxf(acc[4 * q + 2], o.z);
                        acc[4 * q + 3] = fmaxf(acc[4 * q + 3], o.w);
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    put4<TOut>(orow + 8 * q, acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
            }
        }
    }
    wait_vm_lgkm_lds_only();
    wg_barrier();
    store_row(rows - 1);
}

struct MfImpPlan {
    MfImpArgs a;
    int R, S, CB, steps;
    size_t lds_bytes;
    int wgs_per_cu;
};

// Filter shapes with compiled kernels: (R, S) = (3, 3) with C/16 in 1..4,
// (1, 1) with C/16 in {1, 2, 4}.
inline bool imp_compiled(int R, int S, int CB) {
    if (R == 3 && S == 3) return CB >= 1 && CB <= 4;
    if (R == 1 && S == 1) return CB == 1 || CB == 2 || CB == 4;
    return false;
}

// Which layers the kernel runs, and its launch plan.  Requirements: groups
// == 1 (checked by the caller), C a multiple of 16 (a step is 16 channels of
// one tap), K <= 64 (the filter lives in registers), W a multiple of 8
// (16-byte row copies), stride_h == 1 (one new input row per output row),
// at most 4 output stores per thread per row, and every LDS region within
// 160 KB.
inline bool mf_imp_plan(const Geom& g, int out_bytes, const Epi& epi, int cus, MfImpPlan& pl) {
    if (g.C % 16 != 0 || g.K > 64 || g.W % 8 != 0 || g.sh != 1) return false;
    if (epi.pool && (g.P < 2 || g.Q < 2)) return false;
    const int CB = g.C / 16;
    if (!imp_compiled(g.R, g.S, CB)) return false;
    if ((int64_t)g.C * g.H * g.W * 2 >= ((int64_t)1 << 31)) return false;   // 32-bit copy offsets
    MfImpArgs& a = pl.a;
    a.C = g.C; a.K = g.K; a.H = g.H; a.W = g.W; a.P = g.P; a.Q = g.Q;
    a.sw = g.sw; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh; a.dw = g.dw;
    a.span = (g.R - 1) * g.dh + 1;
    a.cg = g.C / 8;
    a.wv = g.W / 8;
    a.CS = a.cg | 1;   // an odd chunk stride: consecutive pixels hit distinct banks
    a.nt = a.span + 1;
    const int wb = std::max(g.Wwin, g.pw + g.W);
    a.row_bytes = wb * a.CS * 16;
    a.nchunks = g.C * g.W / 8;
    a.nd = (a.nchunks + kThreads - 1) / kThreads;
    if (a.nd > kImpMaxCopies) return false;
    a.stage_bytes = std::max(a.nchunks, kThreads) * 16;   // one copy covers 256 positions
    a.plane_bytes = (uint32_t)((int64_t)g.H * g.W * 2);
    a.nblk = (g.Q + 31) / 32;
    a.nkh = g.K > 32 ? 2 : 1;
    const int V = 16 / out_bytes;
    int ostride = (32 * a.nblk + V - 1) / V * V;
    if (((ostride * out_bytes) / 16) % 2 == 0) ostride += V;   // odd 16-byte units per row
    a.ostride = ostride;
    a.pool = epi.pool ? 1 : 0;
    a.relu = epi.relu ? 1 : 0;
    a.Pc = a.pool ? 2 * (g.P / 2) : g.P;
    a.qout = a.pool ? g.Q / 2 : g.Q;
    const int64_t yplane = (int64_t)(a.pool ? g.P / 2 : g.P) * a.qout;
    if ((int64_t)g.K * yplane >= ((int64_t)1 << 31)) return false;   // 32-bit store offsets
    a.yplane = (int)yplane;
    a.se = V;   // the widest store that divides a row
    while (a.se > 1 && a.qout % a.se != 0) a.se >>= 1;
    a.nq = a.qout / a.se;
    a.nsv = (g.K * a.nq + kThreads - 1) / kThreads;
    if (a.nsv > kImpMaxStores) return false;
    const size_t tile = 2 * (size_t)g.K * ostride * out_bytes;
    // two workgroups per CU with the deepest copy-ahead that fits, else one
    size_t lds = 0;
    int wgs = 0, pf = 0;
    for (int w = 2; w >= 1 && wgs == 0; --w)
        for (int p = 3; p >= 1; --p) {
            const size_t bytes = (size_t)a.nt * a.row_bytes + (size_t)(p + 1) * a.stage_bytes + tile + 256;
            if (bytes * w <= 160 * 1024) {
                lds = bytes;
                wgs = w;
                pf = p;
                break;
            }
        }
    if (wgs == 0) return false;
    a.pf = pf;
    a.nstage = pf + 1;
    a.off_stage = a.nt * a.row_bytes;
    a.off_tile = a.off_stage + a.nstage * a.stage_bytes;
    a.off_bias = a.off_tile + (int)tile;
    // bands: about wgs_per_cu workgroups per CU in total, and at least 4
    // output rows a band (fewer would re-read most input rows per row);
    // whole row pairs with the pool
    const int64_t target = (int64_t)cus * wgs;
    int nb = (int)std::min<int64_t>(a.Pc, std::max<int64_t>(1, (target + g.N / 2) / std::max(g.N, 1)));
    a.band = std::max((a.Pc + nb - 1) / nb, std::min(a.Pc, 4));
    if (a.pool) a.band += a.band & 1;
    a.nbands = (a.Pc + a.band - 1) / a.band;
    const int64_t ntask = (int64_t)g.N * a.nbands;
    if (ntask >= ((int64_t)1 << 31)) return false;
    a.ntask = (int)ntask;
    pl.R = g.R; pl.S = g.S; pl.CB = CB;
    pl.steps = g.R * g.S * CB;
    pl.lds_bytes = lds;
    pl.wgs_per_cu = wgs;
    return true;
}

inline int device_cus() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    return cus;
}

template <typename TIn, typename TOut, int R, int S, int CB>
hipError_t launch_imp_one(const MfImpPlan& pl, const void* x, const void* aperm, const void* bias,
                          void* y, hipStream_t st) {
    void (*kfn)(const uint16_t*, const uint16_t*, const TIn*, TOut*, MfImpArgs) =
        conv_mfma_implicit_kernel<TIn, TOut, R, S, CB>;
    if (pl.lds_bytes > 65536 && allow_dynamic_lds(reinterpret_cast<const void*>(kfn), pl.lds_bytes) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kfn, dim3((uint32_t)pl.a.ntask), dim3(kThreads), pl.lds_bytes, st,
                       (const uint16_t*)x, (const uint16_t*)aperm, (const TIn*)bias, (TOut*)y, pl.a);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_imp_t(const MfImpPlan& pl, const void* x, const void* aperm, const void* bias,
                        void* y, hipStream_t st) {
    if (pl.R == 3) {
        switch (pl.CB) {
            case 1: return launch_imp_one<TIn, TOut, 3, 3, 1>(pl, x, aperm, bias, y, st);
            case 2: return launch_imp_one<TIn, TOut, 3, 3, 2>(pl, x, aperm, bias, y, st);
            case 3: return launch_imp_one<TIn, TOut, 3, 3, 3>(pl, x, aperm, bias, y, st);
            default: return launch_imp_one<TIn, TOut, 3, 3, 4>(pl, x, aperm, bias, y, st);
        }
    }
    switch (pl.CB) {
        case 1: return launch_imp_one<TIn, TOut, 1, 1, 1>(pl, x, aperm, bias, y, st);
        case 2: return launch_imp_one<TIn, TOut, 1, 1, 2>(pl, x, aperm, bias, y, st);
        default: return launch_imp_one<TIn, TOut, 1, 1, 4>(pl, x, aperm, bias, y, st);
    }
}

}  // namespace
}  // namespace ciw
