// conv_mfma_impl.hpp -- fp16/bf16 windowed contraction on the gfx950 matrix
// cores: kernels, row-kernel plan and launchers (templates).  Included by
// conv_mfma.hip (entry points, filter prep) and by one file per input type,
// which instantiate the kernels, so the two compile in parallel.
//
// The im2win paper ("Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support ...", §III-D) maps the output to a matrix product
// with M = output channels and N = images x output rows x output columns,
// reducing over the window.  With the HWC window layout the window of output
// (n, h, w) is, for each filter column q, the R*C contiguous elements at
// column w*stride_w + q*dil_w of row (n, h); with dil_w = 1 the whole window
// (S*R*C elements) is one contiguous run.  The reduction index is
// t = (q*R + r)*C + c and the filter operand is F[k][c][r][q] (the filter
// height index varies before the width, §III-C).  Products are exact in fp32 and accumulate in fp32
// (§III-F); the bias is added in fp32 and the result rounded once.
#pragma once

#include <algorithm>

#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMB = 64;       // output channels per workgroup
constexpr int kNB = 64;       // pixels per workgroup
constexpr int kKB = 32;       // reduction step (one 16x16x32 MFMA)
constexpr int kLdsRow = 40;   // 32 + 8 halves: rows 80 B apart

struct MfmaArgs {
    int C, K, R, S, P, Q, sw, dw, pitch;
    int T, RC, npix;                // npix: GEMM columns (4 per output with the pool)
    int relu, pool, Po, Qo;         // epilogue; output extent
    FastDiv fdRC, fdC, fdPQo, fdQo;
};

// Bias, then the optional ReLU (maxNum against 0).
__device__ __forceinline__ float act(float v, float b, int relu) {
    v += b;
    return relu ? fmaxf(v, 0.f) : v;
}

template <typename TIn>
__device__ __forceinline__ f32x4 mfma16x16x32(const uint16_t* a, const uint16_t* b, f32x4 acc);

template <>
__device__ __forceinline__ f32x4 mfma16x16x32<half_t>(const uint16_t* a, const uint16_t* b,
                                                      f32x4 acc) {
    f16x8 va = *reinterpret_cast<const f16x8*>(a);
    f16x8 vb = *reinterpret_cast<const f16x8*>(b);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(va, vb, acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mfma16x16x32<bf16_t>(const uint16_t* a, const uint16_t* b,
                                                      f32x4 acc) {
    bf16x8 va = *reinterpret_cast<const bf16x8*>(a);
    bf16x8 vb = *reinterpret_cast<const bf16x8*>(b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, vb, acc, 0, 0, 0);
}

// Generic tile kernel: 64 output channels x 64 pixels per workgroup, four
// waves each owning a 32x32 quadrant (2x2 MFMA tiles).  Operands go through
// LDS one 32-wide reduction step at a time.  With the 2x2 max-pool, GEMM
// column 4 o + d is pixel d of output o's region, so a region lies in four
// neighbouring lanes and two lane exchanges give its max.
template <typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads) void conv_mfma_generic_kernel(
    const uint16_t* __restrict__ xw, const uint16_t* __restrict__ w,
    const TIn* __restrict__ bias, TOut* __restrict__ y, MfmaArgs a) {
    __shared__ __align__(16) uint16_t As[kMB * kLdsRow];
    __shared__ __align__(16) uint16_t Bs[kNB * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int k0 = blockIdx.y * kMB;
    const int p0 = blockIdx.x * kNB;

    // loader role: row (filter or pixel) and 8-element slot of the step
    const int lrow = tid >> 2;
    const int lslot = (tid & 3) * 8;
    const int kload = k0 + lrow;
    const int pload = p0 + lrow;
    // per-thread window base of its pixel (index precomputation)
    int64_t bbase = -1;
    if (pload < a.npix) {
        const int side = a.pool ? 2 : 1;
        const uint32_t o = a.pool ? (uint32_t)pload >> 2 : (uint32_t)pload;   // output index
        uint32_t n = fdiv(o, a.fdPQo);
        int opix = o - n * (a.Po * a.Qo);
        int h2 = fdiv(opix, a.fdQo);
        int w2 = opix - h2 * a.Qo;
        int h = h2 * side + (a.pool ? (pload >> 1) & 1 : 0);
        int wo = w2 * side + (a.pool ? pload & 1 : 0);
        bbase = ((int64_t)n * a.P + h) * a.pitch + (int64_t)wo * a.sw * a.RC;
    }

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wm = wave >> 1, wn = wave & 1;
    for (int t0 = 0; t0 < a.T; t0 += kKB) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int t = t0 + lslot + i;
            uint16_t av = 0, bv = 0;
            if (t < a.T) {
                uint32_t q = fdiv(t, a.fdRC);
                int rc = t - q * a.RC;
                uint32_t r = fdiv(rc, a.fdC);
                int c = rc - r * a.C;
                if (kload < a.K) av = w[(((int64_t)kload * a.C + c) * a.R + r) * a.S + q];
                if (bbase >= 0) bv = xw[bbase + (int64_t)q * a.dw * a.RC + rc];
            }
            As[lrow * kLdsRow + lslot + i] = av;
            Bs[lrow * kLdsRow + lslot + i] = bv;
        }
        __syncthreads();
        const int kq = (lane >> 4) * 8;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                acc[mi][ni] = mfma16x16x32<TIn>(
                    &As[(wm * 32 + mi * 16 + (lane & 15)) * kLdsRow + kq],
                    &Bs[(wn * 32 + ni * 16 + (lane & 15)) * kLdsRow + kq], acc[mi][ni]);
        __syncthreads();
    }

    // epilogue: lane holds D[4*(lane/16) + i][lane % 16] of each 16x16 tile
    const int PQo = a.Po * a.Qo;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int p = p0 + wn * 32 + ni * 16 + (lane & 15);
        const uint32_t o = a.pool ? (uint32_t)p >> 2 : (uint32_t)p;
        // every lane takes part in the exchanges; a region's four columns
        // are all in range or all out (npix is a multiple of 4)
        const bool store = p < a.npix && (!a.pool || (lane & 3) == 0);
        uint32_t n = fdiv(o, a.fdPQo);
        int opix = o - n * PQo;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = k0 + wm * 32 + mi * 16 + (lane >> 4) * 4 + i;
                float v = act(acc[mi][ni][i], (bias && k < a.K) ? to_f32(bias[k]) : 0.f, a.relu);
                if (a.pool) {
                    v = fmaxf(v, __shfl_xor(v, 1));
                    v = fmaxf(v, __shfl_xor(v, 2));
                }
                if (store && k < a.K) y[((int64_t)n * a.K + k) * PQo + opix] = from_f32<TOut>(v);
            }
    }
}

// ------------------------------------------------------------ row kernel
// Persistent kernel for layers whose filter fits in registers (K <= 64,
// padded reduction <= 640 per phase set).  The GEMM view is the paper's
// (§III-D), output pixels x output channels reduced over the window.  One
// workgroup owns whole window rows (n, h):
//   - each of its four waves keeps the filter fragments of 32 output
//     channels over the whole padded reduction in registers for the life of
//     the kernel;
//   - window rows stream through a ring of LDS buffers, copied from global
//     memory straight into LDS several rows ahead of the row being
//     multiplied (load/compute overlap, §III-D/§III-E);
//   - the window of pixel w is the run of LDS chunks starting at w*D, D =
//     stride_w*R*C, so consecutive pixels read overlapping runs and each
//     window element crosses HBM once per output row (overlapping windows
//     reuse inputs already in cache, the im2win paper §III-C);
//   - the window fragment is the MFMA's first operand, so a lane ends up
//     holding 16 pixels of one output channel, four of them adjacent; they
//     go through an LDS tile so each output row leaves with whole-vector
//     stores.
// Alignment: a window fragment is a 16-byte LDS read, so its start must be
// a multiple of 8 elements.  Pixels are grouped into `nph` phases (w mod
// nph, nph = 8 / gcd(D, 8)) whose window starts share one misalignment
// delta; each phase multiplies a copy of the filter shifted right by delta,
// and reads start delta elements early.  Reduction entries outside the
// window (the shift, the padding to a multiple of 16) are zero in the filter
// and masked to zero in the window fragment, so values outside a window
// never reach a stored output.
// Bank conflicts: the 32 pixels of a fragment start G = D*nph/8 chunks
// apart.  With nph > 1, G is odd and consecutive lanes fall in distinct
// banks.  With nph = 1 the row is stored with one pad chunk after every PAD
// chunks (PAD the largest power of two dividing G, at most 8), which makes
// the lane stride G + G/PAD odd; every run starts on the pad grid, so the
// offset of each reduction step is a compile-time constant.
// Ablation switches of the row kernel (compile definitions; the library is
// built with all of them 0, the ablation variants each set one).  Each
// changes when or how data moves, never the order of a sum:
//   CIW_ABLATE_ROWS_NO_DOUBLE: one row buffer; each row is copied at the
//     iteration that multiplies it and waited for (no copy-ahead).
//   CIW_ABLATE_ROWS_NO_ASYNC: rows go global memory -> registers -> LDS
//     instead of the direct global-to-LDS copy.
//   CIW_ABLATE_ROWS_NO_PAD: no pad chunks in the LDS rows, so with one
//     pixel phase the lanes of a fragment read the same banks (the
//     bank-conflict avoidance that the im2win paper's zig-zag order serves).
//   CIW_ABLATE_ROWS_NO_INDEX: no precomputed indices: plain divisions
//     instead of the multiply-shift ones, and no filter re-layout kernel --
//     each lane gathers its filter fragments from the KCRS filter itself,
//     computing every element's (channel, filter row, filter column).
#ifndef CIW_ABLATE_ROWS_NO_DOUBLE
#define CIW_ABLATE_ROWS_NO_DOUBLE 0
#endif
#ifndef CIW_ABLATE_ROWS_NO_ASYNC
#define CIW_ABLATE_ROWS_NO_ASYNC 0
#endif
#ifndef CIW_ABLATE_ROWS_NO_PAD
#define CIW_ABLATE_ROWS_NO_PAD 0
#endif
#ifndef CIW_ABLATE_ROWS_NO_INDEX
#define CIW_ABLATE_ROWS_NO_INDEX 0
#endif
// The ablation variants are timed and checked on one layer (fp16 in and
// out, 3x3, 64 -> 64 channels, stride 1, no pool); CIW_ROWS_ABLATION_ONLY
// builds only the row-kernel forms that layer uses (one pixel phase, 36
// steps, no masks) and turns every other plan down with
// hipErrorNotSupported, which keeps the variant builds short.
#ifndef CIW_ROWS_ABLATION_ONLY
#define CIW_ROWS_ABLATION_ONLY 0
#endif

struct MfRowArgs {
    int C, K, R, S, P, Q, pitch;   // pitch: window row pitch (elements)
    int D, T;                      // window start stride, window length
    int nph, mblocks;              // pixel phases (1, 2, 4 or 8), 32-pixel blocks per phase
    int nph_log2;
    int G;                         // chunks between window starts (nph == 1)
    int nchunks;                   // 16-byte chunks of a window row
    int copy_chunks;               // LDS chunk positions of a row (pads included)
    int buf_elems;                 // elements per LDS row buffer
    int nbuf;                      // row buffers in the LDS ring
    int nd;                        // row-copy instructions per thread per row
    int ostride;                   // LDS output tile row stride (elements of TOut)
    int vec_store;                 // output rows are whole 16-byte vectors
    int ns;                        // output store instructions per thread per output row
    int rows;                      // row units: N * P, or N * 2 (P / 2) with the pool
    int relu, pool;                // epilogue
    int Po, Qo;                    // output extent (P / 2 x Q / 2 with the pool)
    FastDiv fdPo;
};

constexpr int kMfMaxChunks = 8;    // 16-byte chunks per thread per row copy
constexpr int kPf = 4;             // window fragments read ahead of the multiplies

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename TIn>
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, f32x16 acc);

template <>
__device__ __forceinline__ f32x16 mfma32<half_t>(const uint4& a, const uint4& b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma32<bf16_t>(const uint4& a, const uint4& b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// The window chunk whose copy LDS position q holds: one pad position after
// every PAD chunks, filled with the chunk before it.
template <int PAD>
__device__ __forceinline__ int pad_src(int q) {
    if (PAD == 1) return q;
    const int grp = q / (PAD + 1);
    return grp * PAD + min(q - grp * (PAD + 1), PAD - 1);
}

// Byte offset of reduction step s within a run: 32 bytes a step plus one
// pad chunk for every PAD chunks passed.
template <int PAD>
__device__ constexpr int step_off(int s) {
    return PAD == 1 ? 32 * s : 32 * s + 16 * ((2 * s) / PAD);
}

// Mask of the 8 elements [t0, t0 + 8) that lie inside [lo, hi).
__device__ __forceinline__ uint4 elem_mask(int t0, int lo, int hi) {
    uint32_t m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 2 * i;
        m[i] = ((t >= lo && t < hi) ? 0xffffu : 0u) | ((t + 1 >= lo && t + 1 < hi) ? 0xffff0000u : 0u);
    }
    return make_uint4(m[0], m[1], m[2], m[3]);
}

// Two outputs rounded to a 16-bit type and packed into one word (the
// hardware's packed round-to-nearest-even conversions).
template <typename TOut>
__device__ __forceinline__ uint32_t pack2(float a0, float a1);

template <>
__device__ __forceinline__ uint32_t pack2<half_t>(float a0, float a1) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a0, a1}, f16x2));
}

template <>
__device__ __forceinline__ uint32_t pack2<bf16_t>(float a0, float a1) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a0, a1}, bf16x2));
}

// Two adjacent outputs as one LDS write.
template <typename TOut>
__device__ __forceinline__ void put2(TOut* p, float a0, float a1) {
    *reinterpret_cast<uint32_t*>(p) = pack2<TOut>(a0, a1);
}

template <>
__device__ __forceinline__ void put2<float>(float* p, float a0, float a1) {
    *reinterpret_cast<float2*>(p) = make_float2(a0, a1);
}

// Four adjacent outputs as one LDS write (8 bytes of halves, 16 of floats).
template <typename TOut>
__device__ __forceinline__ void put4(TOut* p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2<TOut>(a0, a1), pack2<TOut>(a2, a3));
}

template <>
__device__ __forceinline__ void put4<float>(float* p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<float4*>(p) = make_float4(a0, a1, a2, a3);
}

// maxNum of two floats as one v_max_f32.  fmaxf would first quiet both
// operands (two more instructions each), which only matters for signaling
// NaNs; the values here are results of arithmetic or stored outputs, whose
// NaNs are quiet.
__device__ __forceinline__ float max_q(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// The two 16-bit outputs of a packed word, as floats (exact).
template <typename TOut>
__device__ __forceinline__ float2 unpack2(uint32_t u);

template <>
__device__ __forceinline__ float2 unpack2<half_t>(uint32_t u) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 h = __builtin_bit_cast(f16x2, u);
    return make_float2((float)h[0], (float)h[1]);
}

template <>
__device__ __forceinline__ float2 unpack2<bf16_t>(uint32_t u) {
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}

// Two / four adjacent tile outputs read back as floats.
template <typename TOut>
__device__ __forceinline__ float2 get2(const TOut* p) {
    return unpack2<TOut>(*reinterpret_cast<const uint32_t*>(p));
}

template <>
__device__ __forceinline__ float2 get2<float>(const float* p) {
    return *reinterpret_cast<const float2*>(p);
}

template <typename TOut>
__device__ __forceinline__ float4 get4(const TOut* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const float2 a = unpack2<TOut>(u.x), b = unpack2<TOut>(u.y);
    return make_float4(a.x, a.y, b.x, b.y);
}

template <>
__device__ __forceinline__ float4 get4<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}

// 2x2 pooling, horizontal half: 2V adjacent outputs (the 16-byte vectors lo,
// hi) to the V maxima of their pairs, each also maxed with `lo3` (0 for the
// ReLU, or a quiet NaN, which maxNum ignores).  Values come from the output
// type, so converting a maximum back is exact.
template <typename TOut>
__device__ __forceinline__ uint4 pool_pairs(uint4 lo, uint4 hi, float lo3) {
    auto word = [&](uint32_t u0, uint32_t u1) {
        const float2 a = unpack2<TOut>(u0), b = unpack2<TOut>(u1);
        return pack2<TOut>(max_q(max_q(a.x, a.y), lo3), max_q(max_q(b.x, b.y), lo3));
    };
    return make_uint4(word(lo.x, lo.y), word(lo.z, lo.w), word(hi.x, hi.y), word(hi.z, hi.w));
}

template <>
__device__ __forceinline__ uint4 pool_pairs<float>(uint4 lo, uint4 hi, float lo3) {
    auto m = [&](uint32_t a, uint32_t b) {
        return __float_as_uint(max_q(max_q(__uint_as_float(a), __uint_as_float(b)), lo3));
    };
    return make_uint4(m(lo.x, lo.y), m(lo.z, lo.w), m(hi.x, hi.y), m(hi.z, hi.w));
}

// ReLU of one 16-byte vector of outputs.
template <typename TOut>
__device__ __forceinline__ uint4 relu_vec(uint4 v) {
    auto word = [](uint32_t u) {
        const float2 a = unpack2<TOut>(u);
        return pack2<TOut>(max_q(a.x, 0.f), max_q(a.y, 0.f));
    };
    return make_uint4(word(v.x), word(v.y), word(v.z), word(v.w));
}

template <>
__device__ __forceinline__ uint4 relu_vec<float>(uint4 v) {
    auto m = [](uint32_t a) { return __float_as_uint(max_q(__uint_as_float(a), 0.f)); };
    return make_uint4(m(v.x), m(v.y), m(v.z), m(v.w));
}

// s_waitcnt with a run-time vector-memory count (the instruction takes an
// immediate): wait until at most n of this wave's vector memory operations
// are outstanding and all its LDS operations are done.
__device__ __forceinline__ void wait_vm_lgkm(int n) {
    asm volatile("" ::: "memory");
    switch (n < 0 ? 0 : (n > 63 ? 63 : n)) {
#define CIW_WAIT_CASE(k) \
    case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | (7 << 4) | (0 << 8)); break;
#define CIW_WAIT_CASE8(b) CIW_WAIT_CASE(b) CIW_WAIT_CASE(b + 1) CIW_WAIT_CASE(b + 2) CIW_WAIT_CASE(b + 3) \
    CIW_WAIT_CASE(b + 4) CIW_WAIT_CASE(b + 5) CIW_WAIT_CASE(b + 6) CIW_WAIT_CASE(b + 7)
        CIW_WAIT_CASE8(0) CIW_WAIT_CASE8(8) CIW_WAIT_CASE8(16) CIW_WAIT_CASE8(24)
        CIW_WAIT_CASE8(32) CIW_WAIT_CASE8(40) CIW_WAIT_CASE8(48) CIW_WAIT_CASE8(56)
#undef CIW_WAIT_CASE8
#undef CIW_WAIT_CASE
    }
    asm volatile("" ::: "memory");
}

// Wait for this wave's LDS operations only.
__device__ __forceinline__ void wait_vm_lgkm_lds_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
}

// Workgroup barrier without the memory fence __syncthreads adds (the waits
// above are placed by hand so row copies can stay in flight across it).
__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wg_barrier_lds() {
    wait_vm_lgkm_lds_only();
    wg_barrier();
}

template <typename TIn, typename TOut, int NSET, int STEPS, bool MASK, int PAD, bool TAILLAST,
          bool POOL>
__global__ __launch_bounds__(kThreads, 2) void conv_mfma_rows_kernel(
    const uint16_t* __restrict__ xw, const uint16_t* __restrict__ aperm,
    const TIn* __restrict__ bias, TOut* __restrict__ y, MfRowArgs a) {
    extern __shared__ __align__(16) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int kh = wave & 1;          // output channels [32 kh, 32 kh + 32)
    const int pb0 = wave >> 1;        // block groups pb0, pb0 + 2, ... (see below)
    const int g = lane >> 5;          // which 8 of a fragment's 16 reduction entries
    const int ml = lane & 31;         // fragment row (pixel) / column (channel)
    const int npb = a.nph * a.mblocks;

    uint16_t* ring = lds;                                                 // nbuf x buf_elems
    TOut* otile0 = reinterpret_cast<TOut*>(lds + a.nbuf * a.buf_elems);  // 2 x K x ostride
    float* bias_l = reinterpret_cast<float*>(otile0 + 2 * a.K * a.ostride);   // 64 floats

    // ---- filter fragments, laid out by the prep kernel in fragment order
    // (phase-shifted, zero-padded): lane holds F[t = 16 s + 8 (lane / 32)
    // + 0..7][k = 32 kh + lane % 32], the second MFMA operand
    uint4 F[NSET][STEPS];
#pragma unroll
    for (int j = 0; j < NSET; ++j) {
        const int pb = min(pb0 * NSET + j, npb - 1);   // set j serves phase pb % nph
        if (CIW_ABLATE_ROWS_NO_INDEX) {
            // aperm is the KCRS filter: entry t of the fragment is filter
            // (k, c, r, q) with t - delta = (q R + r) C + c, by division
            const int dl = ((pb & (a.nph - 1)) * a.D) & 7;
            const int k = kh * 32 + ml;
#pragma clang loop unroll(full)
            for (int s2 = 0; s2 < STEPS; ++s2) {
                uint32_t d[4];
#pragma clang loop unroll(full)
                for (int e = 0; e < 8; ++e) {
                    const int t = 16 * s2 + 8 * g + e - dl;
                    uint32_t v = 0;
                    if (k < a.K && t >= 0 && t < a.T) {
                        const int qr = t / a.C, c = t % a.C;
                        const int q = qr / a.R, r = qr % a.R;
                        v = aperm[(((size_t)k * a.C + c) * a.R + r) * a.S + q];
                    }
                    if (e & 1) d[e >> 1] |= v << 16;
                    else d[e >> 1] = v;
                }
                // opaque from here on: kept in registers like the loaded
                // fragments, not recomputed where they are used
                asm volatile("" : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]));
                F[j][s2] = make_uint4(d[0], d[1], d[2], d[3]);
            }
            continue;
        }
        const uint16_t* fp = aperm + ((size_t)((pb & (a.nph - 1)) * 2 + kh) * STEPS * 64 + lane) * 8;
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2)
            F[j][s2] = *reinterpret_cast<const uint4*>(fp + 512 * s2);
    }
    if (tid < 64) bias_l[tid] = (bias && tid < a.K) ? to_f32(bias[tid]) : 0.f;
    // complete these loads now: the wait counts below cover only row copies
    // and output stores
#pragma unroll
    for (int j = 0; j < NSET; ++j)
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2) asm volatile("" ::"v"(F[j][s2].x));
    wait_vm_lgkm(0);

    // ---- window rows: global -> LDS directly (no registers), into a ring of
    // nbuf row buffers, nbuf - 1 rows ahead of the row being multiplied.
    // Every wave issues exactly a.nd copy instructions per row, so the
    // number of this wave's memory operations after any row's copy is known.
    // Copy instruction j fills LDS positions [256 j, 256 j + 256); the last
    // one is moved back to end at the row's last position (positions it
    // shares with the one before receive the same chunk twice).  A lane's
    // source offsets do not depend on the row and are computed once.
    uint32_t src_off[kMfMaxChunks];
    int pos_base[kMfMaxChunks];
#pragma unroll
    for (int j = 0; j < kMfMaxChunks; ++j) {
        pos_base[j] = (j == a.nd - 1 && a.nd > 1) ? a.copy_chunks - kThreads : j * kThreads;
        const int q = min(pos_base[j] + tid, a.copy_chunks - 1);
        src_off[j] = 16u * (uint32_t)min(pad_src<PAD>(q), a.nchunks - 1);
    }
    // The copies are issued as inline asm: the compiler then neither counts
    // them nor makes the LDS reads that follow wait for every copy in flight
    // (it would drain the ring before each row); the hand-placed waits below
    // order them instead.  M0 holds the wave's LDS destination (lane i writes
    // 16 bytes at M0 + 16 i); the source is the row base (scalar) plus a
    // 32-bit byte offset per lane.
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)ring;
    // Row units: window rows in order, or with the pool the two rows 2j,
    // 2j + 1 of each pooled output row (n, j) = u / 2 (an odd last row of
    // an image reaches no output and is skipped).
    auto window_row = [&](int u) -> int {
        if (!POOL) return u;
        const uint32_t pr = (uint32_t)u >> 1;
        const uint32_t n = CIW_ABLATE_ROWS_NO_INDEX ? pr / (uint32_t)a.Po : fdiv(pr, a.fdPo);
        return (int)(n * a.P + 2 * (pr - n * a.Po)) + (u & 1);
    };
    auto copy_row = [&](int u, int buf) {
        const uint16_t* src = xw + (size_t)window_row(u) * a.pitch;
        const uint32_t dst0 = ring_lds + 2u * (uint32_t)(buf * a.buf_elems) + 1024u * (uint32_t)wave;
#pragma unroll
        for (int j = 0; j < kMfMaxChunks; ++j) {
            if (j < a.nd) {
                if (CIW_ABLATE_ROWS_NO_ASYNC) {
                    // through registers, to the position the direct copy writes
                    const uint4 v = *reinterpret_cast<const uint4*>(
                        reinterpret_cast<const char*>(src) + src_off[j]);
                    *reinterpret_cast<uint4*>(ring + buf * a.buf_elems + 8 * (pos_base[j] + tid)) = v;
                    continue;
                }
                const uint32_t dst = __builtin_amdgcn_readfirstlane(dst0 + 16u * (uint32_t)pos_base[j]);
                asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
                             :: "v"(src_off[j]), "s"(dst), "s"(src) : "memory");
            }
        }
    };

    // each workgroup takes a contiguous run of rows: neighbouring output
    // rows share cache lines, and one workgroup writing them back to back
    // completes those lines while they are still in L2.  With the pool the
    // run is whole pairs, so both rows of a region meet in one workgroup.
    const int unit = POOL ? 2 : 1;                       // row units per output row
    const int groups = a.rows / unit;
    const int per = (groups + (int)gridDim.x - 1) / (int)gridDim.x;
    const int first = blockIdx.x * per * unit;
    if (first >= a.rows) return;
    const int my_rows = min(per * unit, a.rows - first);  // units first .. first + my_rows - 1
    for (int i = 0; i < a.nbuf - 1 && i < my_rows; ++i) copy_row(first + i, i);
    wg_barrier_lds();                // bias_l visible
    const float bias_k = bias_l[kh * 32 + ml];
    // Small filter sets leave registers for two kernel-lifetime helpers: the
    // bias splat, which seeds the accumulators (the first multiply adds onto
    // it, no separate add), and each set's edge masks, which depend only on
    // its phase and so are built once here instead of every row.
    constexpr bool kLean = NSET * STEPS <= 20;
    f32x16 bias_vec;
#pragma unroll
    for (int i = 0; i < 16; ++i) bias_vec[i] = kLean ? bias_k : 0.f;
    uint4 mkf[NSET], mkt[NSET];
    int sfj[NSET];
#pragma unroll
    for (int j = 0; j < NSET; ++j) {
        const int dj = (((pb0 * NSET + j) & (a.nph - 1)) * a.D) & 7;
        sfj[j] = (dj + a.T) / 16;
        mkf[j] = make_uint4(~0u, ~0u, ~0u, ~0u);
        mkt[j] = mkf[j];
        if (MASK && kLean) {
            mkf[j] = elem_mask(8 * g, dj, dj + a.T);
            mkt[j] = elem_mask(16 * (TAILLAST ? STEPS - 1 : sfj[j]) + 8 * g, dj, dj + a.T);
        }
    }

    // output stores: thread's first (k, column vector) and its step per 256
    // vectors, fixed for the kernel
    constexpr int V = 16 / sizeof(TOut);
    const int E = a.vec_store ? V : 1;          // elements per store
    const int nq = a.Qo / E;                    // stores per output row
    const int sk0 = tid / nq, sv0 = tid - sk0 * nq;
    const int dk = kThreads / nq, dv = kThreads - dk * nq;
    const int sc = POOL ? 2 : 1;                // tile columns per output column
    // ReLU is applied to the tile's values as they are stored (ReLU and
    // rounding are monotone, so this equals ReLU before rounding, and it
    // commutes with the pool's max).  With the pool it is a third operand of
    // the pair's max: 0, or a quiet NaN, which maxNum ignores.
    const float relu_lo = a.relu ? 0.f : __builtin_nanf("");

    // ---- output row (n, h) from a tile: K rows of Qo contiguous elements.
    // With the pool the tile already holds the max of the region's two rows
    // and each output is the max of two neighbouring tile columns.
    // Exactly a.ns stores per thread (surplus threads repeat the last one);
    // each tile read is issued one store ahead of its use.
    const int PQo = a.Po * a.Qo;
    auto store_row = [&](int orow_idx, const TOut* tl) {
        const uint32_t n = CIW_ABLATE_ROWS_NO_INDEX ? (uint32_t)orow_idx / (uint32_t)a.Po
                                                    : fdiv(orow_idx, a.fdPo);
        const int h = orow_idx - n * a.Po;
        TOut* yrow = y + (size_t)n * a.K * PQo + (size_t)h * a.Qo;
        int k = sk0, v = sv0;
        // element offsets of store j in the tile (src) and in the output row
        // block (dst); advance to store j + 1
        int src, dst_k, dst_off;
        auto take = [&]() {
            const int kk = min(k, a.K - 1);
            dst_off = kk < k ? (a.Qo - E) : v * E;
            dst_k = kk;
            src = kk * a.ostride + sc * dst_off;
            k += dk;
            v += dv;
            if (v >= nq) {
                v -= nq;
                ++k;
            }
        };
        auto vec_at = [&](int i) {
            const uint4 lo = *reinterpret_cast<const uint4*>(tl + i);
            if (POOL) return pool_pairs<TOut>(lo, *reinterpret_cast<const uint4*>(tl + i + V), relu_lo);
            return a.relu ? relu_vec<TOut>(lo) : lo;
        };
        auto elem_at = [&](int i) {
            if (POOL) return from_f32<TOut>(max_q(max_q(to_f32(tl[i]), to_f32(tl[i + 1])), relu_lo));
            return a.relu ? from_f32<TOut>(max_q(to_f32(tl[i]), 0.f)) : tl[i];
        };
        take();
        if (a.vec_store) {
            uint4 cur = vec_at(src);
            for (int j = 0; j < a.ns; ++j) {
                TOut* dp = yrow + (size_t)dst_k * PQo + dst_off;
                uint4 nxt = cur;
                if (j + 1 < a.ns) {
                    take();
                    nxt = vec_at(src);
                }
                *reinterpret_cast<uint4*>(dp) = cur;
                cur = nxt;
            }
        } else {
            TOut cur = elem_at(src);
            for (int j = 0; j < a.ns; ++j) {
                TOut* dp = yrow + (size_t)dst_k * PQo + dst_off;
                TOut nxt = cur;
                if (j + 1 < a.ns) {
                    take();
                    nxt = elem_at(src);
                }
                *dp = cur;
                cur = nxt;
            }
        }
    };

    // Iteration it: wait for row it's copy, barrier, copy row it + nbuf - 1
    // into the buffer row it - 1 used (every wave is past it now), store
    // row it - 1 from its tile, then multiply row it into the other tile.
    // The stores thus overlap the next row's multiplies, and the barrier
    // that makes row it visible also makes tile it - 1 complete.  With the
    // pool a tile serves a pair of rows: the first writes it, the second
    // takes the max with it in place (each lane rewrites exactly the
    // entries it wrote), and the pair is stored while the next pair's first
    // row multiplies into the other tile.
    const int tile_elems = a.K * a.ostride;
    for (int it = 0; it < my_rows; ++it) {
        const int buf = it % a.nbuf;
        // wait for this row's copy: allow the copies of the rows after it
        // and the output stores issued since it (in iterations lo .. it - 1;
        // a store follows every row, or every second row with the pool) to
        // stay in flight
        const int later_rows = min(a.nbuf - 2, my_rows - 1 - it);
        const int lo = max(it - a.nbuf + 1, 1);
        int later_stores = max(0, it - lo);
        if (POOL) {
            const int lo2 = max(lo, 2);
            later_stores = it - 1 >= lo2 ? (it - 1) / 2 - (lo2 - 1) / 2 : 0;
        }
        if (CIW_ABLATE_ROWS_NO_DOUBLE) {
            // one buffer: once every wave is done with row it - 1, copy row
            // it into it and wait for the copy
            if (it > 0) wg_barrier();
            copy_row(first + it, 0);
            wait_vm_lgkm(0);
        } else {
            wait_vm_lgkm(a.nd * later_rows + a.ns * later_stores);
        }
        wg_barrier();                // row it landed; the tile to store is complete and free
        if (!CIW_ABLATE_ROWS_NO_DOUBLE && it + a.nbuf - 1 < my_rows)
            copy_row(first + it + a.nbuf - 1, (it + a.nbuf - 1) % a.nbuf);
        if (!POOL) {
            if (it > 0) store_row(first + it - 1, otile0 + ((it - 1) & 1) * tile_elems);
        } else if (it >= 2 && (it & 1) == 0) {
            store_row((first + it) / 2 - 1, otile0 + (((it >> 1) - 1) & 1) * tile_elems);
        }
        TOut* otile = otile0 + (POOL ? (it >> 1) & 1 : it & 1) * tile_elems;
        const bool merge = POOL && (it & 1);   // second row of a pair

        const uint16_t* lb = ring + buf * a.buf_elems;
        // Pixel blocks pb = phase + nph * (32-pixel block): the wave takes
        // groups gi = pb0, pb0 + 2, ... of NSET consecutive blocks, block
        // gi * NSET + j with filter set j.  With NSET > 1 (nph = 2 NSET) a
        // group is NSET adjacent phases of one 32-pixel block, so blocks
        // j and j + 1 hold neighbouring pixels and their outputs go to the
        // tile in pairs.
        constexpr int kNph = NSET > 1 ? 2 * NSET : 1;   // nph when NSET > 1
        for (int base = 0; (pb0 + 2 * base) * NSET < npb; ++base) {
            f32x16 accp;   // block j - 1 of a pair, until block j is done
#pragma unroll
            for (int j = 0; j < NSET; ++j) {
            const int pb = (pb0 + 2 * base) * NSET + j;
            if (NSET == 1 && pb >= npb) break;
            const int ph = pb & (a.nph - 1);
            const int mb = pb >> a.nph_log2;
            const int delta = (ph * a.D) & 7;
            const int wpix = a.nph * (32 * mb + ml) + ph;
            // pixels past the row end (never stored) read the last pixel of
            // their phase instead, so reads stay inside the row buffer
            const int wlast = a.Q - 1 >= ph ? a.Q - 1 - ((a.Q - 1 - ph) & (a.nph - 1)) : ph;
            const int wread = min(wpix, wlast);
            // LDS chunk position of the lane's step-0 read: the window start
            // minus delta (a multiple of 8 elements), plus 8 elements for g
            const int run = PAD == 1 ? (wread * a.D - delta) / 8 + g
                                     : wread * (a.G + a.G / PAD) + g;
            const char* rp = reinterpret_cast<const char*>(lb + 8 * run);
            f32x16 acc = bias_vec;
            // window fragments kPf steps ahead of the multiply that uses them
            uint4 bq[kPf];
#pragma unroll
            for (int s2 = 0; s2 < kPf && s2 < STEPS; ++s2)
                bq[s2] = *reinterpret_cast<const uint4*>(rp + step_off<PAD>(s2));
            // Edge masks.  Step 0 holds the window start (entries below
            // delta are masked); step s_full holds its end (entries from
            // delta + T on are masked); later steps lie wholly past the end
            // and are zeroed; the steps between need no mask.  With TAILLAST
            // every phase ends in the last step, so only steps 0 and
            // STEPS - 1 are masked.  Without kLean the masks are rebuilt
            // every row from opaque copies of delta and s_full rather than
            // kept live across the row loop.
            uint4 mk_first = mkf[j], mk_tail = mkt[j];
            int sf = sfj[j];
            if (MASK && !kLean) {
                int dl = delta;
                sf = (delta + a.T) / 16;
                asm volatile("" : "+v"(dl));
                asm volatile("" : "+s"(sf));
                mk_first = elem_mask(8 * g, dl, dl + a.T);
                mk_tail = elem_mask(16 * (TAILLAST ? STEPS - 1 : sf) + 8 * g, dl, dl + a.T);
            }
#pragma unroll
            for (int s2 = 0; s2 < STEPS; ++s2) {
                uint4 b = bq[s2 % kPf];
                if (s2 + kPf < STEPS)
                    bq[s2 % kPf] = *reinterpret_cast<const uint4*>(rp + step_off<PAD>(s2 + kPf));
                if (MASK) {
                    if (s2 == 0) {
                        b.x &= mk_first.x; b.y &= mk_first.y; b.z &= mk_first.z; b.w &= mk_first.w;
                    }
                    if (TAILLAST) {
                        if (s2 == STEPS - 1) {
                            b.x &= mk_tail.x; b.y &= mk_tail.y; b.z &= mk_tail.z; b.w &= mk_tail.w;
                        }
                    } else {
                        // branch-free: keep all before s_full, the tail mask at it
                        const uint32_t keep = s2 < sf ? ~0u : 0u;
                        const uint32_t at = s2 == sf ? ~0u : 0u;
                        b.x &= keep | (at & mk_tail.x); b.y &= keep | (at & mk_tail.y);
                        b.z &= keep | (at & mk_tail.z); b.w &= keep | (at & mk_tail.w);
                    }
                }
                acc = mfma32<TIn>(b, F[j][s2], acc);
            }
            // keep the reads kPf multiplies ahead: the first reads, then one
            // multiply and one read per step
            __builtin_amdgcn_sched_group_barrier(0x100, kPf < STEPS ? kPf : STEPS, 0);
#pragma unroll
            for (int s2 = 0; s2 < STEPS; ++s2) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (s2 + kPf < STEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            // lane holds D[m][n] for channel n = lane % 32 and block pixel
            // m = 8 (i / 4) + 4 (lane / 32) + i % 4; pixels past the row end
            // land in tile columns that are never stored.  The bias is added
            // unless it seeded the sum (adding "+ 0" would not be free: the
            // compiler must keep it for the sign of a zero sum).  The second
            // row of a pooled pair reads back what the first wrote at the
            // same places, all reads before one wait.
            if (!kLean) {
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] += bias_k;
            }
            const int k = kh * 32 + ml;
            if (NSET == 1) {
                if (k < a.K) {
                    TOut* orow = otile + k * a.ostride + a.nph * 32 * mb + ph;
                    if (a.nph == 1) {
                        if (merge) {
                            asm volatile("" ::: "memory");   // keep the reads on this path
                            float4 o[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) o[q] = get4<TOut>(orow + 8 * q + 4 * g);
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                put4<TOut>(orow + 8 * q + 4 * g, max_q(acc[4 * q], o[q].x),
                                           max_q(acc[4 * q + 1], o[q].y), max_q(acc[4 * q + 2], o[q].z),
                                           max_q(acc[4 * q + 3], o[q].w));
                        } else {
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                put4<TOut>(orow + 8 * q + 4 * g, acc[4 * q], acc[4 * q + 1],
                                           acc[4 * q + 2], acc[4 * q + 3]);
                        }
                    } else {
                        auto at = [&](int i) { return orow + a.nph * (8 * (i >> 2) + 4 * g + (i & 3)); };
                        if (merge) {
                            asm volatile("" ::: "memory");
                            float o[16];
#pragma unroll
                            for (int i = 0; i < 16; ++i) o[i] = to_f32(*at(i));
#pragma unroll
                            for (int i = 0; i < 16; ++i) *at(i) = from_f32<TOut>(max_q(acc[i], o[i]));
                        } else {
#pragma unroll
                            for (int i = 0; i < 16; ++i) *at(i) = from_f32<TOut>(acc[i]);
                        }
                    }
                }
            } else if ((j & 1) == 0) {
                accp = acc;
            } else if (k < a.K) {
                // blocks j - 1 and j: phases ph - 1 and ph, neighbouring pixels
                TOut* orow = otile + k * a.ostride + kNph * (32 * mb + 4 * g) + ph - 1;
                auto at = [&](int i) { return orow + kNph * (8 * (i >> 2) + (i & 3)); };
                if (merge) {
                    asm volatile("" ::: "memory");
                    float2 o[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[i] = get2<TOut>(at(i));
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        put2<TOut>(at(i), max_q(accp[i], o[i].x), max_q(acc[i], o[i].y));
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) put2<TOut>(at(i), accp[i], acc[i]);
                }
            }
            }
        }
    }
    // the last row's (pair's) tile
    wait_vm_lgkm_lds_only();
    wg_barrier();
    if (POOL)
        store_row((first + my_rows) / 2 - 1, otile0 + (((my_rows >> 1) - 1) & 1) * tile_elems);
    else
        store_row(first + my_rows - 1, otile0 + ((my_rows - 1) & 1) * tile_elems);
}

// Filter layout for the row kernel, in the order the A fragments are
// loaded: aperm[ph][kh][s][lane][e] holds filter entry (k, t') with
// k = 32 kh + lane % 32 and t' = 16 s + 8 (lane / 32) + e, so one wave's
// load of a whole step is 1 KB of consecutive bytes.  Entry (k, t') is
// F[k][c][r][q] at window-order index t = t' - delta(ph) = (q*R + r)*C + c
// when 0 <= t < T and k < K, else 0 (phase shift and zero padding).
struct PermArgs {
    int C, K, R, S, D, T, steps;
    FastDiv fdSteps, fdC, fdR;
    uint32_t total;                // nph * 2 * steps * 512
};

__global__ __launch_bounds__(kThreads) __attribute__((unused)) void mfma_filter_perm_kernel(
    const uint16_t* __restrict__ w, uint16_t* __restrict__ aperm, PermArgs p) {
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= p.total) return;
    const int e = i & 7;
    const int lane = (i >> 3) & 63;
    const uint32_t rest = i >> 9;                 // (ph * 2 + kh) * steps + s
    const uint32_t phk = fdiv(rest, p.fdSteps);
    const int s = rest - phk * p.steps;
    const int kh = phk & 1;
    const int ph = phk >> 1;
    const int k = kh * 32 + (lane & 31);
    const int t = 16 * s + 8 * (lane >> 5) + e - ((ph * p.D) & 7);
    uint16_t v = 0;
    if (k < p.K && t >= 0 && t < p.T) {
        const uint32_t qr = fdiv(t, p.fdC);
        const int c = t - qr * p.C;
        const uint32_t q = fdiv(qr, p.fdR);
        const int r = qr - q * p.R;
        v = w[(((size_t)k * p.C + c) * p.R + r) * p.S + q];
    }
    aperm[i] = v;
}

struct MfRowPlan {
    MfRowArgs a;
    int nset, steps, pad;
    bool mask, tail_last;
    size_t lds_bytes;
    int wgs_per_cu;
};

int gcd_int(int x, int y) {
    while (y) {
        int t = x % y;
        x = y;
        y = t;
    }
    return x;
}

// Row-kernel plan; false when the layer does not fit it.  Whether a layer
// fits without the epilogue decides whether the filter is re-laid out, so
// an epilogue may only turn a fitting plan down (to the generic kernel),
// never accept one the plain plan rejects.
[[maybe_unused]] bool mf_row_plan(const Geom& g, int out_bytes, MfRowPlan& pl, const Epi& epi = Epi{}) {
    if (g.K > 64 || g.dw != 1) return false;
    MfRowArgs& a = pl.a;
    // window start stride and length in elements, in 64 bits (a huge
    // horizontal stride is legal); a window row must fit LDS anyway
    const int64_t D64 = (int64_t)g.sw * g.R * g.C, T64 = (int64_t)g.S * g.R * g.C;
    if (D64 > (1 << 20) || T64 > (1 << 20)) return false;
    const int D = (int)D64;
    const int T = (int)T64;
    const int nph = 8 / gcd_int(D, 8);
    int maxdelta = 0;
    for (int ph = 0; ph < nph; ++ph) maxdelta = std::max(maxdelta, (ph * D) & 7);
    const int need = (T + maxdelta + 15) / 16;
    const int nset = nph == 1 ? 1 : nph / 2;
    // compiled step counts (a few more steps than needed only cost MFMAs
    // on zero filter entries)
    int steps = 0;
    for (int c : {10, 16, 24, 36, 40})
        if (c >= need) {
            steps = c;
            break;
        }
    if (steps == 0 || nset * steps > 40) return false;
    // masking is needed unless every step lies wholly inside the window;
    // tail_last: every phase's window ends in the last step
    const bool mask = maxdelta > 0 || T != 16 * steps;
    bool tail_last = true;
    for (int ph = 0; ph < nph; ++ph) tail_last = tail_last && ((ph * D) & 7) + T >= 16 * (steps - 1);
    const int mcount = (g.Q + nph - 1) / nph;
    const int mblocks = (mcount + 31) / 32;
    const int nchunks = g.pitchB / 8;
    // row layout: with nph > 1 the lanes of a fragment start an odd number
    // of chunks apart (D * nph / 8 = D / gcd(D, 8)); with nph = 1 they start
    // G = D / 8 chunks apart and a pad chunk after every PAD chunks (PAD the
    // power-of-two part of G, at most 8) makes the stride G + G / PAD odd
    const int G = nph == 1 ? D / 8 : 0;
    int pad = 1;
    if (nph == 1 && !CIW_ABLATE_ROWS_NO_PAD)
        while (pad < 8 && G % (2 * pad) == 0) pad *= 2;
    const int stride = pad == 1 ? D * nph / 8 : G + G / pad;   // chunks between lane starts
    const int copy_chunks = pad == 1 ? nchunks : (nchunks + pad - 1) / pad * (pad + 1);
    if (copy_chunks > kMfMaxChunks * kThreads) return false;
    const int nd = (copy_chunks + kThreads - 1) / kThreads;
    // the furthest LDS chunk a fragment read touches: the last pixel's run
    // over the whole padded reduction (a run starts at the pixel's stride
    // position; g adds one chunk; each step two, plus the pads passed)
    const int wmax = std::max(g.Q - 1, nph - 1);
    const int run_end = 1 + 2 * (steps - 1) + (pad == 1 ? 0 : (2 * (steps - 1)) / pad);
    const int last_chunk = (pad == 1 ? (wmax * D) / 8 : wmax * stride) + run_end;
    // one copy instruction covers 256 positions, so a row shorter than that
    // still takes 256
    int buf_chunks = std::max(std::max(copy_chunks, last_chunk + 1), nd == 1 ? kThreads : 0);
    buf_chunks = (buf_chunks + 15) / 16 * 16;
    const int buf = buf_chunks * 8;
    // output tile: every pixel of every block has a column (pixels past the
    // row end are written but never stored); an odd number of 16-byte units
    // per row spreads the channel rows of a tile write over the banks
    const int V = 16 / out_bytes;
    int ostride = (nph * 32 * mblocks + V - 1) / V * V;
    if (((ostride * out_bytes) / 16) % 2 == 0) ostride += V;
    // two tiles: row it - 1 is stored from one while row it fills the other
    const size_t tile = 2 * (size_t)g.K * ostride * out_bytes + 64 * 4;
    // workgroups per CU, then ring depth, within the 160 KB of LDS of a CU:
    // two workgroups (two waves per SIMD, one multiplying while the other
    // waits at a barrier or stores) beat one with a deeper ring
    int nbuf = 0, wgs = 0;
    for (int w = 2; w >= 1 && nbuf == 0; --w)
        for (int nb = CIW_ABLATE_ROWS_NO_DOUBLE ? 1 : 6; nb >= (CIW_ABLATE_ROWS_NO_DOUBLE ? 1 : 2); --nb)
            if (((size_t)nb * buf * 2 + tile) * w <= 160 * 1024) {
                nbuf = nb;
                wgs = w;
                break;
            }
    if (nbuf == 0) return false;
    // stores per thread of an output row of Qo columns (16-byte vectors when
    // every output row starts on a vector)
    auto stores = [&](int Po, int Qo, int& vec) {
        vec = (Qo % V == 0 && ((int64_t)Po * Qo) % V == 0) ? 1 : 0;
        const int64_t total = vec ? (int64_t)g.K * (Qo / V) : (int64_t)g.K * Qo;
        return (int)((total + kThreads - 1) / kThreads);
    };
    // the wait counts must fit the 6-bit vector-memory counter: a shorter
    // ring when the copies and stores of nbuf - 1 rows would not
    const int nbuf_lds = nbuf;
    int vec_store = 0;
    int ns = stores(g.P, g.Q, vec_store);
    while (nbuf > 2 && (nd + ns) * (nbuf - 1) > 63) --nbuf;
    if ((nd + ns) * (nbuf - 1) > 63) return false;
    if (epi.pool) {   // fewer, narrower output rows
        ns = stores(g.P / 2, g.Q / 2, vec_store);
        nbuf = nbuf_lds;
        while (nbuf > 2 && (nd + ns) * (nbuf - 1) > 63) --nbuf;
        if ((nd + ns) * (nbuf - 1) > 63) return false;
    }
    const size_t lds = (size_t)nbuf * buf * 2 + tile;
    a.C = g.C; a.K = g.K; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
    a.pitch = g.pitchB;
    a.D = D; a.T = T;
    a.nph = nph; a.mblocks = mblocks;
    a.nph_log2 = nph == 1 ? 0 : nph == 2 ? 1 : nph == 4 ? 2 : 3;
    a.G = G;
    a.nchunks = nchunks;
    a.copy_chunks = copy_chunks;
    a.buf_elems = buf;
    a.nbuf = nbuf;
    a.nd = nd;
    a.ostride = ostride;
    a.vec_store = vec_store;
    a.ns = ns;
    a.relu = epi.relu;
    a.pool = epi.pool;
    a.Po = out_rows(g, epi);
    a.Qo = out_cols(g, epi);
    a.fdPo = make_fastdiv(a.Po);
    pl.nset = nset;
    pl.steps = steps;
    pl.pad = pad;
    pl.mask = mask;
    pl.tail_last = tail_last;
    pl.lds_bytes = lds;
    pl.wgs_per_cu = wgs;
    return true;
}

// One compiled kernel: the tail-in-last-step form exists only for masked
// plans (without masks it would be the same kernel).
template <typename TIn, typename TOut, int NS, int M, bool MK, int PD, bool POOL>
hipError_t launch_rows_one(const MfRowPlan& pl, int64_t grid, const void* xw,
                           const void* aperm, const void* bias, void* y, const MfRowArgs& a,
                           hipStream_t st) {
    void (*kfn)(const uint16_t*, const uint16_t*, const TIn*, TOut*, MfRowArgs) =
        conv_mfma_rows_kernel<TIn, TOut, NS, M, MK, PD, false, POOL>;
    if constexpr (MK) {
        if (pl.tail_last) kfn = conv_mfma_rows_kernel<TIn, TOut, NS, M, MK, PD, true, POOL>;
    }
    // more than 64 KB of dynamic LDS per workgroup must be allowed explicitly
    if (pl.lds_bytes > 65536 && allow_dynamic_lds(reinterpret_cast<const void*>(kfn), pl.lds_bytes) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kfn, dim3((uint32_t)grid), dim3(kThreads), pl.lds_bytes, st,
                       (const uint16_t*)xw, (const uint16_t*)aperm, (const TIn*)bias, (TOut*)y, a);
    return hipSuccess;
}

template <typename TIn, typename TOut, bool POOL>
hipError_t launch_rows(const Geom& g, MfRowPlan pl, const void* xw, const void* aperm,
                       const void* bias, void* y, int n_images, hipStream_t st) {
    MfRowArgs a = pl.a;
    // row units: every window row, or both rows of every pooled output row
    const int64_t rows = (int64_t)n_images * (a.pool ? 2 * a.Po : g.P);
    if (rows >= (1ll << 31)) return hipErrorInvalidValue;
    a.rows = (int)rows;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    int64_t grid = (int64_t)cus * pl.wgs_per_cu;   // resident workgroups only
    const int64_t groups = a.pool ? rows / 2 : rows;   // runs are whole pairs with the pool
    if (grid > groups) grid = groups;
#define CIW_MF_LAUNCH(NS, M, MK, PD)                                                           \
    do {                                                                                       \
        const hipError_t e_ = launch_rows_one<TIn, TOut, NS, M, MK, PD, POOL>(pl, grid, xw,        \
                                                                              aperm, bias, y,  \
                                                                              a, st);          \
        if (e_ != hipSuccess) return e_;                                                       \
    } while (0)
#define CIW_MF_STEPS(MK, PD)                                                                   \
    do {                                                                                       \
        if (pl.steps == 10) CIW_MF_LAUNCH(1, 10, MK, PD);                                      \
        else if (pl.steps == 16) CIW_MF_LAUNCH(1, 16, MK, PD);                                 \
        else if (pl.steps == 24) CIW_MF_LAUNCH(1, 24, MK, PD);                                 \
        else if (pl.steps == 36) CIW_MF_LAUNCH(1, 36, MK, PD);                                 \
        else CIW_MF_LAUNCH(1, 40, MK, PD);                                                     \
    } while (0)
#define CIW_MF_PAD(MK)                                                                         \
    do {                                                                                       \
        if (pl.pad == 1) CIW_MF_STEPS(MK, 1);                                                  \
        else if (pl.pad == 2) CIW_MF_STEPS(MK, 2);                                             \
        else if (pl.pad == 4) CIW_MF_STEPS(MK, 4);                                             \
        else CIW_MF_STEPS(MK, 8);                                                              \
    } while (0)
#if CIW_ROWS_ABLATION_ONLY
    if (POOL || pl.nset != 1 || pl.mask || pl.steps != 36 || (pl.pad != 1 && pl.pad != 8))
        return hipErrorNotSupported;
    if (pl.pad == 8) CIW_MF_LAUNCH(1, 36, false, 8);
    else CIW_MF_LAUNCH(1, 36, false, 1);
#else
    if (pl.nset == 1) {
        if (pl.mask) CIW_MF_PAD(true);
        else CIW_MF_PAD(false);
    } else if (pl.nset == 2) {    // several phases: nph > 1, no pad chunks
        if (pl.steps == 10) CIW_MF_LAUNCH(2, 10, true, 1);
        else CIW_MF_LAUNCH(2, 16, true, 1);
    } else {
        CIW_MF_LAUNCH(4, 10, true, 1);
    }
#endif
#undef CIW_MF_PAD
#undef CIW_MF_STEPS
#undef CIW_MF_LAUNCH
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_t(const Geom& g, const void* xw, const void* w, const void* aperm,
                    const void* bias, void* y, int n_images, bool generic, const Epi& epi,
                    hipStream_t st) {
    if (n_images == 0) return hipSuccess;
    MfRowPlan pl;
    if (!generic && aperm && mf_row_plan(g, (int)sizeof(TOut), pl, epi)) {
        // without the re-layout the kernel gathers from the filter itself
        const void* fsrc = CIW_ABLATE_ROWS_NO_INDEX ? w : aperm;
#if CIW_ROWS_ABLATION_ONLY
        if (epi.pool) return hipErrorNotSupported;
        return launch_rows<TIn, TOut, false>(g, pl, xw, fsrc, bias, y, n_images, st);
#else
        return epi.pool ? launch_rows<TIn, TOut, true>(g, pl, xw, fsrc, bias, y, n_images, st)
                        : launch_rows<TIn, TOut, false>(g, pl, xw, fsrc, bias, y, n_images, st);
#endif
    }
#if CIW_ROWS_ABLATION_ONLY
    return hipErrorNotSupported;
#else
    MfmaArgs a;
    a.C = g.C; a.K = g.K; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
    a.sw = g.sw; a.dw = g.dw; a.pitch = g.pitchB;
    a.RC = g.R * g.C;
    a.T = g.S * a.RC;
    a.relu = epi.relu;
    a.pool = epi.pool;
    a.Po = out_rows(g, epi);
    a.Qo = out_cols(g, epi);
    const int64_t npix = (int64_t)n_images * a.Po * a.Qo * (epi.pool ? 4 : 1);
    if (npix >= (1ll << 31)) return hipErrorInvalidValue;
    a.npix = (int)npix;
    a.fdRC = make_fastdiv(a.RC);
    a.fdC = make_fastdiv(g.C);
    a.fdPQo = make_fastdiv(a.Po * a.Qo);
    a.fdQo = make_fastdiv(a.Qo);
    dim3 grid((a.npix + kNB - 1) / kNB, (g.K + kMB - 1) / kMB);
    hipLaunchKernelGGL((conv_mfma_generic_kernel<TIn, TOut>), grid, dim3(kThreads), 0, st,
                       (const uint16_t*)xw, (const uint16_t*)w, (const TIn*)bias, (TOut*)y, a);
    return hipGetLastError();
#endif
}

}  // namespace
}  // namespace ciw
