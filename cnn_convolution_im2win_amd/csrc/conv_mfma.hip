// conv_mfma.hip -- fp16/bf16 windowed contraction on the gfx950 matrix cores.
//
// The im2win paper ("Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support ...", §III-D) maps the output to a matrix product
// with M = output channels and N = images x output rows x output columns,
// reducing over the window.  With the HWC window layout the window of output
// (n, h, w) is, for each filter column q, the R*C contiguous elements at
// column w*stride_w + q*dil_w of row (n, h); with dil_w = 1 the whole window
// (S*R*C elements) is one contiguous run.  The reduction index is
// t = (q*R + r)*C + c and the filter operand is F[k][c][r][q] ("height before
// width", §III-C).  Products are exact in fp32 and accumulate in fp32
// (§III-F); the bias is added in fp32 and the result rounded once.
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
    int T, RC, npix;
    FastDiv fdRC, fdC, fdPQ, fdQ;
};

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
// LDS one 32-wide reduction step at a time.
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
        uint32_t n = fdiv(pload, a.fdPQ);
        int pix = pload - n * (a.P * a.Q);
        int h = fdiv(pix, a.fdQ);
        int wo = pix - h * a.Q;
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
    const int PQ = a.P * a.Q;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        int p = p0 + wn * 32 + ni * 16 + (lane & 15);
        if (p >= a.npix) continue;
        uint32_t n = fdiv(p, a.fdPQ);
        int pix = p - n * PQ;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int k = k0 + wm * 32 + mi * 16 + (lane >> 4) * 4 + i;
                if (k >= a.K) continue;
                float v = acc[mi][ni][i];
                if (bias) v += to_f32(bias[k]);
                y[((int64_t)n * a.K + k) * PQ + pix] = from_f32<TOut>(v);
            }
    }
}

// ------------------------------------------------------------ row kernel
// Persistent kernel for layers whose filter fits in registers (K <= 64,
// padded reduction <= 640 per phase set).  The GEMM view is the paper's
// (§III-D): M = output channels, N = output pixels, reduction over the
// window.  One workgroup owns whole window rows (n, h):
//   - each of its four waves keeps its A operand -- 32 output channels x
//     the whole padded reduction, as v_mfma_f32_32x32x16 fragments -- in
//     registers for the life of the kernel;
//   - window rows stream through two LDS buffers: while one row is
//     multiplied the next row's loads are in flight (double buffering and
//     load/compute overlap, §III-D/§III-E);
//   - the window of pixel w is the contiguous LDS run at w*D, D =
//     stride_w*R*C, so consecutive pixels read overlapping runs and each
//     window element is fetched from HBM once per output row ("elements
//     loaded in a previous window remain in cache", §III-C);
//   - results pass through an LDS tile so each output row leaves with
//     contiguous stores.
// Alignment: a B fragment is a 16-byte LDS read, so its start must be a
// multiple of 8 elements.  Pixels are grouped into `nph` phases (w mod nph,
// nph = 8 / gcd(D, 8)) whose window starts share one misalignment delta;
// each phase multiplies a copy of the filter shifted right by delta, and
// reads start delta elements early.  Reduction entries outside the window
// (the shift, the padding to a multiple of 16) are zero in A and masked to
// zero in B, so values outside a window never reach a stored output.
struct MfRowArgs {
    int C, K, R, S, P, Q, pitch;   // pitch: window row pitch (elements)
    int D, T;                      // window start stride, window length
    int nph, mblocks;              // pixel phases, 32-pixel blocks per phase
    int steps;                     // padded reduction / 16
    int nchunks;                   // 16-byte chunks of a window row
    int copy_chunks;               // chunks copied (nchunks rounded to 8 when swizzled)
    int swz;                       // XOR-swizzle 16-byte chunks within 128-byte groups
    int buf_elems;                 // elements per LDS row buffer
    int ostride;                   // LDS output tile row stride (elements of TOut)
    int vec_store;                 // output rows are whole 16-byte vectors
    int rows;                      // N * P
    FastDiv fdP, fdCp, fdR, fdRS;
};

constexpr int kMfMaxChunks = 8;    // 16-byte chunks per thread per row copy

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

// LDS position of 16-byte chunk ch when swizzled: its low four bits XORed
// with bits 3..6, a permutation of each group of 16 chunks (256 bytes) that
// spreads window starts 24 or 72 chunks apart over distinct banks.
__device__ __forceinline__ int swz_pos(int ch, int on) {
    return on ? (ch ^ ((ch >> 3) & 15)) : ch;
}

// The chunk stored at LDS position p (inverse of swz_pos).
__device__ __forceinline__ int swz_chunk_at(int p, int on) {
    if (!on) return p;
    const int z = p ^ (((p >> 4) & 7) << 1);
    return z ^ ((z >> 3) & 1);
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

template <typename TIn, typename TOut, int NSET, int STEPS, bool MASK>
__global__ __launch_bounds__(kThreads, 2) void conv_mfma_rows_kernel(
    const uint16_t* __restrict__ xw, const uint16_t* __restrict__ aperm,
    const TIn* __restrict__ bias, TOut* __restrict__ y, MfRowArgs a) {
    extern __shared__ __align__(16) uint16_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kh = wave & 1;          // output channels [32 kh, 32 kh + 32)
    const int pb0 = wave >> 1;        // pixel blocks pb0, pb0 + 2, ...
    const int g = lane >> 5;          // which 8 of a fragment's 16 reduction entries
    const int ml = lane & 31;         // fragment column
    const int npb = a.nph * a.mblocks;
    constexpr int Tp = STEPS * 16;

    uint16_t* rowbuf = lds;                                              // 2 x buf_elems
    float* otile = reinterpret_cast<float*>(lds + 2 * a.buf_elems);      // K x ostride fp32
    float* bias_l = otile + a.K * a.ostride;                             // 64 floats

    // ---- A fragments, from the filter the prep kernel laid out as
    // aperm[phase][64 output channels][Tp] (phase-shifted, zero-padded):
    // lane holds A[m = lane % 32][16 s + 8 (lane / 32) + 0..7]
    uint4 A[NSET][STEPS];
#pragma unroll
    for (int j = 0; j < NSET; ++j) {
        const int pb = min(pb0 + 2 * j, npb - 1);
        const uint16_t* ap = aperm + ((size_t)(pb % a.nph) * 64 + kh * 32 + ml) * Tp + 8 * g;
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2)
            A[j][s2] = *reinterpret_cast<const uint4*>(ap + 16 * s2);
    }
    // wait for them here, not at their first use inside the row loop (where
    // the wait would also drain the next row's prefetch)
#pragma unroll
    for (int j = 0; j < NSET; ++j)
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2) asm volatile("" ::"v"(A[j][s2].x));

    // ---- window rows: global -> registers -> LDS (chunk positions swizzled).
    // Loads are unconditional (clamped addresses) so they all issue at once.
    uint4 stg[kMfMaxChunks];
    auto load_row = [&](int row) {
        const uint4* src = reinterpret_cast<const uint4*>(xw + (size_t)row * a.pitch);
#pragma unroll
        for (int j = 0; j < kMfMaxChunks; ++j) {
            if (j * kThreads < a.copy_chunks) {
                const int p = min(tid + j * kThreads, a.copy_chunks - 1);
                const int ch = min(swz_chunk_at(p, a.swz), a.nchunks - 1);
                stg[j] = src[ch];
            }
        }
    };
    auto store_row = [&](int buf) {
        uint4* dst = reinterpret_cast<uint4*>(rowbuf + buf * a.buf_elems);
#pragma unroll
        for (int j = 0; j < kMfMaxChunks; ++j) {
            const int p = tid + j * kThreads;
            if (p < a.copy_chunks)
                dst[p] = swz_chunk_at(p, a.swz) < a.nchunks ? stg[j] : make_uint4(0u, 0u, 0u, 0u);
        }
    };

    int row = blockIdx.x;
    if (row >= a.rows) return;
    // zero the row buffers once: chunks past copy_chunks are read only by
    // pixels past the end of the row, and must hold finite values
    for (int i = tid * 8; i < 2 * a.buf_elems; i += kThreads * 8)
        *reinterpret_cast<uint4*>(rowbuf + i) = make_uint4(0u, 0u, 0u, 0u);
    if (tid < 64) bias_l[tid] = (bias && tid < a.K) ? to_f32(bias[tid]) : 0.f;
    __syncthreads();
    load_row(row);
    store_row(0);
    __syncthreads();

    const int PQ = a.P * a.Q;
    for (int it = 0; row < a.rows; ++it, row += gridDim.x) {
        const int buf = it & 1;
        const int next = row + gridDim.x;
        if (next < a.rows) load_row(next);

        const uint16_t* lb = rowbuf + buf * a.buf_elems;
        float* ot = otile;
        // blocks pb0 + 2 j; block j uses the fragments of set j % NSET
        for (int base = 0; pb0 + 2 * base < npb; base += NSET)
#pragma unroll
        for (int j = 0; j < NSET; ++j) {
            const int pb = pb0 + 2 * (base + j);
            if (pb >= npb) break;
            const int ph = pb % a.nph;
            const int mb = pb / a.nph;
            const int delta = (ph * a.D) & 7;
            const int wpix = a.nph * (32 * mb + ml) + ph;
            // pixels past the row end (never stored) read the last pixel of
            // their phase instead, so reads stay inside the row buffer
            const int wlast = a.Q - 1 >= ph ? a.Q - 1 - (a.Q - 1 - ph) % a.nph : ph;
            const int wread = min(wpix, wlast);
            // first element of the run this lane reads: window start minus
            // delta (a multiple of 8), then 16 per step
            const int chunk0 = (wread * a.D - delta) / 8 + g;
            // steps [1, s_full) hold only window entries; with MASK the
            // first step (when delta > 0) and the steps from s_full on are
            // masked (without MASK the plan guarantees there are none)
            const int s_full = (delta + a.T) / 16;
            f32x16 acc;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.f;
            // B fragments double-buffered in registers: the read of step
            // s + 1 is in flight while step s multiplies
            uint4 bn = *reinterpret_cast<const uint4*>(lb + 8 * swz_pos(chunk0, a.swz));
#pragma unroll
            for (int s2 = 0; s2 < STEPS; ++s2) {
                uint4 b = bn;
                if (s2 + 1 < STEPS)
                    bn = *reinterpret_cast<const uint4*>(
                        lb + 8 * swz_pos(chunk0 + 2 * (s2 + 1), a.swz));
                if (MASK && ((s2 == 0 && delta > 0) || s2 >= s_full)) {
                    const uint4 mk = elem_mask(16 * s2 + 8 * g, delta, delta + a.T);
                    b.x &= mk.x; b.y &= mk.y; b.z &= mk.z; b.w &= mk.w;
                }
                acc = mfma32<TIn>(A[j][s2], b, acc);
            }
            // lane holds D[m][n] for n = lane % 32, m = 8 (i / 4) + 4 (lane / 32) + i % 4
            if (wpix < a.Q) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int k = kh * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                    if (k < a.K) ot[k * a.ostride + wpix] = acc[i];
                }
            }
        }
        if (next < a.rows) store_row(buf ^ 1);
        __syncthreads();

        // ---- output row (n, h): K rows of Q contiguous elements
        const uint32_t n = fdiv(row, a.fdP);
        const int h = row - n * a.P;
        TOut* yrow = y + (size_t)n * a.K * PQ + (size_t)h * a.Q;
        if (a.vec_store) {
            constexpr int V = 16 / sizeof(TOut);   // outputs per 16-byte store
            const int vq = a.Q / V;
            for (int i = tid; i < a.K * vq; i += kThreads) {
                const int k = i / vq;
                const int v = i - k * vq;
                const float b = bias_l[k];
                const float* src = ot + k * a.ostride + v * V;
                union {
                    uint4 u;
                    TOut e[V];
                } pk;
#pragma unroll
                for (int e = 0; e < V; ++e) pk.e[e] = from_f32<TOut>(src[e] + b);
                *reinterpret_cast<uint4*>(yrow + (size_t)k * PQ + v * V) = pk.u;
            }
        } else {
            for (int i = tid; i < a.K * a.Q; i += kThreads) {
                const int k = i / a.Q;
                const int wq = i - k * a.Q;
                yrow[(size_t)k * PQ + wq] = from_f32<TOut>(ot[k * a.ostride + wq] + bias_l[k]);
            }
        }
        __syncthreads();   // the output tile is rewritten by the next row
    }
}

// Filter layout for the row kernel: aperm[ph][k][t'] = F[k][c][r][q] at
// window-order index t = t' - delta(ph) = (q*R + r)*C + c when 0 <= t < T
// and k < K, else 0; 64 output channels and Tp = 16*steps entries per phase.
struct PermArgs {
    int C, K, R, S, D, T, nph, Tp;
    FastDiv fdTp, fdC, fdR;
    uint32_t total;
};

__global__ __launch_bounds__(kThreads) void mfma_filter_perm_kernel(
    const uint16_t* __restrict__ w, uint16_t* __restrict__ aperm, PermArgs p) {
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= p.total) return;
    const uint32_t pk = fdiv(i, p.fdTp);
    const int tp = i - pk * p.Tp;
    const int k = pk & 63;
    const int ph = pk >> 6;
    const int t = tp - ((ph * p.D) & 7);
    uint16_t e = 0;
    if (k < p.K && t >= 0 && t < p.T) {
        const uint32_t qr = fdiv(t, p.fdC);
        const int c = t - qr * p.C;
        const uint32_t q = fdiv(qr, p.fdR);
        const int r = qr - q * p.R;
        e = w[(((size_t)k * p.C + c) * p.R + r) * p.S + q];
    }
    aperm[i] = e;
}

struct MfRowPlan {
    MfRowArgs a;
    int nset, steps;
    bool mask;
    size_t lds_bytes;
};

int gcd_int(int x, int y) {
    while (y) {
        int t = x % y;
        x = y;
        y = t;
    }
    return x;
}

// Row-kernel plan; false when the layer does not fit it.
bool mf_row_plan(const Geom& g, int out_bytes, MfRowPlan& pl) {
    if (g.K > 64 || g.dw != 1) return false;
    MfRowArgs& a = pl.a;
    const int D = g.sw * g.R * g.C;
    const int T = g.S * g.R * g.C;
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
    // masking is needed unless every step lies wholly inside the window
    const bool mask = maxdelta > 0 || T != 16 * steps;
    const int mcount = (g.Q + nph - 1) / nph;
    const int mblocks = (mcount + 31) / 32;
    const int nchunks = g.pitchB / 8;
    // bank conflicts of the fragment reads: the 32 lanes of a half-wave read
    // chunks D*nph/8 apart; count 16-lane groups that miss one of 16 bank
    // groups (64 banks) and 8-lane groups that miss one of 8 (32 banks),
    // without and with the swizzle, and keep the better layout
    const int sp = D * nph / 8;
    auto conflicts = [&](int on) {
        int bad = 0;
        for (int base = 0; base < 64; ++base) {
            int pos[32];
            for (int m = 0; m < 32; ++m) {
                const int ch = base + m * sp;
                pos[m] = on ? (ch ^ ((ch >> 3) & 15)) : ch;
            }
            for (int ph = 0; ph < 32; ph += 16) {
                int seen = 0;
                for (int m = ph; m < ph + 16; ++m) seen |= 1 << (pos[m] & 15);
                bad += seen != 0xffff;
            }
            for (int ph = 0; ph < 32; ph += 8) {
                int seen = 0;
                for (int m = ph; m < ph + 8; ++m) seen |= 1 << (pos[m] & 7);
                bad += seen != 0xff;
            }
        }
        return bad;
    };
    const int swz = conflicts(1) < conflicts(0) ? 1 : 0;
    const int copy_chunks = swz ? (nchunks + 15) / 16 * 16 : nchunks;
    if (copy_chunks > kMfMaxChunks * kThreads) return false;
    // the furthest chunk any fragment read touches (the last pixel's window
    // over the whole padded reduction), rounded to 256 bytes
    const int wmax = std::max(g.Q - 1, nph - 1);   // furthest pixel whose window is read
    const int last_chunk = (wmax * D) / 8 + 2 * steps + 1;
    int buf_chunks = std::max(copy_chunks, last_chunk + 1);
    buf_chunks = (buf_chunks + 15) / 16 * 16;
    const int buf = buf_chunks * 8;
    const int ostride = (g.Q + 3) / 4 * 4;
    const size_t lds = (size_t)2 * buf * 2 + (size_t)g.K * ostride * 4 + 64 * 4;
    const int crs = g.C * g.R * g.S;
    if (lds > 65536) return false;
    (void)crs;
    a.C = g.C; a.K = g.K; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
    a.pitch = g.pitchB;
    a.D = D; a.T = T;
    a.nph = nph; a.mblocks = mblocks;
    a.steps = steps;
    a.nchunks = nchunks;
    a.copy_chunks = copy_chunks;
    a.swz = swz;
    a.buf_elems = buf;
    a.ostride = ostride;
    const int V = 16 / out_bytes;
    a.vec_store = (g.Q % V == 0 && ((int64_t)g.P * g.Q) % V == 0) ? 1 : 0;
    a.fdP = make_fastdiv(g.P);
    a.fdCp = make_fastdiv(g.C);
    a.fdR = make_fastdiv(g.R);
    a.fdRS = make_fastdiv(g.R * g.S);
    pl.nset = nset;
    pl.steps = steps;
    pl.mask = mask;
    pl.lds_bytes = lds;
    return true;
}

template <typename TIn, typename TOut>
hipError_t launch_rows(const Geom& g, MfRowPlan pl, const void* xw, const void* aperm,
                       const void* bias, void* y, int n_images, hipStream_t st) {
    MfRowArgs a = pl.a;
    const int64_t rows = (int64_t)n_images * g.P;
    if (rows >= (1ll << 31)) return hipErrorInvalidValue;
    a.rows = (int)rows;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    int64_t grid = (int64_t)cus * 2;   // two resident workgroups per CU
    if (grid > rows) grid = rows;
#define CIW_MF_LAUNCH(NS, M, MK)                                                               \
    hipLaunchKernelGGL((conv_mfma_rows_kernel<TIn, TOut, NS, M, MK>), dim3((uint32_t)grid),     \
                       dim3(kThreads), pl.lds_bytes, st, (const uint16_t*)xw, (const uint16_t*)aperm, \
                       (const TIn*)bias, (TOut*)y, a)
    if (pl.nset == 1 && !pl.mask) {
        if (pl.steps == 10) CIW_MF_LAUNCH(1, 10, false);
        else if (pl.steps == 16) CIW_MF_LAUNCH(1, 16, false);
        else if (pl.steps == 24) CIW_MF_LAUNCH(1, 24, false);
        else if (pl.steps == 36) CIW_MF_LAUNCH(1, 36, false);
        else CIW_MF_LAUNCH(1, 40, false);
    } else if (pl.nset == 1) {
        if (pl.steps == 10) CIW_MF_LAUNCH(1, 10, true);
        else if (pl.steps == 16) CIW_MF_LAUNCH(1, 16, true);
        else if (pl.steps == 24) CIW_MF_LAUNCH(1, 24, true);
        else if (pl.steps == 36) CIW_MF_LAUNCH(1, 36, true);
        else CIW_MF_LAUNCH(1, 40, true);
    } else if (pl.nset == 2) {
        if (pl.steps == 10) CIW_MF_LAUNCH(2, 10, true);
        else CIW_MF_LAUNCH(2, 16, true);
    } else {
        CIW_MF_LAUNCH(4, 10, true);
    }
#undef CIW_MF_LAUNCH
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_t(const Geom& g, const void* xw, const void* w, const void* aperm,
                    const void* bias, void* y, int n_images, bool generic, hipStream_t st) {
    if (n_images == 0) return hipSuccess;
    MfRowPlan pl;
    if (!generic && aperm && mf_row_plan(g, (int)sizeof(TOut), pl))
        return launch_rows<TIn, TOut>(g, pl, xw, aperm, bias, y, n_images, st);
    MfmaArgs a;
    a.C = g.C; a.K = g.K; a.R = g.R; a.S = g.S; a.P = g.P; a.Q = g.Q;
    a.sw = g.sw; a.dw = g.dw; a.pitch = g.pitchB;
    a.RC = g.R * g.C;
    a.T = g.S * a.RC;
    a.npix = n_images * g.P * g.Q;
    a.fdRC = make_fastdiv(a.RC);
    a.fdC = make_fastdiv(g.C);
    a.fdPQ = make_fastdiv(g.P * g.Q);
    a.fdQ = make_fastdiv(g.Q);
    dim3 grid((a.npix + kNB - 1) / kNB, (g.K + kMB - 1) / kMB);
    hipLaunchKernelGGL((conv_mfma_generic_kernel<TIn, TOut>), grid, dim3(kThreads), 0, st,
                       (const uint16_t*)xw, (const uint16_t*)w, (const TIn*)bias, (TOut*)y, a);
    return hipGetLastError();
}

}  // namespace

size_t mfma_prep_bytes(const Geom& g) {
    MfRowPlan pl;
    // the plan with 4-byte outputs needs the most LDS; size for any output type
    if (!mf_row_plan(g, 2, pl) && !mf_row_plan(g, 4, pl)) return 0;
    return (size_t)pl.a.nph * 64 * pl.steps * 16 * sizeof(uint16_t);
}

hipError_t launch_mfma_prep(const Geom& g, ciw_dtype out, const void* w, void* aperm,
                            hipStream_t st) {
    MfRowPlan pl;
    if (!mf_row_plan(g, elem_bytes(out), pl)) return hipSuccess;   // generic kernel: no prep
    PermArgs p;
    p.C = g.C; p.K = g.K; p.R = g.R; p.S = g.S;
    p.D = pl.a.D; p.T = pl.a.T; p.nph = pl.a.nph; p.Tp = pl.steps * 16;
    p.fdTp = make_fastdiv(p.Tp);
    p.fdC = make_fastdiv(g.C);
    p.fdR = make_fastdiv(g.R);
    p.total = (uint32_t)(p.nph * 64 * p.Tp);
    hipLaunchKernelGGL(mfma_filter_perm_kernel, dim3((p.total + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, st, (const uint16_t*)w, (uint16_t*)aperm, p);
    return hipGetLastError();
}

hipError_t launch_conv_mfma(const Geom& g, ciw_dtype in, ciw_dtype out, const void* xw,
                            const void* w, const void* aperm, const void* bias, void* y,
                            int n_images, bool generic, hipStream_t st) {
    if (in == CIW_F16)
        return out == CIW_F32
                   ? launch_t<half_t, float>(g, xw, w, aperm, bias, y, n_images, generic, st)
                   : launch_t<half_t, half_t>(g, xw, w, aperm, bias, y, n_images, generic, st);
    return out == CIW_F32
               ? launch_t<bf16_t, float>(g, xw, w, aperm, bias, y, n_images, generic, st)
               : launch_t<bf16_t, bf16_t>(g, xw, w, aperm, bias, y, n_images, generic, st);
}

}  // namespace ciw
