// conv_fp32_m16.hip -- fp32 dense windowed contraction on the gfx950 matrix
// cores with the whole channel sum in one workgroup
// (v_mfma_f32_16x16x4_f32), over the CHW window tensor.
//
// The contraction is the im2win paper's windowed dot product (§III-C): for
// output (n, k, h, w) the sum over channels c and filter taps (r, q) of
// w[k][c][r][q] times the window element xw[n][c][h][(w*stride_w +
// q*dil_w)*R + r].  The fp32 form of the paper runs it on CUDA cores
// (§III-F); here it runs on the fp32 matrix instruction.
//
// A workgroup owns 16 output channels and 48 consecutive output pixels of
// one image (three 16 x 16 MFMA tiles) and the whole channel sum, so no
// partial sums leave it.  Its eight waves split the channels into eight
// contiguous ranges; a wave streams its own range in groups of 4 channels
// (one MFMA reduction step per filter tap): the group's filter rows
// (16 x 4 x R*S, 16-byte loads) and its window rows (the rows its 48 pixels
// span, 16-byte loads) go from registers into the wave's own LDS buffer,
// two groups' loads in flight, and the next group's operands are read while
// a group multiplies.  No wave reads another's buffer, so the loop has no
// barrier (LDS operations of one wave are processed in order).  At the end
// the eight waves' sums are added through LDS in wave order, then the bias
// and ReLU: results are deterministic.
//
// Against the split-channel kernel of conv_fp32_mfma.hip this removes the
// partial sums (written and read back) and the second kernel; the price is
// that each workgroup reads its 16 channels' filter rows whole (the
// workgroups of one channel block share them through their XCD's L2) and
// that 16 x 16 tiles need twice the LDS reads per multiply of 32 x 32 ones.
#include <algorithm>

#include "internal.hpp"
#include "device_common.hpp"

namespace ciw {
namespace {

constexpr int kT = 512;       // 8 waves
constexpr int kWaves = 8;
constexpr int kM = 16;        // output channels per workgroup
constexpr int kTiles = 3;     // pixel tiles of 16
constexpr int kPix = 48;      // output pixels per workgroup
constexpr int kG = 4;         // channels per group: the MFMA's reduction width
constexpr int kMaxP = 10;     // 16-byte loads per lane per group (at most)
// groups whose loads are in flight: 4, or 2 where four groups' registers
// would not fit beside the rest (more than 6 loads a group)
#ifndef CIW_M16_DEPTH
#define CIW_M16_DEPTH 4
#endif
template <int NP>
constexpr int depth_for() { return NP <= 6 ? CIW_M16_DEPTH : 2; }

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct M16Args {
    int C, K, PQ, P, Q, pitch, sw, dw, R;
    int pgroups;      // pixel groups (of 48) per image
    int kblocks;      // 16-channel output blocks
    int nimg;         // images
    int ntask;
    int gA, gB;       // channel groups of waves 0-3 and of waves 4-7
    int nrow;         // window rows staged per channel (rows 48 pixels span, at most)
    int rq4;          // 16-byte pieces of a channel's staged rows: nrow * pitch / 4
    int AS;           // LDS row stride of a group's filter rows (floats)
    int BS;           // LDS stride between a group's channels (floats)
    int buf;          // floats per buffer: 16 * AS + 4 * BS (256 more follow it)
    int relu;
    // in-LDS form: the staged zero-padded input rows of the group's channels
    int H, W, sh, ph, pw, dh;
    int Hr;           // staged rows a channel
    int npc;          // 16-byte pieces of a channel's staged rows (at most)
    int zoff;         // a channel's zero run: (R - 1) * dil_h * W + 1 zeros
};

// RS: filter taps (9 or 1); NP: 16-byte loads (and LDS stores) per lane per
// group of its window pieces (with the filter's), or with IMP of its input
// rows (after the filter's); D (even): groups whose loads are in flight.
// IMP: the in-LDS form.  xw is then x itself: a group stages, per channel,
// the input rows its 48 pixels' windows span, Hr rows of W elements end to
// end as in x (rows outside the image stay zero), and the window element of
// output (h, w) at tap (r, q) is staged row (h - h0) * stride_h + r * dil_h
// (h0 the first pixel's row), column w * stride_w - pad_w + q * dil_w, or 0
// where that column is outside the image.  The window tensor is never
// written.
template <int RS, int NP, int D, bool IMP>
__global__ __launch_bounds__(kT, 1) void conv_fp32_mfma16_kernel(
    const float* __restrict__ xw, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ y, M16Args a) {
    extern __shared__ __align__(16) float smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15;      // A row (output channel) / B column (pixel) of the lane
    const int kk = lane >> 4;     // reduction entry: channel kk of the group

    // task = (channel block, image, pixel group), pixel group fastest; with
    // the grid a multiple of 8 the tasks of one XCD are consecutive
    // (dispatch is round-robin over 8), so the pixel groups reading one
    // channel block's filter rows meet in one L2
    int task = blockIdx.x;
    if ((a.ntask & 7) == 0) task = (int)(blockIdx.x & 7) * (a.ntask >> 3) + (int)(blockIdx.x >> 3);
    const int pg = task % a.pgroups;
    const int rest = task / a.pgroups;
    const int n_img = rest % a.nimg;
    const int kb = rest / a.nimg;
    const int k0 = kb * kM;
    const int p0 = pg * kPix;
    // the bias of the thread's (at most two) outputs of the final sum,
    // requested now so that its latency is not paid at the end
    static_assert(kM * kPix <= 2 * kT, "two final-sum outputs a thread");
    float bpre[2] = {0.f, 0.f};
    if (bias != nullptr) {
#pragma unroll
        for (int j = 0; j < 2; ++j) bpre[j] = bias[min(k0 + min(tid + j * kT, kM * kPix - 1) / kPix, a.K - 1)];
    }
    const int h_lo = p0 / a.Q;

    // Waves 0-3 take gA groups of 4 channels each and waves 4-7 gB <= gA:
    // waves t and t + 4 share a SIMD, and the older one is issued first
    // whenever both are ready, so it gets through its groups faster (with
    // equal shares the younger one was measured finishing 20% of the
    // kernel later).
    const int c_lo = wave < 4 ? wave * a.gA * kG : (4 * a.gA + (wave - 4) * a.gB) * kG;
    const int ngr = max(0, min(wave < 4 ? a.gA : a.gB, (a.C - c_lo) / kG));   // C is a multiple of 4

    // Per-lane load plan, the same for every group (only the channel base
    // moves).  A group is 16 * RS filter pieces (row k, piece f of the
    // group's 4 * RS floats of filter row k0 + k) followed by 4 * rq4
    // window pieces (channel ch, piece o4 of its nrow staged rows); piece
    // e = lane + 64 u is the lane's u-th load.  Every load is issued (a
    // fixed number in flight on every path, so the compiler waits for
    // exactly the group it stores): a piece outside the tensors reads a
    // clamped address and needs no zeroing (a filter row past K only feeds
    // output channels that are never stored, and no pixel's window reaches
    // a row past P), and a lane past the group's pieces writes its own
    // slot past the buffer.  Each load address is a per-lane pointer moved
    // by a per-lane step each group; it stops at the wave's last group, so
    // the loads issued past it stay in bounds.
    // With IMP the filter's pieces take the first kNA loads and the input
    // rows the next NP: a channel's staged rows inside the image are nv
    // elements end to end in x (so are they in LDS, from delta on, which
    // puts them on 16-byte boundaries), cut into 16-byte pieces, the last
    // one moved back to end at the last element (it then overlaps the one
    // before and may sit off a 16-byte boundary).  Staged rows outside the
    // image are zeroed once: they sit at the same positions for every group.
    const int nA = kM * RS;
    const int nP = nA + kG * a.rq4;
    constexpr int kNA = (kM * RS + 63) / 64;
    constexpr int kNL = IMP ? kNA + NP : NP;    // 16-byte loads a group
    const float* src[kNL];
    uint32_t step[kNL], dst[kNL];
    const int g0 = ngr > 0 ? c_lo : 0;   // first channel loaded (a wave with no channels reads channel 0)
    // IMP: the staged rows inside the image, [r_lo, r_hi]; delta puts row
    // r_lo's first element on a 16-byte boundary
    const int r_lo = IMP ? max(0, a.ph - h_lo * a.sh) : 0;
    const int r_hi = IMP ? min(a.Hr - 1, a.H - 1 + a.ph - h_lo * a.sh) : 0;
    const int nv = IMP ? max(0, r_hi - r_lo + 1) * a.W : 0;
    const int delta = IMP ? (4 - (r_lo * a.W) % 4) % 4 : 0;
    if constexpr (IMP) {
        const int npc = (nv + 3) / 4;
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int e = lane + 64 * u;
            const int ch = e / a.npc, i = e - ch * a.npc;
            const bool ok = ch < kG && i < npc;           // (then nv >= W >= 4)
            const int start = ok ? min(4 * i, nv - 4) : 0;
            const int ih0 = h_lo * a.sh - a.ph + r_lo;    // image row of staged row r_lo
            src[kNA + u] = ok ? xw + (((size_t)n_img * a.C + g0 + ch) * a.H + ih0) * a.W + start
                              : xw + ((size_t)n_img * a.C + g0) * a.H * a.W;
            step[kNA + u] = (uint32_t)(kG * a.H * a.W * 4);
            dst[kNA + u] = ok ? 4u * (uint32_t)(kM * a.AS + ch * a.BS + delta + r_lo * a.W + start)
                              : 4u * (uint32_t)a.buf + 16u * lane;
        }
    }
#pragma unroll
    for (int u = 0; u < (IMP ? kNA : NP); ++u) {
        const int e = lane + 64 * u;
        if (e < nA || IMP) {
            const int ec = min(e, nA - 1);
            const int k = ec / RS, f = ec - k * RS;
            const int kr = min(k0 + k, a.K - 1);
            src[u] = w + ((size_t)kr * a.C + g0) * RS + 4 * f;
            step[u] = kG * RS * 4;
            dst[u] = e < nA ? 4u * (uint32_t)(k * a.AS + 4 * f) : 4u * (uint32_t)a.buf + 16u * lane;
        } else {
            const int eb = min(e, nP - 1) - nA;
            const int ch = eb / a.rq4, o4 = eb - ch * a.rq4;
            const int row = min(h_lo + (4 * o4) / a.pitch, a.P - 1);
            const int col = (4 * o4) % a.pitch;
            src[u] = xw + (((size_t)n_img * a.C + g0 + ch) * a.P + row) * a.pitch + col;
            step[u] = (uint32_t)(kG * a.P * a.pitch * 4);
            dst[u] = e < nP ? 4u * (uint32_t)(kM * a.AS + ch * a.BS + 4 * o4) : 4u * (uint32_t)a.buf + 16u * lane;
        }
    }

    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    struct Fetched {
        u32x4 r[kNL];
    };
    // the loads of the next group (group j: the pointers sit at group
    // min(j, ngr - 1))
    int at = 0;   // group the pointers sit at
    auto fetch = [&](Fetched& f) {
#pragma unroll
        for (int u = 0; u < kNL; ++u) f.r[u] = *reinterpret_cast<const u32x4*>(src[u]);
        const bool adv = at + 1 < ngr;
        at += adv ? 1 : 0;
#pragma unroll
        for (int u = 0; u < kNL; ++u)
            src[u] = reinterpret_cast<const float*>(reinterpret_cast<const char*>(src[u]) + (adv ? step[u] : 0u));
    };
    // the wave's buffer: filter rows [16][AS], then the window rows [4][BS],
    // then 64 16-byte slots that lanes with no piece write (so every store
    // is unconditional: no branches between the multiplies)
    char* wbase = reinterpret_cast<char*>(smem + wave * (a.buf + 256));
    auto stash = [&](const Fetched& f) {
#pragma unroll
        for (int u = 0; u < kNL; ++u) *reinterpret_cast<u32x4*>(wbase + dst[u]) = f.r[u];
    };
    if constexpr (IMP) {
        // the staged rows' padding: zero once (no group writes it)
        for (int i = lane; i < a.BS; i += 64)
            reinterpret_cast<u32x4*>(wbase + 4 * kM * a.AS)[i] = u32x4{0u, 0u, 0u, 0u};
    }

    // the lane's window offsets: pixel tile t3, column m of the tile (past
    // the image's last pixel: that pixel, read but never stored)
    constexpr int S = RS == 9 ? 3 : 1;
    constexpr int R = S;
    // off[t3][q]: the lane's window element of tile t3, filter row 0,
    // filter column q (the window tensor's R values of a column adjacent;
    // in LDS, staged row (h - h0) * stride_h, column w * stride_w - pad_w
    // + q * dil_w), filter row r rstep * r further on.  In LDS a column
    // outside the image points at the channel's zero run instead, which
    // holds zeros at every filter row's distance.
    int off[kTiles][S];
#pragma unroll
    for (int t3 = 0; t3 < kTiles; ++t3) {
        const int px = min(p0 + 16 * t3 + m, a.PQ - 1);
        const int hh = px / a.Q, ww = px - hh * a.Q;
#pragma unroll
        for (int q = 0; q < S; ++q) {
            if constexpr (IMP) {
                const int col = ww * a.sw - a.pw + q * a.dw;
                off[t3][q] = col >= 0 && col < a.W ? delta + (hh - h_lo) * a.sh * a.W + col : a.zoff;
            } else {
                off[t3][q] = (hh - h_lo) * a.pitch + (ww * a.sw + q * a.dw) * a.R;
            }
        }
    }
    const int rstep = IMP ? a.dh * a.W : 1;

    f32x4 acc[kTiles];
#pragma unroll
    for (int t3 = 0; t3 < kTiles; ++t3) acc[t3] = f32x4{0.f, 0.f, 0.f, 0.f};

    // a group's operands: lane (m, kk) takes filter row m, channel kk, tap
    // t and, per tile, the window element of channel kk, pixel m, tap t
    struct Ops {
        float av[RS];
        float bv[kTiles][RS];
    };
    const float* Ap = reinterpret_cast<const float*>(wbase) + m * a.AS + kk * RS;
    const float* Bp = reinterpret_cast<const float*>(wbase) + kM * a.AS + kk * a.BS;
    auto read_ops = [&](Ops& o) {
#pragma unroll
        for (int t = 0; t < RS; ++t) o.av[t] = Ap[t];
#pragma unroll
        for (int t3 = 0; t3 < kTiles; ++t3)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < S; ++q) o.bv[t3][r * S + q] = Bp[off[t3][q] + r * rstep];
    };
    auto multiply = [&](const Ops& o) {
#pragma unroll
        for (int t = 0; t < RS; ++t)
#pragma unroll
            for (int t3 = 0; t3 < kTiles; ++t3)
                acc[t3] = __builtin_amdgcn_mfma_f32_16x16x4f32(o.av[t], o.bv[t3][t], acc[t3], 0, 0, 0);
    };
    // Interleave a group's multiplies with the next group's stores, loads
    // and operand reads (which all follow its stores: same buffer), so the
    // wave issues memory operations between matrix instructions.
    auto interleave = [&]() {
        constexpr int kR = RS + (kTiles * RS + 1) / 2;    // operand reads (some paired)
        constexpr int kSteps = RS * kTiles / 3;           // groups of 3 multiplies
        constexpr int kRper = (kR + kSteps - 3) / (kSteps - 2);
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);          // MFMA
            if (i < 2) __builtin_amdgcn_sched_group_barrier(0x200, (kNL + 1) / 2, 0);   // DS write
            else __builtin_amdgcn_sched_group_barrier(0x100, kRper, 0);               // DS read
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);          // VMEM read
        }
    };
    // One step: store group g + 1 (its loads were issued D steps earlier),
    // issue the loads of group g + 1 + D into the registers it leaves, read
    // group g + 1's operands, and multiply group g (whose operands were read
    // in the step before).  One LDS buffer a wave: its reads and stores are
    // processed in order.
    Fetched f[D];
    Ops ops[2];
    auto step_g = [&](Fetched& fs, Ops& next, const Ops& cur, bool mul) {
        stash(fs);
        // the operand reads stay after the stores (the interleaving below
        // must not move a store past a read of the same buffer)
        asm volatile("" ::: "memory");
        fetch(fs);
        read_ops(next);
        if (mul) multiply(cur);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int i = 0; i < D; ++i) {
        fetch(f[i]);   // groups 0 .. D - 1
        __builtin_amdgcn_sched_barrier(0);
    }
    stash(f[0]);
    asm volatile("" ::: "memory");
    fetch(f[0]);       // group D
    read_ops(ops[0]);
    __builtin_amdgcn_sched_barrier(0);
    // steps g = j .. j + D - 1 (group g + 1's registers: f[(g + 1) % D];
    // group g's operands: ops[g % 2]), D a multiple of 2
    int j = 0;
    for (; j + D <= ngr; j += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) step_g(f[(i + 1) % D], ops[(i + 1) & 1], ops[i & 1], true);
    }
#pragma unroll
    for (int i = 0; i + 1 < D; ++i)
        if (j + i < ngr) step_g(f[(i + 1) % D], ops[(i + 1) & 1], ops[i & 1], true);

    // ---- the waves' sums, added in wave order.  Each wave puts its tiles
    // in its own buffer (after its own last reads of it); lane l
    // holds D[4 (l / 16) + i][l % 16] of each tile: output channel
    // 4 (l / 16) + i, pixel l % 16.
#pragma unroll
    for (int t3 = 0; t3 < kTiles; ++t3)
#pragma unroll
        for (int i = 0; i < 4; ++i) reinterpret_cast<float*>(wbase)[(t3 * 4 + i) * 64 + lane] = acc[t3][i];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int o = tid + j * kT;
        if (o >= kM * kPix) break;
        const int ch = o / kPix, px = o - ch * kPix;
        const int t3 = px >> 4, l = 16 * (ch >> 2) + (px & 15), i = ch & 3;
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) s += smem[v * (a.buf + 256) + (t3 * 4 + i) * 64 + l];
        const int k = k0 + ch, p = p0 + px;
        if (k < a.K && p < a.PQ) {
            if (bias) s += bpre[j];
            if (a.relu) s = fmaxf(s, 0.f);
            y[((size_t)n_img * a.K + k) * a.PQ + p] = s;
        }
    }
}

struct M16Plan {
    M16Args a;
    int np;       // loads per lane per group (window pieces, or input elements)
    size_t lds;
};

template <int RS, bool IMP>
using M16Fn = void (*)(const float*, const float*, const float*, float*, M16Args);

template <int NP, bool IMP>
constexpr int depth_of() { return depth_for<IMP ? NP + 3 : NP>(); }

template <int RS, bool IMP>
M16Fn<RS, IMP> m16_kernel(int np) {
    switch (np) {
        case 1: return conv_fp32_mfma16_kernel<RS, 1, depth_of<1, IMP>(), IMP>;
        case 2: return conv_fp32_mfma16_kernel<RS, 2, depth_of<2, IMP>(), IMP>;
        case 3: return conv_fp32_mfma16_kernel<RS, 3, depth_of<3, IMP>(), IMP>;
        case 4: return conv_fp32_mfma16_kernel<RS, 4, depth_of<4, IMP>(), IMP>;
        case 5: return conv_fp32_mfma16_kernel<RS, 5, depth_of<5, IMP>(), IMP>;
        case 6: return conv_fp32_mfma16_kernel<RS, 6, depth_of<6, IMP>(), IMP>;
        case 7: return conv_fp32_mfma16_kernel<RS, 7, depth_of<7, IMP>(), IMP>;
        case 8: return conv_fp32_mfma16_kernel<RS, 8, depth_of<8, IMP>(), IMP>;
        case 9: return conv_fp32_mfma16_kernel<RS, 9, depth_of<9, IMP>(), IMP>;
        default: return conv_fp32_mfma16_kernel<RS, 10, depth_of<10, IMP>(), IMP>;
    }
}

// Layers this kernel runs: fp32, 3x3 or 1x1 filters, C a multiple of 4
// (16-byte filter loads), a group's window pieces (or, in LDS, input
// elements) within kMaxP loads a lane, the eight waves' buffers within
// 160 KB of LDS.
bool m16_plan(const Geom& g, int n_images, bool imp, M16Plan& pl) {
    if (!((g.R == 3 && g.S == 3) || (g.R == 1 && g.S == 1))) return false;
    if (g.C % kG != 0 || g.C <= 0 || g.K <= 0 || g.P <= 0 || g.Q <= 0) return false;
    M16Args& a = pl.a;
    const int RS = g.R * g.S;
    a.C = g.C; a.K = g.K; a.P = g.P; a.Q = g.Q; a.pitch = g.pitchA; a.sw = g.sw; a.dw = g.dw; a.R = g.R;
    a.H = g.H; a.W = g.W; a.sh = g.sh; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh;
    const int64_t PQ = (int64_t)g.P * g.Q;
    a.PQ = (int)PQ;
    a.pgroups = (int)((PQ + kPix - 1) / kPix);
    a.kblocks = (g.K + kM - 1) / kM;
    // rows spanned by 48 consecutive pixels: at most floor(47 / Q) + 2
    a.nrow = std::min(g.P, (kPix - 1) / g.Q + 2);
    a.AS = kG * RS;
    if (imp) {
        // pieces of 4 elements need rows of at least 4
        if (g.W < 4) return false;
        const int64_t hr = (int64_t)(a.nrow - 1) * g.sh + (int64_t)(g.R - 1) * g.dh + 1;
        const int64_t per_ch = hr * g.W;                // staged elements a channel
        const int64_t npc = (per_ch + 3) / 4;
        const int64_t np = (kG * npc + 63) / 64;
        if (np + (kM * RS + 63) / 64 > kMaxP || per_ch > (1 << 20)) return false;
        a.Hr = (int)hr;
        a.npc = (int)npc;
        a.rq4 = 0;
        // [shift <= 3][staged rows][<= 3][zero run], the run read for taps in
        // the horizontal padding
        a.zoff = (int)round_up(per_ch + 3, 4);
        a.BS = a.zoff + (int)round_up((int64_t)(g.R - 1) * g.dh * g.W + 1, 4) + 4;
        pl.np = (int)np;
        // 32-bit offsets: the step between groups of x
        if ((int64_t)kG * g.H * g.W * 4 >= ((int64_t)1 << 32)) return false;
    } else {
        if ((int64_t)a.nrow * g.pitchA % 4 != 0) return false;
        a.rq4 = a.nrow * g.pitchA / 4;
        const int64_t pieces = (int64_t)kM * RS + (int64_t)kG * a.rq4;
        if (pieces > (int64_t)kMaxP * 64) return false;
        pl.np = (int)((pieces + 63) / 64);
        a.Hr = a.npc = a.zoff = 0;
        a.BS = a.nrow * g.pitchA + 4;
        if ((int64_t)kG * g.P * g.pitchA * 4 >= ((int64_t)1 << 32)) return false;
    }
    // the groups split over the waves, an eighth of a wave's share moved
    // from each of waves 4-7 to its SIMD partner
    const int ngr = (g.C / kG + kWaves - 1) / kWaves;
    a.gA = ngr + ngr / 8;
    a.gB = ngr - ngr / 8;
    a.buf = kM * a.AS + kG * a.BS;
    if (a.buf < kTiles * 4 * 64) a.buf = kTiles * 4 * 64;   // room for the final sums
    a.nimg = n_images;
    const int64_t ntask = (int64_t)n_images * a.pgroups * a.kblocks;
    if (ntask >= ((int64_t)1 << 31) || ntask == 0) return false;
    a.ntask = (int)ntask;
    pl.lds = (size_t)kWaves * (a.buf + 256) * sizeof(float);
    return pl.lds <= 160 * 1024;
}

}  // namespace

int fp32_m16_tasks(const Geom& g, int n_images, bool imp) {
    M16Plan pl;
    return m16_plan(g, n_images, imp, pl) ? pl.a.ntask : 0;
}

hipError_t launch_conv_fp32_m16(const Geom& g, const float* xw, const float* w, const float* bias,
                                float* y, int n_images, const Epi& epi, bool imp, hipStream_t st) {
    M16Plan pl;
    if (n_images == 0) return hipSuccess;
    if (epi.pool || !m16_plan(g, n_images, imp, pl)) return hipErrorNotSupported;
    pl.a.relu = epi.relu;
    void (*kfn)(const float*, const float*, const float*, float*, M16Args) =
        imp ? (g.R == 3 ? m16_kernel<9, true>(pl.np) : m16_kernel<1, true>(pl.np))
            : (g.R == 3 ? m16_kernel<9, false>(pl.np) : m16_kernel<1, false>(pl.np));
    if (pl.lds > 65536 && allow_dynamic_lds(reinterpret_cast<const void*>(kfn), pl.lds) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(kfn, dim3((uint32_t)pl.a.ntask), dim3(kT), pl.lds, st, xw, w, bias, y, pl.a);
    return hipGetLastError();
}

}  // namespace ciw
