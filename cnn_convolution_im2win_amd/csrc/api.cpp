// api.cpp -- the C ABI of include/conv_im2win.h: argument validation, shape
// and workspace arithmetic, batch chunking and kernel dispatch.
//
// Every check runs before the first launch, so an error status means nothing
// was enqueued.  State kept between calls: the record of which kernels were
// allowed more than 64 KB of dynamic LDS (below), and the per-device
// addresses of the allocation-free entry point's workspace array.
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <utility>

#include "internal.hpp"

using namespace ciw;

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;   // int32 indexing in the kernels

// Output extent along one axis (floor formula); <= 0 when the dilated
// window does not fit the padded input.
int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d) {
    int64_t span = d * (k - 1) + 1;
    int64_t padded = in + 2 * p;
    if (padded < span) return 0;
    return (padded - span) / s + 1;
}

bool dtype_ok(int t) { return t == CIW_F32 || t == CIW_F16 || t == CIW_BF16; }

// The integer a caller passed for an enum parameter, read from its bytes: a
// C caller may pass any int, and loading an enum object that holds a value
// outside the enumeration's range is undefined in C++.  Every entry point
// checks its enum arguments this way before using them.
template <typename E>
int raw(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}
bool layout_ok(int l) { return l == CIW_WIN_CHW || l == CIW_WIN_HWC; }

// Product of non-negative extents, false if it reaches 2^62 (then the
// tensor is far past int32 indexing whatever the other factors are).  Every
// partial product is checked, so no multiplication can overflow int64.
bool mul_ok(std::initializer_list<int64_t> factors, int64_t* out) {
    const int64_t cap = (int64_t)1 << 62;
    int64_t p = 1;
    for (int64_t f : factors) {
        if (f < 0) return false;
        if (f != 0 && p > cap / f) return false;
        p *= f;
    }
    *out = p;
    return true;
}

// True when the product of the extents is below 2^31 (int32 indexing).
bool below_2_31(std::initializer_list<int64_t> factors) {
    int64_t p = 0;
    return mul_ok(factors, &p) && p < kMaxElems;
}

// a1: validate a descriptor and resolve the geometry.  Problems whose
// tensors exceed int32 indexing, or whose dilated filter is taller than the
// repack's LDS tile can hold (more than 4096 input rows), are unsupported.
// Extents come from the caller and may be as large as 2^31 - 1 each, so
// every product below is formed with overflow checks.
ciw_status resolve(const ciw_conv_desc* d, ciw_dtype dt, Geom* g) {
    if (!d || !dtype_ok(dt)) return CIW_ERR_INVALID_ARG;
    if (d->N < 0 || d->C < 1 || d->H < 1 || d->W < 1 || d->K < 1 || d->R < 1 || d->S < 1)
        return CIW_ERR_INVALID_ARG;
    if (d->stride_h < 1 || d->stride_w < 1 || d->pad_h < 0 || d->pad_w < 0 || d->dil_h < 1 ||
        d->dil_w < 1 || d->groups < 1)
        return CIW_ERR_INVALID_ARG;
    if (d->C % d->groups || d->K % d->groups) return CIW_ERR_INVALID_ARG;
    const int64_t limit = kMaxElems - 1;
    if (d->N > limit || d->C > limit || d->H > limit || d->W > limit || d->K > limit ||
        d->R > limit || d->S > limit)
        return CIW_ERR_UNSUPPORTED;
    int64_t P = out_extent(d->H, d->R, d->stride_h, d->pad_h, d->dil_h);
    int64_t Q = out_extent(d->W, d->S, d->stride_w, d->pad_w, d->dil_w);
    if (P < 1 || Q < 1) return CIW_ERR_INVALID_ARG;
    if ((int64_t)d->dil_h * (d->R - 1) + 1 > 4096) return CIW_ERR_UNSUPPORTED;
    const int64_t eb = elem_bytes(dt);
    // (Q - 1) * stride_w <= W + 2 pad_w < 2^33 and dil_w * (S - 1) < 2^62:
    // no overflow here
    const int64_t wwin = (Q - 1) * d->stride_w + (int64_t)d->dil_w * (d->S - 1) + 1;
    if (wwin >= kMaxElems) return CIW_ERR_UNSUPPORTED;
    // every tensor the kernels index must stay below 2^31 elements
    const int64_t N = d->N > 0 ? d->N : 1;
    if (!below_2_31({N, d->C, d->H, d->W}) || !below_2_31({d->K, d->C / d->groups, d->R, d->S}) ||
        !below_2_31({N, d->K, P, Q}) || !below_2_31({N, wwin, d->R, d->C}))
        return CIW_ERR_UNSUPPORTED;
    const int64_t lenA = wwin * d->R;   // < 2^31 by the check above
    const int64_t lenB = lenA * d->C;
    const int64_t pitchA = round_up(lenA, 16 / eb);
    const int64_t pitchB = round_up(lenB, 16 / eb);
    if (!below_2_31({N, d->C, P, pitchA}) || !below_2_31({N, P, pitchB})) return CIW_ERR_UNSUPPORTED;
    g->N = (int)d->N; g->C = (int)d->C; g->H = (int)d->H; g->W = (int)d->W;
    g->K = (int)d->K; g->R = (int)d->R; g->S = (int)d->S; g->P = (int)P; g->Q = (int)Q;
    g->sh = d->stride_h; g->sw = d->stride_w; g->ph = d->pad_h; g->pw = d->pad_w;
    g->dh = d->dil_h; g->dw = d->dil_w; g->G = d->groups;
    g->Wwin = (int)wwin;
    g->elem = (int)eb;
    g->lenA = (int)lenA; g->pitchA = (int)pitchA;
    g->lenB = (int)lenB; g->pitchB = (int)pitchB;
    return CIW_OK;
}

int64_t window_bytes_per_image(const Geom& g, ciw_win_layout lay) {
    return lay == CIW_WIN_CHW ? (int64_t)g.C * g.P * g.pitchA * g.elem
                              : (int64_t)g.P * g.pitchB * g.elem;
}

enum Path { PATH_FP32, PATH_MFMA, PATH_DW };

Path path_of(const Geom& g, ciw_dtype in, bool depthwise) {
    if (depthwise) return PATH_DW;
    return in == CIW_F32 ? PATH_FP32 : PATH_MFMA;
}

ciw_win_layout layout_of(Path p) { return p == PATH_MFMA ? CIW_WIN_HWC : CIW_WIN_CHW; }

// a8: workspace of one chunk of n images = its window tensor (+ fp32 partial sums).
int64_t chunk_workspace(const Geom& g, Path p, int64_t n) {
    int64_t bytes = round_up(window_bytes_per_image(g, layout_of(p)) * n, 256);
    if (p == PATH_FP32) {
        int s = fp32_splits(g, (int)n);
        if (s > 1) bytes += (int64_t)s * n * g.K * g.P * g.Q * 4;
    } else if (p == PATH_MFMA) {
        bytes += round_up((int64_t)mfma_prep_bytes(g), 256);   // re-laid-out filter
    }
    return bytes;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

ciw_status from_hip(hipError_t e) { return e == hipSuccess ? CIW_OK : CIW_ERR_HIP; }

// ---- the allocation-free entry point's workspace.
// A file-scope device array: each GPU the library runs on holds its own copy
// (CIW_NOALLOC_SCRATCH_BYTES) from the first use until the process ends.  In
// host code the name `scratch` is only a stand-in for the symbol, never a
// device address: the address of a device's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that pointer reaches kernels.  Every conv2d_fwd_noalloc call on
// a GPU uses the same array, so calls that overlap on one GPU (other
// streams, other threads) race on it.  Nothing in it needs clearing between
// calls: each call's repack writes every byte of the window tensor it
// reads, and every other workspace region a kernel reads is fully written
// earlier in the same call.
static __device__ __align__(256) unsigned char scratch[CIW_NOALLOC_SCRATCH_BYTES];

// The current device's copy of `scratch` (CIW_ERR_HIP if the runtime cannot
// give its address).
ciw_status scratch_of_current_device(void** out) {
    static std::mutex mu;
    static std::map<int, void*> ptrs;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CIW_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    auto it = ptrs.find(dev);
    if (it == ptrs.end()) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) return CIW_ERR_HIP;
        it = ptrs.emplace(dev, p).first;
    }
    *out = it->second;
    return CIW_OK;
}

// noalloc: the workspace is this device's copy of `scratch` (ws and
// ws_bytes are ignored), fetched after every check, before the first launch.
ciw_status run_conv(const ciw_conv_desc* desc, ciw_dtype in, ciw_dtype out, const void* x,
                    const void* w, const void* bias, void* y, void* ws, size_t ws_bytes,
                    uint32_t flags, void* stream, bool depthwise, bool noalloc = false) {
    if (noalloc) {
        // a window tensor prepared by the caller cannot be in the library's array
        if (flags & CIW_FLAG_WINDOW_READY) return CIW_ERR_INVALID_ARG;
        ws = nullptr;
        ws_bytes = CIW_NOALLOC_SCRATCH_BYTES;
    }
    Geom g;
    ciw_status s = resolve(desc, in, &g);
    if (s != CIW_OK) return s;
    if (!dtype_ok(out)) return CIW_ERR_INVALID_ARG;
    // allowed (in -> out) pairs
    if (in == CIW_F32 ? out != CIW_F32 : (out != in && out != CIW_F32)) return CIW_ERR_INVALID_ARG;
    if (flags & ~(CIW_FLAG_WINDOW_READY | CIW_FLAG_NO_SPLIT | CIW_FLAG_GENERIC | CIW_FLAG_RELU |
                  CIW_FLAG_MAXPOOL2 | CIW_FLAG_IMPLICIT | CIW_FLAG_FP32_MFMA | CIW_FLAG_FP32_VALU))
        return CIW_ERR_INVALID_ARG;
    const bool implicit = (flags & CIW_FLAG_IMPLICIT) != 0;
    if ((flags & CIW_FLAG_FP32_MFMA) && (flags & CIW_FLAG_FP32_VALU)) return CIW_ERR_INVALID_ARG;
    if (implicit && (flags & (CIW_FLAG_WINDOW_READY | CIW_FLAG_GENERIC))) return CIW_ERR_INVALID_ARG;
    Epi epi;
    epi.relu = (flags & CIW_FLAG_RELU) != 0;
    epi.pool = (flags & CIW_FLAG_MAXPOOL2) != 0;
    if (epi.pool && (g.P < 2 || g.Q < 2)) return CIW_ERR_INVALID_ARG;   // no 2x2 region
    if (depthwise) {
        if (!(g.G == g.C && g.K == g.C)) return g.G == 1 ? CIW_ERR_INVALID_ARG : CIW_ERR_UNSUPPORTED;
    } else if (g.G != 1) {
        return CIW_ERR_UNSUPPORTED;
    }
    if (implicit && depthwise) {
        // windows built in LDS from x; no workspace
        if (!dw_implicit_supported(g, epi)) return CIW_ERR_UNSUPPORTED;
        if (g.N == 0) return CIW_OK;
        if (!x || !w || !y || !aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) ||
            (bias && !aligned(bias, elem_bytes(in))))
            return CIW_ERR_INVALID_ARG;
        (void)hipGetLastError();
        return from_hip(launch_conv_dw_implicit(g, in, out, x, w, bias, y, epi, (hipStream_t)stream));
    }
    if (g.N == 0) return CIW_OK;   // empty batch: nothing to do
    const bool ready = (flags & CIW_FLAG_WINDOW_READY) != 0;
    size_t imp_need = 0;   // workspace of the in-LDS kernels (may be 0: then ws may be NULL)
    if (implicit) {
        const bool ok = in == CIW_F32 ? fp32_implicit_workspace(g, epi, &imp_need)
                                      : implicit_workspace(g, out, epi, &imp_need);
        if (!ok) return CIW_ERR_UNSUPPORTED;
    }
    const bool ws_needed = !noalloc && !(implicit && imp_need == 0);
    if ((!ready && !x) || !w || !y || (!ws && ws_needed)) return CIW_ERR_INVALID_ARG;
    if ((x && !aligned(x, 16)) || !aligned(w, 16) || !aligned(y, 16) || !aligned(ws, 16) ||
        (bias && !aligned(bias, elem_bytes(in))))
        return CIW_ERR_INVALID_ARG;

    if (implicit) {
        // window rows built in LDS from x: no chunks, the workspace holds
        // at most the re-laid-out filter
        if (ws_bytes < imp_need) return CIW_ERR_WORKSPACE;
        if (noalloc && imp_need > 0 && (s = scratch_of_current_device(&ws)) != CIW_OK) return s;
        (void)hipGetLastError();
        if (in == CIW_F32)
            return from_hip(launch_conv_fp32_implicit(g, (const float*)x, (const float*)w, (const float*)bias,
                                                      (float*)y, (float*)ws, epi, (hipStream_t)stream));
        return from_hip(launch_conv_implicit(g, in, out, x, w, bias, y, ws, epi, (hipStream_t)stream));
    }

    const Path p = path_of(g, in, depthwise);
    const ciw_win_layout lay = layout_of(p);
    const bool no_split = (flags & CIW_FLAG_NO_SPLIT) != 0;
    const bool generic = (flags & CIW_FLAG_GENERIC) != 0;
    const Fp32Kernel fp32_kernel = (flags & CIW_FLAG_FP32_MFMA) ? FP32_MATRIX
                                   : (flags & CIW_FLAG_FP32_VALU) ? FP32_VECTOR : FP32_AUTO;

    // chunk size: the most images whose workspace fits (the full batch if it does)
    int64_t nc = 0;
    if (ready) {
        if ((int64_t)ws_bytes < chunk_workspace(g, p, g.N)) return CIW_ERR_WORKSPACE;
        nc = g.N;
    } else {
        int64_t per = window_bytes_per_image(g, lay);
        int64_t hi = per > 0 ? (int64_t)ws_bytes / per : 0;
        if (hi > g.N) hi = g.N;
        for (int64_t n = hi; n >= 1; --n)
            if (chunk_workspace(g, p, n) <= (int64_t)ws_bytes) {
                nc = n;
                break;
            }
        if (nc == 0) return CIW_ERR_WORKSPACE;
    }

    if (noalloc && (s = scratch_of_current_device(&ws)) != CIW_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    (void)hipGetLastError();   // clear a stale error so launch checks report our own
    // the matrix-core kernel's filter copy sits after the window tensor of
    // the largest chunk; written once, used by every chunk
    unsigned char* aperm = nullptr;
    if (p == PATH_MFMA && !generic && mfma_prep_bytes(g) > 0) {
        aperm = (unsigned char*)ws + round_up(window_bytes_per_image(g, lay) * nc, 256);
        hipError_t e = launch_mfma_prep(g, out, w, aperm, st);
        if (e != hipSuccess) return from_hip(e);
    }
    const int64_t x_img = (int64_t)g.C * g.H * g.W * g.elem;
    const int64_t y_img = (int64_t)g.K * out_rows(g, epi) * out_cols(g, epi) * elem_bytes(out);
    unsigned char* wsb = (unsigned char*)ws;
    for (int64_t n0 = 0; n0 < g.N; n0 += nc) {
        const int n = (int)((g.N - n0) < nc ? (g.N - n0) : nc);
        const unsigned char* xc = x ? (const unsigned char*)x + n0 * x_img : nullptr;
        unsigned char* yc = (unsigned char*)y + n0 * y_img;
        if (!ready) {
            hipError_t e = launch_transform(g, in, lay, xc, wsb, n, st);
            if (e != hipSuccess) return from_hip(e);
        }
        hipError_t e;
        if (p == PATH_FP32) {
            // one slice count for every chunk, sized for the largest chunk, so a
            // smaller last chunk's partial sums fit where the first chunk's did
            int splits = no_split ? 1 : fp32_splits(g, (int)nc);
            float* partials = (float*)(wsb + round_up(window_bytes_per_image(g, lay) * nc, 256));
            e = launch_conv_fp32(g, (const float*)wsb, (const float*)w, (const float*)bias,
                                 (float*)yc, n, partials, splits, generic, fp32_kernel, epi, st);
        } else if (p == PATH_MFMA) {
            e = launch_conv_mfma(g, in, out, wsb, w, aperm, bias, yc, n, generic, epi, st);
        } else {
            e = launch_conv_dw(g, in, out, wsb, w, bias, yc, n, generic, epi, st);
        }
        if (e != hipSuccess) return from_hip(e);
    }
    return CIW_OK;
}

}  // namespace

hipError_t ciw::allow_dynamic_lds(const void* fn, size_t bytes) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, size_t> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    size_t& have = done[{dev, fn}];
    if (have >= bytes) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) have = bytes;
    return e;
}

extern "C" {

ciw_status conv_im2win_output_dims(const ciw_conv_desc* desc, int64_t* P, int64_t* Q) {
    Geom g;
    ciw_status s = resolve(desc, CIW_F32, &g);
    if (s != CIW_OK) return s;
    if (P) *P = g.P;
    if (Q) *Q = g.Q;
    return CIW_OK;
}

ciw_status conv2d_output_dims(const ciw_conv_desc* desc, uint32_t flags, int64_t* P, int64_t* Q) {
    Geom g;
    ciw_status s = resolve(desc, CIW_F32, &g);
    if (s != CIW_OK) return s;
    Epi epi;
    epi.pool = (flags & CIW_FLAG_MAXPOOL2) != 0;
    if (epi.pool && (g.P < 2 || g.Q < 2)) return CIW_ERR_INVALID_ARG;
    if (P) *P = out_rows(g, epi);
    if (Q) *Q = out_cols(g, epi);
    return CIW_OK;
}

ciw_status conv_im2win_window_geometry(const ciw_conv_desc* desc, ciw_dtype dtype,
                                       ciw_win_layout layout, int64_t* rows_per_image,
                                       int64_t* row_elems, int64_t* row_pitch) {
    if (!layout_ok(raw(layout)) || !dtype_ok(raw(dtype))) return CIW_ERR_INVALID_ARG;
    Geom g;
    ciw_status s = resolve(desc, dtype, &g);
    if (s != CIW_OK) return s;
    const bool chw = layout == CIW_WIN_CHW;
    if (rows_per_image) *rows_per_image = chw ? (int64_t)g.C * g.P : g.P;
    if (row_elems) *row_elems = chw ? g.lenA : g.lenB;
    if (row_pitch) *row_pitch = chw ? g.pitchA : g.pitchB;
    return CIW_OK;
}

ciw_status conv_im2win_window_bytes(const ciw_conv_desc* desc, ciw_dtype dtype,
                                    ciw_win_layout layout, int64_t n_images, size_t* bytes) {
    if (!layout_ok(raw(layout)) || !dtype_ok(raw(dtype))) return CIW_ERR_INVALID_ARG;
    if (!bytes || n_images < 0) return CIW_ERR_INVALID_ARG;
    Geom g;
    ciw_status s = resolve(desc, dtype, &g);
    if (s != CIW_OK) return s;
    int64_t total = 0;
    if (!mul_ok({window_bytes_per_image(g, layout), n_images}, &total)) return CIW_ERR_UNSUPPORTED;
    *bytes = (size_t)total;
    return CIW_OK;
}

ciw_status conv_im2win_transform(const ciw_conv_desc* desc, ciw_dtype dtype,
                                 ciw_win_layout layout, const void* x, void* x_win,
                                 void* stream) {
    if (!layout_ok(raw(layout)) || !dtype_ok(raw(dtype))) return CIW_ERR_INVALID_ARG;
    Geom g;
    ciw_status s = resolve(desc, dtype, &g);
    if (s != CIW_OK) return s;
    if (g.N == 0) return CIW_OK;
    if (!x || !x_win || !aligned(x, 16) || !aligned(x_win, 16)) return CIW_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return from_hip(launch_transform(g, dtype, layout, x, x_win, g.N, (hipStream_t)stream));
}

ciw_status conv2d_workspace_bytes(const ciw_conv_desc* desc, ciw_dtype in_dtype,
                                  int64_t n_images, size_t* bytes) {
    if (!bytes || n_images < 1 || !dtype_ok(raw(in_dtype))) return CIW_ERR_INVALID_ARG;
    Geom g;
    ciw_status s = resolve(desc, in_dtype, &g);
    if (s != CIW_OK) return s;
    bool dw = g.G > 1;
    if (dw && !(g.G == g.C && g.K == g.C)) return CIW_ERR_UNSUPPORTED;
    // a chunk never holds more than the batch (a larger n_images describes
    // the same single chunk); this also keeps the products below in range
    if (n_images > g.N && g.N > 0) n_images = g.N;
    *bytes = (size_t)chunk_workspace(g, path_of(g, in_dtype, dw), n_images);
    return CIW_OK;
}

ciw_status conv2d_implicit_workspace_bytes(const ciw_conv_desc* desc, ciw_dtype in_dtype,
                                           ciw_dtype out_dtype, uint32_t flags, size_t* bytes) {
    if (!bytes || !dtype_ok(raw(in_dtype)) || !dtype_ok(raw(out_dtype))) return CIW_ERR_INVALID_ARG;
    Geom g;
    ciw_status s = resolve(desc, in_dtype, &g);
    if (s != CIW_OK) return s;
    if (in_dtype == CIW_F32 ? out_dtype != CIW_F32 : (out_dtype != in_dtype && out_dtype != CIW_F32))
        return CIW_ERR_INVALID_ARG;
    Epi epi;
    epi.relu = (flags & CIW_FLAG_RELU) != 0;
    epi.pool = (flags & CIW_FLAG_MAXPOOL2) != 0;
    if (epi.pool && (g.P < 2 || g.Q < 2)) return CIW_ERR_INVALID_ARG;
    if (g.G > 1) {   // depthwise: no workspace
        if (!(g.G == g.C && g.K == g.C) || !dw_implicit_supported(g, epi)) return CIW_ERR_UNSUPPORTED;
        *bytes = 0;
        return CIW_OK;
    }
    size_t need = 0;
    const bool ok = in_dtype == CIW_F32 ? fp32_implicit_workspace(g, epi, &need)
                                        : implicit_workspace(g, out_dtype, epi, &need);
    if (!ok) return CIW_ERR_UNSUPPORTED;
    *bytes = need;
    return CIW_OK;
}

ciw_status conv2d_fwd(const ciw_conv_desc* desc, ciw_dtype in_dtype, ciw_dtype out_dtype,
                      const void* x, const void* w, const void* bias, void* y, void* workspace,
                      size_t workspace_bytes, uint32_t flags, void* stream) {
    if (!dtype_ok(raw(in_dtype)) || !dtype_ok(raw(out_dtype))) return CIW_ERR_INVALID_ARG;
    return run_conv(desc, in_dtype, out_dtype, x, w, bias, y, workspace, workspace_bytes, flags,
                    stream, false);
}

ciw_status conv2d_fwd_noalloc(const ciw_conv_desc* desc, ciw_dtype in_dtype, ciw_dtype out_dtype,
                              const void* x, const void* w, const void* bias, void* y,
                              uint32_t flags, void* stream) {
    if (!dtype_ok(raw(in_dtype)) || !dtype_ok(raw(out_dtype))) return CIW_ERR_INVALID_ARG;
    return run_conv(desc, in_dtype, out_dtype, x, w, bias, y, nullptr, 0, flags, stream, false,
                    true);
}

ciw_status conv2d_dw_fwd(const ciw_conv_desc* desc, ciw_dtype in_dtype, ciw_dtype out_dtype,
                         const void* x, const void* w, const void* bias, void* y,
                         void* workspace, size_t workspace_bytes, uint32_t flags,
                         void* stream) {
    if (!dtype_ok(raw(in_dtype)) || !dtype_ok(raw(out_dtype))) return CIW_ERR_INVALID_ARG;
    return run_conv(desc, in_dtype, out_dtype, x, w, bias, y, workspace, workspace_bytes, flags,
                    stream, true);
}

const char* conv_im2win_status_string(ciw_status status) {
    switch (raw(status)) {
        case CIW_OK: return "success";
        case CIW_ERR_INVALID_ARG: return "invalid argument";
        case CIW_ERR_UNSUPPORTED: return "unsupported convolution";
        case CIW_ERR_WORKSPACE: return "workspace too small";
        case CIW_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

}  // extern "C"
