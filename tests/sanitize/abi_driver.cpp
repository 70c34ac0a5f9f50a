// abi_driver.cpp -- the library's host code (descriptor validation, output
// extents, window geometry, workspace and chunk arithmetic, the per-kernel
// plans) run under AddressSanitizer and UndefinedBehaviorSanitizer through
// the C ABI, on a few thousand descriptors: valid layers of every size, the
// edges (zero and one-pixel outputs, padding past the filter's reach), and
// invalid or wrapping ones (negative, zero, 2^31 .. 2^62 extents, products
// that wrap 64 bits).  Extents the library reports are checked against the
// same formulas evaluated here in 128-bit arithmetic.  The convolution
// entry points are called only when no GPU is visible: there every call
// stops at argument validation or at the first HIP call, which fails.
// Exit status 0: clean.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "conv_im2win.h"

typedef __int128 i128;

static uint64_t rs = 88172645463325252ull;
static uint64_t next() {
    rs ^= rs << 13;
    rs ^= rs >> 7;
    rs ^= rs << 17;
    return rs;
}
static int64_t pick(const int64_t* v, int n) { return v[next() % (uint64_t)n]; }

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { ++fails; if (fails < 20) { fprintf(stderr, __VA_ARGS__); fprintf(stderr, "\n"); } } } while (0)

// expected output extent, or -1 when no window fits
static i128 extent(i128 in, i128 k, i128 s, i128 p, i128 d) {
    const i128 span = d * (k - 1) + 1;
    if (in + 2 * p < span) return -1;
    return (in + 2 * p - span) / s + 1;
}

int main() {
    int ndev = 0;
    const bool gpu = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0;
    const int64_t ext[] = {0, 1, 2, 3, 7, 13, 14, 16, 32, 56, 64, 224, 512, 1000, 4096, 65535,
                           (1ll << 31) - 1, 1ll << 31, 1ll << 40, (1ll << 62) + 3, -1, -7};
    const int64_t small[] = {1, 1, 1, 2, 3, 3, 3, 5, 7, 11};
    const int64_t chan[] = {1, 2, 3, 8, 16, 32, 48, 64, 128, 512, 1024};
    const int32_t st[] = {1, 1, 1, 2, 3, 0, -1, 1 << 30};
    const int32_t pd[] = {0, 1, 1, 2, 3, 5, -1, 1 << 30};
    const int32_t dl[] = {1, 1, 1, 2, 3, 0, -2, 1 << 30};
    int valid = 0, checked = 0;
    for (int it = 0; it < 6000; ++it) {
        ciw_conv_desc d;
        const int mode = (int)(next() % 4);   // 0: wild extents; else a plausible layer
        d.N = mode == 0 ? pick(ext, 22) : pick(small, 10);
        d.C = mode == 0 ? pick(ext, 22) : pick(chan, 11);
        d.H = mode == 0 ? pick(ext, 22) : pick(ext, 13);
        d.W = mode == 0 ? pick(ext, 22) : pick(ext, 13);
        d.K = mode == 0 ? pick(ext, 22) : pick(chan, 11);
        d.R = mode == 0 ? pick(ext, 22) : pick(small, 10);
        d.S = mode == 0 ? pick(ext, 22) : pick(small, 10);
        d.stride_h = st[next() % 8]; d.stride_w = st[next() % 8];
        d.pad_h = pd[next() % 8]; d.pad_w = pd[next() % 8];
        d.dil_h = dl[next() % 8]; d.dil_w = dl[next() % 8];
        d.groups = (next() % 5 == 0) ? (int32_t)(d.C > 0 && d.C < (1 << 30) ? d.C : 1) : 1;
        if (next() % 7 == 0) d.groups = (int32_t)(next() % 5) - 1;

        int64_t P = -1, Q = -1;
        const ciw_status s = conv_im2win_output_dims(&d, &P, &Q);
        const bool sane = d.N >= 0 && d.C >= 1 && d.H >= 1 && d.W >= 1 && d.K >= 1 && d.R >= 1 &&
                          d.S >= 1 && d.stride_h >= 1 && d.stride_w >= 1 && d.pad_h >= 0 &&
                          d.pad_w >= 0 && d.dil_h >= 1 && d.dil_w >= 1 && d.groups >= 1;
        if (!sane) {
            CHECK(s != CIW_OK, "accepted an invalid descriptor (iteration %d)", it);
            continue;
        }
        const i128 eP = extent(d.H, d.R, d.stride_h, d.pad_h, d.dil_h);
        const i128 eQ = extent(d.W, d.S, d.stride_w, d.pad_w, d.dil_w);
        if (s == CIW_OK) {
            ++valid;
            CHECK(eP >= 1 && eQ >= 1 && P == (int64_t)eP && Q == (int64_t)eQ,
                  "output extent (%lld, %lld) on iteration %d", (long long)P, (long long)Q, it);
        } else {
            // refusals: no window fits, or a tensor too large to index
            CHECK(s == CIW_ERR_INVALID_ARG || s == CIW_ERR_UNSUPPORTED, "status %d", (int)s);
            continue;
        }
        for (uint32_t flags : {0u, (uint32_t)CIW_FLAG_RELU, (uint32_t)CIW_FLAG_MAXPOOL2}) {
            int64_t Po = -1, Qo = -1;
            const ciw_status so = conv2d_output_dims(&d, flags, &Po, &Qo);
            if (so == CIW_OK)
                CHECK((flags & CIW_FLAG_MAXPOOL2) ? (Po == P / 2 && Qo == Q / 2) : (Po == P && Qo == Q),
                      "pooled extent");
        }
        for (int dt = 0; dt < 3; ++dt)
            for (int lay = 0; lay < 2; ++lay) {
                int64_t rows = 0, elems = 0, pitch = 0;
                const ciw_status sg = conv_im2win_window_geometry(&d, (ciw_dtype)dt, (ciw_win_layout)lay,
                                                                  &rows, &elems, &pitch);
                for (int64_t n : {(int64_t)0, (int64_t)1, (int64_t)3, d.N, (int64_t)1 << 40}) {
                    size_t bytes = 0;
                    const ciw_status sb = conv_im2win_window_bytes(&d, (ciw_dtype)dt, (ciw_win_layout)lay, n, &bytes);
                    if (sg == CIW_OK && sb == CIW_OK) {
                        ++checked;
                        const i128 want = (i128)rows * pitch * (dt == 0 ? 4 : 2) * n;
                        CHECK((i128)bytes == want, "window bytes on iteration %d", it);
                    }
                }
                if (sg == CIW_OK) CHECK(elems <= pitch && pitch % (dt == 0 ? 4 : 8) == 0, "pitch");
            }
        for (int dt = 0; dt < 3; ++dt) {
            // (not monotone in the chunk: the fp32 channel slices fall as
            // the chunk grows; the library searches the chunk from the top)
            for (int64_t n : {(int64_t)1, (int64_t)2, (int64_t)5, d.N, (int64_t)1 << 50}) {
                size_t bytes = 0;
                (void)conv2d_workspace_bytes(&d, (ciw_dtype)dt, n, &bytes);
            }
            for (uint32_t flags : {(uint32_t)CIW_FLAG_IMPLICIT, (uint32_t)(CIW_FLAG_IMPLICIT | CIW_FLAG_RELU),
                                   (uint32_t)(CIW_FLAG_IMPLICIT | CIW_FLAG_MAXPOOL2)}) {
                size_t bytes = 0;
                (void)conv2d_implicit_workspace_bytes(&d, (ciw_dtype)dt, (ciw_dtype)dt, flags, &bytes);
                (void)conv2d_implicit_workspace_bytes(&d, (ciw_dtype)dt, CIW_F32, flags, &bytes);
            }
        }
        if (!gpu) {
            // the convolution entry points: argument checks, chunk arithmetic
            // for small workspaces, then the first HIP call fails
            char buf[64];
            void* p = buf;
            for (size_t ws : {(size_t)0, (size_t)64, (size_t)1 << 20, (size_t)1 << 40}) {
                (void)conv2d_fwd(&d, CIW_F32, CIW_F32, p, p, nullptr, p, p, ws, 0, nullptr);
                (void)conv2d_fwd(&d, CIW_F16, CIW_F16, p, p, p, p, p, ws, CIW_FLAG_RELU, nullptr);
                (void)conv2d_fwd(&d, CIW_BF16, CIW_F32, p, p, p, p, p, ws, CIW_FLAG_IMPLICIT, nullptr);
                (void)conv2d_dw_fwd(&d, CIW_F32, CIW_F32, p, p, p, p, p, ws, 0, nullptr);
            }
            (void)conv2d_fwd_noalloc(&d, CIW_F16, CIW_F16, p, p, nullptr, p, 0, nullptr);
            (void)conv_im2win_transform(&d, CIW_F32, CIW_WIN_CHW, p, p, nullptr);
            CHECK(conv2d_fwd(&d, CIW_F32, CIW_F32, nullptr, p, nullptr, p, p, 64, 0, nullptr) != CIW_OK,
                  "accepted a null input");
        }
    }
    for (int s = -6; s <= 1; ++s) (void)conv_im2win_status_string((ciw_status)s);
    // enum arguments outside their enumerations (a C caller may pass any int)
    {
        ciw_conv_desc d = {1, 16, 8, 8, 16, 3, 3, 1, 1, 1, 1, 1, 1, 1};
        int64_t a = 0, b = 0, c = 0;
        size_t bytes = 0;
        for (int bad : {-1, 3, 7, 1 << 20}) {
            CHECK(conv_im2win_window_geometry(&d, (ciw_dtype)bad, CIW_WIN_CHW, &a, &b, &c) == CIW_ERR_INVALID_ARG, "dtype %d", bad);
            CHECK(conv_im2win_window_geometry(&d, CIW_F32, (ciw_win_layout)bad, &a, &b, &c) == CIW_ERR_INVALID_ARG, "layout %d", bad);
            CHECK(conv_im2win_window_bytes(&d, (ciw_dtype)bad, CIW_WIN_HWC, 1, &bytes) == CIW_ERR_INVALID_ARG, "dtype %d", bad);
            CHECK(conv2d_workspace_bytes(&d, (ciw_dtype)bad, 1, &bytes) == CIW_ERR_INVALID_ARG, "dtype %d", bad);
            CHECK(conv2d_implicit_workspace_bytes(&d, (ciw_dtype)bad, CIW_F16, CIW_FLAG_IMPLICIT, &bytes) == CIW_ERR_INVALID_ARG, "dtype %d", bad);
            CHECK(conv2d_implicit_workspace_bytes(&d, CIW_F16, (ciw_dtype)bad, CIW_FLAG_IMPLICIT, &bytes) == CIW_ERR_INVALID_ARG, "dtype %d", bad);
            char buf[64];
            CHECK(conv2d_fwd(&d, (ciw_dtype)bad, CIW_F32, buf, buf, nullptr, buf, buf, 64, 0, nullptr) == CIW_ERR_INVALID_ARG, "dtype %d", bad);
            CHECK(conv2d_dw_fwd(&d, CIW_F32, (ciw_dtype)bad, buf, buf, nullptr, buf, buf, 64, 0, nullptr) == CIW_ERR_INVALID_ARG, "dtype %d", bad);
            CHECK(conv2d_fwd_noalloc(&d, (ciw_dtype)bad, CIW_F16, buf, buf, nullptr, buf, 0, nullptr) == CIW_ERR_INVALID_ARG, "dtype %d", bad);
            CHECK(conv_im2win_transform(&d, CIW_F16, (ciw_win_layout)bad, buf, buf, nullptr) == CIW_ERR_INVALID_ARG, "layout %d", bad);
        }
    }
    CHECK(conv_im2win_output_dims(nullptr, nullptr, nullptr) != CIW_OK, "null descriptor");
    if (fails) {
        fprintf(stderr, "%d check(s) failed\n", fails);
        return 1;
    }
    printf("host ABI under ASan/UBSan: clean (%d valid descriptors, %d window sizes checked, GPU %s)\n",
           valid, checked, gpu ? "visible: convolution entry points not called" : "absent");
    return 0;
}
