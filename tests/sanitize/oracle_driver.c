/*
 * oracle_driver.c -- runs every entry point of the CPU oracle
 * (oracle/conv_oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer
 * on small layers chosen for their edges: padding wider than the filter's
 * reach, dilation, strides larger than the filter, grouped and depthwise
 * channels, 1x1 filters, one-pixel outputs, odd extents for the pool.  Every
 * buffer is allocated at exactly the size the oracle may touch, so a read or
 * write past it stops the run.  It also checks that the window-tensor
 * convolution (O3 on O2) agrees with the direct one (O1), so a driver that
 * ran on wrong sizes would not pass quietly.  Exit status 0: clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_out_dims(const int64_t* d, int64_t* P, int64_t* Q);
void oracle_conv2d(const int64_t* d, const double* x, const double* w, const double* b, double* y);
void oracle_conv2d_points(const int64_t* d, const double* x, const double* w, const double* b,
                          const int64_t* idx, int64_t npts, double* out);
int64_t oracle_win_width(const int64_t* d);
int64_t oracle_row_pitch(int64_t row_elems, int64_t elem_bytes);
int64_t oracle_row_elems(const int64_t* d, int layout);
void oracle_im2win(const int64_t* d, int layout, int64_t elem_bytes, const void* x, void* out);
void oracle_window_conv(const int64_t* d, int layout, const double* xw, const double* w,
                        const double* b, double* y);
void oracle_relu_pool(const int64_t* shape, int relu, int pool, const double* y, double* out);

static uint64_t rng_state = 12345;
static double rnd(void) {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) / 9007199254740992.0 - 0.5;
}

static double* fill(int64_t n) {
    double* a = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) a[i] = rnd();
    return a;
}

static int run(int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S,
               int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw, int64_t G) {
    const int64_t d[14] = {N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, G};
    int64_t P, Q;
    if (oracle_out_dims(d, &P, &Q)) return 0;   /* no output: nothing to run */
    double* x = fill(N * C * H * W);
    double* w = fill(K * (C / G) * R * S);
    double* b = fill(K);
    double* y = fill(N * K * P * Q);
    oracle_conv2d(d, x, w, b, y);
    /* a few points, the corners included */
    int64_t idx[4 * 4] = {0, 0, 0, 0, N - 1, K - 1, P - 1, Q - 1, 0, K - 1, P - 1, 0, N - 1, 0, 0, Q - 1};
    double pts[4];
    oracle_conv2d_points(d, x, w, b, idx, 4, pts);
    int bad = 0;
    for (int i = 0; i < 4; ++i) {
        const int64_t* p = idx + 4 * i;
        const double ref = y[((p[0] * K + p[1]) * P + p[2]) * Q + p[3]];
        if (fabs(pts[i] - ref) > 1e-12 * (1.0 + fabs(ref))) bad = 1;
    }
    /* the window tensor in both layouts, at every element size the library
     * uses, then O3 on the fp64 one */
    for (int layout = 0; layout < 2; ++layout) {
        const int64_t len = oracle_row_elems(d, layout);
        const int64_t rows = layout == 0 ? N * C * P : N * P;
        for (int eb = 2; eb <= 8; eb *= 2) {
            const int64_t pitch = oracle_row_pitch(len, eb);
            unsigned char* xs = (unsigned char*)malloc((size_t)(N * C * H * W * eb));
            for (int64_t i = 0; i < N * C * H * W * eb; ++i) xs[i] = (unsigned char)(i * 7);
            unsigned char* xw = (unsigned char*)malloc((size_t)(rows * pitch * eb));
            oracle_im2win(d, layout, eb, xs, xw);
            free(xs);
            free(xw);
        }
        if (G == 1 || layout == 0) {
            const int64_t pitch = oracle_row_pitch(len, 8);
            double* xw = (double*)malloc((size_t)(rows * pitch) * sizeof(double));
            oracle_im2win(d, layout, 8, x, xw);
            double* y3 = (double*)malloc((size_t)(N * K * P * Q) * sizeof(double));
            oracle_window_conv(d, layout, xw, w, b, y3);
            for (int64_t i = 0; i < N * K * P * Q; ++i)
                if (fabs(y3[i] - y[i]) > 1e-9 * (1.0 + fabs(y[i]))) bad = 1;
            free(y3);
            free(xw);
        }
    }
    /* O5 with and without the pool */
    const int64_t shape[4] = {N, K, P, Q};
    for (int relu = 0; relu < 2; ++relu)
        for (int pool = 0; pool < 2; ++pool) {
            const int64_t n_out = pool ? N * K * (P / 2) * (Q / 2) : N * K * P * Q;
            double* o = (double*)malloc((size_t)(n_out > 0 ? n_out : 1) * sizeof(double));
            oracle_relu_pool(shape, relu, pool, y, o);
            free(o);
        }
    free(x); free(w); free(b); free(y);
    if (bad) fprintf(stderr, "mismatch on layer N%lld C%lld H%lld W%lld K%lld %lldx%lld\n",
                     (long long)N, (long long)C, (long long)H, (long long)W, (long long)K,
                     (long long)R, (long long)S);
    return bad;
}

int main(void) {
    int bad = 0;
    /*       N  C   H   W  K  R  S sh sw ph pw dh dw G */
    bad |= run(1, 3, 7, 9, 4, 3, 3, 1, 1, 1, 1, 1, 1, 1);
    bad |= run(2, 4, 5, 6, 3, 3, 2, 2, 1, 4, 5, 1, 1, 1);    /* padding past the filter's reach */
    bad |= run(1, 2, 9, 8, 2, 3, 3, 1, 2, 2, 3, 2, 3, 1);    /* dilation, dil_h != dil_w */
    bad |= run(2, 6, 8, 7, 6, 2, 2, 3, 3, 0, 1, 1, 1, 3);    /* stride past the filter, groups */
    bad |= run(1, 5, 4, 5, 5, 3, 3, 1, 1, 1, 1, 1, 1, 5);    /* depthwise */
    bad |= run(3, 4, 3, 3, 2, 1, 1, 1, 1, 0, 0, 1, 1, 1);    /* 1x1 */
    bad |= run(1, 2, 3, 3, 2, 3, 3, 1, 1, 0, 0, 1, 1, 1);    /* one output pixel */
    bad |= run(2, 3, 5, 7, 4, 7, 7, 2, 2, 3, 3, 1, 1, 1);    /* stem-like, odd output for the pool */
    bad |= run(1, 1, 1, 1, 1, 1, 1, 1, 1, 0, 0, 1, 1, 1);    /* smallest */
    bad |= run(1, 2, 4, 4, 2, 3, 3, 1, 1, 0, 0, 2, 2, 1);    /* dilated filter wider than the input: no output */
    if (bad) return 1;
    printf("oracle under ASan/UBSan: clean\n");
    return 0;
}
