/*
 * conv_oracle.c -- CPU oracle for forward 2-D convolution and the im2win
 * window tensor.  TEST INFRASTRUCTURE: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library; it is plain C, fp64, no intrinsics,
 * no fast-math, and deliberately slow and obvious.
 *
 * Pages it follows:
 *   [IM2WIN]  "Enabling Memory-efficient Im2win Convolution with
 *             Multi-precision Support on GPU CUDA and Tensor Cores"
 *   [OCL]     "OpenCL-Benchmarks" (atranitell), "Setting: normal" kernel
 *   [CS149]   "CS149 L9: Running DNNs Efficiently on GPUs ...",
 *             "The direct version: seven nested loops"
 *
 * Descriptor: every entry point takes `const int64_t d[14]` =
 *   { N, C, H, W, K, R, S, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups }
 * Tensors are dense row-major: x[N][C][H][W], w[K][C/groups][R][S], b[K],
 * y[N][K][P][Q].
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

enum { DN, DC, DH, DW, DK, DR, DS, DSH, DSW, DPH, DPW, DDH, DDW, DG, DLEN };

/* Output extent along one axis: the number of window positions whose
 * (dilated) extent fits in the zero-padded input.  [OCL] passes out_h/out_w
 * in as arguments; this is the usual floor formula, restated as a count. */
static int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p, int64_t dil) {
    int64_t span = dil * (k - 1) + 1;
    int64_t padded = in + 2 * p;
    if (padded < span || s <= 0) return 0;
    return (padded - span) / s + 1;
}

int oracle_out_dims(const int64_t* d, int64_t* P, int64_t* Q) {
    *P = out_extent(d[DH], d[DR], d[DSH], d[DPH], d[DDH]);
    *Q = out_extent(d[DW], d[DS], d[DSW], d[DPW], d[DDW]);
    return (*P > 0 && *Q > 0) ? 0 : -1;
}

/* x with zero padding: the bounds test of the [OCL] kernel, which skips taps
 * that fall outside [0,H) x [0,W). */
static double x_at(const int64_t* d, const double* x, int64_t n, int64_t c,
                   int64_t ih, int64_t iw) {
    if (ih < 0 || ih >= d[DH] || iw < 0 || iw >= d[DW]) return 0.0;
    return x[((n * d[DC] + c) * d[DH] + ih) * d[DW] + iw];
}

/* One output element of the direct convolution (cross-correlation: input and
 * filter indices advance together, no flip), bias added after the sum, as in
 * the [OCL] kernel.  Grouped: output channel k sees input channels
 * [g*C/G, (g+1)*C/G) with g = k / (K/G). */
static double direct_point(const int64_t* d, const double* x, const double* w,
                           const double* b, int64_t n, int64_t k, int64_t h,
                           int64_t wo) {
    const int64_t Cg = d[DC] / d[DG], Kg = d[DK] / d[DG];
    const int64_t c0 = (k / Kg) * Cg;
    double acc = 0.0;
    for (int64_t c = 0; c < Cg; ++c)
        for (int64_t r = 0; r < d[DR]; ++r)
            for (int64_t q = 0; q < d[DS]; ++q) {
                int64_t ih = h * d[DSH] - d[DPH] + r * d[DDH];
                int64_t iw = wo * d[DSW] - d[DPW] + q * d[DDW];
                acc += x_at(d, x, n, c0 + c, ih, iw) *
                       w[((k * Cg + c) * d[DR] + r) * d[DS] + q];
            }
    return b ? acc + b[k] : acc;
}

/* O1: the seven-loop direct convolution ([CS149] "seven nested loops";
 * [IM2WIN] §III-C notes im2win has the same loop nest and complexity).
 * Parallel over (n, k) only. */
void oracle_conv2d(const int64_t* d, const double* x, const double* w,
                   const double* b, double* y) {
    int64_t P, Q;
    if (oracle_out_dims(d, &P, &Q)) return;
    const int64_t NK = d[DN] * d[DK];
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t nk = 0; nk < NK; ++nk) {
        int64_t n = nk / d[DK], k = nk % d[DK];
        for (int64_t h = 0; h < P; ++h)
            for (int64_t wo = 0; wo < Q; ++wo)
                y[(nk * P + h) * Q + wo] = direct_point(d, x, w, b, n, k, h, wo);
    }
}

/* O1 at chosen outputs: idx holds npts quadruples (n, k, h, w). */
void oracle_conv2d_points(const int64_t* d, const double* x, const double* w,
                          const double* b, const int64_t* idx, int64_t npts,
                          double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npts; ++i)
        out[i] = direct_point(d, x, w, b, idx[4 * i], idx[4 * i + 1],
                              idx[4 * i + 2], idx[4 * i + 3]);
}

/* ------------------------------------------------------------------ im2win */
/* Columns of the padded input that the windows of one output row touch:
 * the last window starts at column (Q-1)*stride_w and spans dil_w*(S-1)+1.
 * ([IM2WIN] §III-B: the window tensor keeps each input element of a row band
 * once, instead of once per window as im2col does.) */
int64_t oracle_win_width(const int64_t* d) {
    int64_t P, Q;
    if (oracle_out_dims(d, &P, &Q)) return 0;
    return (Q - 1) * d[DSW] + d[DDW] * (d[DS] - 1) + 1;
}

/* Row pitch in elements: the row length rounded up to 16 bytes. */
int64_t oracle_row_pitch(int64_t row_elems, int64_t elem_bytes) {
    int64_t v = 16 / elem_bytes;
    return (row_elems + v - 1) / v * v;
}

/* Elements of one window-tensor row: layout 0 (channel-planar) holds one
 * channel, layout 1 (channel-innermost) holds all C channels. */
int64_t oracle_row_elems(const int64_t* d, int layout) {
    int64_t ww = oracle_win_width(d);
    return layout == 0 ? ww * d[DR] : ww * d[DR] * d[DC];
}

/* O2: the im2win repack, as a pure copy of element bit patterns.
 *
 * [IM2WIN] §III-B/§III-C: one window-tensor row holds the R input rows that
 * feed one output row, laid out column by column with the R values of a
 * column adjacent ("height before width"), so the window of output column w
 * is the contiguous run that starts stride_w*R elements after the window of
 * column w-1.  [IM2WIN] §III-D uses the NHWC order on tensor cores: there
 * the C channels of each (column, filter-row) pair are innermost.
 *
 *   layout 0: xw[n][c][h][ (x*R + r) ]        , pitch = roundup(Wwin*R)
 *   layout 1: xw[n][h][ (x*R + r)*C + c ]     , pitch = roundup(Wwin*R*C)
 * value = x[n][c][h*stride_h - pad_h + r*dil_h][x - pad_w], zero outside the
 * input; the tail of each row from the row length up to the pitch is zero. */
void oracle_im2win(const int64_t* d, int layout, int64_t elem_bytes,
                   const void* xv, void* outv) {
    int64_t P, Q;
    if (oracle_out_dims(d, &P, &Q)) return;
    const unsigned char* x = (const unsigned char*)xv;
    unsigned char* out = (unsigned char*)outv;
    const int64_t N = d[DN], C = d[DC], H = d[DH], W = d[DW], R = d[DR];
    const int64_t ww = oracle_win_width(d);
    const int64_t len = oracle_row_elems(d, layout);
    const int64_t pitch = oracle_row_pitch(len, elem_bytes);
    const int64_t rows = layout == 0 ? N * C * P : N * P;
    memset(out, 0, (size_t)(rows * pitch * elem_bytes));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < C; ++c)
            for (int64_t h = 0; h < P; ++h)
                for (int64_t xc = 0; xc < ww; ++xc)
                    for (int64_t r = 0; r < R; ++r) {
                        int64_t ih = h * d[DSH] - d[DPH] + r * d[DDH];
                        int64_t iw = xc - d[DPW];
                        int64_t dst;
                        if (layout == 0)
                            dst = ((n * C + c) * P + h) * pitch + xc * R + r;
                        else
                            dst = (n * P + h) * pitch + (xc * R + r) * C + c;
                        if (ih < 0 || ih >= H || iw < 0 || iw >= W) continue;
                        int64_t src = ((n * C + c) * H + ih) * W + iw;
                        memcpy(out + dst * elem_bytes, x + src * elem_bytes,
                               (size_t)elem_bytes);
                    }
}

/* O3: convolution that reads its inputs only from an fp64 window tensor made
 * by O2.  The window of output (n,k,h,w) is, for each filter column q, the R
 * (layout 0) or R*C (layout 1) contiguous elements starting at column
 * w*stride_w + q*dil_w; the filter is read height before width ([IM2WIN]
 * §III-C).  Must agree with O1 up to rounding order. */
void oracle_window_conv(const int64_t* d, int layout, const double* xw,
                        const double* w, const double* b, double* y) {
    int64_t P, Q;
    if (oracle_out_dims(d, &P, &Q)) return;
    const int64_t C = d[DC], K = d[DK], R = d[DR], S = d[DS];
    const int64_t Cg = C / d[DG], Kg = K / d[DG];
    const int64_t len = oracle_row_elems(d, layout);
    const int64_t pitch = oracle_row_pitch(len, 8);  /* fp64 copy: 16 B = 2 */
    const int64_t NK = d[DN] * K;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t nk = 0; nk < NK; ++nk) {
        int64_t n = nk / K, k = nk % K, c0 = (k / Kg) * Cg;
        for (int64_t h = 0; h < P; ++h)
            for (int64_t wo = 0; wo < Q; ++wo) {
                double acc = 0.0;
                for (int64_t c = 0; c < Cg; ++c)
                    for (int64_t q = 0; q < S; ++q)
                        for (int64_t r = 0; r < R; ++r) {
                            int64_t col = wo * d[DSW] + q * d[DDW];
                            double v;
                            if (layout == 0)
                                v = xw[((n * C + c0 + c) * P + h) * pitch + col * R + r];
                            else
                                v = xw[(n * P + h) * pitch + (col * R + r) * C + c0 + c];
                            acc += v * w[((k * Cg + c) * R + r) * S + q];
                        }
                y[(nk * P + h) * Q + wo] = b ? acc + b[k] : acc;
            }
    }
}

/* O5: the fused epilogue of the conv -> scale/bias -> max-pool chain
 * ([CS149] "Fusion: keep intermediates out of memory", slides 56-57),
 * applied to a biased convolution output y[N][K][P][Q] (O1's result):
 *   - relu != 0: each value becomes max(v, 0) (the ReLU of [CS149] slide 14);
 *   - pool != 0: out[n][k][j][i] is the largest of the 2x2 region
 *     y[n][k][2j .. 2j+1][2i .. 2i+1] ("max over each 2x2 region", slide 23):
 *     non-overlapping regions, so out is [N][K][P/2][Q/2] (floor: an odd
 *     last row or column belongs to no region and is dropped).
 * Every maximum is IEEE-754 maxNum (C's fmax): a NaN loses to a number.
 * shape = { N, K, P, Q }. */
static double act(double v, int relu) { return relu ? fmax(v, 0.0) : v; }

void oracle_relu_pool(const int64_t* shape, int relu, int pool, const double* y, double* out) {
    const int64_t N = shape[0], K = shape[1], P = shape[2], Q = shape[3];
    if (!pool) {
        for (int64_t i = 0; i < N * K * P * Q; ++i) out[i] = act(y[i], relu);
        return;
    }
    const int64_t P2 = P / 2, Q2 = Q / 2;
    for (int64_t nk = 0; nk < N * K; ++nk)
        for (int64_t j = 0; j < P2; ++j)
            for (int64_t i = 0; i < Q2; ++i) {
                double m = act(y[(nk * P + 2 * j) * Q + 2 * i], relu);
                for (int64_t dy = 0; dy < 2; ++dy)
                    for (int64_t dx = 0; dx < 2; ++dx)
                        m = fmax(m, act(y[(nk * P + 2 * j + dy) * Q + 2 * i + dx], relu));
                out[(nk * P2 + j) * Q2 + i] = m;
            }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
