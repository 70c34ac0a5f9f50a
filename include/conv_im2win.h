/*
 * conv_im2win.h -- C ABI of the im2win forward-convolution library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the im2win ("image to window") paradigm of "Enabling
 * Memory-efficient Im2win Convolution with Multi-precision Support on GPU
 * CUDA and Tensor Cores" (below: the im2win paper):
 *   1. the input is repacked once into a window tensor in which the inputs
 *      of every output row sit in one contiguous row (§III-B, §III-C);
 *   2. a windowed dot product contracts each output's contiguous window with
 *      the filter (§III-C), in fp32 on the vector ALUs or the fp32 matrix
 *      cores and in fp16/bf16 on the matrix cores with fp32 accumulation
 *      (§III-D, §III-F).
 * The problem statement (N, C, H, W, K, R, S, stride, padding, dilation,
 * bias; zero padding; cross-correlation; bias added after the sum) is the one
 * of the OpenCL-Benchmarks page's direct "conv2d" kernel ("Setting: normal").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *   never allocates, frees or synchronises; work is enqueued on `stream`
 *   (a hipStream_t; NULL means the null stream) and completes
 *   asynchronously.  Calls on different streams may run concurrently if
 *   their buffers do not overlap.  The only state kept between calls is,
 *   per device, which kernels have already been allowed more than 64 KB of
 *   dynamic LDS (set once, under a lock, on a kernel's first launch).
 * - Arguments are validated BEFORE anything is enqueued; on any error status
 *   nothing has been launched and no buffer has been touched.
 * - Tensors are dense and contiguous: x is NCHW [N][C][H][W]; the filters w
 *   are KCRS [K][C/groups][R][S] (R = filter height, S = filter width); bias
 *   is [K] and may be NULL; y is NCHW [N][K][P][Q] ([N][K][P/2][Q/2] with
 *   CIW_FLAG_MAXPOOL2).
 * - x, w, y and workspace must be 16-byte aligned; bias must be aligned to
 *   its element size.  Every tensor must hold fewer than 2^31 elements.
 * - Element types: input, filter and bias share `in_dtype`.  Allowed
 *   (in -> out) pairs: F32->F32, F16->F16, F16->F32, BF16->BF16, BF16->F32.
 *   Products are accumulated in fp32, the bias is added in fp32, and the
 *   result is rounded once (round-to-nearest-even) to the output type.
 */
#ifndef CONV_IM2WIN_H
#define CONV_IM2WIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CIW_OK = 0,
    CIW_ERR_INVALID_ARG = -1,   /* bad descriptor, NULL/misaligned pointer, bad dtype pair */
    CIW_ERR_UNSUPPORTED = -2,   /* valid convolution this library does not run (e.g. groups
                                   other than 1 or C, a tensor with >= 2^31 elements) */
    CIW_ERR_WORKSPACE = -3,     /* workspace smaller than one image needs */
    CIW_ERR_HIP = -4            /* a HIP launch or runtime call failed */
} ciw_status;

typedef enum { CIW_F32 = 0, CIW_F16 = 1, CIW_BF16 = 2 } ciw_dtype;

/* Window-tensor layouts.
 * CIW_WIN_CHW (channel-planar): one row per (n, c, output row h):
 *     xw[n][c][h][x*R + r]
 * CIW_WIN_HWC (channel-innermost, the NHWC-based variant the im2win paper
 *     uses on tensor cores, §III-D): one row per (n, output row h):
 *     xw[n][h][(x*R + r)*C + c]
 * with value x[n][c][h*stride_h - pad_h + r*dil_h][x - pad_w] (zero outside
 * the input) for columns x in [0, Wwin), Wwin = (Q-1)*stride_w +
 * dil_w*(S-1) + 1.  Rows are padded with zeros to a pitch that is a multiple
 * of 16 bytes.  The window of output (h, w) is, for each filter column q, the
 * R (CHW) or R*C (HWC) contiguous elements at column w*stride_w + q*dil_w;
 * with dil_w = 1 the whole window is one contiguous run (the filter height
 * index varies before the width, §III-C). */
typedef enum { CIW_WIN_CHW = 0, CIW_WIN_HWC = 1 } ciw_win_layout;

/* Convolution descriptor.  groups must divide C and K; the library runs
 * groups == 1 (dense) and groups == C == K (depthwise). */
typedef struct {
    int64_t N, C, H, W;        /* input batch, channels, height, width */
    int64_t K, R, S;           /* output channels, filter height, filter width */
    int32_t stride_h, stride_w;
    int32_t pad_h, pad_w;      /* zero padding on each side */
    int32_t dil_h, dil_w;      /* dilation (>= 1) */
    int32_t groups;
} ciw_conv_desc;

/* conv2d_fwd / conv2d_dw_fwd flags. */
#define CIW_FLAG_WINDOW_READY 0x1u  /* workspace already holds the full-batch window tensor
                                       of x (made by conv_im2win_transform with the layout
                                       the call uses); the repack is skipped, x may be NULL */
#define CIW_FLAG_NO_SPLIT     0x2u  /* fp32 dense: never split the channel sum across
                                       workgroups (a single pass, no partial sums) */
#define CIW_FLAG_GENERIC      0x4u  /* use the shape-generic kernels only (testing aid) */
/* Fused epilogue ("CS149 L9: Running DNNs Efficiently on GPUs ...", "Fusion:
 * keep intermediates out of memory": conv -> scale/bias -> max pool, with the
 * ReLU and 2x2 pooling of its slides 14 and 23).  Applied to the biased fp32
 * sums inside the contraction kernels, so the unpooled output never reaches
 * memory.  Maxima are IEEE-754 maxNum (a NaN loses to a number). */
#define CIW_FLAG_RELU         0x8u  /* y = max(y, 0) after the bias */
#define CIW_FLAG_MAXPOOL2     0x10u /* y[n][k][j][i] = max of the 2x2 region at rows 2j..2j+1,
                                       columns 2i..2i+1 (after the ReLU, if any): y is
                                       [N][K][P/2][Q/2] (floor; an odd last row or column
                                       is dropped).  CIW_ERR_INVALID_ARG if P or Q < 2. */

/* On-the-fly windows: the contraction builds its windows in LDS straight
 * from x and never writes the window tensor to memory (the im2win paper's
 * memory concern, §III-B and the processing strategies of §IV-D1, taken to
 * its end).  The result is the same sum in another order.
 *   conv2d_fwd, fp16/bf16 input, one of three kernels:
 *   - 3x3 filters, stride_h 1, C a multiple of 16 up to 64, K <= 64, W a
 *     multiple of 8, no pool: one kernel, filter re-layout included, no
 *     workspace;
 *   - the other layers with C a multiple of 16 that the row-band kernel
 *     runs (see conv2d_implicit_workspace_bytes), with the fused pool: the
 *     workspace holds a re-laid-out copy of the filter;
 *   - layers with few input channels and an even horizontal stride (C R <=
 *     22, such as the 3-channel 7x7 stride-2 stem), no pool: one kernel,
 *     filter included, no workspace;
 *   conv2d_fwd, fp32 (3x3 and 1x1 filters, no pool), one of two kernels:
 *   - C a multiple of 4: the whole-sum matrix-core kernel (16 output
 *     channels x 48 pixels and the whole channel sum a workgroup) with each
 *     group of 4 channels' input rows staged in LDS; no workspace;
 *   - otherwise the split matrix-core kernel with each pixel block's
 *     zero-padded input rows staged in LDS; the workspace holds only the
 *     channel slices' partial sums (0 bytes when the sum is not split);
 *   conv2d_dw_fwd (any input type): each workgroup stages whole zero-padded
 *     input planes in LDS and computes their outputs there; no workspace.
 * conv2d_implicit_workspace_bytes gives the workspace (0 bytes: workspace
 * may be NULL); layers none of these kernels run return
 * CIW_ERR_UNSUPPORTED.  Not allowed with CIW_FLAG_WINDOW_READY or
 * CIW_FLAG_GENERIC (CIW_ERR_INVALID_ARG). */
#define CIW_FLAG_IMPLICIT     0x20u
/* fp32 dense (conv2d_fwd) kernel choice.  By default the contraction runs
 * on the matrix cores: with the whole channel sum in one workgroup
 * (v_mfma_f32_16x16x4_f32, 16 output channels x 48 pixels; 3x3 and 1x1
 * filters, C a multiple of 4, no CIW_FLAG_MAXPOOL2; one kernel, no partial
 * sums), else with the channel sum split over workgroups
 * (v_mfma_f32_32x32x2_f32; 3x3 and 1x1 filters, output rows of at most 192
 * pixels, no pool) where that plan has at least 4 slices; otherwise on the
 * vector ALUs.  CIW_FLAG_FP32_MFMA forces the matrix cores wherever one of
 * those kernels runs the layer, CIW_FLAG_FP32_VALU forces the vector ALUs
 * (both: CIW_ERR_INVALID_ARG).  Every sum is deterministic (fixed orders)
 * and the same sum in another order.  Ignored for fp16/bf16;
 * CIW_FLAG_GENERIC implies the vector ALUs; with CIW_FLAG_NO_SPLIT only the
 * whole-sum kernel or the vector ALUs run. */
#define CIW_FLAG_FP32_MFMA    0x40u
#define CIW_FLAG_FP32_VALU    0x80u

/* Output extent: P = floor((H + 2 pad_h - dil_h (R-1) - 1) / stride_h) + 1,
 * Q likewise.  The OpenCL-Benchmarks page's conv2d kernel takes out_h and
 * out_w as arguments without saying how they are formed; its layer table
 * ("Convolution Ops Analysis": 13x13 in, 3x3, stride 1, padding 1, 13x13
 * out) fits this floor formula, the reading taken here.  Returns
 * CIW_ERR_INVALID_ARG if the descriptor is invalid or the window does not
 * fit the padded input, CIW_ERR_UNSUPPORTED if a tensor of the layer has
 * 2^31 or more elements. */
ciw_status conv_im2win_output_dims(const ciw_conv_desc* desc, int64_t* P, int64_t* Q);

/* Extent of the output conv2d_fwd / conv2d_dw_fwd write with these flags:
 * (P, Q) as above, or (P/2, Q/2) with CIW_FLAG_MAXPOOL2, the max over each
 * 2x2 region ("CS149 L9", slide 23; the pool fused after the conv as in
 * "Fusion: keep intermediates out of memory"); CIW_ERR_INVALID_ARG if P or
 * Q < 2.  Other flag bits are ignored here. */
ciw_status conv2d_output_dims(const ciw_conv_desc* desc, uint32_t flags, int64_t* P, int64_t* Q);

/* Geometry of the window tensor of ONE image (the im2win paper, §III-B:
 * one row per output row holding the input columns its windows cover;
 * §III-D for the channel-innermost variant): number of rows (C*P for CHW,
 * P for HWC), elements per row before padding, and the row pitch in
 * elements.  Any output pointer may be NULL. */
ciw_status conv_im2win_window_geometry(const ciw_conv_desc* desc, ciw_dtype dtype,
                                       ciw_win_layout layout, int64_t* rows_per_image,
                                       int64_t* row_elems, int64_t* row_pitch);

/* Bytes of the window tensor of n_images images, pitch included: the
 * memory cost of the repack that the im2win paper weighs against the
 * im2col matrix (§III-B).  CIW_ERR_UNSUPPORTED if the size does not fit in
 * 62 bits. */
ciw_status conv_im2win_window_bytes(const ciw_conv_desc* desc, ciw_dtype dtype,
                                    ciw_win_layout layout, int64_t n_images, size_t* bytes);

/* im2win repack (the im2win paper §III-B, §III-C; §III-D for the HWC
 * layout).  Writes the full-batch window tensor of x, pitch tails zeroed, to
 * x_win (conv_im2win_window_bytes(desc, dtype, layout, N) bytes, 16-byte
 * aligned).  A pure data movement: the result is bit-exact. */
ciw_status conv_im2win_transform(const ciw_conv_desc* desc, ciw_dtype dtype,
                                 ciw_win_layout layout, const void* x, void* x_win,
                                 void* stream);

/* Workspace conv2d_fwd / conv2d_dw_fwd need to process n_images images per
 * chunk (the window tensor of the chunk plus any partial sums): the
 * single-batch / mini-batch / full-batch processing strategies of the im2win
 * paper (§IV-D1) are n_images = 1, 1 < n_images < N and n_images = N (a
 * larger n_images gives the n_images = N size).  The minimum usable
 * workspace is the n_images = 1 size. */
ciw_status conv2d_workspace_bytes(const ciw_conv_desc* desc, ciw_dtype in_dtype,
                                  int64_t n_images, size_t* bytes);

/* Workspace conv2d_fwd / conv2d_dw_fwd need with CIW_FLAG_IMPLICIT for this
 * layer, output type and epilogue flags.  CIW_ERR_UNSUPPORTED for layers no
 * in-LDS kernel runs.
 * Depthwise (groups == C == K): 0 bytes; unsupported if a zero-padded input
 * plane and its filter exceed 48 KB of LDS.
 * Dense fp16/bf16 (groups == 1), the first kernel that runs the layer:
 *   - 0 bytes: 3x3 filter, stride_h 1, C a multiple of 16 up to 64, K <= 64,
 *     W a multiple of 8, no CIW_FLAG_MAXPOOL2;
 *   - the re-laid-out filter: C a multiple of 16, K <= 64, W a multiple of 8,
 *     stride_h == 1, a 3x3 filter with C <= 64 or 1x1 with C in {16, 32, 64},
 *     a stored output row needing at most 4 stores per thread (K*Qs/E <=
 *     1024, where Qs is Q, or Q/2 with CIW_FLAG_MAXPOOL2, and E the largest
 *     power of two that divides Qs with E * output element bytes <= 16);
 *     ReLU and the 2x2 max-pool fused;
 *   - 0 bytes: C R <= 22, K <= 64, stride_w even, dil_w == 1, W a multiple of
 *     8, 6 <= S + d <= 8 where d = (L - pad_w) mod 2 and L is pad_w rounded
 *     up to a multiple of 4, no CIW_FLAG_MAXPOOL2 (ReLU fused);
 *   all with K times the output plane and an image of x below 2^31 elements.
 * Dense fp32, 3x3 or 1x1 filter, no CIW_FLAG_MAXPOOL2, the first kernel
 *   that runs the layer:
 *   - 0 bytes: C a multiple of 4, W >= 4, and the input rows that 48
 *     consecutive output pixels span, rows = (n - 1) stride_h + (R - 1)
 *     dil_h + 1 with n = min(P, floor(47 / Q) + 2), with rows * W <= 448
 *     for 3x3 (576 for 1x1);
 *   - Q <= 192, C >= 2, and the zero-padded input rows of one 16-channel
 *     chunk of a pixel block at most 5120 elements; the workspace is the
 *     channel slices' partial sums, splits x N x K x P x Q x 4 bytes (0 when
 *     the sum is not split). */
ciw_status conv2d_implicit_workspace_bytes(const ciw_conv_desc* desc, ciw_dtype in_dtype,
                                           ciw_dtype out_dtype, uint32_t flags, size_t* bytes);

/* Dense forward convolution (groups == 1), im2win method: for each batch
 * chunk, the repack into `workspace` followed by the windowed contraction
 * (the im2win paper §III-C..§III-F; the problem statement is that of the
 * OpenCL-Benchmarks page's conv2d kernel).  fp32 uses the CHW window layout
 * and the fp32 matrix cores or the vector ALUs (see CIW_FLAG_FP32_MFMA);
 * fp16/bf16 use the HWC layout and the matrix cores with fp32
 * accumulation.  The chunk size is the largest number of images whose
 * workspace (conv2d_workspace_bytes) fits in workspace_bytes, capped at N;
 * CIW_ERR_WORKSPACE if not even one image fits.  With
 * CIW_FLAG_WINDOW_READY the workspace must hold the full-batch window
 * tensor at offset 0 and be at least conv2d_workspace_bytes(desc, in, N).
 * With CIW_FLAG_IMPLICIT the window rows are built in LDS instead (see that
 * flag) and the workspace must hold conv2d_implicit_workspace_bytes. */
ciw_status conv2d_fwd(const ciw_conv_desc* desc, ciw_dtype in_dtype, ciw_dtype out_dtype,
                      const void* x, const void* w, const void* bias, void* y,
                      void* workspace, size_t workspace_bytes, uint32_t flags,
                      void* stream);

/* Size of the device array conv2d_fwd_noalloc uses as its workspace. */
#define CIW_NOALLOC_SCRATCH_BYTES (32u << 20)

/* conv2d_fwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is
 * a file-scope device array of the library, CIW_NOALLOC_SCRATCH_BYTES bytes
 * per GPU, held from the first call on that GPU until the process ends; the
 * batch is processed in chunks of as many images as fit in it (see
 * conv2d_workspace_bytes), with CIW_FLAG_IMPLICIT the array holds the
 * in-LDS path's workspace (the re-laid-out filter or the fp32 partial
 * sums; nothing for the single-kernel forms).  Same arguments, flags and results as conv2d_fwd
 * otherwise.  Errors (before anything is enqueued): CIW_ERR_WORKSPACE if
 * one image's workspace (or the CIW_FLAG_IMPLICIT workspace) exceeds the
 * array; CIW_ERR_INVALID_ARG with CIW_FLAG_WINDOW_READY (the array cannot
 * hold a window tensor the caller prepared); CIW_ERR_HIP if the runtime
 * cannot give the array's address.  The library calls no allocating routine
 * on this path.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams or threads) race and must be ordered by
 * the caller. */
ciw_status conv2d_fwd_noalloc(const ciw_conv_desc* desc, ciw_dtype in_dtype, ciw_dtype out_dtype,
                              const void* x, const void* w, const void* bias, void* y,
                              uint32_t flags, void* stream);

/* Depthwise forward convolution (groups == C == K, one filter per channel;
 * "Diagonalwise Refactorization: An Efficient Training Method for Depthwise
 * Convolutions", abstract: each input channel is convolved with its own
 * filter, which equals a dense convolution whose filter is zero off the
 * channel diagonal): the CHW window tensor, then a per-channel windowed dot
 * product (bandwidth-bound).  Same arguments, workspace and flag rules as
 * conv2d_fwd; w is [C][1][R][S]. */
ciw_status conv2d_dw_fwd(const ciw_conv_desc* desc, ciw_dtype in_dtype, ciw_dtype out_dtype,
                         const void* x, const void* w, const void* bias, void* y,
                         void* workspace, size_t workspace_bytes, uint32_t flags,
                         void* stream);

/* Static description of a status code (never NULL).  A convenience of
 * this library: no passage of the pages defines error statuses. */
const char* conv_im2win_status_string(ciw_status status);

#ifdef __cplusplus
}
#endif

#endif /* CONV_IM2WIN_H */
