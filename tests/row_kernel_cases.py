"""Layers that exercise each specialisation of the matrix-core row kernel.

Each was chosen from the kernel's geometry (the notes say which pad period,
phase count, filter-set count, masking and store mode it lands on).  Used
by the GPU parity test of the row kernel and by the CPU model of its
indexing; no torch here.
"""
import workloads

L = workloads.Layer
CASES = {
    # pad 8 (G = 24), no masks, K = 40: the second channel half partly valid
    "pad8_c64_k40": L("c", N=2, C=64, H=7, W=29, K=40, R=3, S=3, pad=(1, 1), dtype="f16",
                      out_dtype="f16"),
    # stride 2: pad 8, masked tail
    "pad8_c32_s2": L("c", N=2, C=32, H=9, W=37, K=64, R=3, S=3, stride=(2, 2), pad=(1, 1),
                     dtype="bf16", out_dtype="bf16"),
    # pad 4 (G = 12), two pixel blocks, fp32 output
    "pad4_c32_f32out": L("c", N=1, C=32, H=6, W=45, K=24, R=3, S=3, pad=(1, 1), dtype="f16",
                         out_dtype="f32"),
    # pad 2 (G = 6), Q = 13: element stores
    "pad2_c16_q13": L("c", N=3, C=16, H=5, W=13, K=64, R=3, S=3, pad=(1, 1), dtype="f16",
                      out_dtype="f16"),
    # G = 15 odd: no pad chunks, masked
    "pad1_c40": L("c", N=1, C=40, H=5, W=33, K=50, R=3, S=3, pad=(1, 1), dtype="bf16",
                  out_dtype="bf16"),
    # 1x1, G = 16: pad period capped at 8, vector stores
    "pad8cap_1x1_c128": L("c", N=2, C=128, H=4, W=40, K=64, R=1, S=1, dtype="f16",
                          out_dtype="f16"),
    # 1x1, G = 1, three pixel blocks, fp32 output
    "pad1_1x1_c8": L("c", N=2, C=8, H=5, W=70, K=17, R=1, S=1, dtype="bf16", out_dtype="f32"),
    # D = 18: four phases, two filter sets, shortened ring
    "nset2_c6": L("c", N=2, C=6, H=7, W=50, K=64, R=3, S=3, pad=(1, 1), dtype="f16",
                  out_dtype="f16"),
    # D = 9: eight phases, four filter sets
    "nset4_c3": L("c", N=2, C=3, H=6, W=90, K=33, R=3, S=3, pad=(1, 1), dtype="bf16",
                  out_dtype="bf16"),
    # D = 36: two phases, one set
    "nph2_c12": L("c", N=1, C=12, H=6, W=41, K=64, R=3, S=3, pad=(1, 1), dtype="f16",
                  out_dtype="f16"),
    # the 7x7 stride-2 stem on a smaller image
    "stem_small": L("c", N=1, C=3, H=30, W=75, K=64, R=7, S=7, stride=(2, 2), pad=(3, 3),
                    dtype="bf16", out_dtype="bf16"),
    # K = 20: the second channel half has no valid channel
    "k20_c64": L("c", N=1, C=64, H=5, W=17, K=20, R=3, S=3, pad=(1, 1), dtype="f16",
                 out_dtype="f16"),
    # a row needing all eight copy instructions per thread
    "long_row_c64": L("c", N=1, C=64, H=3, W=70, K=64, R=3, S=3, pad=(1, 1), dtype="f16",
                      out_dtype="f16"),
    # 1x5 filter, G = 6: pad 2
    "c48_1x5": L("c", N=2, C=48, H=9, W=21, K=64, R=1, S=5, pad=(0, 2), dtype="bf16",
                 out_dtype="bf16"),
}
