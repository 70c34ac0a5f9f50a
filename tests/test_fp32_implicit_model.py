"""CPU model of the in-LDS form of the fp32 matrix-core contraction
(conv_fp32_mfma_kernel with IMP, csrc/conv_fp32_mfma.hip): per pixel block
and chunk of 16 channels, every channel's zero-padded input rows are staged
in LDS straight from x ([Hr][Wpl] a channel, Wpl the padded columns the
windows touch), and the window of output (h, w) at tap (r, q) is the staged
element (h stride_h + r dil_h, w stride_w + q dil_w).

The model mirrors the plan (pixel block rows, staged extent, elements per
thread), replays each thread's staging map (the same positions every chunk,
only the channel base moves), checks every staging write and every operand
read against the staged region of its channel, and multiplies out the
outputs from the staged data; they must equal the oracle's convolution."""
import numpy as np
import pytest

import oracle

KCH = 16
THREADS = 512
MAX_BI = 10
MAX_PIX = 192


def plan(C, H, W, K, R, S, sh, sw, ph, pw, dh, dw):
    if (R, S) not in ((3, 3), (1, 1)):
        return None
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    if P < 1 or Q < 1 or Q > MAX_PIX or C < 2:
        return None
    HB = min(P, MAX_PIX // Q)
    Hr = (HB - 1) * sh + (R - 1) * dh + 1
    Wpl = (Q - 1) * sw + dw * (S - 1) + 1
    if KCH * Hr * Wpl > MAX_BI * THREADS:
        return None
    return dict(P=P, Q=Q, HB=HB, Hr=Hr, Wpl=Wpl, BS=Hr * Wpl + 4, nBI=KCH * Hr * Wpl)


def replay(x, w, sh, sw, ph, pw, dh, dw, a):
    C, H, W = x.shape
    K, _, R, S = w.shape
    P, Q, HB, Hr, Wpl, BS = (a[k] for k in ("P", "Q", "HB", "Hr", "Wpl", "BS"))
    y = np.zeros((K, P, Q))
    per_ch = Hr * Wpl
    for h0 in range(0, P, HB):
        rows = min(HB, P - h0)
        npx = rows * Q
        for cc in range(0, C, KCH):
            nc = min(KCH, C - cc)
            Bs = np.full(KCH * BS, np.nan)
            written = np.zeros(KCH * BS, dtype=int)
            # every thread's staging map
            for tid in range(THREADS):
                for u in range(MAX_BI):
                    e = tid + u * THREADS
                    if e >= a["nBI"]:
                        continue
                    cl, rr = divmod(e, per_ch)
                    yy, xx = divmod(rr, Wpl)
                    iy, ix = h0 * sh - ph + yy, xx - pw
                    dst = cl * BS + yy * Wpl + xx
                    assert 0 <= dst < KCH * BS and dst < cl * BS + per_ch
                    inside = 0 <= iy < H and 0 <= ix < W
                    Bs[dst] = x[cc + cl, iy, ix] if (cl < nc and inside) else 0.0
                    written[dst] += 1
            # operand reads: pixel block pixels (clamped to the last), every tap
            for px in range(32 * ((npx + 31) // 32)):
                pc = min(px, npx - 1)
                hh, ww = divmod(pc, Q)
                pxoff = hh * sh * Wpl + ww * sw
                for cl in range(KCH):
                    for r in range(R):
                        for q in range(S):
                            off = cl * BS + pxoff + r * dh * Wpl + q * dw
                            assert cl * BS <= off < cl * BS + per_ch
                            assert written[off] == 1
                if px < npx:
                    for cl in range(nc):
                        win = np.array([[Bs[cl * BS + pxoff + r * dh * Wpl + q * dw] for q in range(S)]
                                        for r in range(R)])
                        y[:, h0 + hh, ww] += np.einsum("krs,rs->k", w[:, cc + cl], win)
    return y


SHAPES = [
    # C, H, W, K, R, sh, sw, pad, dil
    (512, 13, 13, 8, 3, 1, 1, 1, 1),    # the 1x512x13x13 layer's geometry (K cut for time)
    (16, 32, 32, 8, 3, 1, 1, 1, 1),     # several pixel blocks
    (20, 9, 11, 5, 3, 2, 1, 0, 1),      # stride_h 2, ragged last chunk
    (18, 10, 12, 4, 3, 1, 2, 2, 2),     # stride_w 2, dilation 2, padding 2
    (33, 7, 7, 3, 1, 1, 1, 0, 1),       # 1x1
]


@pytest.mark.parametrize("shape", SHAPES)
def test_fp32_implicit_model_matches_oracle(shape):
    C, H, W, K, R, sh, sw, pad, dil = shape
    a = plan(C, H, W, K, R, R, sh, sw, pad, pad, dil, dil)
    assert a is not None
    rng = np.random.default_rng(sum(shape))
    x = rng.standard_normal((C, H, W))
    w = rng.standard_normal((K, C, R, R))
    y = replay(x, w, sh, sw, pad, pad, dil, dil, a)
    ref = oracle.conv2d(x[None], w, None, (sh, sw), (pad, pad), (dil, dil), 1)[0]
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())


def test_plan_of_the_mid_layer():
    """1x512x13x13: one pixel block of all 13 rows, 15 x 15 staged
    elements a channel, 3600 a chunk (at most 8 a thread)."""
    a = plan(512, 13, 13, 1024, 3, 3, 1, 1, 1, 1, 1, 1)
    assert (a["HB"], a["Hr"], a["Wpl"], a["nBI"]) == (13, 15, 15, 3600)
    assert -(-a["nBI"] // THREADS) == 8


m = pytest.importorskip("cnn_convolution_im2win_amd")
from tests.test_fp32_m16_model import plan as m16_plan  # noqa: E402


def test_eligibility_matches_library():
    """The fp32 layers this model's plan or the whole-sum kernel's in-LDS
    plan accepts are exactly those for which the library accepts
    CIW_FLAG_IMPLICIT."""
    rng = np.random.default_rng(11)
    for _ in range(80):
        C = int(rng.choice([1, 2, 3, 16, 48, 512]))
        H, W = int(rng.integers(1, 40)), int(rng.choice([5, 13, 56, 150, 200]))
        K, R = int(rng.integers(1, 70)), int(rng.choice([1, 3, 5]))
        sh, sw, pad, dil = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(0, 3)), int(rng.integers(1, 3))
        d = m.make_desc((2, C, H, W), (K, C, R, R), (sh, sw), pad, dil, 1)
        try:
            m.conv_im2win_output_dims(d)
        except m.Im2winError:
            continue
        try:
            m.conv2d_implicit_workspace_bytes(d, m.CIW_F32, m.CIW_F32, m.CIW_FLAG_IMPLICIT)
            ok = True
        except m.Im2winError:
            ok = False
        pl = plan(C, H, W, K, R, R, sh, sw, pad, pad, dil, dil)
        # the whole-sum kernel's in-LDS form takes the layers it fits first
        whole = m16_plan(2, C, H, W, K, R, R, sh, sw, pad, pad, dil, dil, imp=True)
        assert (pl is not None or whole is not None) == ok, (C, H, W, K, R, sh, sw, pad, dil)
