"""CPU model of the depthwise in-LDS kernel (conv_dw_implicit_kernel): its
plan, the staging of x into zero-padded planes (16-byte loads for fp32
planes whose area is a multiple of 4, else element positions stepped by a
fixed increment), and the two strip forms (7 outputs down a column; with the
2x2 pool, 4 pooled outputs down a pooled column).  Every LDS position is
bounds-checked against its plane, every output is written exactly once, and
the outputs equal the oracle's.

The kernel builds each window from a zero-padded copy of the input plane;
the sum is the same as in the direct convolution of the im2win paper's
problem statement (§III-A), in another order.
"""
import numpy as np
import pytest

import oracle

THREADS = 256
LDS_BYTES = 48 * 1024
KSH, KPS = 7, 4


def plan(N, C, H, W, R, S, sh, sw, ph, pw, dh, dw, pool):
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    a = dict(H=H, W=W, P=P, Q=Q, R=R, S=S, ph=ph, pw=pw, pool=pool)
    a["Wp"] = W + 2 * pw

    def plane_of(hp):
        while (hp * a["Wp"]) % 4:
            hp += 1
        return hp

    bytes_of = lambda hp: (hp * a["Wp"] + R * S + 1) * 4
    a["Hp"] = plane_of(H + 2 * ph)
    if bytes_of(a["Hp"]) > LDS_BYTES:
        return None
    nstrip = (P // 2 + KPS - 1) // KPS if pool else (P + KSH - 1) // KSH
    rows = 2 * KPS if pool else KSH
    a["strip"] = (R, S, sh, sw, dh, dw) == (3, 3, 1, 1, 1, 1)
    if a["strip"]:
        hs = plane_of(max(a["Hp"], nstrip * rows + 2))
        if bytes_of(hs) <= LDS_BYTES:
            a["Hp"] = hs
        else:
            a["strip"] = False
    # two columns a lane (no pool, Qo even)
    a["pairs"] = a["strip"] and not pool and Q % 2 == 0 and a["Wp"] % 2 == 0
    planes = N * C
    per = min(LDS_BYTES // bytes_of(a["Hp"]), max(1, 16 * THREADS // (H * W)))
    per = max(1, min(per, max(1, planes // 1024)))
    if a["strip"]:
        spp = (Q // 2 if pool or a["pairs"] else Q) * nstrip
        it = -(-per * spp // THREADS)
        per2 = (it - 1) * THREADS // spp
        if it > 1 and per2 >= 1 and (it - 1) * per < it * per2:
            per = per2
    a.update(per=per, planes=planes, nstrip=nstrip, Po=P // 2 if pool else P,
             Qo=Q // 2 if pool else Q)
    HW = H * W
    a["dQ"], a["dH"], a["dW"] = THREADS // HW, (THREADS % HW) // W, (THREADS % HW) % W
    a["vec4"] = HW % 4 == 0 and W >= 4
    return a


def stage(xp, a, np_, fp32):
    """The planes of one workgroup in LDS, as the kernel writes them."""
    H, W, Hp, Wp, ph, pw = a["H"], a["W"], a["Hp"], a["Wp"], a["ph"], a["pw"]
    HW, HpWp = H * W, Hp * Wp
    lds = np.zeros(np_ * HpWp)
    written = np.zeros(np_ * HpWp, dtype=int)
    flat = xp.reshape(-1)
    total = np_ * HW
    if fp32 and a["vec4"]:
        total4 = total // 4
        for tid in range(THREADS):
            for e0 in range(tid, total4, 4 * THREADS):
                for u in range(4):
                    e4 = e0 + u * THREADS
                    if e4 < total4:
                        q, r = divmod(4 * e4, HW)
                        hh, ww = divmod(r, W)
                        row = q * HpWp + (hh + ph) * Wp + pw
                        for j in range(4):
                            c = ww + j
                            off = row + (c if c < W else c - W + Wp)
                            assert q * HpWp <= off < (q + 1) * HpWp
                            lds[off] = flat[4 * e4 + j]
                            written[off] += 1
    else:
        step = a["dQ"] * HpWp + a["dH"] * Wp + a["dW"]
        for tid in range(THREADS):
            for e0 in range(tid, total, 16 * THREADS):
                q0, r0 = divmod(e0, HW)
                hh, ww = divmod(r0, W)
                off = q0 * HpWp + (hh + ph) * Wp + ww + pw
                for u in range(16):
                    if e0 + u * THREADS < total:
                        assert 0 <= off < np_ * HpWp
                        lds[off] = flat[e0 + u * THREADS]
                        written[off] += 1
                    ww += a["dW"]
                    hh += a["dH"]
                    off += step
                    if ww >= W:
                        ww -= W
                        hh += 1
                        off += Wp - W
                    if hh >= H:
                        hh -= H
                        off += HpWp - H * Wp
    # every interior position once, padding untouched (zero)
    want = np.zeros((np_, Hp, Wp), dtype=int)
    want[:, ph:ph + H, pw:pw + W] = 1
    assert np.array_equal(written.reshape(np_, Hp, Wp), want)
    return lds


def strip_outputs(lds, wts, bias, a, np_, relu):
    """The strip forms over one workgroup's planes (pooled, two columns a
    lane, one column a lane); every read bounds-checked, the pair form's
    8-byte reads and two-element stores checked for alignment."""
    Hp, Wp, P, Q, Po, Qo = a["Hp"], a["Wp"], a["P"], a["Q"], a["Po"], a["Qo"]
    HpWp = Hp * Wp
    y = np.full((np_, Po, Qo), np.nan)

    def rd(q, r, c):
        assert 0 <= r < Hp and 0 <= c < Wp
        return lds[q * HpWp + r * Wp + c]

    rows = 2 * KPS if a["pool"] else KSH
    if a["pairs"]:
        qh = Qo // 2
        assert Wp % 2 == 0 and HpWp % 2 == 0 and Qo % 2 == 0 and (P * Qo) % 2 == 0
        for it in range(np_ * qh * a["nstrip"]):
            q, r = divmod(it, qh * a["nstrip"])
            st, cp = divmod(r, qh)
            oh0 = st * KSH
            w = wts[q].reshape(3, 3)
            base = q * HpWp + oh0 * Wp + 2 * cp
            assert base % 2 == 0                       # 8-byte aligned float2 reads
            patch = np.array([[rd(q, oh0 + rr, 2 * cp + cc) for cc in range(4)]
                              for rr in range(rows + 2)])
            for i in range(KSH):
                if oh0 + i < P:
                    assert ((oh0 + i) * Qo + 2 * cp) % 2 == 0   # two-element store aligned
                    for j in range(2):
                        v = float(np.sum(patch[i:i + 3, j:j + 3] * w)) + bias[q]
                        assert np.isnan(y[q, oh0 + i, 2 * cp + j])
                        y[q, oh0 + i, 2 * cp + j] = max(v, 0.0) if relu else v
        return y
    per_plane = Qo * a["nstrip"]
    for it in range(np_ * per_plane):
        q, r = divmod(it, per_plane)
        st, ow = divmod(r, Qo)
        w = wts[q].reshape(3, 3)
        if a["pool"]:
            oi0 = st * KPS
            patch = np.array([[rd(q, 2 * oi0 + rr, 2 * ow + cc) for cc in range(4)]
                              for rr in range(rows + 2)])
            for i in range(KPS):
                if oi0 + i < Po:
                    vals = []
                    for d in range(4):
                        dr, dc = 2 * i + d // 2, d % 2
                        v = float(np.sum(patch[dr:dr + 3, dc:dc + 3] * w)) + bias[q]
                        vals.append(max(v, 0.0) if relu else v)
                    assert np.isnan(y[q, oi0 + i, ow])
                    y[q, oi0 + i, ow] = max(vals)
        else:
            oh0 = st * KSH
            patch = np.array([[rd(q, oh0 + rr, ow + cc) for cc in range(3)]
                              for rr in range(rows + 2)])
            for i in range(KSH):
                if oh0 + i < P:
                    v = float(np.sum(patch[i:i + 3] * w)) + bias[q]
                    assert np.isnan(y[q, oh0 + i, ow])
                    y[q, oh0 + i, ow] = max(v, 0.0) if relu else v
    return y


CASES = [
    # N, C, H, W, pad, pool, relu
    (2, 8, 14, 14, 1, False, False),    # the 14x14 layer's plane shape
    (2, 8, 14, 14, 1, True, True),
    (1, 3, 13, 9, 1, False, True),      # plane area odd: stepped staging
    (1, 3, 13, 9, 1, True, False),
    (1, 2, 6, 6, 0, True, True),        # float4s across row ends, no padding
    (1, 2, 22, 8, 2, False, False),     # strips past P, pad 2
    (1, 1, 70, 70, 1, True, True),      # a plane over two load rounds
    (1, 3, 10, 11, 1, False, False),    # Q odd: one column a lane
    (2, 4, 9, 7, 0, False, True),       # Q odd, no padding
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("fp32", [True, False])
def test_strip_model_matches_oracle(case, fp32):
    N, C, H, W, pad, pool, relu = case
    a = plan(N, C, H, W, 3, 3, 1, 1, pad, pad, 1, 1, pool)
    assert a is not None and a["strip"]
    rng = np.random.default_rng(sum(case[:5]))
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((C, 1, 3, 3)) * 0.3
    b = rng.uniform(-0.1, 0.1, C)
    planes = x.reshape(N * C, H, W)
    got = np.empty((N * C, a["Po"], a["Qo"]))
    for p0 in range(0, N * C, a["per"]):
        np_ = min(a["per"], N * C - p0)
        lds = stage(planes[p0:p0 + np_], a, np_, fp32)
        cs = [(p0 + i) % C for i in range(np_)]
        got[p0:p0 + np_] = strip_outputs(lds, w[cs, 0], b[cs], a, np_, relu)
    ref = oracle.conv2d(x, w, b, 1, pad, 1, C)
    ref = oracle.relu_pool(ref, relu=relu, pool=pool)
    assert not np.isnan(got).any()
    np.testing.assert_allclose(got.reshape(ref.shape), ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_plan_of_the_depthwise_layer():
    """128x512x14x14: 18 planes a workgroup with and without the pool, so
    every thread computes one pass of strips (252 of 256 threads busy:
    without the pool a two-column strip each, with it a pooled strip each),
    planes padded to 16 / 18 rows."""
    a = plan(128, 512, 14, 14, 3, 3, 1, 1, 1, 1, 1, 1, False)
    assert a["strip"] and a["pairs"] and a["per"] == 18 and a["Hp"] == 16 and a["vec4"]
    assert a["per"] * (a["Qo"] // 2) * a["nstrip"] == 252
    a = plan(128, 512, 14, 14, 3, 3, 1, 1, 1, 1, 1, 1, True)
    assert a["strip"] and a["per"] == 18 and a["Hp"] == 18
    assert a["per"] * a["Qo"] * a["nstrip"] <= THREADS


def test_eligibility_agrees_with_library():
    """This model's plan exists exactly when the library runs the layer in
    LDS (conv2d_implicit_workspace_bytes: 0 bytes, else unsupported)."""
    import ctypes
    import cnn_convolution_im2win_amd as ciw
    from cnn_convolution_im2win_amd import _lib
    rng = np.random.default_rng(4)
    shapes = [(1, 4, 14, 14, 3, 1, 1), (1, 2, 100, 100, 3, 1, 1), (1, 2, 104, 104, 3, 1, 1),
              (1, 2, 110, 110, 3, 1, 1), (2, 3, 9, 11, 5, 2, 2), (1, 2, 1, 1, 1, 1, 0)]
    for _ in range(30):
        R = int(rng.choice([1, 3, 5]))
        # C >= 2: with C = 1 the layer is an ordinary (groups = 1) convolution
        shapes.append((1, int(rng.integers(2, 9)), int(rng.integers(1, 120)), int(rng.integers(1, 120)),
                       R, int(rng.integers(1, 3)), int(rng.integers(0, 3))))
    for N, C, H, W, R, s, p in shapes:
        if H + 2 * p < R or W + 2 * p < R:
            continue
        a = plan(N, C, H, W, R, R, s, s, p, p, 1, 1, False)
        desc = ciw.make_desc((N, C, H, W), (C, 1, R, R), (s, s), (p, p), (1, 1), C)
        out = ctypes.c_size_t(12345)
        st = _lib.load().conv2d_implicit_workspace_bytes(ctypes.byref(desc), ciw.CIW_F32, ciw.CIW_F32,
                                                         0, ctypes.byref(out))
        if a is None:
            assert st == _lib.CIW_ERR_UNSUPPORTED, (N, C, H, W, R, s, p)
        else:
            assert st == 0 and out.value == 0, (N, C, H, W, R, s, p)
