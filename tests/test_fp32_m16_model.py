"""CPU model of the whole-channel-sum fp32 matrix-core contraction
(conv_fp32_mfma16_kernel, csrc/conv_fp32_m16.hip).

A workgroup owns 16 output channels x 48 consecutive output pixels of one
image and the whole channel sum; wave v streams its own contiguous channel range
in groups of 4 (the 16x16x4 MFMA's reduction width; waves 0-3 take an eighth
more groups than waves 4-7): the group's filter rows
(16 rows x 4 R S floats, 16-byte pieces) and the rows of the CHW window
tensor its 48 pixels span (nrow rows of each of the 4 channels, 16-byte
pieces) go into the wave's own LDS buffer; lane (m, kk) then reads filter
row m, channel kk, tap t, and window element kk, pixel m of each tile,
tap t.

The model mirrors the plan, replays every lane's loads (clamped addresses
must stay inside w and the window tensor; pieces outside the tensors must
never be read as operands of a stored output), every LDS write (inside the
wave's buffer, each slot once) and every operand read (inside the slots the
group wrote), and multiplies the outputs out from the replayed buffers in
the kernel's order: they must match the oracle's convolution.

The in-LDS form (IMP) is replayed too: a group's filter pieces as above, then
each channel's staged rows inside the image, end to end as in x, in 16-byte
pieces (the last one moved back to end at the last element), stored from a
shift that puts them on 16-byte boundaries; rows outside the image and the
channel's zero run stay zero from the one clearing at the start; the window
element of pixel (h, w) at tap (r, q) is read at staged row (h - h_lo)
stride_h + r dil_h, column w stride_w - pad_w + q dil_w, or from the zero
run where that column is outside the image."""
import numpy as np
import pytest

import oracle

WAVES, M, TILES, PIX, G, MAX_P = 8, 16, 3, 48, 4, 10
LDS = 160 * 1024


def plan(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, imp=False):
    if (R, S) not in ((3, 3), (1, 1)) or C % G or C <= 0 or K <= 0:
        return None
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    if P < 1 or Q < 1:
        return None
    Wwin = (Q - 1) * sw + dw * (S - 1) + 1
    pitch = -(-Wwin * R // 4) * 4
    RS = R * S
    PQ = P * Q
    a = dict(P=P, Q=Q, PQ=PQ, pitch=pitch, RS=RS)
    a["pgroups"] = -(-PQ // PIX)
    a["kblocks"] = -(-K // M)
    a["nrow"] = min(P, (PIX - 1) // Q + 2)
    a["imp"] = imp
    if imp:
        if W < 4:
            return None
        Hr = (a["nrow"] - 1) * sh + (R - 1) * dh + 1
        per_ch = Hr * W
        npc = -(-per_ch // 4)
        np_ = -(-G * npc // 64)
        if np_ + -(-M * R * S // 64) > MAX_P or per_ch > (1 << 20) or G * H * W * 4 >= 2 ** 32:
            return None
        zoff = -(-(per_ch + 3) // 4) * 4
        a.update(Hr=Hr, npc=npc, rq4=0, zoff=zoff, BS=zoff + -(-((R - 1) * dh * W + 1) // 4) * 4 + 4,
                 np=np_, H=H, W=W, sh=sh, ph=ph, pw=pw, dh=dh)
    else:
        if a["nrow"] * pitch % 4:
            return None
        a["rq4"] = a["nrow"] * pitch // 4
        pieces = M * RS + G * a["rq4"]
        if pieces > MAX_P * 64 or G * P * pitch * 4 >= 2 ** 32:
            return None
        a["np"] = -(-pieces // 64)
        a["BS"] = a["nrow"] * pitch + 4
    ngr = -(-(C // G) // WAVES)
    a["gA"], a["gB"] = ngr + ngr // 8, ngr - ngr // 8
    a["AS"] = G * RS
    a["buf"] = max(M * a["AS"] + G * a["BS"], TILES * 4 * 64)
    a["ntask"] = N * a["pgroups"] * a["kblocks"]
    if a["ntask"] >= 2 ** 31:
        return None
    a["lds"] = WAVES * (a["buf"] + 256) * 4
    return a if a["lds"] <= LDS else None


def replay(xw, w, a, N, C, K, R, S, sw, dw):
    """xw: the CHW window tensor [N*C*P, pitch], or with a["imp"] x itself
    [N][C][H][W]; returns y [N][K][P*Q]."""
    imp = a["imp"]
    P, Q, PQ, pitch, RS = a["P"], a["Q"], a["PQ"], a["pitch"], a["RS"]
    AS, BS, buf, rq4, nrow = a["AS"], a["BS"], a["buf"], a["rq4"], a["nrow"]
    kAL = -(-M * RS // 64)
    wflat = w.reshape(-1)
    xflat = xw.reshape(-1)
    y = np.full((N, K, PQ), np.nan)
    stored = np.zeros((N, K, PQ), dtype=int)
    lanes = np.arange(64)
    m, kk = lanes & 15, lanes >> 4
    span = a["BS"] if imp else nrow * pitch     # a channel's readable words
    for task in range(a["ntask"]):
        pg = task % a["pgroups"]
        rest = task // a["pgroups"]
        n, kb = rest % N, rest // N
        k0, p0 = kb * M, pg * PIX
        h_lo = p0 // Q
        # the lanes' window offsets (clamped pixels)
        px = np.minimum(p0 + 16 * np.arange(TILES)[:, None] + m[None, :], PQ - 1)   # [tile][lane]
        hh, ww = px // Q, px % Q
        assert np.all(hh - h_lo < nrow) and np.all(hh - h_lo >= 0)
        # off[t3][q][lane]: filter row 0, column q; row r is rstep * r further on
        if imp:
            r_lo = max(0, a["ph"] - h_lo * a["sh"])
            r_hi = min(a["Hr"] - 1, a["H"] - 1 + a["ph"] - h_lo * a["sh"])
            nv = max(0, r_hi - r_lo + 1) * a["W"]
            delta = (4 - (r_lo * a["W"]) % 4) % 4
            col = ww[:, None, :] * sw - a["pw"] + np.arange(S)[None, :, None] * dw
            inside = (col >= 0) & (col < a["W"])
            off = np.where(inside, delta + (hh - h_lo)[:, None, :] * a["sh"] * a["W"] + col, a["zoff"])
            rstep = a["dh"] * a["W"]
        else:
            off = (hh - h_lo)[:, None, :] * pitch + (ww[:, None, :] * sw + np.arange(S)[None, :, None] * dw) * R
            rstep = 1
        red = np.zeros((WAVES, TILES, 64, 4))
        for v in range(WAVES):
            gA, gB = a["gA"], a["gB"]
            c_lo = (v * gA if v < 4 else 4 * gA + (v - 4) * gB) * G
            ngr = max(0, min(gA if v < 4 else gB, (C - c_lo) // G))
            acc = np.zeros((TILES, 16, 16))     # [tile][channel row][pixel col]
            # one buffer a wave: filter rows [16][AS], window rows [4][BS], then
            # 64 dummy 16-byte slots; the in-LDS form clears the window rows once
            buf_arr = np.full(buf + 256, np.nan)
            if imp:
                buf_arr[M * AS:M * AS + G * BS] = 0.0
            for j in range(ngr):
                c = c_lo + G * j
                wrote = np.zeros(buf + 256, dtype=int)
                nA = M * RS
                nP = nA + G * rq4
                g0 = c_lo if ngr > 0 else 0
                nLA = -(-nA // 64) if imp else a["np"]     # 16-byte loads a group
                for u in range(nLA):
                    for l in range(64):
                        e = l + 64 * u
                        if imp and e >= nA:
                            dst = buf + 4 * l                  # past the group's filter pieces
                            val = np.full(4, np.nan)
                        elif e < nA:
                            k, f = divmod(e, RS)
                            kr = min(k0 + k, K - 1)
                            src = (kr * C + g0) * RS + 4 * f + j * G * RS
                            assert 0 <= src and src + 4 <= wflat.size
                            # a clamped row only feeds output rows that are never stored
                            val = wflat[src:src + 4] if k0 + k < K else np.full(4, np.nan)
                            dst = k * AS + 4 * f
                            assert dst + 4 <= M * AS
                        else:
                            eb = min(e, nP - 1) - nA
                            ch, o4 = divmod(eb, rq4)
                            row = min(h_lo + (4 * o4) // pitch, P - 1)
                            col = (4 * o4) % pitch
                            src = ((n * C + g0 + ch) * P + row) * pitch + col + j * G * P * pitch
                            assert 0 <= src and src + 4 <= xflat.size
                            # a clamped row is never part of a pixel's window
                            val = xflat[src:src + 4] if h_lo + (4 * o4) // pitch < P else np.full(4, np.nan)
                            if e < nP:
                                dst = M * AS + ch * BS + 4 * o4
                                assert M * AS + ch * BS <= dst and dst + 4 <= M * AS + ch * BS + nrow * pitch
                            else:
                                dst = buf + 4 * l
                        buf_arr[dst:dst + 4] = val
                        wrote[dst:dst + 4] += 1
                if imp:
                    H, W = a["H"], a["W"]
                    npc = -(-nv // 4)
                    ih0 = h_lo * a["sh"] - a["ph"] + r_lo
                    for u in range(a["np"]):
                        for l in range(64):
                            e = l + 64 * u
                            ch, i = divmod(e, a["npc"])
                            ok = ch < G and i < npc
                            if ok:
                                assert nv >= 4
                                start = min(4 * i, nv - 4)
                                src = ((n * C + g0 + ch) * H + ih0) * W + start + j * G * H * W
                                dst = M * AS + ch * BS + delta + r_lo * W + start
                                # inside the channel's staged rows, before its zero run
                                assert M * AS + ch * BS <= dst and dst + 4 <= M * AS + ch * BS + a["zoff"]
                                assert dst + 4 <= M * AS + ch * BS + delta + (r_hi + 1) * W
                                wrote[dst:dst + 4] = 1
                            else:
                                src = ((n * C + g0) * H) * W + j * G * H * W
                                dst = buf + 4 * l
                            assert 0 <= src and src + 4 <= xflat.size
                            buf_arr[dst:dst + 4] = xflat[src:src + 4]
                Abuf, Bbuf = buf_arr[:M * AS], buf_arr[M * AS:M * AS + G * BS]
                wrote_a, wrote_b = wrote[:M * AS], wrote[M * AS:M * AS + G * BS]
                assert wrote_a.max() <= 1 and wrote_b.max() <= 1
                assert M * AS + G * BS <= buf
                # operand reads: A[m][kk][t], B[kk][pixel m of tile t3][t]
                aidx = m[:, None] * AS + kk[:, None] * RS + np.arange(RS)[None, :]     # [lane][t]
                assert np.all(wrote_a[aidx] == 1)
                av = Abuf[aidx]
                for t3 in range(TILES):
                    bidx = np.stack([kk * BS + off[t3][t % S] + (t // S) * rstep for t in range(RS)], axis=1)
                    assert np.all(bidx >= kk[:, None] * BS) and np.all(bidx < kk[:, None] * BS + span)
                    if not imp:
                        assert np.all(wrote_b[bidx] == 1)
                    bv = Bbuf[bidx]
                    # 16x16x4 step per tap: D[i][jcol] += sum_k A[i][k] B[k][jcol],
                    # A lane (m, kk) = row m, k = kk; B lane (m, kk) = col m, k = kk
                    for t in range(RS):
                        Am = np.zeros((16, 4))
                        Bm = np.zeros((4, 16))
                        Am[m, kk] = av[:, t]
                        Bm[kk, m] = bv[:, t]
                        with np.errstate(invalid="ignore"):
                            acc[t3] += Am @ Bm
            # lane l holds D[4 (l / 16) + i][l % 16]
            for t3 in range(TILES):
                for i in range(4):
                    red[v, t3, :, i] = acc[t3][4 * (lanes >> 4) + i, lanes & 15]
        for o in range(M * PIX):
            ch, p = divmod(o, PIX)
            t3, l, i = p >> 4, 16 * (ch >> 2) + (p & 15), ch & 3
            k, pp = k0 + ch, p0 + p
            if k < K and pp < PQ:
                s = 0.0
                for v in range(WAVES):
                    s += red[v, t3, l, i]
                y[n, k, pp] = s
                stored[n, k, pp] += 1
    assert np.all(stored == 1)
    return y


SHAPES = [
    # N, C, H, W, K, R, stride, pad, dil
    (1, 32, 13, 13, 40, 3, 1, 1, 1),     # the mid layer's geometry, K ragged: pixel groups of 4-5 rows
    (2, 20, 9, 11, 17, 3, (2, 1), 0, 1),  # stride_h 2, waves with 1 group and none, two images
    (1, 12, 10, 24, 16, 3, (1, 2), 2, 2),  # stride_w 2, dilation 2, padding 2: 7 window loads a lane
    (1, 8, 7, 7, 9, 1, 1, 0, 1),          # 1x1
    (1, 36, 4, 30, 20, 3, 1, 1, 1),       # 30-pixel rows: groups of 2-3 rows, odd group counts
    (1, 12, 10, 12, 16, 3, (1, 2), 2, 2),  # stride_w 2, dilation 2 in LDS: 13 staged rows, 624 elements
]


@pytest.mark.parametrize("imp", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_m16_model_matches_oracle(shape, imp):
    N, C, H, W, K, R, stride, pad, dil = shape
    sh, sw = stride if isinstance(stride, tuple) else (stride, stride)
    a = plan(N, C, H, W, K, R, R, sh, sw, pad, pad, dil, dil, imp)
    if a is None:
        # the two forms' limits differ: 9 staged rows of 24 elements x 4
        # channels are more than 10 loads a lane in LDS, and 6 pixel groups'
        # 9 window rows of 28 floats more than 10 pieces a lane
        assert (shape, imp) in (((1, 12, 10, 24, 16, 3, (1, 2), 2, 2), True),
                                ((1, 12, 10, 12, 16, 3, (1, 2), 2, 2), False))
        return
    rng = np.random.default_rng(sum(shape[:6]))
    x = rng.standard_normal((N, C, H, W)).astype(np.float32).astype(np.float64)
    w = rng.standard_normal((K, C, R, R))
    if imp:
        src = x
    else:
        # the fp32 window tensor (16-byte pitch of 4 floats), widened
        src = oracle.im2win(x.astype(np.float32), R, R, (sh, sw), (pad, pad), (dil, dil)).astype(np.float64)
        assert src.shape == (N * C * a["P"], a["pitch"])
    y = replay(src, w, a, N, C, K, R, R, sw, dil)
    ref = oracle.conv2d(x, w, None, (sh, sw), (pad, pad), (dil, dil), 1).reshape(N, K, -1)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())


def test_plan_of_the_mid_layer():
    """1x512x13x13 -> 1024: 4 pixel groups x 64 channel blocks = 256
    workgroups; 18 groups of 4 channels for each of waves 0-3, 14 for each of
    waves 4-7; 5 window rows of 48 floats a
    channel: 144 + 240 16-byte pieces a group, 6 loads a lane; 58 KB of LDS."""
    a = plan(1, 512, 13, 13, 1024, 3, 3, 1, 1, 1, 1, 1, 1)
    assert (a["pgroups"], a["kblocks"], a["ntask"]) == (4, 64, 256)
    assert (a["gA"], a["gB"], a["nrow"], a["pitch"], a["np"]) == (18, 14, 5, 48, 6)
    assert a["lds"] == 8 * (16 * 36 + 4 * 244 + 256) * 4


def test_plan_of_the_mid_layer_in_lds():
    """In LDS: 7 staged rows of 13 elements a channel, 23 16-byte pieces, 92
    a group: 2 loads a lane beside the filter's 3; a 27-word zero run."""
    a = plan(1, 512, 13, 13, 1024, 3, 3, 1, 1, 1, 1, 1, 1, imp=True)
    assert (a["Hr"], a["npc"], a["np"], a["zoff"], a["BS"]) == (7, 23, 2, 96, 128)
    assert a["lds"] == 8 * (16 * 36 + 4 * 128 + 256) * 4
