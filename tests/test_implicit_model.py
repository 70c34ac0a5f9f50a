"""CPU model of the in-LDS window kernel (conv_mfma_implicit_kernel).

Host-logic test: the kernel's launch plan, every address it computes (row
copies into the staging ring, the 8x8 transposes into the window-row
buffers, the window-fragment reads, the output tile and the stores) and its
hand-placed wait counts are replayed here in Python on small layers, each
access bounds-checked against the buffer it must stay in.  The replay also
carries the data: staged rows, transposed rows and the fragment products are
evaluated in numpy and the result is compared with the fp64 oracle, so a
wrong index (a transposed operand, a wrong tap or channel) fails here before
the kernel ever runs on a GPU.  The plan is tied to the library through
conv2d_implicit_workspace_bytes (eligibility and workspace size).
"""
import ctypes
import itertools

import numpy as np
import pytest

import oracle
from tests.test_band_model import band_plan

THREADS = 256
MAX_COPIES = 4
MAX_STORES = 4
LDS_CU = 160 * 1024


class G:   # resolved geometry, as the library's resolve() computes it
    def __init__(self, N, C, H, W, K, R, S, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1):
        self.N, self.C, self.H, self.W, self.K, self.R, self.S = N, C, H, W, K, R, S
        self.sh, self.sw, self.ph, self.pw, self.dh, self.dw = sh, sw, ph, pw, dh, dw
        self.P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
        self.Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
        self.Wwin = (self.Q - 1) * sw + dw * (S - 1) + 1


def compiled(R, S, CB):
    if (R, S) == (3, 3):
        return 1 <= CB <= 4
    if (R, S) == (1, 1):
        return CB in (1, 2, 4)
    return False


def plan(g, out_bytes, relu=False, pool=False, cus=256):
    if g.C % 16 or g.K > 64 or g.W % 8 or g.sh != 1:
        return None
    if pool and (g.P < 2 or g.Q < 2):
        return None
    CB = g.C // 16
    if not compiled(g.R, g.S, CB):
        return None
    if g.C * g.H * g.W * 2 >= 2 ** 31:
        return None
    a = dict(span=(g.R - 1) * g.dh + 1, cg=g.C // 8, wv=g.W // 8)
    a["nt"] = a["span"] + 1
    a["CS"] = a["cg"] | 1
    wb = max(g.Wwin, g.pw + g.W)
    a["wb"] = wb
    a["row_bytes"] = wb * a["CS"] * 16
    a["nchunks"] = g.C * g.W // 8
    a["nd"] = -(-a["nchunks"] // THREADS)
    if a["nd"] > MAX_COPIES:
        return None
    a["stage_bytes"] = max(a["nchunks"], THREADS) * 16
    a["plane_bytes"] = g.H * g.W * 2
    a["nblk"] = -(-g.Q // 32)
    a["nkh"] = 2 if g.K > 32 else 1
    V = 16 // out_bytes
    ost = -(-(32 * a["nblk"]) // V) * V
    if (ost * out_bytes // 16) % 2 == 0:
        ost += V
    a["ostride"] = ost
    a["pool"] = int(pool)
    a["Pc"] = 2 * (g.P // 2) if pool else g.P
    a["qout"] = g.Q // 2 if pool else g.Q
    a["yplane"] = (g.P // 2 if pool else g.P) * a["qout"]
    if g.K * a["yplane"] >= 2 ** 31:
        return None
    se = V
    while se > 1 and a["qout"] % se:
        se //= 2
    a["se"] = se
    a["nq"] = a["qout"] // se
    a["nsv"] = -(-(g.K * a["nq"]) // THREADS)
    if a["nsv"] > MAX_STORES:
        return None
    tile = 2 * g.K * ost * out_bytes
    lds = wgs = pf = 0
    for w in (2, 1):
        for p in (3, 2, 1):
            b = a["nt"] * a["row_bytes"] + (p + 1) * a["stage_bytes"] + tile + 256
            if b * w <= LDS_CU:
                lds, wgs, pf = b, w, p
                break
        if wgs:
            break
    if not wgs:
        return None
    a.update(pf=pf, nstage=pf + 1, lds=lds, wgs=wgs, tile=tile)
    a["off_stage"] = a["nt"] * a["row_bytes"]
    a["off_tile"] = a["off_stage"] + a["nstage"] * a["stage_bytes"]
    a["off_bias"] = a["off_tile"] + tile
    target = cus * wgs
    Pc = a["Pc"]
    nb = min(Pc, max(1, (target + g.N // 2) // max(g.N, 1)))
    a["band"] = max(-(-Pc // nb), min(Pc, 4))
    if pool:
        a["band"] += a["band"] & 1
    a["nbands"] = -(-Pc // a["band"])
    a["ntask"] = g.N * a["nbands"]
    a["steps"] = g.R * g.S * CB
    a["CB"] = CB
    a["out_bytes"] = out_bytes
    return a


def prep_filter(w16, g, a):
    """mfma_implicit_filter_kernel: aperm[kh][s][lane][e]."""
    steps, CB = a["steps"], a["CB"]
    wbits = np.ascontiguousarray(w16).view(np.uint16)
    out = np.zeros(2 * steps * 512, dtype=np.uint16)
    for i in range(out.size):
        e, lane, rest = i & 7, (i >> 3) & 63, i >> 9
        kh, s = divmod(rest, steps)
        k = kh * 32 + (lane & 31)
        cb, q, r = s % CB, (s // CB) % g.S, s // (CB * g.S)
        c = 16 * cb + 8 * (lane >> 5) + e
        if k < g.K:
            out[i] = wbits[k, c, r, q]
    return out


def stores_at(i, a):
    """The step of output row i stores row i - 1: every row, or with the
    pool the second row of each pair."""
    return i >= 1 and (not a["pool"] or (i - 1) % 2 == 1)


def tile_of(i, a):
    return (i >> a["pool"]) & 1


def later_ops(j, a, J):
    """Vector-memory operations a wave issues after the copy of row j, up to
    the wait for it (prologue copies rows 0..pf; step v copies row
    v + pf + 1, then stores output row v - span if that step stores)."""
    pf, nd, nsv, span = a["pf"], a["nd"], a["nsv"], a["span"]
    dma = lambda v: nd if v + pf + 1 < J else 0
    st = lambda v: nsv if stores_at(v - span + 1, a) else 0
    if j <= pf:
        c = nd * (min(pf + 1, J) - 1 - j)
        c += sum(dma(v) + st(v) for v in range(j - 1))
    else:
        c = st(j - pf - 1) + sum(dma(v) + st(v) for v in range(j - pf, j - 1))
    return c


def issue_log(a, J):
    """The kernel's vector-memory issue order for one band: ('dma', row) and
    ('st', output row) events, and the index of each wait's target."""
    log = [("dma", j) for j in range(min(a["pf"] + 1, J))]
    waits = {0: len(log)}
    for v in range(J):
        if v + 1 < J:
            waits[v + 1] = len(log)
        if v + a["pf"] + 1 < J:
            log += [("dma", v + a["pf"] + 1)] * 1
        i = v - a["span"] + 1
        if stores_at(i, a):
            log += [("st", i - 1)]
    return log, waits


def emulate(x16, w16, b, g, a, relu):
    """Replays the kernel on the CPU; returns y (fp64, before output rounding
    is applied by the caller) and checks every access.  Outputs go through
    the two tiles and the store plan, as in the kernel; `wrote` records
    which output row each tile element last held."""
    N, C, H, W, K = g.N, g.C, g.H, g.W, g.K
    pool = a["pool"]
    Po, Qo = (g.P // 2, g.Q // 2) if pool else (g.P, g.Q)
    xbytes = x16.reshape(-1).view(np.uint8)
    img_bytes = C * H * W * 2
    aperm = prep_filter(w16, g, a)
    y = np.full((N, K, Po, Qo), np.nan)
    yflat = y.reshape(-1)
    stores = store_plan(g, a)
    seen = np.zeros(a["ntask"], dtype=bool)
    span, cg, CS, wv = a["span"], a["cg"], a["CS"], a["wv"]
    nd, nchunks = a["nd"], a["nchunks"]
    steps, CB = a["steps"], a["CB"]
    # filter as the kernel's registers see it: F[kh][s] -> [lane][8]
    Freg = aperm.reshape(2, steps, 64, 8).view(np.float16).astype(np.float64)
    bias = np.zeros(64) if b is None else np.concatenate([b.astype(np.float64), np.zeros(64 - K)])
    for blk in range(a["ntask"]):
        task = (blk & 7) * (a["ntask"] >> 3) + (blk >> 3) if a["ntask"] % 8 == 0 else blk
        assert 0 <= task < a["ntask"] and not seen[task]
        seen[task] = True
        n, band = divmod(task, a["nbands"])
        h0 = band * a["band"]
        rows = min(a["band"], a["Pc"] - h0)
        assert rows >= 1 and (not pool or (h0 % 2 == 0 and rows % 2 == 0))
        tile = np.full((2, K, a["ostride"]), np.nan)
        wrote = np.full((2, K, a["ostride"]), -1)

        def store_row(i):
            t = tile_of(i, a)
            yrow = n * K * a["yplane"] + ((h0 + i) >> pool) * a["qout"]
            for (src, dst) in stores:
                k, c0 = divmod(src, a["ostride"])
                if pool:
                    cols = list(range(c0, c0 + 2 * a["se"]))
                else:
                    cols = list(range(c0, c0 + a["se"]))
                assert all(wrote[t, k, c] == i and c < g.Q for c in cols)
                vals = tile[t, k, cols]
                if pool:
                    vals = np.maximum(vals[0::2], vals[1::2])
                yflat[yrow + dst:yrow + dst + a["se"]] = vals
        J = rows + span - 1
        lds = np.zeros(a["lds"], dtype=np.uint8)
        # copy plan
        pos_base, src_off = [], []
        for j in range(MAX_COPIES):
            pb = nchunks - THREADS if (j == nd - 1 and nd > 1) else j * THREADS
            pos_base.append(pb)
            offs = []
            for tid in range(THREADS):
                p = min(pb + tid, nchunks - 1)
                gi, rest = p % cg, p // cg
                offs.append((8 * gi + (rest & 7)) * a["plane_bytes"] + 16 * (rest >> 3))
            src_off.append(offs)

        def copy_row(j):
            hin = min(max(h0 - g.ph + j, 0), H - 1)
            src = n * img_bytes + hin * W * 2
            slot0 = a["off_stage"] + (j % a["nstage"]) * a["stage_bytes"]
            for jj in range(nd):
                for tid in range(THREADS):
                    wave, lane = divmod(tid, 64)
                    dst = slot0 + 1024 * wave + 16 * pos_base[jj] + 16 * lane
                    assert slot0 <= dst and dst + 16 <= slot0 + a["stage_bytes"]
                    s0 = src_off[jj][tid]
                    assert 0 <= s0 and hin * W * 2 + s0 + 16 <= img_bytes
                    lds[dst:dst + 16] = xbytes[src + s0:src + s0 + 16]

        def transpose_row(j):
            hin = h0 - g.ph + j
            inside = 0 <= hin < H
            t0 = (j % a["nt"]) * a["row_bytes"]
            s0 = a["off_stage"] + (j % a["nstage"]) * a["stage_bytes"]
            for it in range(4 * cg * wv):
                jp, rest = it & 3, it >> 2
                gi, xv = rest % cg, rest // cg
                v = np.zeros((8, 2), dtype=np.uint16)   # [channel e][column 2jp + c]
                for e in range(8):
                    o = s0 + 16 * ((xv * 8 + e) * cg + gi) + 4 * jp
                    assert s0 <= o and o + 4 <= s0 + a["stage_bytes"]
                    if inside:
                        v[e] = lds[o:o + 4].view(np.uint16)
                for c in range(2):
                    o = t0 + 16 * ((g.pw + 8 * xv + 2 * jp + c) * CS + gi)
                    assert t0 <= o and o + 16 <= t0 + a["row_bytes"]
                    lds[o:o + 16] = v[:, c].copy().view(np.uint8)

        for j in range(min(a["pf"] + 1, J)):
            copy_row(j)
        # the wait counts: the op waited for is exactly later_ops back from
        # the end of what has been issued
        log, waits = issue_log(a, J)
        for j, pos in waits.items():
            ops = [e for e in log[:pos]]
            k = max(idx for idx, e in enumerate(ops) if e == ("dma", j))
            assert sum(nd if e[0] == "dma" else a["nsv"] for e in ops[k + 1:]) == later_ops(j, a, J)
        transpose_row(0)
        done = {0}
        for u in range(J):
            i = u - span + 1
            if stores_at(i, a):
                # the tile it reads is not the one this step's multiply writes
                assert tile_of(i - 1, a) != tile_of(i, a)
                store_row(i - 1)
            if u + a["pf"] + 1 < J:
                # the staging buffer it overwrites held row u, transposed already
                assert u in done
                copy_row(u + a["pf"] + 1)
            i = u - span + 1
            if u + 1 < J:
                # the buffer it overwrites held row u + 1 - nt, whose last reader
                # (output row u + 1 - nt) was multiplied in an earlier step
                assert u + 1 - a["nt"] < i or u + 1 - a["nt"] < 0
                transpose_row(u + 1)
                done.add(u + 1)
            if i < 0:
                continue
            # the rows output row i reads were transposed in earlier steps
            for r in range(g.R):
                assert i + r * g.dh <= u and (i + r * g.dh) in done
            soff = [((i + r * g.dh) % a["nt"]) * a["row_bytes"] for r in range(g.R)]
            for kh in range(a["nkh"]):
                for bb in range(a["nblk"]):
                    acc = np.tile(bias[kh * 32:kh * 32 + 32], (32, 1))   # [pixel][channel]
                    for s in range(steps):
                        cb, q, r = s % CB, (s // CB) % g.S, s // (CB * g.S)
                        A = np.zeros((32, 16))
                        for lane in range(64):
                            ml, gg = lane & 31, lane >> 5
                            wr = min(32 * bb + ml, g.Q - 1)
                            o = (wr * g.sw * CS + gg) * 16 + soff[r] + q * g.dw * CS * 16 + 32 * cb
                            assert soff[r] <= o and o + 16 <= soff[r] + a["row_bytes"]
                            A[ml, 8 * gg:8 * gg + 8] = lds[o:o + 16].view(np.float16).astype(np.float64)
                        Bm = np.zeros((16, 32))
                        for lane in range(64):
                            Bm[8 * (lane >> 5):8 * (lane >> 5) + 8, lane & 31] = Freg[kh, s, lane]
                        acc += A @ Bm
                    if relu:
                        acc = np.maximum(acc, 0)
                    t = tile_of(i, a)
                    for ml in range(32):
                        w_ = 32 * bb + ml
                        assert w_ < a["ostride"]
                        for kk in range(32):
                            k = kh * 32 + kk
                            if k < K:
                                v = acc[ml, kk]
                                if pool and i % 2 == 1:
                                    # the first row of the pair, same lane
                                    assert wrote[t, k, w_] == i - 1
                                    v = max(v, tile[t, k, w_])
                                tile[t, k, w_] = v
                                wrote[t, k, w_] = i
        store_row(rows - 1)
    assert seen.all()
    return y


def store_plan(g, a):
    """(tile offset, y offset) of every store of one output row, over all
    threads: idx = tid + 256 j, surplus threads repeating the last."""
    out = []
    for tid in range(THREADS):
        for j in range(a["nsv"]):
            idx = min(tid + THREADS * j, g.K * a["nq"] - 1)
            k, v = divmod(idx, a["nq"])
            out.append((k * a["ostride"] + ((v * a["se"]) << a["pool"]),
                        k * a["yplane"] + v * a["se"]))
    return out


def store_indices_ok(g, a):
    """The store plan: every (k, vector) of an output row exactly covered,
    reads inside the tile row, writes inside the output row block, and both
    aligned to the store's width."""
    E, eb = a["se"], a["out_bytes"]
    span = E << a["pool"]          # tile elements one store reads
    covered = set()
    for src, dst in store_plan(g, a):
        k = src // a["ostride"]
        assert src + span <= g.K * a["ostride"] and (src + span - 1) // a["ostride"] == k
        assert (src - k * a["ostride"]) + span <= g.Q
        assert dst + E <= g.K * a["yplane"] and (dst - k * a["yplane"]) + E <= a["qout"]
        assert (src * eb) % min(16, span * eb) == 0 and (dst * eb) % (E * eb) == 0
        covered.add((k, dst - k * a["yplane"]))
    assert len(covered) == g.K * a["nq"]
    assert E * eb in (2, 4, 8, 16) and a["qout"] % E == 0


CASES = [
    # N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw
    (1, 16, 5, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1),
    (2, 32, 7, 16, 40, 3, 3, 1, 1, 1, 1, 1, 1),
    (1, 64, 6, 8, 64, 3, 3, 1, 1, 0, 0, 1, 1),
    (2, 48, 5, 8, 33, 3, 3, 1, 2, 2, 1, 1, 1),
    (1, 16, 9, 16, 24, 3, 3, 1, 1, 2, 2, 2, 2),
    (3, 32, 4, 8, 64, 1, 1, 1, 1, 0, 0, 1, 1),
    (1, 64, 3, 40, 64, 3, 3, 1, 1, 1, 1, 1, 1),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("out_bytes,cus,pool", [(2, 256, False), (4, 256, False), (2, 1, False),
                                                (2, 256, True), (4, 1, True)])
def test_emulated_kernel_matches_oracle(case, out_bytes, cus, pool):
    N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw = case
    g = G(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw)
    a = plan(g, out_bytes, pool=pool, cus=cus)
    assert a is not None
    rng = np.random.default_rng(7)
    x = rng.standard_normal((N, C, H, W)).astype(np.float16)
    w = (rng.standard_normal((K, C, R, S)) * 0.2).astype(np.float16)
    b = rng.uniform(-0.1, 0.1, K).astype(np.float16)
    relu = out_bytes == 4
    got = emulate(x, w, b, g, a, relu)
    ref = oracle.conv2d(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64),
                        (sh, sw), (ph, pw), (dh, dw), 1)
    ref = oracle.relu_pool(ref, relu=relu, pool=pool)
    assert not np.isnan(got).any()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-9 * max(1.0, np.abs(ref).max()))
    store_indices_ok(g, a)


@pytest.mark.parametrize("out_bytes", [2, 4])
def test_plan_resnet_layer(out_bytes):
    """The 128x64x56x56 -> 64 3x3 layer: with fp16 output two workgroups per
    CU and 512 bands of 14 rows; with fp32 output (a tile twice the size)
    one workgroup per CU.  Store plan and wait counts valid."""
    g = G(128, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1, 1, 1)
    a = plan(g, out_bytes)
    assert a is not None
    if out_bytes == 2:
        assert a["wgs"] == 2 and a["ntask"] == 512 and a["band"] == 14
    assert a["lds"] * a["wgs"] <= LDS_CU
    store_indices_ok(g, a)
    J = a["band"] + a["span"] - 1
    for j in range(J):
        assert later_ops(j, a, J) >= 0


def test_plan_agrees_with_library():
    """Eligibility and workspace: this model's plan and the library agree."""
    import cnn_convolution_im2win_amd as ciw
    from cnn_convolution_im2win_amd import _lib
    rng = np.random.default_rng(3)
    shapes = list(CASES) + [
        (128, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1, 1, 1),
        (1, 24, 8, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1),      # C not a multiple of 16
        (1, 16, 8, 12, 8, 3, 3, 1, 1, 1, 1, 1, 1),     # W not a multiple of 8
        (1, 16, 8, 8, 80, 3, 3, 1, 1, 1, 1, 1, 1),     # K > 64
        (1, 16, 9, 8, 8, 3, 3, 2, 1, 1, 1, 1, 1),      # stride_h 2
        (1, 80, 8, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1),      # C/16 = 5 not compiled
        (1, 16, 8, 8, 8, 5, 5, 1, 1, 2, 2, 1, 1),      # 5x5 not compiled
        (1, 32, 8, 8, 8, 1, 1, 1, 1, 0, 0, 1, 1),
        (1, 48, 8, 8, 8, 1, 1, 1, 1, 0, 0, 1, 1),      # 1x1 with C/16 = 3 not compiled
        (2, 64, 4, 256, 64, 3, 3, 1, 1, 1, 1, 1, 1),   # too many stores per thread
    ]
    for _ in range(40):
        C = int(rng.choice([16, 32, 48, 64]))
        R = int(rng.choice([1, 3]))
        shapes.append((int(rng.integers(1, 4)), C, int(rng.integers(3, 20)),
                       8 * int(rng.integers(1, 12)), int(rng.integers(1, 70)), R, R, 1,
                       int(rng.integers(1, 3)), int(rng.integers(0, 3)),
                       int(rng.integers(0, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 3))))
    for s in shapes:
        N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw = s
        g = G(*s)
        if g.P < 1 or g.Q < 1:
            continue
        desc = ciw.make_desc((N, C, H, W), (K, C, R, S), (sh, sw), (ph, pw), (dh, dw), 1)
        for (dt, ob), pool in itertools.product(((ciw.CIW_F16, 2), (ciw.CIW_BF16, 2),
                                                  (ciw.CIW_F16, 4)), (False, True)):
            out_dt = dt if ob == 2 else ciw.CIW_F32
            a = plan(g, ob, pool=pool)
            out = ctypes.c_size_t()
            flags = _lib.CIW_FLAG_MAXPOOL2 if pool else 0
            st = _lib.load().conv2d_implicit_workspace_bytes(ctypes.byref(desc), dt, out_dt, flags,
                                                             ctypes.byref(out))
            # the band kernel (3x3, no pool; no workspace) takes the layers it
            # runs before this kernel
            band = band_plan(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, pool=pool)
            if pool and (g.P < 2 or g.Q < 2):
                assert st == _lib.CIW_ERR_INVALID_ARG, s
            elif band is not None:
                assert st == 0 and out.value == 0, s
            elif a is None:
                assert st == _lib.CIW_ERR_UNSUPPORTED, s
            else:
                assert st == 0, s
                assert out.value == 2 * a["steps"] * 512 * 2
