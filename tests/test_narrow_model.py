"""CPU model of the few-channel in-LDS kernel (conv_mfma_narrow_kernel,
csrc/conv_narrow_impl.hpp): the fp16/bf16 contraction for layers such as the
3-channel 7x7 stride-2 stem.  It keeps a ring of zero-padded input rows in
LDS ([slot][channel][column]), reduces in (channel,
filter row, filter column) order, and reads each lane's 8 entries of an MFMA
step as one strip of a row, masked to the filter's columns.

The model mirrors the plan and replays, for every band of a layer, the
prologue (padding columns cleared, the first step's rows copied in,
the filter staged) and every step (each block's fragment reads, the next
step's rows copied into the ring, output stores).  It checks:
  * every LDS access lies inside the kernel's allocation and inside the slot
    and channel row it is meant for; fragment reads are 4-byte aligned;
  * a slot is read only while it holds the row the read needs (each slot is
    tagged with the input row it holds), never a row the step does not have,
    and no copy writes a slot that the same step reads;
  * copies never write padding columns, and every entry a fragment keeps
    was written; only the last step's second pair may be missing (C R odd),
    and its fragment is cleared;
  * every global load lies inside x, and every output is stored exactly
    once, inside y;
  * the outputs multiplied out from the fragments the kernel would read
    (masked as the kernel masks them) equal the oracle's convolution.
The plan is tied to the library through conv2d_implicit_workspace_bytes:
for layers whose channel count is not a multiple of 16 (which no other
in-LDS kernel runs), the library takes the flag exactly when the model's
plan accepts the layer, with 0 bytes of workspace."""
import numpy as np
import pytest

import oracle
import workloads

THREADS = 256
WAVES = THREADS // 64
MAX_IT, MAX_IT0, MAX_FILT = 6, 8, 6
LDS = 80 * 1024


def ceil_div(a, b):
    return -(-a // b)


def narrow_plan(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, pool=False, cus=256, out_bytes=2):
    """Python mirror of narrow_plan(): None if the kernel does not run the layer."""
    if pool or dw != 1 or sw % 2 or K > 64 or W % 8:
        return None
    CR = C * R
    if CR > 22:
        return None
    L = ceil_div(pw, 4) * 4
    d = (L - pw) & 1
    if S + d > 8 or S + d < 6:
        return None
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    if P < 1 or Q < 1:
        return None
    if C * H * W >= 2 ** 31 or K * P * Q * out_bytes >= 2 ** 32:
        return None
    span = (R - 1) * dh + 1
    col0 = L - pw - d
    keep = [d <= e < d + S for e in range(8)]
    cols = max(L + W, (Q - 1) * sw + col0 + 8)
    RB = ceil_div(cols, 8) * 8 * 2
    slot_bytes = C * RB
    if slot_bytes * (2 * span - 1) > LDS:
        return None
    wv = W // 8
    filt_elems = K * CR * S
    filt_bytes = ceil_div(filt_elems * 2, 16) * 16 + 32   # 16 bytes of slack below and above
    if filt_elems * 2 // 16 > MAX_FILT * THREADS:
        return None
    eb = out_bytes
    tiles = WAVES * 64 * (32 * eb + 16)
    region = max(filt_bytes, tiles)   # the staged filter, then the output tiles
    Nn = max(N, 1)
    nb = max(1, min(P, ceil_div(2 * cus, Nn)))
    band = ceil_div(P, nb)
    nbands = ceil_div(P, band)
    per_row = C * wv
    SR = NR = lds = 0
    for sr in range(min(band, 16), 0, -1):
        nr = (2 * sr - 1) * sh + span
        r0 = (sr - 1) * sh + span
        need = (nr + span - 1) * slot_bytes + region   # ring and mirror slots
        if need <= LDS and sr * sh * per_row <= MAX_IT * THREADS and \
                r0 * per_row <= MAX_IT0 * THREADS:
            SR, NR, lds = sr, nr, need
            break
    if SR == 0:
        return None
    return dict(N=N, C=C, H=H, W=W, K=K, R=R, S=S, P=P, Q=Q, sh=sh, sw=sw, ph=ph, pw=pw, dh=dh,
                CR=CR, span=span, L=L, d=d, col0=col0, keep=keep, RB=RB, slot_bytes=slot_bytes,
                NR=NR, SR=SR, wv=wv, nl=L // 4, nr=(RB // 2 - L - W) // 4, band=band,
                nbands=nbands, ntask=N * nbands, filt_elems=filt_elems, filt_bytes=filt_bytes,
                ring_bytes=NR * slot_bytes, mirror_lim=(span - 1) * slot_bytes,
                filt_off=(NR + span - 1) * slot_bytes, tiles=tiles, lds=lds,
                staged=Q % (16 // eb) == 0, vec=Q % 4 == 0, out_bytes=eb, KS=ceil_div(CR, 2))


def replay(pl, x, wf, bias=None):
    """Replay every band; returns y (fp64) built from the LDS contents."""
    N, C, H, W, K, R, S, P, Q = (pl[k] for k in ("N", "C", "H", "W", "K", "R", "S", "P", "Q"))
    sh, sw, ph, dh = pl["sh"], pl["sw"], pl["ph"], pl["dh"]
    CR, span, L, d, col0, keep = (pl[k] for k in ("CR", "span", "L", "d", "col0", "keep"))
    RB, SB, NR, SR, wv, KS = (pl[k] for k in ("RB", "slot_bytes", "NR", "SR", "wv", "KS"))
    per_row = C * wv
    assert pl["filt_off"] + 16 + 2 * pl["filt_elems"] + 16 <= pl["filt_off"] + pl["filt_bytes"] <= pl["lds"]
    assert pl["filt_off"] + pl["tiles"] <= pl["lds"] <= LDS
    assert 2 * KS - 1 <= CR <= 2 * KS and (span - 1) < NR
    y = np.full((N, K, P, Q), np.nan)
    written = np.zeros((N, K, P, Q), dtype=np.int64)
    kmask = np.array(keep)
    assert kmask[2:6].all(), "only a fragment's first and last words are masked"
    # filter fragments F[ct][ks][lane] (8 entries), built as the kernel builds
    # them: the staged filter starts 16 bytes into its region (unwritten
    # half-words are NaN), entry 0 of (k, u) is half-word (k C R + u) S - d + 8,
    # read as aligned words, shifted into place, masked to the taps
    fbytes = pl["filt_bytes"]
    staged = np.full(fbytes // 2, np.nan)
    staged[8:8 + pl["filt_elems"]] = wf.reshape(-1)
    F = np.zeros((2, KS, 64, 8))
    for ct in range(2):
        for ks in range(KS):
            for lane in range(64):
                k, u = 32 * ct + lane % 32, 2 * ks + lane // 32
                ok = k < K and u < CR
                e0 = (k * CR + u) * S - d + 8 if ok else 8
                word = e0 >> 1   # five aligned words from there, shifted into place
                assert 0 <= 4 * word and 4 * (word + 5) <= fbytes, "a filter read leaves the region"
                vals = staged[e0:e0 + 8]
                if ok:
                    assert not np.isnan(vals[kmask]).any()
                    F[ct, ks, lane] = np.where(kmask, vals, 0.0)
                    for e in range(8):   # the taps the entries must hold
                        if kmask[e]:
                            assert vals[e] == wf[k, u // R, u % R, e - d]
    bk = np.zeros(64)
    if bias is not None:
        bk[:K] = bias
    for task in range(pl["ntask"]):
        n, bi = divmod(task, pl["nbands"])
        h0 = bi * pl["band"]
        rows = min(pl["band"], P - h0)
        nsteps = ceil_div(rows, SR)
        orow = lambda t: min(t * SR, rows)
        rb = lambda t: (orow(t + 1) - 1) * sh + span
        xr0 = h0 * sh - ph
        NS = NR + span - 1                            # ring slots and their mirrors
        ring = np.full(NS * SB // 2, np.nan)         # LDS ring, one entry per 16-bit element
        wr = np.zeros(NS * SB // 2, dtype=bool)      # entry written
        pad = np.zeros(NS * SB // 2, dtype=bool)     # padding columns
        tag = np.full(NS, -1)                         # band input row a slot holds

        # zeros: per slot, each channel row's nl + nr padding words
        per_c = pl["nl"] + pl["nr"]
        units = C * per_c
        for it in range(NS * units):
            slot, u = divmod(it, units)
            c, k = divmod(u, per_c)
            off = slot * SB + c * RB + (8 * k if k < pl["nl"] else 2 * (L + W) + 8 * (k - pl["nl"]))
            lo = slot * SB + c * RB
            assert lo <= off and off + 8 <= lo + RB
            col = (off - lo) // 2
            assert col + 4 <= L or col >= L + W, "zeroes an input column"
            assert off % 8 == 0
            ring[off // 2:off // 2 + 4] = 0.0
            wr[off // 2:off // 2 + 4] = True
            pad[off // 2:off // 2 + 4] = True
        # every padding column was cleared
        for slot in range(NS):
            for c in range(C):
                row = slot * SB // 2 + c * RB // 2 + np.arange(RB // 2)
                cols = np.arange(RB // 2)
                assert np.array_equal(pad[row], (cols < L) | (cols >= L + W))

        def copy_rows(j0, j1, max_per_thread):
            nitems = (j1 - j0) * per_row
            assert nitems <= max_per_thread * THREADS
            for it in range(nitems):
                jr, rem = divmod(it, per_row)
                c, vv = divmod(rem, wv)
                j = j0 + jr
                slot = j % NR
                dst = slot * SB + c * RB + (L + 8 * vv) * 2
                lo = slot * SB + c * RB
                assert dst % 8 == 0 and lo <= dst and dst + 16 <= lo + RB
                xrow = xr0 + j
                # every item's load is issued, from row 0 where the row is padding
                goff = 2 * (c * H * W + (xrow if 0 <= xrow < H else 0) * W + 8 * vv)
                assert 0 <= goff and goff + 16 <= 2 * C * H * W
                vals = x[n, c, xrow, 8 * vv:8 * vv + 8] if 0 <= xrow < H else 0.0
                for d_ in ([dst, dst + pl["ring_bytes"]] if dst < pl["mirror_lim"] else [dst]):
                    idx = d_ // 2 + np.arange(8)
                    assert not pad[idx].any(), "a copy writes a padding column"
                    ring[idx] = vals
                    wr[idx] = True
            for j in range(j0, j1):
                tag[j % NR] = j
                if j % NR < span - 1:
                    tag[j % NR + NR] = j   # the mirror slot

        copy_rows(0, rb(0), MAX_IT0)
        for t in range(nsteps):
            o0 = orow(t)
            npx = (orow(t + 1) - o0) * Q
            nblk = ceil_div(npx, 32)
            pix0 = o0 * Q
            need = set()
            for b in range(nblk):
                acc = np.zeros((2, 32, 32))   # [ct][pixel m][channel n]
                acc += bk.reshape(2, 1, 32)
                for lane in range(64):
                    ml, g = lane % 32, lane // 32
                    pb = pix0 + min(32 * b + ml, npx - 1)
                    i, q = divmod(pb, Q)
                    jb = i * sh
                    s0 = jb % NR
                    colb = (q * sw + col0) * 2
                    for ks in range(KS):
                        u = 2 * ks + g
                        c, r = (u // R, u % R) if u < CR else (0, 0)
                        s = s0 + r * dh            # no wrap: the mirror slots continue the ring
                        assert s < NS
                        off = s * SB + c * RB + colb
                        lo = s * SB + c * RB
                        assert off % 4 == 0 and lo <= off and off + 16 <= lo + RB
                        vals = ring[off // 2:off // 2 + 8].copy()
                        if u < CR:
                            j = jb + r * dh
                            assert j < rb(t), "reads a row this step does not have"
                            assert tag[s] == j, "slot holds another row"
                            need.add(s)
                            assert wr[off // 2:off // 2 + 8][kmask].all(), "keeps an unwritten entry"
                        else:
                            assert ks == KS - 1 and g == 1, "only the last step's second pair may be unused"
                        tailm = not (ks == KS - 1 and u >= CR)
                        vals = np.where(kmask & tailm, vals, 0.0)
                        for ct in range(2):
                            # lane (ml, g) is row m = ml of the window operand and column
                            # n = ml of the filter operand, both with k = 8 g + e
                            acc[ct, ml, :] += F[ct, ks, 32 * g:32 * g + 32, :] @ vals
                # stores: pixels below npx, channels below K, each exactly once
                ps = 32 * b + np.arange(32)
                pm = ps < npx
                hh, ww = np.divmod(pix0 + ps[pm], Q)
                for ct in range(2):
                    if 32 * ct >= K:
                        break
                    ks_ = np.arange(32 * ct, 32 * ct + 32)
                    km = ks_ < K
                    kk = ks_[km]
                    y[n, kk[:, None], h0 + hh[None, :], ww[None, :]] = acc[ct][np.ix_(pm, km)].T
                    np.add.at(written, (n, kk[:, None], h0 + hh[None, :], ww[None, :]), 1)
                if pl["staged"]:
                    # the wave's tile: 64 channel rows of 32 outputs; every
                    # lane writes its 4-output runs of both halves, then reads
                    # NRD 16-byte pieces and stores them
                    eb = pl["out_bytes"]
                    ostr, cpr = 32 * eb + 16, 2 * eb
                    wave = b % 4
                    assert (wave + 1) * 64 * ostr <= pl["tiles"]
                    written_t = np.zeros((64, 32 * eb), dtype=bool)
                    for lane in range(64):
                        ml, g = lane % 32, lane // 32
                        for ct in range(2 if K > 32 else 1):
                            for jq in range(4):
                                o = (8 * jq + 4 * g) * eb
                                written_t[32 * ct + ml, o:o + 4 * eb] = True
                    for lane in range(64):
                        for r in range(64 * cpr // 64):
                            piece = lane + 64 * r
                            kk, seg = divmod(piece, cpr)
                            assert kk * ostr + 16 * seg + 16 <= 64 * ostr
                            p = 32 * b + seg * (16 // eb)
                            if kk < K and p < npx:   # a stored piece was written, never crosses the step's end
                                assert p + 16 // eb <= npx
                                assert written_t[kk, 16 * seg:16 * seg + 16].all()
            if t + 1 < nsteps:
                new = {j % NR for j in range(rb(t), rb(t + 1))}
                new |= {s_ + NR for s_ in new if s_ < span - 1}
                assert not (new & need), "a copy overwrites a slot the step reads"
                copy_rows(rb(t), rb(t + 1), MAX_IT)
    assert np.all(written == 1), "an output is stored twice or never"
    return y


SHAPES = [
    # (N, C, H, W, K, R, S, stride, pad, dil_h, cus)
    (1, 3, 40, 224, 64, 7, 7, (2, 2), (3, 3), 1, 1),    # the stem's rows and filter, a few bands
    (2, 3, 23, 40, 40, 7, 7, (2, 2), (3, 3), 1, 2),     # K not a multiple of 32, ragged rows
    (1, 2, 30, 64, 24, 5, 5, (1, 2), (2, 1), 1, 1),     # 5x5 (pad_w 1: a trailing entry masked), stride_h 1
    (1, 4, 26, 32, 33, 5, 6, (3, 2), (1, 1), 2, 1),     # dilation_h 2, stride_h 3, S = 6
    (1, 1, 17, 16, 8, 7, 7, (2, 4), (0, 3), 1, 1),      # one channel, stride_w 4, no row padding
    (2, 3, 12, 8, 64, 3, 7, (2, 2), (1, 5), 1, 2),      # pad_w 5 (L = 8, d = 1), 6 pairs
    (2, 3, 112, 64, 64, 7, 7, (2, 2), (3, 3), 1, 1),    # one band an image: the ring wraps, mirrors read
    (2, 2, 70, 48, 24, 5, 6, (1, 2), (2, 1), 2, 1),     # the same with stride_h 1, dil_h 2
]


@pytest.mark.parametrize("shape", SHAPES)
def test_narrow_model_against_oracle(shape):
    N, C, H, W, K, R, S, (sh, sw), (ph, pw), dh, cus = shape
    pl = narrow_plan(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, 1, cus=cus)
    assert pl is not None
    rng = np.random.default_rng(sum(shape[:7]))
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((K, C, R, S))
    b = rng.standard_normal(K)
    y = replay(pl, x, w, b)
    ref = oracle.conv2d(x, w, b, (sh, sw), (ph, pw), (dh, 1), 1)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_narrow_model_masks_other_windows_columns():
    """Infinities in x reach exactly the outputs whose windows hold them: the
    leading and trailing entries of a strip (other windows' columns) are
    masked, not multiplied by the filter's zeros (0 x Inf would be NaN)."""
    N, C, H, W, K, R, S, sh, sw, ph, pw = 1, 3, 24, 64, 40, 7, 7, 2, 2, 3, 3
    pl = narrow_plan(N, C, H, W, K, R, S, sh, sw, ph, pw, 1, 1, cus=1)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((K, C, R, S))
    for c, h, col, v in ((0, 3, 10, np.inf), (1, 11, 33, -np.inf), (2, 20, 63, np.inf), (1, 0, 0, np.nan)):
        x[0, c, h, col] = v
    with np.errstate(invalid="ignore"):   # Inf - Inf and NaN in channels never stored
        y = replay(pl, x, w)
    ref = oracle.conv2d(x, w, None, (sh, sw), (ph, pw), 1, 1)
    assert np.isfinite(ref).sum() > 0 and (~np.isfinite(ref)).sum() > 0
    np.testing.assert_array_equal(np.isnan(y), np.isnan(ref))
    np.testing.assert_array_equal(np.isinf(y), np.isinf(ref))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(y[fin], ref[fin], rtol=1e-12, atol=1e-12 * np.abs(ref[fin]).max())


def test_narrow_plan_of_the_stem():
    L = workloads.LAYERS["stem_7x7_s2_bf16"]
    pl = narrow_plan(L.N, L.C, L.H, L.W, L.K, 7, 7, 2, 2, 3, 3, 1, 1)
    # four bands of 28 rows an image (512 workgroups, two per CU), steps of
    # 8 rows (28 blocks of 32 pixels, 7 a wave) and a last one of 4, 37 ring
    # slots and 6 mirror slots of 3 channel rows of 232 columns, 11 steps of
    # 16 reduction entries
    assert (pl["band"], pl["nbands"], pl["ntask"], pl["SR"], pl["NR"], pl["KS"]) == \
        (28, 4, 512, 8, 37, 11)
    assert (pl["L"], pl["d"], pl["col0"], pl["RB"]) == (4, 1, 0, 464)
    assert pl["keep"] == [False] + [True] * 7
    # the filter's region then holds the four waves' 64-row output tiles
    assert pl["staged"] and pl["lds"] == 43 * 3 * 464 + 4 * 64 * 80 <= LDS


m = pytest.importorskip("cnn_convolution_im2win_amd")


def test_narrow_eligibility_matches_library():
    """For channel counts no other in-LDS kernel takes (not a multiple of
    16), the library accepts CIW_FLAG_IMPLICIT with 0 bytes of workspace
    exactly when the model's plan accepts the layer."""
    rng = np.random.default_rng(11)
    cases = [(128, 3, 224, 224, 64, 7, 7, 2, 2, 3, 3, 1)]
    for _ in range(80):
        R = int(rng.integers(1, 9))
        cases.append((int(rng.integers(1, 5)), int(rng.choice([1, 2, 3, 4, 5, 7])), int(rng.integers(3, 40)),
                      int(rng.choice([8, 16, 24, 40, 64])), int(rng.integers(1, 80)), R,
                      int(rng.integers(1, 9)), int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 4])),
                      int(rng.integers(0, 5)), int(rng.integers(0, 6)), int(rng.integers(1, 3))))
    seen = 0
    for N, C, H, W, K, R, S, sh, sw, ph, pw, dh in cases:
        for pool in (False, True):
            d = m.make_desc((N, C, H, W), (K, C, R, S), (sh, sw), (ph, pw), (dh, 1), 1)
            try:
                P, Q = m.conv_im2win_output_dims(d)
            except m.Im2winError:
                continue
            if pool and (P < 2 or Q < 2):
                continue
            flags = m.CIW_FLAG_IMPLICIT | (m.CIW_FLAG_MAXPOOL2 if pool else 0)
            for dt in (m.CIW_BF16, m.CIW_F16):
                for out in (dt, m.CIW_F32):
                    try:
                        nbytes = m.conv2d_implicit_workspace_bytes(d, dt, out, flags)
                    except m.Im2winError:
                        nbytes = None
                    pl = narrow_plan(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, 1, pool=pool,
                                     out_bytes=4 if out == m.CIW_F32 else 2)
                    assert (pl is not None) == (nbytes == 0), (N, C, H, W, K, R, S, sh, sw, ph, pw, dh, pool)
                    seen += pl is not None
    assert seen > 20
