"""CPU model of the band kernel (conv_mfma_band_kernel, csrc/conv_band_impl.hpp):
the fp16/bf16 3x3 contraction that keeps a ring of transposed input rows in
LDS and computes SR output rows per step.

The model mirrors the kernel's plan and replays, for every band of a layer,
the prologue (padding columns zeroed, first step's rows transposed into the
ring, filter staged above them) and every step (ring reads of each task,
the next step's rows transposed into the ring, output stores).  It checks:
  * every LDS access (zeroing, transposes, filter staging and reads,
    fragment reads) lies inside the kernel's LDS allocation and inside the
    ring slot / column / chunk it is meant for;
  * no transpose writes a ring slot that the same step's tasks read, and a
    slot is read only after the row it must hold has been written (each slot
    is tagged with the input row it holds);
  * padding columns are zero when read and never overwritten;
  * every global load lies inside x and w, and every output is stored
    exactly once, inside y;
  * the outputs computed from the replayed ring contents (the fragments each
    task would read, times the filter fragments, in numpy) equal the
    oracle's convolution.
The plan is tied to the library through conv2d_implicit_workspace_bytes:
the layers the model accepts are exactly those for which the library
reports the band kernel's workspace (0 bytes), apart from the few-channel
layers (C not a multiple of 16) that another no-workspace kernel runs."""
import math

import numpy as np
import pytest

import oracle
import workloads

THREADS = 512
LDS_MAX = 160 * 1024


def band_plan(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, pool=False, cus=256, out_bytes=2):
    """Python mirror of band_plan(): None if the kernel does not run the layer."""
    if R != 3 or S != 3 or C % 16 or C > 64 or K > 64 or W % 8 or sh != 1 or pool:
        return None
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    if P < 1 or Q < 1:
        return None
    span = 2 * dh + 1
    cg = C // 8
    CS = cg | 1
    wb = max(pw + W, (Q - 1) * sw + 2 * dw + 1)
    row_bytes = wb * CS * 16
    wv = W // 8
    nkh = 2 if K > 32 else 1
    CB = C // 16
    filt_bytes = nkh * 9 * CB * 64 * 16
    raw_bytes = nkh * CB * 32 * 18 * 16          # the stager waves' raw filter pieces
    Nn = max(N, 1)
    nb = max(1, min(P, (cus + Nn - 1) // Nn))
    band = max((P + nb - 1) // nb, min(P, 8))
    nbands = (P + band - 1) // band
    per_row = cg * wv
    SR = SR0 = NR = lds = 0
    for sr in range(min(band, 16), 0, -1):
        nr = 2 * sr + span - 1
        sr0 = max(1, sr // 2)
        while sr0 > 1 and (sr0 + span - 1) * per_row > THREADS:
            sr0 -= 1
        r0 = sr0 + span - 1
        need = max(nr * row_bytes, max(r0 * row_bytes, raw_bytes) + filt_bytes)
        if need <= LDS_MAX and sr * per_row <= THREADS and r0 * per_row <= THREADS:
            SR, SR0, NR, lds = sr, sr0, nr, need
            break
    if SR == 0:
        return None
    # per-wave output tiles for the staged stores, where they fit
    tiles = 8 * (1024 // (32 * out_bytes)) * (32 * out_bytes + 16)
    staged = Q % (16 // out_bytes) == 0 and lds + tiles <= LDS_MAX
    ostage_off = lds
    if staged:
        lds += tiles
    return dict(dv=(sw == 1 and dw == 1 and Q % 2 == 0), staged=staged, ostage_off=ostage_off, out_bytes=out_bytes, N=N, C=C, H=H, W=W, K=K, P=P, Q=Q, sw=sw, ph=ph, pw=pw, dh=dh, dw=dw, span=span,
                SR=SR, SR0=SR0, NR=NR, CS=CS, wb=wb, row_bytes=row_bytes, wv=wv, band=band,
                nbands=nbands, ntask=N * nbands, nkh=nkh, CB=CB, cg=cg,
                filt_off=max((SR0 + span - 1) * row_bytes, raw_bytes), raw_bytes=raw_bytes, lds=lds)


def replay(pl, x, wf, dv_rule=None):
    """Replay every band; returns y (fp64) built from the ring contents.
    dv_rule (tests only) replaces the kernel's choice of neighbour lane for
    filter column 1: a function (ml, wc, Q) -> bool array, True for m + 1."""
    N, C, H, W, K, P, Q = (pl[k] for k in ("N", "C", "H", "W", "K", "P", "Q"))
    CS, NR, SR, span, wb, cg, wv = (pl[k] for k in ("CS", "NR", "SR", "span", "wb", "cg", "wv"))
    SR0 = pl["SR0"]
    rb_bytes, CB, nkh = pl["row_bytes"], pl["CB"], pl["nkh"]
    sw, ph, pw, dh, dw = (pl[k] for k in ("sw", "ph", "pw", "dh", "dw"))
    assert NR * rb_bytes <= pl["lds"] <= LDS_MAX
    assert pl["filt_off"] + nkh * 9 * CB * 1024 <= pl["lds"]
    y = np.full((N, K, P, Q), np.nan)
    written = np.zeros((N, K, P, Q), dtype=np.int64)
    # ring contents: value[slot][col][channel] and tags
    for task in range(pl["ntask"]):
        n, bi = divmod(task, pl["nbands"])
        h0 = bi * pl["band"]
        rows = min(pl["band"], P - h0)
        nsteps = 1 if rows <= SR0 else 1 + (rows - SR0 + SR - 1) // SR
        orow = lambda t: 0 if t == 0 else min(SR0 + (t - 1) * SR, rows)
        rb = lambda t: orow(t + 1) + span - 1
        ring = np.full((NR, wb, C), np.nan)          # NaN: never written
        tag = np.full(NR, -1)                         # input row a slot holds (-1: none)
        padded = np.zeros((NR, wb), dtype=bool)       # padding column zeroed

        def zero_pads(s0, s1):
            for s in range(s0, s1):
                for col in list(range(pw)) + list(range(pw + W, wb)):
                    ring[s, col, :] = 0.0
                    padded[s, col] = True

        def transpose_rows(j0, j1):
            """All items of rows [j0, j1) (the kernel spreads them over threads)."""
            nitems = (j1 - j0) * cg * wv
            for it in range(nitems):
                gi, rest = it % cg, it // cg
                xv, j = rest % wv, j0 + rest // wv
                hin = h0 - ph + j
                slot = j % NR
                cols = pw + 8 * xv + np.arange(8)
                assert cols[0] >= pw and cols[-1] < pw + W and cols[-1] < wb
                assert not padded[slot, cols].any()     # never overwrites a padding column
                chans = slice(8 * gi, 8 * gi + 8)
                if 0 <= hin < H:
                    assert 8 * gi + 7 < C and 8 * xv + 7 < W
                    ring[slot, cols, chans] = x[n, chans, hin, 8 * xv:8 * xv + 8].T
                else:
                    ring[slot, cols, chans] = 0.0
            for j in range(j0, j1):
                tag[j % NR] = j

        # prologue
        r0 = rb(0)
        zero_pads(0, r0)
        assert r0 * cg * wv <= THREADS            # one item per thread
        if nsteps > 1:
            assert (rb(1) - r0) * cg * wv <= THREADS
        transpose_rows(0, r0)
        # filter staging lies above the first step's slots
        assert pl["filt_off"] >= r0 * rb_bytes
        zero_pads(r0, NR)
        for t in range(nsteps):
            npx = (orow(t + 1) - orow(t)) * Q
            nblk = (npx + 31) // 32
            pix0 = orow(t) * Q
            assert orow(t + 1) - orow(t) <= SR
            need = set()
            for b in range(nblk):
                for kh in range(nkh):
                    pls = np.minimum(32 * b + np.arange(32), npx - 1)
                    pb = pix0 + pls
                    i, wc = pb // Q, pb % Q
                    valid = 32 * b + np.arange(32) < npx
                    # DV: filter column 1's fragment comes from lane m + 1's
                    # column-0 fragment, or lane m - 1's column-2 fragment
                    nxt = (np.arange(32) != 31) & (wc != Q - 1)
                    if dv_rule is not None:
                        nxt = dv_rule(np.arange(32), wc, Q)
                    src = np.where(nxt, np.arange(32) + 1, np.arange(32) - 1)
                    if pl["dv"]:
                        inb = (src >= 0) & (src < 32)
                        assert np.all(inb[valid]), "takes a fragment from the other half or outside the wave"
                        s = np.clip(src, 0, 31)
                        q_src = np.where(nxt, 0, 2)
                        # same output row, and the source's column equals the direct read's
                        assert np.all((i[s] == i)[valid])
                        assert np.all((wc[s] * sw + q_src * dw == wc * sw + dw)[valid])
                    acc = np.zeros((32, 32))
                    for r in range(3):
                        j = i + r * dh
                        slot = j % NR
                        assert np.all(j < rb(t)), "reads a row this step does not have"
                        assert np.all(tag[slot] == j), "slot holds another row"
                        need.update(int(v) for v in np.unique(slot))
                        for q in range(3):
                            col = wc * sw + q * dw
                            assert np.all(col < wb)
                            for cb in range(CB):
                                for g in range(2):
                                    c0 = 16 * cb + 8 * g
                                    # LDS byte offset of the lane's 16-byte read, inside its slot
                                    off = slot * rb_bytes + (col * CS + 2 * cb + g) * 16
                                    assert np.all(off + 16 <= (slot + 1) * rb_bytes)
                                    frag = ring[slot, col, c0:c0 + 8]        # [32 pixels][8]
                                    if pl["dv"] and q == 1:
                                        # the kernel never reads column 1; use what the
                                        # DPP shifts hand over (0 from outside the half)
                                        fa = ring[slot, wc * sw, c0:c0 + 8]
                                        fb = ring[slot, wc * sw + 2 * dw, c0:c0 + 8]
                                        z = np.zeros((1, 8))
                                        from_next = np.concatenate([fa[1:], z])
                                        from_prev = np.concatenate([z, fb[:-1]])
                                        frag = np.where(nxt[:, None], from_next, from_prev)
                                    assert not np.isnan(frag).any(), "reads an unwritten chunk"
                                    kk = np.arange(32 * kh, 32 * kh + 32)
                                    fk = np.zeros((32, 8))
                                    ok = kk < K
                                    fk[ok] = wf[kk[ok], c0:c0 + 8, r, q]
                                    acc += frag @ fk.T
                    if pl["staged"]:
                        eb = pl["out_bytes"]
                        rpr, ostr = 1024 // (32 * eb), 32 * eb + 16
                        lpr = 64 // rpr
                        tile0 = pl["ostage_off"]
                        for wave in range(8):   # every wave's tile lies inside LDS
                            assert tile0 + wave * rpr * ostr + rpr * ostr <= pl["lds"]
                        for lane in range(64):
                            rr, seg = lane // lpr, lane % lpr
                            assert rr * ostr + 16 * seg + 16 <= rpr * ostr
                            p = 32 * b + seg * (16 // eb)
                            if p < npx:   # a stored 16-byte run never crosses the step's end
                                assert p + 16 // eb <= npx
                    ks = np.arange(32 * kh, 32 * kh + 32)
                    ps = 32 * b + np.arange(32)
                    km, pm = ks < K, ps < npx
                    hh, ww = np.divmod(pix0 + ps[pm], Q)
                    kk = ks[km]
                    y[n, kk[:, None], h0 + hh[None, :], ww[None, :]] = acc[np.ix_(pm, km)].T
                    np.add.at(written, (n, kk[:, None], h0 + hh[None, :], ww[None, :]), 1)
            # the next step's rows go to slots this step does not read
            if t + 1 < nsteps:
                assert (rb(t + 1) - rb(t)) * cg * wv <= THREADS
                new = {j % NR for j in range(rb(t), rb(t + 1))}
                assert not (new & need), "transpose overwrites a slot the step reads"
                transpose_rows(rb(t), rb(t + 1))
    assert np.all(written == 1), "an output is stored twice or never"
    return y


SHAPES = [
    # (N, C, H, W, K, sw, pad, dil)
    (3, 64, 56, 56, 64, 1, 1, 1),      # the fp16 layer's geometry (two bands an image)
    (2, 32, 20, 24, 40, 1, 1, 1),      # K not a multiple of 32, Q = 24
    (1, 16, 9, 16, 8, 1, 0, 1),        # no padding, Q = 14 (scalar stores)
    (2, 48, 13, 16, 64, 2, 1, 1),      # stride_w 2
    (1, 64, 12, 8, 33, 1, 2, 2),       # dilation 2, padding 2
    (5, 16, 30, 40, 24, 1, 1, 1),      # several steps with a short last one
    (1, 64, 70, 64, 64, 1, 1, 1),      # one image: narrow bands
]


@pytest.mark.parametrize("shape", SHAPES)
def test_band_model_against_oracle(shape):
    N, C, H, W, K, sw, pad, dil = shape
    pl = band_plan(N, C, H, W, K, 3, 3, 1, sw, pad, pad, dil, dil)
    assert pl is not None
    rng = np.random.default_rng(sum(shape))
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((K, C, 3, 3))
    y = replay(pl, x, w)
    ref = oracle.conv2d(x, w, None, (1, sw), (pad, pad), (dil, dil), 1)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def filter_copy_check(C, K, piece_of=None):
    """Replay the prologue's coalesced filter copy for one layer (see
    test_band_filter_pieces); piece_of(ml, g, i) (tests only) replaces the
    kernel's read-back index ml PPR + RS g + i.  Raises AssertionError on
    any mismatch or out-of-range access."""
    pl = band_plan(2, C, 12, 16, K, 3, 3, 1, 1, 1, 1, 1, 1)
    assert pl is not None
    RS, PPR = 9, 18
    nkh, CB = pl["nkh"], pl["CB"]
    if piece_of is None:
        piece_of = lambda ml, g, i: ml * PPR + RS * g + i
    wflat = np.arange(K * C * RS, dtype=np.int64)     # halves of KCRS, each its own index
    area = 32 * PPR * 16
    assert nkh * CB * area == pl["raw_bytes"] <= pl["filt_off"]
    assert pl["filt_off"] + nkh * RS * CB * 1024 <= pl["lds"]
    for wave in range(nkh * CB):
        fkh, fcb = wave % nkh, wave // nkh
        lds = np.full(area // 2, -1, dtype=np.int64)   # the wave's area, in halves
        for i in range(RS):
            for lane in range(64):
                j = 64 * i + lane
                run = j // PPR
                k = min(32 * fkh + run, K - 1)
                h0 = (k * C + 16 * fcb) * RS + 8 * (j - run * PPR)   # first half of the load
                assert h0 % 8 == 0 and 0 <= h0 and h0 + 8 <= K * C * RS
                lds[(64 * i + lane) * 8:(64 * i + lane) * 8 + 8] = wflat[h0:h0 + 8]
        assert (lds >= 0).all()
        for lane in range(64):
            ml, g = lane % 32, lane // 32
            pieces = [piece_of(ml, g, i) for i in range(RS)]
            assert all(0 <= q < 32 * PPR for q in pieces), "reads outside the wave's area"
            got = np.concatenate([lds[q * 8:q * 8 + 8] for q in pieces])
            k = 32 * fkh + ml
            if k >= K:
                continue                                 # masked to zero by the perm
            c0 = 16 * fcb + 8 * g
            want = wflat.reshape(K, C, RS)[k, c0:c0 + 8, :].reshape(-1)
            assert np.array_equal(got, want), (wave, lane)


@pytest.mark.parametrize("C,K", [(16, 8), (32, 40), (48, 64), (64, 64), (64, 33), (16, 64)])
def test_band_filter_pieces(C, K):
    """The prologue's coalesced filter copy: load i of lane L of stager wave
    (fkh, fcb) takes 16-byte piece 64 i + L of the wave's slice, the pieces
    go to the wave's LDS area in that order, and lane (ml, g) reads back
    pieces ml PPR + RS g + i.  Replayed on a KCRS filter of distinct values:
    every load lies inside the filter, every raw area lies below the
    fragment staging, and each lane's read-back is F[k][c0 .. c0 + 7][taps]
    (k = 32 fkh + ml, c0 = 16 fcb + 8 g), the lanes past K dropped."""
    filter_copy_check(C, K)


@pytest.mark.parametrize("name,piece_of", [
    ("channel halves swapped", lambda ml, g, i: ml * 18 + 9 * (1 - g) + i),
    ("run stride of a half", lambda ml, g, i: ml * 9 + 9 * g + i),
    ("pieces reversed", lambda ml, g, i: ml * 18 + 9 * g + (8 - i)),
])
def test_band_filter_copy_mutants_caught(name, piece_of):
    with pytest.raises(AssertionError):
        filter_copy_check(64, 64, piece_of)


# Plausible mistakes in the neighbour-lane rule; each must be caught (by the
# source-column check or by the comparison with the oracle) on some layer.
DV_MUTANTS = {
    "ignores row ends": lambda ml, wc, Q: ml != 31,
    "ignores the half's last lane": lambda ml, wc, Q: wc != Q - 1,
    "always the previous lane": lambda ml, wc, Q: np.zeros(32, dtype=bool),
    "off by one at the row end": lambda ml, wc, Q: (ml != 31) & (wc != Q - 2),
}


@pytest.mark.parametrize("name", sorted(DV_MUTANTS))
def test_band_model_catches_wrong_neighbour_rule(name):
    caught = False
    for shape in SHAPES:
        N, C, H, W, K, sw, pad, dil = shape
        pl = band_plan(N, C, H, W, K, 3, 3, 1, sw, pad, pad, dil, dil)
        if not pl["dv"]:
            continue
        rng = np.random.default_rng(sum(shape))
        x = rng.standard_normal((N, C, H, W))
        w = rng.standard_normal((K, C, 3, 3))
        try:
            y = replay(pl, x, w, dv_rule=DV_MUTANTS[name])
        except AssertionError:
            caught = True
            break
        ref = oracle.conv2d(x, w, None, (1, sw), (pad, pad), (dil, dil), 1)
        if not np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max()):
            caught = True
            break
    assert caught, f"the model accepts the mutant rule: {name}"


def test_band_plan_of_the_fp16_layer():
    L = workloads.LAYERS["resnet_3x3_fp16"]
    pl = band_plan(L.N, L.C, L.H, L.W, L.K, 3, 3, 1, 1, 1, 1, 1, 1)
    # one band of 28 rows per CU, steps of 4, 8, 8 and 8 rows, 18 ring slots of 58 x 9 chunks,
    # then eight 16-channel x 32-pixel output tiles (rows padded to 80 bytes)
    assert (pl["band"], pl["nbands"], pl["ntask"], pl["SR0"], pl["SR"], pl["NR"]) == \
        (28, 2, 256, 4, 8, 18)
    assert pl["row_bytes"] == 58 * 9 * 16 and pl["staged"]
    assert pl["lds"] == 18 * 58 * 9 * 16 + 8 * 16 * 80 <= 160 * 1024


m = pytest.importorskip("cnn_convolution_im2win_amd")

from tests.test_narrow_model import narrow_plan  # noqa: E402


def test_band_eligibility_matches_library():
    """The layers the model's plan accepts are exactly those for which the
    library reports 0 bytes of in-LDS workspace (the band kernel's)."""
    rng = np.random.default_rng(7)
    cases = [(2, 64, 56, 56, 64, 3, 1, 1, 1), (1, 64, 56, 56, 64, 3, 1, 1, 2)]
    for _ in range(60):
        C = int(rng.choice([8, 16, 32, 48, 64, 80]))
        cases.append((int(rng.integers(1, 5)), C, int(rng.integers(3, 40)),
                      int(rng.choice([8, 16, 24, 12, 56, 112])), int(rng.integers(1, 80)),
                      int(rng.choice([1, 3])), int(rng.integers(1, 3)), int(rng.integers(0, 3)),
                      int(rng.integers(1, 3))))
    for N, C, H, W, K, R, sw, pad, dil in cases:
        for pool in (False, True):
            d = m.make_desc((N, C, H, W), (K, C, R, R), (1, sw), pad, dil, 1)
            try:
                P, Q = m.conv_im2win_output_dims(d)
            except m.Im2winError:
                continue
            if pool and (P < 2 or Q < 2):
                continue
            flags = m.CIW_FLAG_IMPLICIT | (m.CIW_FLAG_MAXPOOL2 if pool else 0)
            try:
                nbytes = m.conv2d_implicit_workspace_bytes(d, m.CIW_F16, m.CIW_F16, flags)
            except m.Im2winError:
                nbytes = None
            pl = band_plan(N, C, H, W, K, R, R, 1, sw, pad, pad, dil, dil, pool=pool)
            # the few-channel kernel (no workspace either) takes some layers
            # with C not a multiple of 16, which the band kernel never runs
            few = C % 16 != 0 and narrow_plan(N, C, H, W, K, R, R, 1, sw, pad, pad, dil, dil,
                                             pool=pool) is not None
            assert (pl is not None or few) == (nbytes == 0), (N, C, H, W, K, R, sw, pad, dil, pool)
