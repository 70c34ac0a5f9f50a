"""CPU model of the matrix-core row kernel's plan and indexing (host logic).

The row kernel (`conv_mfma_rows_kernel`) reads and writes LDS and global
memory through indices that depend on its plan: the pad period of the LDS
row layout, pixel phases, ring depth, copy instructions per row, the output
tile and the hand-placed `s_waitcnt` counts that keep row copies in flight.
This model restates that plan and walks every access the kernel makes for a
layer, checking that

- every row-copy lane writes inside its ring buffer and reads inside the row;
- every LDS position of the row is filled, and window chunk c sits at its
  padded position;
- every fragment read stays in the buffer, and every unmasked fragment entry
  is the pixel's own window element (so masks cover exactly the rest);
- every tile column stays inside the tile row; the incremental store indices
  equal the divided ones;
- each wait count equals the number of the wave's vector-memory operations
  issued after the row's copy (so it waits for exactly that copy), and fits
  the 6-bit counter;
- with the fused 2x2 max-pool: runs are whole row pairs inside one image,
  every window row read exists, the pooled stores read tile columns inside
  the tile row, and the wait counts hold for stores after every second row.

The plan is restated from conv_mfma_impl.hpp and must change with it; the
first test ties it to the library: for half-precision layers the workspace
the library asks for includes the re-laid-out filter, nph * steps * 2 KB,
which only exists when the library's plan accepts the layer.
"""
import math

import numpy as np
import pytest

import workloads
from tests import row_kernel_cases

TH = 256            # threads per workgroup
MAX_CHUNKS = 8      # copy instructions per thread per row


def out_dims(L):
    P = (L.H + 2 * L.pad[0] - L.dil[0] * (L.R - 1) - 1) // L.stride[0] + 1
    Q = (L.W + 2 * L.pad[1] - L.dil[1] * (L.S - 1) - 1) // L.stride[1] + 1
    return P, Q


def pitch_b(L, Q):
    wwin = (Q - 1) * L.stride[1] + L.dil[1] * (L.S - 1) + 1
    return (wwin * L.R * L.C + 7) // 8 * 8


def plan(L, out_bytes, pool=False):
    """The row-kernel plan, or None when the layer goes to the generic kernel."""
    P, Q = out_dims(L)
    C, K, R, S, sw = L.C, L.K, L.R, L.S, L.stride[1]
    if K > 64 or L.dil[1] != 1:
        return None
    D, T = sw * R * C, S * R * C
    nph = 8 // math.gcd(D, 8)
    maxdelta = max((ph * D) & 7 for ph in range(nph))
    need = (T + maxdelta + 15) // 16
    nset = 1 if nph == 1 else nph // 2
    steps = next((c for c in (10, 16, 24, 36, 40) if c >= need), 0)
    if steps == 0 or nset * steps > 40:
        return None
    mask = maxdelta > 0 or T != 16 * steps
    mblocks = ((Q + nph - 1) // nph + 31) // 32
    nchunks = pitch_b(L, Q) // 8
    G = D // 8 if nph == 1 else 0
    pad = 1
    if nph == 1:
        while pad < 8 and G % (2 * pad) == 0:
            pad *= 2
    stride = D * nph // 8 if pad == 1 else G + G // pad
    copy = nchunks if pad == 1 else (nchunks + pad - 1) // pad * (pad + 1)
    if copy > MAX_CHUNKS * TH:
        return None
    nd = (copy + TH - 1) // TH
    wmax = max(Q - 1, nph - 1)
    run_end = 1 + 2 * (steps - 1) + (0 if pad == 1 else (2 * (steps - 1)) // pad)
    last = ((wmax * D) // 8 if pad == 1 else wmax * stride) + run_end
    bufc = max(copy, last + 1, TH if nd == 1 else 0)
    bufc = (bufc + 15) // 16 * 16
    V = 16 // out_bytes
    ostride = (nph * 32 * mblocks + V - 1) // V * V
    if ((ostride * out_bytes) // 16) % 2 == 0:
        ostride += V
    tile = 2 * K * ostride * out_bytes + 256
    nbuf = wgs = 0
    for w in (2, 1):
        if nbuf:
            break
        for nb in (6, 5, 4, 3, 2):
            if (nb * bufc * 8 * 2 + tile) * w <= 160 * 1024:
                nbuf, wgs = nb, w
                break
    if nbuf == 0:
        return None

    def stores(Po, Qo):
        vec = 1 if (Qo % V == 0 and (Po * Qo) % V == 0) else 0
        total = K * (Qo // V) if vec else K * Qo
        return vec, (total + TH - 1) // TH

    nbuf_lds = nbuf
    vec, ns = stores(P, Q)
    while nbuf > 2 and (nd + ns) * (nbuf - 1) > 63:
        nbuf -= 1
    if (nd + ns) * (nbuf - 1) > 63:
        return None
    Po, Qo = P, Q
    if pool:
        Po, Qo = P // 2, Q // 2
        vec, ns = stores(Po, Qo)
        nbuf = nbuf_lds
        while nbuf > 2 and (nd + ns) * (nbuf - 1) > 63:
            nbuf -= 1
        if (nd + ns) * (nbuf - 1) > 63:
            return None
    return dict(P=P, Q=Q, K=K, D=D, T=T, nph=nph, nset=nset, steps=steps, mask=mask,
                mblocks=mblocks, nchunks=nchunks, G=G, pad=pad, copy=copy, nd=nd, bufc=bufc,
                V=V, ostride=ostride, nbuf=nbuf, wgs=wgs, lds=nbuf * bufc * 16 + tile, vec=vec,
                ns=ns, pool=pool, Po=Po, Qo=Qo)


def pad_src(q, pad):
    if pad == 1:
        return q
    grp = q // (pad + 1)
    return grp * pad + min(q - grp * (pad + 1), pad - 1)


def pad_pos(ch, pad):
    return ch if pad == 1 else ch + ch // pad


def step_off(s, pad):
    return 32 * s if pad == 1 else 32 * s + 16 * ((2 * s) // pad)


def has_store(it, pool):
    """A store follows every row (of row it - 1), or with the pool every
    second row (of pair it / 2 - 1, at even it)."""
    return it >= 2 and it % 2 == 0 if pool else it >= 1


def check_waits(nbuf, nd, ns, my_rows, pool=False):
    """Iteration it: wait, barrier, copy row it + nbuf - 1, the stores due,
    multiplies; the prologue copies rows 0 .. nbuf - 2."""
    ops = []
    for i in range(min(nbuf - 1, my_rows)):
        ops += [("c", i)] * nd
    for it in range(my_rows):
        later_rows = min(nbuf - 2, my_rows - 1 - it)
        lo = max(it - nbuf + 1, 1)
        later_stores = max(0, it - lo)
        if pool:
            lo2 = max(lo, 2)
            later_stores = (it - 1) // 2 - (lo2 - 1) // 2 if it - 1 >= lo2 else 0
        w = nd * later_rows + ns * later_stores
        assert 0 <= w <= 63
        last_copy = max(i for i, o in enumerate(ops) if o == ("c", it))
        assert w == len(ops) - 1 - last_copy, (nbuf, nd, ns, my_rows, pool, it)
        if it + nbuf - 1 < my_rows:
            ops += [("c", it + nbuf - 1)] * nd
        if has_store(it, pool):
            ops += [("s", it - 1)] * ns


def check_pool_schedule(p, N, grid):
    """Row units of every workgroup: whole pairs of one image, window rows in
    range; tiles alternate per pair and a stored tile is never the one the
    same iteration multiplies into or merges."""
    P, Po = p["P"], p["Po"]
    rows = N * 2 * Po
    groups = rows // 2
    per = (groups + grid - 1) // grid
    seen = []
    for b in range(grid):
        first = b * per * 2
        if first >= rows:
            continue
        my_rows = min(per * 2, rows - first)
        assert first % 2 == 0 and my_rows % 2 == 0
        for it in range(my_rows):
            u = first + it
            pr = u >> 1
            n, j = divmod(pr, Po)
            wrow = n * P + 2 * j + (u & 1)
            assert n < N and 2 * j + 1 < P and 0 <= wrow < N * P
            seen.append(u)
            tile = (it >> 1) & 1
            if has_store(it, True):
                stored_pair = (first + it) // 2 - 1
                assert stored_pair == pr - 1
                assert ((it >> 1) - 1) & 1 != tile
        # the epilogue stores the last pair
        assert (first + my_rows) // 2 - 1 == (first + my_rows - 1) >> 1
    assert sorted(seen) == list(range(rows))


def check_layer(L, out_bytes, pool=False):
    p = plan(L, out_bytes, pool)
    if p is None:
        return None
    bufc, pad, Q = p["bufc"], p["pad"], p["Q"]
    assert p["lds"] * p["wgs"] <= 160 * 1024
    assert (L.K * p["ostride"] * out_bytes) % 16 == 0
    # row copy: position -> chunk it holds
    held = {}
    for j in range(p["nd"]):
        base = p["copy"] - TH if (j == p["nd"] - 1 and p["nd"] > 1) else j * TH
        assert base >= 0
        for tid in range(TH):
            pos = base + tid
            assert 0 <= pos < bufc
            ch = min(pad_src(min(pos, p["copy"] - 1), pad), p["nchunks"] - 1)
            assert 0 <= ch < p["nchunks"]
            assert held.setdefault(pos, ch) == ch
    assert all(q in held for q in range(p["copy"]))
    assert all(held[pad_pos(ch, pad)] == ch for ch in range(p["nchunks"]))
    # fragment reads of every block, lane and step
    for pb in range(p["nph"] * p["mblocks"]):
        ph, mb = pb % p["nph"], pb // p["nph"]
        delta = (ph * p["D"]) & 7
        s_full = (delta + p["T"]) // 16
        for ml in range(32):
            w = p["nph"] * (32 * mb + ml) + ph
            wl = Q - 1 - ((Q - 1 - ph) % p["nph"]) if Q - 1 >= ph else ph
            wr = min(w, wl)
            assert p["nph"] * (32 * mb + ml) + ph < p["ostride"]      # tile column
            for g in (0, 1):
                if pad == 1:
                    assert (wr * p["D"] - delta) % 8 == 0 and wr * p["D"] >= delta
                    run = (wr * p["D"] - delta) // 8 + g
                else:
                    run = wr * (p["G"] + p["G"] // pad) + g
                for s in range(p["steps"]):
                    pos = (run * 16 + step_off(s, pad)) // 16
                    assert 0 <= pos < bufc
                    t0 = 16 * s + 8 * g
                    masked = p["mask"] and (s == 0 and delta > 0 or s >= s_full)
                    if not masked and w < Q:
                        assert delta <= t0 and t0 + 8 <= delta + p["T"]
                        assert held.get(pos) == (wr * p["D"] + t0 - delta) // 8
    # stores: incremental (k, v) equal the divided ones; the tile columns a
    # store reads (two per output with the pool) lie inside the tile row
    E = p["V"] if p["vec"] else 1
    Qo = p["Qo"]
    sc = 2 if pool else 1
    nq = Qo // E
    total = L.K * nq
    dk, dv = TH // nq, TH % nq
    for tid in range(TH):
        k, v = tid // nq, tid % nq
        for j in range(p["ns"]):
            i = min(tid + j * TH, total - 1)
            kk = min(k, L.K - 1)
            off = Qo - E if kk < k else v * E
            assert (kk, off) == (i // nq, (i % nq) * E)
            src = sc * off
            assert src % E == 0 and src + sc * E <= min(Q, p["ostride"])
            k, v = k + dk, v + dv
            if v >= nq:
                v, k = v - nq, k + 1
    for my_rows in range(1, 9):
        if not pool or my_rows % 2 == 0:
            check_waits(p["nbuf"], p["nd"], p["ns"], my_rows, pool)
    if pool:
        for N in (1, 2, 3):
            for grid in (1, 2, 3, 7, 512):
                check_pool_schedule(p, N, grid)
    return p


def test_plan_matches_library_filter_size():
    m = pytest.importorskip("cnn_convolution_im2win_amd")
    layers = [workloads.LAYERS["resnet_3x3_fp16"], workloads.LAYERS["stem_7x7_s2_bf16"]]
    layers += list(row_kernel_cases.CASES.values())
    rng = np.random.default_rng(5)
    layers += [workloads.random_layer(rng, dtype="f16", max_hw=40, max_c=70, max_k=80)
               for _ in range(200)]
    for L in layers:
        code = m.CIW_F16 if L.dtype == "f16" else m.CIW_BF16
        d = m.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, L.groups)
        win = m.conv_im2win_window_bytes(d, code, m.CIW_WIN_HWC, L.N)
        extra = m.conv2d_workspace_bytes(d, code, L.N) - (win + 255) // 256 * 256
        p2, p4 = plan(L, 2), plan(L, 4)
        p = p2 or p4
        want = 0 if p is None else (p["nph"] * p["steps"] * 2048 + 255) // 256 * 256
        assert extra == want, (L, extra, want)


@pytest.mark.parametrize("name", ["resnet_3x3_fp16", "stem_7x7_s2_bf16"])
def test_model_full_layers(name):
    L = workloads.LAYERS[name]
    assert check_layer(L, 2) is not None and check_layer(L, 4) is not None
    assert check_layer(L, 2, pool=True) is not None and check_layer(L, 4, pool=True) is not None


def test_model_coverage_layers_reach_every_specialisation():
    seen = set()
    for L in row_kernel_cases.CASES.values():
        ob = 4 if L.out_dtype == "f32" else 2
        p = check_layer(L, ob)
        assert p is not None, L
        if p["P"] >= 2 and p["Q"] >= 2:
            pp = check_layer(L, ob, pool=True)
            assert pp is not None, L
            seen.add(("pool_vec", pp["vec"]))
        seen.add(("pad", p["pad"]))
        seen.add(("nset", p["nset"]))
        seen.add(("mask", p["mask"]))
        seen.add(("vec", p["vec"]))
    want = {("pad", 1), ("pad", 2), ("pad", 4), ("pad", 8), ("nset", 1), ("nset", 2),
            ("nset", 4), ("mask", True), ("mask", False), ("vec", 0), ("vec", 1),
            ("pool_vec", 0), ("pool_vec", 1)}
    assert want <= seen, want - seen


def test_model_random_layers():
    rng = np.random.default_rng(0)
    rows = 0
    for i in range(1200):
        L = workloads.random_layer(rng, dtype="f16", max_hw=40, max_c=70, max_k=80)
        p = check_layer(L, 2 if i % 2 else 4)
        rows += p is not None
        if p is not None and p["P"] >= 2 and p["Q"] >= 2 and i % 3 == 0:
            check_layer(L, 2 if i % 2 else 4, pool=True)
    for i in range(300):
        L = workloads.random_layer(rng, dtype="f16", max_hw=300, max_c=8, max_k=64)
        rows += check_layer(L, 2 if i % 2 else 4) is not None
    assert rows > 300


def test_wait_counts_every_ring_depth():
    for nbuf in range(2, 7):
        for nd in range(1, MAX_CHUNKS + 1):
            for ns in range(1, 40):
                if (nd + ns) * (nbuf - 1) > 63:
                    continue
                for my_rows in range(1, 12):
                    check_waits(nbuf, nd, ns, my_rows)
                    if my_rows % 2 == 0:
                        check_waits(nbuf, nd, ns, my_rows, pool=True)
