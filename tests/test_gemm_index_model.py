"""CPU model of the GEMM engine's operand staging (csrc/muon_gemm.h): the
direct global -> LDS loads of DmaFeed, the fragment reads of frag(), and the
tile walks decode_sym / decode_full, restated here from the kernel source.

For both tile sizes and both operand layouts it checks that
  * every load stays inside the operand buffer and inside its LDS stage,
  * the loads of one K step place each element of the TILE x 32 operand
    slice exactly once, and every fragment read finds the element the MFMA
    expects (row / column mn, depth k) under the stored swizzle,
  * the tile walks visit every tile of a matrix exactly once, in range.
A change to the engine's indexing that breaks one of these fails here, on the
CPU, before any GPU run.  (Index arithmetic only: no kernel runs.)"""
import numpy as np
import pytest

BK = 32


def lanes():
    return np.arange(64)


# ---------------------------------------------------------------- loads ----
def dma_elements(tile, mn_layout, ld, mn0, kt, waves=4):
    """(mn, k) element and LDS element offset of every 16-byte piece one K
    step loads, for an operand with leading dimension `ld` (elements)."""
    lpw = tile // 64
    l = lanes()
    out_mn, out_k, out_lds = [], [], []
    for w in range(waves):
        for q in range(lpw):
            lds0 = (w * lpw + q) * 512 + 8 * l          # element offset in the stage
            if not mn_layout:
                row = l >> 2
                c = (l & 3) ^ (2 * ((row >> 3) & 1))
                # byte offset: (mn0 + 16 lpw w + 16 q + row) * 2 ld + 2 BK kt + 16 c
                mn = mn0 + 16 * lpw * w + 16 * q + row
                k = BK * kt + 8 * c
            else:
                cpr, r_ = tile // 8, 512 // tile
                row = l // cpr
                c = (l % cpr) ^ (2 * ((r_ * (q & 1) + row) & 3) + 8 * (w & 1))
                k = BK * kt + r_ * lpw * w + r_ * q + row
                mn = mn0 + 8 * c
            out_mn.append(mn)
            out_k.append(k)
            out_lds.append(lds0)
    return np.concatenate(out_mn), np.concatenate(out_k), np.concatenate(out_lds)


def stored_position(tile, mn_layout, mn_rel, k_rel):
    """Element offset in the stage where the reader expects (mn_rel, k_rel)."""
    if not mn_layout:
        c = k_rel // 8
        return mn_rel * BK + ((c ^ (2 * ((mn_rel >> 3) & 1))) * 8) + k_rel % 8
    c = mn_rel // 8
    return k_rel * tile + ((c ^ (2 * (k_rel & 3) + 8 * ((k_rel >> 3) & 1))) * 8) + mn_rel % 8


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("mn_layout", [False, True])
def test_one_step_of_loads_fills_the_stage_exactly(tile, mn_layout):
    ld = 4 * tile + 64 if not mn_layout else 3 * tile
    mn0 = tile                                     # second tile row
    kt = 5
    mn, k, lds = dma_elements(tile, mn_layout, ld, mn0, kt)
    # 8 elements per 16-byte piece
    step = np.arange(8)
    zero = np.zeros(8, dtype=np.int64)
    mn_all = (mn[:, None] + (step if mn_layout else zero)).ravel()
    k_all = (k[:, None] + (zero if mn_layout else step)).ravel()
    lds_all = (lds[:, None] + np.arange(8)).ravel()
    te = tile * BK
    assert lds_all.min() >= 0 and lds_all.max() < te
    assert len(np.unique(lds_all)) == te             # every stage element written once
    # each LDS element receives the element the readers expect there
    want = stored_position(tile, mn_layout, mn_all - mn0, k_all - BK * kt)
    assert np.array_equal(want, lds_all)
    assert mn_all.min() == mn0 and mn_all.max() == mn0 + tile - 1
    assert k_all.min() == BK * kt and k_all.max() == BK * kt + BK - 1


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("mn_layout", [False, True])
@pytest.mark.parametrize("extent", [(1, 1), (3, 2), (16, 9)])
def test_loads_stay_inside_the_operand(tile, mn_layout, extent):
    """The last tile of a matrix, every K step including the three clamped
    steps past the end (which re-read the last step)."""
    tiles_mn, k_steps4 = extent
    K = 4 * BK * k_steps4                          # K is a multiple of 128
    n_mn = tiles_mn * tile
    ld = K if not mn_layout else n_mn
    rows = n_mn if not mn_layout else K
    kt_n = K // BK
    for kt in range(kt_n + 3):
        kc = min(kt, kt_n - 1)
        mn, k, _ = dma_elements(tile, mn_layout, ld, n_mn - tile, kc)
        if not mn_layout:
            first = mn * ld + k
            last = first + 7
        else:
            first = k * ld + mn
            last = first + 7
        assert first.min() >= 0 and last.max() < rows * ld


# ------------------------------------------------------------ fragments ----
@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("mn_layout", [False, True])
def test_fragment_reads_find_their_elements(tile, mn_layout):
    """frag(): lane l holds row (or column) rowbase + (l & 15), depth
    8 (l >> 4) .. +7; K-contiguous stages are read with one 16-byte read,
    MN-contiguous ones with two transposing 8-byte reads."""
    l = lanes()
    te = tile * BK
    for rowbase in range(0, tile, 16):
        mn_rel = rowbase + (l & 15)
        if not mn_layout:
            row = mn_rel
            c = (l >> 4) ^ (2 * ((row >> 3) & 1))
            addr = row * BK + c * 8                      # 8 elements from here
            for j in range(8):
                assert np.array_equal(addr + j, stored_position(tile, False, mn_rel, 8 * (l >> 4) + j))
        else:
            g, i = l >> 4, l & 15
            m = rowbase + 4 * (i & 3)
            k = 8 * g + (i >> 2)
            off = (((m >> 3) ^ (2 * (i >> 2) + 8 * (g & 1))) << 3) + (m & 4)
            for half, kk in enumerate((k, k + 4)):
                base = kk * tile + off                   # 4 elements (8 bytes) per lane
                assert base.min() >= 0 and base.max() + 3 < te
                # the transposing read: in each 16-lane group, lane 4a + b gets
                # element b of the pieces addressed by lanes a, a + 4, a + 8, a + 12
                for grp in range(4):
                    lg = np.arange(16) + 16 * grp
                    for a in range(4):
                        for b in range(4):
                            dst = 16 * grp + 4 * a + b
                            src_lanes = lg[[a, a + 4, a + 8, a + 12]]
                            got = base[src_lanes] + b            # elements lane dst receives
                            want = stored_position(tile, True, np.full(4, rowbase + dst % 16),
                                                   8 * grp + 4 * half + np.arange(4))
                            assert np.array_equal(got, want), (tile, rowbase, dst)


# ----------------------------------------------------------- tile walks ----
def decode_sym(u, t, gm=8):
    lo = 0
    while True:
        hi = min(lo + gm, t)
        band = (hi - lo) * t - (lo + hi - 1) * (hi - lo) // 2
        if u < band or hi == t:
            break
        u -= band
        lo = hi
    hi = min(lo + gm, t)
    tj = lo
    while True:
        rows = min(tj, hi - 1) - lo + 1
        if u < rows or tj == t - 1:
            break
        u -= rows
        tj += 1
    return lo + u, tj


def decode_full(u, tm, tn, gm=8):
    group = u // (gm * tn)
    first = group * gm
    g = min(tm - first, gm)
    local = u - group * gm * tn
    return first + local % g, local // g


@pytest.mark.parametrize("t", [1, 2, 7, 8, 9, 16, 17, 33])
def test_symmetric_walk_covers_the_upper_triangle(t):
    n = t * (t + 1) // 2
    got = [decode_sym(u, t) for u in range(n)]
    assert sorted(got) == sorted((i, j) for i in range(t) for j in range(i, t))


@pytest.mark.parametrize("tm,tn", [(1, 1), (1, 5), (5, 1), (8, 16), (9, 3), (56, 16), (16, 56), (17, 17)])
def test_full_walk_covers_the_grid(tm, tn):
    got = [decode_full(u, tm, tn) for u in range(tm * tn)]
    assert sorted(got) == [(i, j) for i in range(tm) for j in range(tn)]


def xcd_remap(b, nb):
    per, rem = nb >> 3, nb & 7
    x, i = b & 7, b >> 3
    return x * per + min(x, rem) + i


@pytest.mark.parametrize("nb", [1, 7, 8, 9, 255, 256, 1000, 30464])
def test_xcd_remap_is_a_permutation(nb):
    assert sorted(xcd_remap(b, nb) for b in range(nb)) == list(range(nb))


# ------------------------------------------------------------ epilogues ----
def tswz(col):
    return ((col & 3) << 2) | ((col >> 2) & 3)


def tpos(tile, row, col):
    return col * tile + ((((row >> 2) ^ tswz(col)) << 2) | (row & 3))


def acc_layout(tile):
    """(row, col) of accumulator element e of block (bi, bj) for every lane of
    every wave, as the symmetric epilogue sees them: 4 consecutive rows of
    one column per lane and block."""
    wt, nb = tile // 2, tile // 32
    rows, cols = [], []
    for w in range(4):
        row_a, row_b = wt * (w >> 1), wt * (w & 1)
        l = lanes()
        for bi in range(nb):
            for bj in range(nb):
                rr = row_a + 16 * bi + 4 * (l >> 4)
                cc = row_b + 16 * bj + (l & 15)
                for e in range(4):
                    rows.append(rr + e)
                    cols.append(cc)
    return np.concatenate(rows), np.concatenate(cols)


@pytest.mark.parametrize("tile", [128, 256])
def test_symmetric_epilogue_staging_and_both_stores(tile):
    """store_sym stages each accumulator at tpos(row, col); store_staged then
    writes the mirror (column col of the tile as a row) with 16-byte reads and
    the tile itself (rows) with transposing reads.  Every element lands at the
    right place of the output, and every read stays inside the staging tile."""
    rows, cols = acc_layout(tile)
    pos = tpos(tile, rows, cols)
    assert len(np.unique(pos)) == tile * tile and pos.min() >= 0 and pos.max() < tile * tile
    where = np.empty(tile * tile, dtype=np.int64)        # staging position -> row * tile + col
    where[pos] = rows * tile + cols
    # mirror: item (col, k) reads the 16 bytes at unit pair (2k) ^ (f & 14), then
    # swaps the halves when f is odd; element j must be (row 8k + j, col)
    cpl = tile // 8
    for col in range(tile):
        f = tswz(col)
        for k in range(cpl):
            base = col * tile + ((2 * k) ^ (f & 14)) * 4
            got = where[base:base + 8]
            if f & 1:
                got = np.concatenate([got[4:], got[:4]])
            assert np.array_equal(got, (8 * k + np.arange(8)) * tile + col), (col, k)
    # tile rows: block (rb, cb), lane (g, i) addresses column cb + 8 g + (i >> 2)
    # (and + 4), rows rb + 4 (i & 3) .. + 3; through the transposing read lane
    # i of group g must receive row rb + i, columns cb + 8 g .. + 7
    l = lanes()
    g, i = l >> 4, l & 15
    for rb in range(0, tile, 16):
        for cb in range(0, tile, 32):
            col = cb + 8 * g + (i >> 2)
            for half, cc in enumerate((col, col + 4)):
                base = tpos(tile, rb + 4 * (i & 3), cc)
                assert base.min() >= 0 and base.max() + 3 < tile * tile
                for grp in range(4):
                    lg = np.arange(16) + 16 * grp
                    for a in range(4):
                        for b in range(4):
                            dst = 4 * a + b
                            got = where[base[lg[[a, a + 4, a + 8, a + 12]]] + b]
                            want = (rb + dst) * tile + cb + 8 * grp + 4 * half + np.arange(4)
                            assert np.array_equal(got, want), (rb, cb, grp, dst)


@pytest.mark.parametrize("tile", [128, 256])
def test_x_update_epilogue_staging(tile):
    """k_xupdate stages lane (row rl + 16 bi, columns cl + 16 bj .. + 3) as one
    8-byte unit u = col / 4 at unit u ^ (row & 31) of its row, then writes
    16-byte row chunks; each chunk must hold columns 8 ch .. 8 ch + 7."""
    wt, nb = tile // 2, tile // 32
    units = tile // 4
    where = -np.ones((tile, units), dtype=np.int64)
    for w in range(4):
        l = lanes()
        rl = wt * (w >> 1) + (l & 15)
        cl = wt * (w & 1) + 4 * (l >> 4)
        for bi in range(nb):
            for bj in range(nb):
                r = rl + 16 * bi
                u = (cl + 16 * bj) >> 2
                phys = u ^ (r & 31)
                assert phys.max() < units
                assert (where[r, phys] == -1).all()
                where[r, phys] = u
    assert (where >= 0).all()
    for r in range(tile):
        for ch in range(tile // 8):
            assert where[r, (2 * ch) ^ (r & 31)] == 2 * ch
            assert where[r, (2 * ch + 1) ^ (r & 31)] == 2 * ch + 1


@pytest.mark.parametrize("tile", [128, 256])
def test_c_epilogue_reads_its_tile_of_a(tile):
    """k_gram2 reads A[c0 + cc][r0 + rr .. + 3] (the tile's own A values, by
    symmetry) for every accumulator: inside A for the last tile pair."""
    rows, cols = acc_layout(tile)
    m_pad = 3 * tile
    r0 = c0 = m_pad - tile
    first = (c0 + cols) * m_pad + r0 + (rows & ~3)
    assert first.min() >= 0 and (first + 3).max() < m_pad * m_pad


def c_epilogue_a_staging(tile, ld, r0, c0):
    """At TILE 256, store_sym<GRAM2> brings the mirrored A tile into LDS with
    direct loads: wave w, load q covers 1 KB block blk = w BPW + q (columns
    blk CPB .. + CPB - 1, CPB = 64 / (tile / 8)); lane l reads 16 bytes of A
    row c0 + col at column r0 + 8 (u ^ (col & 15)), u = l % (tile / 8), and
    they land at LDS element 512 blk + 8 l.  Returns, per 16-byte piece, the
    A element offset of its first element and its LDS element offset."""
    upc = tile // 8
    cpb = 64 // upc
    bpw = tile // cpb // 4
    l = lanes()
    src, dst = [], []
    for w in range(4):
        for q in range(bpw):
            blk = w * bpw + q
            col = blk * cpb + l // upc
            u = l % upc
            base = (c0 + blk * cpb) * ld + r0                  # wave-uniform, elements
            voff_bytes = (l // upc) * 2 * ld + 16 * (u ^ (col & 15))
            assert (voff_bytes < 2**32).all()
            src.append(base + voff_bytes // 2)
            dst.append(512 * blk + 8 * l)
    return np.concatenate(src), np.concatenate(dst)


def test_c_epilogue_a_tile_staging():
    """The staged copy holds every element of the mirrored tile exactly once,
    inside A and inside the 128 KB of LDS, and the 8-byte read of each
    accumulator's A values (rows rr .. rr + 3 of column cc at unit
    (rr >> 3) ^ (cc & 15)) finds A[c0 + cc][r0 + rr .. rr + 3]."""
    tile = 256
    m_pad = 3 * tile
    for r0, c0 in ((0, 0), (m_pad - tile, 0), (0, m_pad - tile), (m_pad - tile, m_pad - tile)):
        src, dst = c_epilogue_a_staging(tile, m_pad, r0, c0)
        assert src.min() >= 0 and (src + 7).max() < m_pad * m_pad
        assert dst.min() >= 0 and (dst + 7).max() < tile * tile
        assert len(np.unique(dst)) == len(dst) == tile * tile // 8
        lds = np.full(tile * tile, -1, dtype=np.int64)       # LDS element -> A offset
        for j in range(8):
            lds[dst + j] = src + j
        assert (lds >= 0).all()
        want = ((c0 + np.arange(tile))[:, None] * m_pad + r0 + np.arange(tile)[None, :]).ravel()
        assert np.array_equal(np.sort(lds), np.sort(want))
        rows, cols = acc_layout(tile)                          # per block: e = 0 .. 3, 64 lanes each
        first = (np.arange(len(rows)) // 64) % 4 == 0
        rr, cc = rows[first], cols[first]                      # first row of each piece
        assert (rr % 4 == 0).all()
        pos = cc * tile + ((((rr >> 3) ^ (cc & 15)) << 3) | (rr & 7))
        for e in range(4):
            assert np.array_equal(lds[pos + e], (c0 + cc) * m_pad + r0 + rr + e)


def test_c_epilogue_a_reads_are_bank_conflict_free():
    """Each 32-lane half of a wave's 8-byte read of the staged A tile touches
    each of the 64 four-byte banks exactly once."""
    tile, wt, nb = 256, 128, 8
    l = lanes()
    for w in range(4):
        row_a, row_b = wt * (w >> 1), wt * (w & 1)
        for bi in range(nb):
            for bj in range(nb):
                rr = row_a + 16 * bi + 4 * (l >> 4)
                cc = row_b + 16 * bj + (l & 15)
                byte = 2 * (cc * tile + ((((rr >> 3) ^ (cc & 15)) << 3) | (rr & 7)))
                banks = np.stack([(byte // 4) % 64, (byte // 4 + 1) % 64], axis=1)
                for half in (slice(0, 32), slice(32, 64)):
                    b = banks[half].ravel()
                    assert len(np.unique(b)) == 64, (w, bi, bj)


# ------------------------------------- rotated C-phase walk (never kept) ----
def ring_schedule(kt_n, stages=4, ahead=3):
    """gemm_tile's stage ring: (step whose data a load fetches, stage it lands
    in, step in whose body it is issued) for the prologue and the loop, with
    the clamp that makes loads past the end re-read the last step."""
    ev = [(min(kt, kt_n - 1), kt % stages, -1) for kt in range(ahead)]
    for kt in range(kt_n):
        nxt = kt + ahead
        ev.append((min(nxt, kt_n - 1), nxt % stages, kt))
    return ev


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("m_pad_tiles", [1, 2, 3, 16])
def test_rotated_c_walk_stays_in_bounds_and_in_ring_order(tile, m_pad_tiles):
    """A C-phase K walk rotated to end on the A columns its epilogue reads
    (start at krot = ((ti + 1) TILE / 32) mod kt_n, step kr = (kc + krot) mod
    kt_n for the clamped step kc) reads every K step of A exactly once, from
    inside A, for every upper tile (ti, tj); a stage is refilled only after
    the step that last read it (same ring as the unrotated walk: the rotation
    changes addresses, not the schedule); and the walk's last TILE / 32 steps
    are the epilogue's columns.  (Index arithmetic of the walk as described;
    the fault seen with that change is not explained by it.)"""
    m_pad = m_pad_tiles * tile
    kt_n = m_pad // BK
    for ti in range(m_pad_tiles):
        for tj in range(ti, m_pad_tiles):
            krot = ((ti + 1) * tile // BK) % kt_n
            seen = []
            for kc, stage, issued_in in ring_schedule(kt_n):
                kr = (kc + krot) % kt_n
                for mn_layout in (False,):                  # C reads A K-contiguous
                    for row0 in (ti * tile, tj * tile):
                        mn, k, lds = dma_elements(tile, mn_layout, m_pad, row0, kr)
                        assert mn.min() >= 0 and (mn * m_pad + k + 7).max() < m_pad * m_pad
                        assert lds.min() >= 0 and (lds + 7).max() < tile * BK
                # a load issued in step s refills stage (s + 3) % 4, last read in step s - 1
                if issued_in >= 0:
                    assert stage == (issued_in + 3) % 4 and (issued_in - 1) % 4 == stage
                seen.append(kr)
            walk = seen[:kt_n]                           # the steps the loop consumes
            assert sorted(walk) == list(range(kt_n))
            tail = walk[-(tile // BK):] if kt_n >= tile // BK else walk
            assert sorted(tail) == list(range(ti * tile // BK, (ti + 1) * tile // BK))[-len(tail):]
