"""Host-side models of the LDS fragment layouts the bf16 kernels rely on (no GPU).

The matrix-core operand order: slot e of lane l in a k16 step carries contraction index
16u + perm_row(e, l // 32), the row order of an output block (register r of C holds row
8(r // 4) + 4(l // 32) + r % 4).  A fragment of a tile that a product contracts over its rows is
read from the row tile with the transposing LDS read, whose lane rule (measured on the GPU with an
in-bounds probe of two address patterns) is: within each group of 16 lanes, lane i receives as
element j the element i % 4 of the 8 bytes addressed by lane 4j + i // 4.

Tiles read that way have rows of D + 32 elements, and tiles also read as rows (16-byte A-operand
fragments) have the low two bits of each 16-byte chunk index XORed with (r >> 2) & 3
(saf_device.h: tile_off, TileLane).  These tests check, for every lane and slot, that the
addresses the kernels issue deliver exactly the operand order above, that every access stays
inside the tile and is aligned, that the one-XOR second bases equal the direct formula, and that
both reads are free of bank conflicts under the LDS model measured with probes on the GPU: 64
banks of 4 bytes; the transposing read served 32 lanes per pass, the 16-byte read 16 lanes."""
import itertools

import pytest


def perm_row(e, hi):
    return 8 * (e >> 2) + 4 * hi + (e & 3)


def tr_read(addr_of_lane, mem):
    """One ds_read_b64_tr_b16: addr_of_lane[l] is lane l's element address (4 consecutive
    16-bit values).  Returns the 4 values each lane receives."""
    out = []
    for l in range(64):
        g, i = l // 16, l % 16
        vals = []
        for j in range(4):
            src = 16 * g + 4 * j + i // 4
            vals.append(mem[addr_of_lane[src] + i % 4])
        out.append(vals)
    return out


def ldr(d):
    return d + 32


def tile_off(d, sw, r, c):
    ch = c >> 3
    if sw:
        ch = (ch & ~3) | ((ch & 3) ^ ((r >> 2) & 3))
    return r * ldr(d) + 8 * ch + (c & 7)


def lane_bases(d, sw, lane):
    """TileLane: (rb0, tb0) and the derived second bases rb(1), tb(1)."""
    l32, hi, i = lane & 31, lane >> 5, lane & 15
    rb0 = tile_off(d, sw, l32, 8 * hi)
    tb0 = tile_off(d, sw, 4 * hi + (i >> 2), 16 * ((lane >> 4) & 1) + 4 * (i & 3))
    rb1 = rb0 ^ 16
    tb1 = (tb0 ^ 16 if sw else tb0) + 8 * ldr(d)
    return rb0, rb1, tb0, tb1


def tr_addresses(d, sw, row0, cc):
    """Per-lane element addresses of tile_tr_frag's two reads."""
    lo, hi = [], []
    for lane in range(64):
        _, _, tb0, tb1 = lane_bases(d, sw, lane)
        lo.append(row0 * ldr(d) + 32 * cc + tb0)
        hi.append(row0 * ldr(d) + 32 * cc + tb1)
    return lo, hi


def row_addresses(d, sw, row_base, t):
    """Per-lane element addresses of tile_row_frag (8 consecutive elements each)."""
    out = []
    for lane in range(64):
        rb0, rb1, _, _ = lane_bases(d, sw, lane)
        out.append(row_base * ldr(d) + 32 * (t >> 1) + (rb1 if t & 1 else rb0))
    return out


def tile_mem(rows, d, sw):
    mem = [None] * (rows * ldr(d))
    for r, c in itertools.product(range(rows), range(d)):
        mem[tile_off(d, sw, r, c)] = (r, c)  # each element names its own row and column
    return mem


def banks_max(addrs, nbytes, lanes_per_pass):
    worst = 0
    for p0 in range(0, 64, lanes_per_pass):
        cnt = [0] * 64
        for l in range(p0, p0 + lanes_per_pass):
            dw = 2 * addrs[l] // 4
            for k in range(nbytes // 4):
                cnt[(dw + k) % 64] += 1
        worst = max(worst, max(cnt))
    return worst


def test_probe_patterns_follow_the_rule():
    """The rule reproduces what the probe printed for both of its address patterns."""
    mem = list(range(4096))
    a = tr_read([4 * l for l in range(64)], mem)
    assert a[0] == [0, 16, 32, 48] and a[17] == [65, 81, 97, 113] and a[63] == [207, 223, 239, 255]
    b = tr_read([(l % 16) * 64 + (l // 16) * 4 for l in range(64)], mem)
    assert b[0] == [0, 256, 512, 768] and b[4] == [64, 320, 576, 832]
    assert b[16] == [4, 260, 516, 772] and b[63] == [207, 463, 719, 975]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("sw", [False, True])
def test_second_bases_equal_the_direct_formula(d, sw):
    """rb(1) and tb(1), one XOR from the first bases, are the offsets tile_off gives directly."""
    for lane in range(64):
        l32, hi, i = lane & 31, lane >> 5, lane & 15
        _, rb1, _, tb1 = lane_bases(d, sw, lane)
        if sw:  # rb1 is only used on swizzled tiles (the forward's V tile is never read as rows)
            assert rb1 == tile_off(d, sw, l32, 16 + 8 * hi)
        assert tb1 == tile_off(d, sw, 4 * hi + (i >> 2) + 8, 16 * ((lane >> 4) & 1) + 4 * (i & 3))


@pytest.mark.parametrize("rows,d", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("sw", [False, True])
def test_transposing_read_gives_the_operand_order(rows, d, sw):
    mem = tile_mem(rows, d, sw)
    for row0 in range(0, rows, 16):
        for cc in range(d // 32):
            lo, hi = tr_addresses(d, sw, row0, cc)
            for a in lo + hi:  # every 8-byte read inside the tile, 8-byte aligned, never padding
                assert 0 <= a and a + 3 < rows * ldr(d) and (2 * a) % 8 == 0
                assert a % ldr(d) + 3 < d
            vlo, vhi = tr_read(lo, mem), tr_read(hi, mem)
            for lane in range(64):
                frag = vlo[lane] + vhi[lane]
                for e in range(8):
                    assert frag[e] == (row0 + perm_row(e, lane >> 5), 32 * cc + (lane & 31))


@pytest.mark.parametrize("rows,d", [(64, 64), (64, 128), (128, 128)])
def test_row_read_gives_the_a_operand(rows, d):
    """Lane l reads row row_base + l % 32, columns 16t + 8(l // 32) .. +7, contiguous."""
    mem = tile_mem(rows, d, True)
    for row_base in range(0, rows, 32):
        for t in range(d // 16):
            for lane, a in enumerate(row_addresses(d, True, row_base, t)):
                assert a % 8 == 0 and 0 <= a and a + 7 < rows * ldr(d)
                want = [(row_base + (lane & 31), 16 * t + 8 * (lane >> 5) + k) for k in range(8)]
                assert mem[a:a + 8] == want


@pytest.mark.parametrize("d", [64, 128])
def test_reads_are_free_of_bank_conflicts(d):
    for row0, cc in itertools.product(range(0, 64, 16), range(d // 32)):
        for sw in (False, True):
            for addrs in tr_addresses(d, sw, row0, cc):
                assert banks_max(addrs, 8, 32) == 1
    for row_base, t in itertools.product((0, 32), range(d // 16)):
        assert banks_max(row_addresses(d, True, row_base, t), 16, 16) == 1


@pytest.mark.parametrize("d", [64, 128])
def test_padded_rows_of_d_plus_8_conflict(d):
    """The layout these replace (rows of D + 8 elements): its transposing reads were 2-way (D = 64)
    and 4-way (D = 128) conflicted, half the measured read rate at D = 128."""
    ld = d + 8
    addrs = []
    for lane in range(64):
        i = lane & 15
        r = 4 * (lane >> 5) + (i >> 2)
        c = 16 * ((lane >> 4) & 1) + 4 * (i & 3)
        addrs.append(r * ld + c)
    assert banks_max(addrs, 8, 32) == (2 if d == 64 else 4)


@pytest.mark.parametrize("d,rows,nt", [(64, 64, 256), (128, 64, 256), (128, 128, 512), (64, 128, 512)])
def test_staging_writes_cover_the_tile_once(d, rows, nt):
    """Chunks::store_tile: chunk idx of the tile (row idx / (d/8), chunk idx % (d/8)) lands at
    tile_off; every element of every row is written exactly once, inside the tile."""
    cpr = d // 8
    seen = set()
    for sw in (False, True):
        seen.clear()
        for idx in range(rows * cpr):
            r, ch = idx // cpr, idx % cpr
            a = tile_off(d, sw, r, 8 * ch)
            assert a % 8 == 0 and a + 7 < rows * ldr(d) and a % ldr(d) + 7 < d
            for k in range(8):
                assert a + k not in seen
                seen.add(a + k)
        assert len(seen) == rows * d


def test_a_planted_address_mistake_is_caught():
    """Swapping the two 4-row reads (a plausible slip) breaks the order the test checks."""
    d, rows = 64, 64
    mem = tile_mem(rows, d, True)
    lo, hi = tr_addresses(d, True, 0, 0)
    frag = tr_read(hi, mem)[0] + tr_read(lo, mem)[0]
    assert [frag[e] for e in range(8)] != [(perm_row(e, 0), 0) for e in range(8)]


# ---- [dimension][key] tiles (saf_device.h: kt_off, KtLane, kt_frag) -------------------------------
KKT = 128


def kt_off(r, c):
    return r * KKT + ((((c >> 5) ^ r) & 3) << 5) + (c & 31)


def kt_base(lane, cb):
    hi, i = lane >> 5, lane & 15
    return kt_off(8 * hi + (i >> 2), 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (i & 3))


def kt_addresses(cb, t):
    """Per-lane element addresses of kt_frag's two reads (rows +0..3 and +4..7 of 16t + 8hi)."""
    lo = [kt_base(l, cb) + 16 * t * KKT for l in range(64)]
    return lo, [a + 4 * KKT for a in lo]


def kt_mem():
    mem = [None] * (KKT * KKT)
    for r, c in itertools.product(range(KKT), range(KKT)):
        assert mem[kt_off(r, c)] is None  # one slot per element: the XOR is a bijection per row
        mem[kt_off(r, c)] = (r, c)
    return mem


def test_kt_read_gives_the_natural_b_operand():
    """Slot e of lane l: contraction row 16t + 8(l // 32) + e (the order of a row fragment of the
    other operand), column 32 cb + l % 32."""
    mem = kt_mem()
    for cb, t in itertools.product(range(4), range(8)):
        lo, hi = kt_addresses(cb, t)
        for a in lo + hi:
            assert 0 <= a and a + 3 < KKT * KKT and (2 * a) % 8 == 0
        vlo, vhi = tr_read(lo, mem), tr_read(hi, mem)
        for lane in range(64):
            frag = vlo[lane] + vhi[lane]
            assert frag == [(16 * t + 8 * (lane >> 5) + e, 32 * cb + (lane & 31)) for e in range(8)]


def test_kt_read_is_free_of_bank_conflicts():
    for cb, t in itertools.product(range(4), range(8)):
        for addrs in kt_addresses(cb, t):
            assert banks_max(addrs, 8, 32) == 1


def test_kt_staging_writes():
    """The staging of a key block: thread chunk idx -> key idx % 128, dimensions 8 (idx // 128) ..
    +7, one 2-byte store each.  Every element is written once; a wave's 64 stores of one dimension
    touch each 4-byte word at most twice (its two halves), so no two lanes meet on a bank with
    different words."""
    seen = set()
    for idx in range(KKT * KKT // 8):
        key, d0 = idx & 127, 8 * (idx >> 7)
        for e in range(8):
            a = kt_off(d0 + e, key)
            assert a not in seen
            seen.add(a)
    assert len(seen) == KKT * KKT
    for w0, e in itertools.product(range(0, KKT * KKT // 8, 64), range(8)):
        words = {}
        for idx in range(w0, w0 + 64):
            a = kt_off(8 * (idx >> 7) + e, idx & 127)
            words.setdefault((a // 2) % 64, set()).add(a // 2)
        assert all(len(v) == 1 for v in words.values())


def test_kt_without_the_xor_conflicts():
    """Unpadded rows without the XOR: the four rows of a pass share one 16-bank segment."""
    addrs = []
    for lane in range(64):
        hi, i = lane >> 5, lane & 15
        addrs.append((8 * hi + (i >> 2)) * KKT + 16 * ((lane >> 4) & 1) + 4 * (i & 3))
    assert banks_max(addrs, 8, 32) == 4


# ---- stored dS subtiles (saf_bwd.hip: bwd_kv's dS store, bwd_dq_ds's ds_tr_off) ------------------
# The wide key-block kernel stores each 32 x 32 subtile of dS as its two B-operand fragments:
# element u * 512 + L * 8 + e holds dS[query 16u + perm_row(e, L // 32)][key L % 32].  bwd_dq_ds
# copies the 1024 elements into LDS in four quarters (u, L // 32) of 256 elements placed DS_BLK
# elements apart, and reads the dQ product's B operand (lane = query, slots = keys) back with the
# transposing read.
DS_BLK = 288


def ds_lds_pos(raw):
    """LDS element position of stored element `raw` (0 .. 1023) within a subtile's region."""
    return (raw // 256) * DS_BLK + raw % 256


def ds_tr_off(lane, ub, rd):
    """Element address lane `lane` issues for read rd (keys +0..3 / +8..11) of k16 step ub."""
    jp, a, g, hi = (lane & 15) >> 2, lane & 3, (lane >> 4) & 1, lane >> 5
    key = 16 * ub + 8 * rd + 4 * hi + jp
    return (2 * g + (a & 1)) * DS_BLK + 8 * key + 4 * (a >> 1)


def ds_subtile_mem():
    """The LDS region after the copy: each element names its (query, key)."""
    mem = [None] * (4 * DS_BLK)
    for u, L, e in itertools.product(range(2), range(64), range(8)):
        raw = 512 * u + 8 * L + e
        q, key = 16 * u + perm_row(e, L // 32), L % 32
        assert mem[ds_lds_pos(raw)] is None
        mem[ds_lds_pos(raw)] = (q, key)
    return mem


def test_stored_ds_read_gives_the_dq_b_operand():
    """Slot e of lane l: dS[query l % 32][key 16 ub + perm_row(e, l // 32)], the order in which the
    K^T fragment (tile_tr_frag of the K row tile) carries the keys."""
    mem = ds_subtile_mem()
    for ub in range(2):
        lo = [ds_tr_off(l, ub, 0) for l in range(64)]
        hi = [ds_tr_off(l, ub, 1) for l in range(64)]
        for a in lo + hi:  # 8-byte aligned, inside the region, never padding
            assert (2 * a) % 8 == 0 and 0 <= a and a + 3 < 4 * DS_BLK and a % DS_BLK + 3 < 256
        vlo, vhi = tr_read(lo, mem), tr_read(hi, mem)
        for lane in range(64):
            frag = vlo[lane] + vhi[lane]
            assert frag == [(lane & 31, 16 * ub + perm_row(e, lane >> 5)) for e in range(8)]


def test_stored_ds_copy_and_reads_are_free_of_bank_conflicts():
    """The copy (lane L writes its 16 bytes of fragment u) and both reads of each k16 step; with
    the quarters 256 elements apart (no padding) the reads would be 4-way conflicted."""
    for u in range(2):
        assert banks_max([ds_lds_pos(512 * u + 8 * L) for L in range(64)], 16, 16) == 1
    for ub, rd in itertools.product(range(2), range(2)):
        assert banks_max([ds_tr_off(l, ub, rd) for l in range(64)], 8, 32) == 1
    unpadded = [ds_tr_off(l, 0, 0) - ((2 * ((l >> 4) & 1) + (l & 1)) * (DS_BLK - 256)) for l in range(64)]
    assert banks_max(unpadded, 8, 32) == 4
