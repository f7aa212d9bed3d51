"""Host-side models of the LDS fragment layouts the bf16 kernels rely on (no GPU).

The matrix-core operand order: slot e of lane l in a k16 step carries contraction index
16u + perm_row(e, l // 32), the row order of an output block (register r of C holds row
8(r // 4) + 4(l // 32) + r % 4).  A fragment of a tile that a product contracts over its rows is
read from the row-major tile with the transposing LDS read, whose lane rule (measured on the GPU
with an in-bounds probe of two address patterns) is: within each group of 16 lanes, lane i
receives as element j the element i % 4 of the 8 bytes addressed by lane 4j + i // 4.  These
tests check that the addresses the kernels give each lane (tr_frag) then deliver exactly the
operand order above, for every lane and slot, and that every read stays inside the tile."""
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


def tr_frag_addresses(row0, col0, ldp):
    """The two per-lane element addresses tr_frag issues (row-major tile, row stride ldp)."""
    lo, hi = [], []
    for lane in range(64):
        i = lane & 15
        r = row0 + 4 * (lane >> 5) + (i >> 2)
        c = col0 + 16 * ((lane >> 4) & 1) + 4 * (i & 3)
        lo.append(r * ldp + c)
        hi.append((r + 8) * ldp + c)
    return lo, hi


def test_probe_patterns_follow_the_rule():
    """The rule reproduces what the probe printed for both of its address patterns."""
    mem = list(range(4096))
    a = tr_read([4 * l for l in range(64)], mem)
    assert a[0] == [0, 16, 32, 48] and a[17] == [65, 81, 97, 113] and a[63] == [207, 223, 239, 255]
    b = tr_read([(l % 16) * 64 + (l // 16) * 4 for l in range(64)], mem)
    assert b[0] == [0, 256, 512, 768] and b[4] == [64, 320, 576, 832]
    assert b[16] == [4, 260, 516, 772] and b[63] == [207, 463, 719, 975]


@pytest.mark.parametrize("rows,d", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_tr_frag_gives_the_operand_order(rows, d):
    ldp = d + 8  # padded bf16 row of the kernels' tiles
    mem = [None] * (rows * ldp)
    for r, c in itertools.product(range(rows), range(d)):
        mem[r * ldp + c] = (r, c)  # each element names its own row and column
    for row0 in range(0, rows, 16):
        for col0 in range(0, d, 32):
            lo, hi = tr_frag_addresses(row0, col0, ldp)
            for a in lo + hi:  # every 8-byte read inside the tile, 8-byte aligned
                assert 0 <= a and a + 3 < rows * ldp and (2 * a) % 8 == 0
                assert a % ldp + 3 < d  # never into the row padding
            vlo, vhi = tr_read(lo, mem), tr_read(hi, mem)
            for lane in range(64):
                frag = vlo[lane] + vhi[lane]
                for e in range(8):
                    assert frag[e] == (row0 + perm_row(e, lane >> 5), col0 + (lane & 31))


def test_a_planted_address_mistake_is_caught():
    """Swapping the two 4-row reads (a plausible slip) breaks the order the test checks."""
    ldp, rows, d = 72, 64, 64
    mem = [None] * (rows * ldp)
    for r, c in itertools.product(range(rows), range(d)):
        mem[r * ldp + c] = (r, c)
    lo, hi = tr_frag_addresses(0, 0, ldp)
    frag = tr_read(hi, mem)[0] + tr_read(lo, mem)[0]
    assert [frag[e] for e in range(8)] != [(perm_row(e, 0), 0) for e in range(8)]
