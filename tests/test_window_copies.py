"""Host model of the replaced heads' distance windows (saf_device.h: win_store, win_base,
win_read4) and of the residues the kernels rely on (no GPU).

A window of WIN entries is kept in 4 copies WINP = win_pad(WIN) floats apart (WIN rounded up to 64,
plus 16); copy c holds entry y + c at index y.  A lane whose 4 consecutive entries start at x with x % 4 == c reads them as
one aligned float4 at index x - c of copy c.  The kernels take c as a per-lane constant, so the
residue of every start they read must not depend on anything but the lane."""
import itertools

import pytest


def win_store(win, winp, x, v):
    for c in range(4):
        if x >= c:
            win[c * winp + x - c] = v


def win_pad(n):
    return ((n + 63) & ~63) + 16


def window(n):
    winp = win_pad(n)
    win = [None] * (4 * winp)
    for x in range(n):
        win_store(win, winp, x, x)  # each entry names itself
    return win, winp


@pytest.mark.parametrize("n", [192, 256, 384, 160, 97])
def test_reads_are_aligned_and_exact(n):
    win, winp = window(n)
    for x in range(0, n - 3):
        c = x % 4
        a = c * winp - c + x  # win_base(win, winp, c) + x
        assert a % 4 == 0 and 0 <= a and a + 3 < 4 * winp
        assert win[a:a + 4] == [x, x + 1, x + 2, x + 3]


def test_forward_residue_is_a_lane_constant():
    """Forward, replaced item: lane query qi = q0 + 32w + l32 reads entries xr - 3 .. xr with
    xr = (qi - q0) + BK - 1 - kk, kk = 32s + 8g + 4hi, and uses copy l32 % 4."""
    for BK, W in ((128, 8), (128, 4), (32, 2)):
        win = BK + 32 * W
        for w, l32, s, g, hi in itertools.product(range(W), range(32), range(BK // 32), range(4), range(2)):
            kk = 32 * s + 8 * g + 4 * hi
            xr = 32 * w + l32 + BK - 1 - kk
            assert (xr - 3) % 4 == l32 % 4 and 0 <= xr - 3 and xr < win


def test_backward_residue_is_a_lane_constant():
    """Backward, replaced item: the lane's key kj = kb0 + 32kg + l32 reads entries xr .. xr+3 with
    xr = qr + kb0 + BKV - 1 - kj, qr = row0 + 8g + 4hi (row0 a multiple of 32), from copy
    (3 - l32) % 4."""
    for BKV, BQ in ((128, 64), (128, 128), (128, 32)):
        win = BQ + BKV
        for kg, l32, row0, g, hi in itertools.product(range(BKV // 32), range(32), range(0, BQ, 32), range(4), range(2)):
            qr = row0 + 8 * g + 4 * hi
            xr = qr + BKV - 1 - (32 * kg + l32)  # kb0 cancels
            assert xr % 4 == (3 - l32) % 4 and 0 <= xr and xr + 3 < win


def test_a_planted_shift_mistake_is_caught():
    """Storing copy c shifted up instead of down (a plausible slip) returns other entries."""
    n = 192
    winp = win_pad(n)
    win = [None] * (4 * winp)
    for x in range(n):
        for c in range(4):
            if x + c < winp:
                win[c * winp + x + c] = x
    x = 5
    a = (x % 4) * winp - (x % 4) + x
    assert win[a:a + 4] != [5, 6, 7, 8]


def _banks(addrs):
    """Worst bank multiplicity of one 16-lane pass of 16-byte reads (64 banks of 4 bytes)."""
    cnt = [0] * 64
    for a in addrs:
        for k in range(4):
            cnt[(a + k) % 64] += 1
    return max(cnt)


@pytest.mark.parametrize("n", [192, 256, 384, 160])
def test_reads_of_consecutive_lanes_are_free_of_bank_conflicts(n):
    """A 16-lane pass reads 16 consecutive starts: ascending from a start = 0 mod 4 (forward:
    xr - 3 = 32w + l32 + BK - 4 - kk) or descending from a start = 3 mod 4 (backward: xr = qr + BKV
    - 1 - 32kg - l32), i.e. 4 indices of the 4 copies, which the copy stride spreads over all banks.
    Copies WIN rounded to 4 apart (the first layout) put them on the same banks 4-way."""
    winp = win_pad(n)
    for x0 in range(16, n - 20):
        if x0 % 4 == 0:
            starts = [x0 + j for j in range(16)]
        elif x0 % 4 == 3:
            starts = [x0 - j for j in range(16)]
        else:
            continue
        assert _banks([(x % 4) * winp - x % 4 + x for x in starts]) == 1
    tight = (n + 3) & ~3
    if tight % 64 == 0:
        starts = [100 + j for j in range(16)]
        assert _banks([(x % 4) * tight - x % 4 + x for x in starts]) == 4
