"""The bwd_kv work grid (saf_internal.h: kv_grid_blocks, kv_grid_item), run on the host (no GPU).

The grid lists the key/value heads that have an ordinary query head (the first B * n_kv_ord slots of
the key/value order) before the replaced-only ones, each section by rows of one key block, lowest
(heaviest) key block first, a row's width padded to a multiple of 8.  These tests compile the
header's own functions into a small host program and check, for assorted shapes: every (slot, key
block) is listed exactly once (only the first section's when the replaced-only heads run in a
kernel of their own), padding blocks report no item, blockIdx % 8 (the XCD) depends only on the slot
within a section, and a section's key blocks never decrease along the grid."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def grid_prog(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("grid") / "grid_map")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
           "-I" + os.path.join(ROOT, "fixed_pattern_mixed_amd", "csrc"), "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "grid_map.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run_grid(exe, B, Hkv, nko, nkb, rep_sec):
    out = subprocess.run([exe, str(B), str(Hkv), str(nko), str(nkb), str(int(rep_sec))],
                         capture_output=True, text=True, check=True).stdout.split("\n")
    n = int(out[0])
    rows = [tuple(int(v) for v in line.split()) for line in out[1:1 + n]]
    assert len(rows) == n
    return rows


SHAPES = [  # B, Hkv, key/value heads with an ordinary query head, key blocks
    (2, 16, 12, 64), (8, 12, 9, 32), (1, 8, 8, 16), (1, 8, 0, 16), (3, 5, 2, 7), (2, 16, 16, 1),
    (1, 3, 1, 5), (4, 12, 6, 64),
]


@pytest.mark.parametrize("B,Hkv,nko,nkb", SHAPES, ids=["B%dKV%dO%dN%d" % s for s in SHAPES])
@pytest.mark.parametrize("rep_sec", [True, False], ids=["both", "first"])
def test_kv_grid(grid_prog, B, Hkv, nko, nkb, rep_sec):
    rows = run_grid(grid_prog, B, Hkv, nko, nkb, rep_sec)
    s1 = B * nko
    listed = [(x, bh, kb) for x, (ok, bh, kb) in enumerate(rows) if ok]
    want = {(bh, kb) for bh in range(s1 if not rep_sec else B * Hkv) for kb in range(nkb)}
    got = [(bh, kb) for _, bh, kb in listed]
    assert len(got) == len(set(got)) and set(got) == want
    # padding: every unlisted block is a pad column of its row (a row's width is a multiple of 8)
    assert len(rows) % 8 == 0
    for sec_lo, sec_hi in ((0, s1), (s1, B * Hkv)):
        sec = [(x, bh, kb) for x, bh, kb in listed if sec_lo <= bh < sec_hi]
        xcd = {}
        for x, bh, kb in sec:
            assert xcd.setdefault(bh, x % 8) == x % 8  # one XCD per slot within the section
            assert (bh - sec_lo) % 8 == x % 8
        kbs = [kb for _, _, kb in sorted(sec)]
        assert kbs == sorted(kbs)  # heaviest (lowest) key blocks first


# ---- the stored dS (saf_internal.h: ord_rank, ds_bytes; bwd_kv stores, bwd_dq_ds reads) ----------
@pytest.fixture(scope="module")
def ds_prog(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("ds") / "ds_index")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
           "-I" + os.path.join(ROOT, "fixed_pattern_mixed_amd", "csrc"), "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "ds_index.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _masks():
    import random
    rnd = random.Random(5)
    out = ["0001" * 4, "0" * 12, "1" * 7 + "0", "0" * 256, "01" * 128]
    out += ["".join(rnd.choice("01") for _ in range(H)) for H in (63, 64, 65, 130, 200, 256)]
    return [m if "0" in m else m[:-1] + "0" for m in out]


@pytest.mark.parametrize("mask", _masks(), ids=lambda m: "H%d" % len(m))
def test_stored_ds_slots_and_size(ds_prog, mask):
    """An ordinary head's slice of the stored dS is b * n_ord + (its rank among the ordinary
    heads): the ranks number the ordinary heads 0, 1, ... in head order (the replaced-head mask
    spans several 64-bit words for H > 64), so the B * n_ord slices tile the region once; the region
    is 2 bytes per element of the 32 x 32 subtiles on or below the diagonal, 1024 per subtile."""
    for B, T in ((1, 1), (2, 8192), (3, 97), (1, 65536)):
        out = subprocess.run([ds_prog, str(B), str(T), mask], capture_output=True, text=True,
                             check=True).stdout.split("\n")
        n_ord, nbytes = (int(v) for v in out[0].split())
        ranks = [tuple(int(v) for v in line.split()) for line in out[1:1 + n_ord]]
        assert n_ord == mask.count("0")
        assert [h for h, _ in ranks] == [h for h, c in enumerate(mask) if c == "0"]
        assert [r for _, r in ranks] == list(range(n_ord))
        n32 = (T + 31) // 32
        assert nbytes == 2 * B * n_ord * (n32 * (n32 + 1) // 2) * 1024


def test_stored_ds_subtile_index_is_a_packing():
    """Subtile (ib, jb <= ib) of a slice at ib (ib + 1) / 2 + jb: every index of [0, n32 (n32 + 1) / 2)
    once, and a query block's subtiles contiguous (the order bwd_dq_ds reads them)."""
    for n32 in (1, 2, 7, 256):
        idx = [ib * (ib + 1) // 2 + jb for ib in range(n32) for jb in range(ib + 1)]
        assert idx == list(range(n32 * (n32 + 1) // 2))
