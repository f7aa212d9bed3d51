"""The C-ABI library on the CPU: it loads, exports every entry point include/saf.h declares, sizes
its workspaces, and rejects invalid arguments before any HIP call (so no GPU is needed here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "saf.h")

saf = pytest.importorskip("fixed_pattern_mixed_amd")

FAKE = 0x100000  # an aligned, never-dereferenced stand-in pointer: each case fails validation first
SIZE_MAX = 2 ** 64 - 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(saf_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"saf_attn_fwd", "saf_attn_bwd", "saf_calibrate", "saf_last_error"} <= set(names)
    lib = ctypes.CDLL(saf.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), "libsaf.so does not export " + n


def test_workspace_sizes():
    pat = saf.saf_pattern_size(12, 4096)
    assert pat >= 12 * 3 * 4096 * 4
    assert saf.saf_attn_fwd_workspace_size(8, 12, 4096, 64) == pat
    assert saf.saf_attn_bwd_workspace_size(8, 12, 4096, 64) == pat + 8 * 12 * 4096 * 4
    assert saf.saf_attn_bwd_workspace_size(0, 12, 4096, 64) == 0
    n = saf.saf_calibrate_workspace_size(32, 16, 8192, 128)
    assert n >= 32 * 16 * 8192 * 4 + 16 * 64 * 128 * 8
    assert saf.saf_attn_bwd_workspace_size(8, 12, 4096, 96) == SIZE_MAX
    assert saf.saf_calibrate_workspace_size(1, 16, 8192, 128) == SIZE_MAX


def _mask(*bits):
    return (ctypes.c_uint8 * len(bits))(*bits)


def fwd(dt=1, B=2, H=4, T=64, d=64, q=FAKE, k=FAKE, v=FAKE, rep=None, a=FAKE, r=FAKE, pat=64,
        scale=0.0, o=FAKE, lse=FAKE, ws=FAKE, ws_n=0):
    rep = _mask(0, 0, 0, 1) if rep is None else rep
    return saf.saf_attn_fwd(dt, B, H, T, d, q, k, v, rep, a, r, pat, None, scale, o, lse, ws, ws_n,
                            None)


def bwd(dt=1, B=2, H=4, T=64, d=64, q=FAKE, k=FAKE, v=FAKE, o=FAKE, g=FAKE, lse=FAKE, rep=None,
        a=FAKE, r=FAKE, pat=64, scale=0.0, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, ws_n=0):
    rep = _mask(0, 0, 0, 1) if rep is None else rep
    return saf.saf_attn_bwd(dt, B, H, T, d, q, k, v, o, g, lse, rep, a, r, pat, None, scale, dq,
                            dk, dv, ws, ws_n, None)



def test_stored_ds_workspace_size():
    """The larger backward workspace with room for the stored dS: bf16, d = 128, Hkv = H and an
    ordinary head; 2 bytes per entry of the 32 x 32 subtiles on or below the diagonal of each
    ordinary slice, after the plain workspace (256-byte aligned); the plain size elsewhere."""
    f = saf.saf_attn_bwd_ds_workspace_size
    for B, H, T, R in [(2, 16, 8192, 4), (1, 4, 257, 1), (3, 2, 33, 0), (1, 2, 1, 1)]:
        base = saf.saf_attn_bwd_workspace_size(B, H, T, 128)
        n32 = (T + 31) // 32
        extra = 2 * B * (H - R) * (n32 * (n32 + 1) // 2) * 1024
        assert f(saf.SAF_BF16, B, H, H, T, 128, R) == base + (extra + 255) // 256 * 256
    assert f(saf.SAF_BF16, 2, 16, 16, 8192, 128, 4) - saf.saf_attn_bwd_workspace_size(2, 16, 8192, 128) == 1616904192  # 1.6 GB at the 1B shape
    base = saf.saf_attn_bwd_workspace_size(2, 8, 512, 128)
    assert f(saf.SAF_F32, 2, 8, 8, 512, 128, 1) == base          # fp32: dQ forms S and dP again
    assert f(saf.SAF_BF16, 2, 8, 2, 512, 128, 1) == base         # grouped key/value heads
    assert f(saf.SAF_BF16, 2, 8, 8, 512, 128, 8) == base         # no ordinary head
    assert f(saf.SAF_BF16, 2, 8, 8, 512, 64, 1) == saf.saf_attn_bwd_workspace_size(2, 8, 512, 64)
    assert f(saf.SAF_BF16, 0, 8, 8, 512, 128, 1) == 0
    for bad in [(saf.SAF_BF16, 2, 8, 3, 512, 128, 1), (saf.SAF_BF16, 2, 8, 8, 512, 128, 9),
                (saf.SAF_BF16, 2, 8, 8, 512, 128, -1), (saf.SAF_BF16, 2, 8, 8, 512, 96, 1),
                (saf.SAF_BF16, 2, 8, 8, 65537, 128, 1), (7, 2, 8, 8, 512, 128, 1)]:
        assert f(*bad) == SIZE_MAX, bad

@pytest.mark.parametrize("case,kw,status", [
    ("unsupported d", dict(d=96), saf.SAF_ERR_UNSUPPORTED),
    ("too many heads", dict(H=300, rep=_mask(*([0] * 300))), saf.SAF_ERR_UNSUPPORTED),
    ("T too long", dict(T=70000, pat=70000), saf.SAF_ERR_UNSUPPORTED),
    ("negative T", dict(T=-1), saf.SAF_ERR_INVALID_ARG),
    ("no heads", dict(H=0), saf.SAF_ERR_INVALID_ARG),
    ("unknown dtype", dict(dt=7), saf.SAF_ERR_INVALID_ARG),
    ("null q", dict(q=None), saf.SAF_ERR_INVALID_ARG),
    ("misaligned v", dict(v=FAKE + 2), saf.SAF_ERR_INVALID_ARG),
    ("null mask", dict(rep=ctypes.POINTER(ctypes.c_uint8)()), saf.SAF_ERR_INVALID_ARG),
    ("null a with a replaced head", dict(a=None), saf.SAF_ERR_INVALID_ARG),
    ("pattern shorter than T", dict(pat=63), saf.SAF_ERR_INVALID_ARG),
    ("null lse", dict(lse=None), saf.SAF_ERR_INVALID_ARG),
    ("NaN scale", dict(scale=float("nan"), ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
    ("short workspace for the pattern", dict(ws_n=100), saf.SAF_ERR_INVALID_ARG),
    ("null workspace for the pattern", dict(ws=None, ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
])
def test_forward_rejects(case, kw, status):
    assert fwd(**kw) == status, saf.saf_last_error()
    assert saf.saf_last_error() != ""


def test_forward_empty_calls_are_noops():
    assert fwd(B=0, q=None, k=None, v=None, o=None, lse=None) == saf.SAF_OK
    assert fwd(T=0, q=None, k=None, v=None, o=None, lse=None) == saf.SAF_OK


def test_ordinary_only_layer_needs_no_pattern():
    # no replaced head: a / r may be NULL; the call then fails on the missing lse, not on a / r
    st = fwd(rep=_mask(0, 0, 0, 0), a=None, r=None, lse=None)
    assert st == saf.SAF_ERR_INVALID_ARG and "lse" in saf.saf_last_error()


def test_replaced_only_layer_needs_no_qk():
    st = fwd(rep=_mask(1, 1, 1, 1), q=None, k=None, lse=None)
    assert st == saf.SAF_ERR_INVALID_ARG and "lse" in saf.saf_last_error()


@pytest.mark.parametrize("case,kw,status", [
    ("unsupported d", dict(d=32), saf.SAF_ERR_UNSUPPORTED),
    ("null ws", dict(ws=None, ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
    ("short ws", dict(ws_n=100), saf.SAF_ERR_INVALID_ARG),
    ("misaligned ws", dict(ws=FAKE + 16, ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
    ("null dk", dict(dk=None, ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
    ("null dout", dict(g=None, ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
    ("pattern shorter than T", dict(pat=10, ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
])
def test_backward_rejects(case, kw, status):
    assert bwd(**kw) == status, saf.saf_last_error()


@pytest.mark.parametrize("case,dt,N,H,T,d,status", [
    ("one sequence", 1, 1, 4, 64, 64, saf.SAF_ERR_INVALID_ARG),
    ("unsupported d", 1, 4, 4, 64, 80, saf.SAF_ERR_UNSUPPORTED),
    ("unknown dtype", 5, 4, 4, 64, 64, saf.SAF_ERR_INVALID_ARG),
    ("no heads", 1, 4, 0, 64, 64, saf.SAF_ERR_INVALID_ARG),
])
def test_calibrate_rejects(case, dt, N, H, T, d, status):
    st = saf.saf_calibrate(dt, N, H, T, d, FAKE, FAKE, 0.0, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == status, saf.saf_last_error()


@pytest.mark.parametrize("case,H,P,a,pat,n,status", [
    ("no heads", 0, 64, FAKE, FAKE, 1 << 20, saf.SAF_ERR_INVALID_ARG),
    ("too many heads", 300, 64, FAKE, FAKE, 1 << 20, saf.SAF_ERR_UNSUPPORTED),
    ("null a", 4, 64, None, FAKE, 1 << 20, saf.SAF_ERR_INVALID_ARG),
    ("null buffer", 4, 64, FAKE, None, 1 << 20, saf.SAF_ERR_INVALID_ARG),
    ("misaligned buffer", 4, 64, FAKE, FAKE + 64, 1 << 20, saf.SAF_ERR_INVALID_ARG),
    ("short buffer", 4, 64, FAKE, FAKE, 64, saf.SAF_ERR_INVALID_ARG),
])
def test_pattern_prepare_rejects(case, H, P, a, pat, n, status):
    rep = _mask(*([0, 0, 0, 1] * 75)[:max(H, 1)])
    assert saf.saf_pattern_prepare(H, rep, a, FAKE, P, pat, n, None) == status, saf.saf_last_error()


def test_pattern_prepare_without_replaced_heads_is_noop():
    assert saf.saf_pattern_prepare(4, _mask(0, 0, 0, 0), None, None, 64, None, 0, None) == saf.SAF_OK


def test_calibrate_short_workspace():
    need = saf.saf_calibrate_workspace_size(4, 2, 64, 64)
    st = saf.saf_calibrate(1, 4, 2, 64, 64, FAKE, FAKE, 0.0, FAKE, FAKE, None, FAKE, need - 1, None)
    assert st == saf.SAF_ERR_INVALID_ARG and "workspace" in saf.saf_last_error()


def test_single_hip_runtime_in_process():
    """The binding must share PyTorch's HIP runtime (one libamdhip64 mapped in the process)."""
    assert len(saf._hip_runtimes()) == 1, saf._hip_runtimes()


def pgrad(dt=1, B=2, H=4, T=64, d=64, v=FAKE, o=FAKE, g=FAKE, lse=FAKE, rep=None, a=FAKE, r=FAKE,
          pat=64, da=FAKE, dr=FAKE, ws=FAKE, ws_n=0):
    rep = _mask(0, 0, 0, 1) if rep is None else rep
    return saf.saf_attn_bwd_pattern(dt, B, H, T, d, v, o, g, lse, rep, a, r, pat, None, da, dr, ws,
                                    ws_n, None)


@pytest.mark.parametrize("case,kw,status", [
    ("unsupported d", dict(d=96), saf.SAF_ERR_UNSUPPORTED),
    ("unknown dtype", dict(dt=3), saf.SAF_ERR_INVALID_ARG),
    ("null a", dict(a=None), saf.SAF_ERR_INVALID_ARG),
    ("pattern shorter than T", dict(pat=32), saf.SAF_ERR_INVALID_ARG),
    ("null da", dict(da=None), saf.SAF_ERR_INVALID_ARG),
    ("misaligned dr", dict(dr=FAKE + 2), saf.SAF_ERR_INVALID_ARG),
    ("null v", dict(v=None, ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
    ("null lse", dict(lse=None, ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
    ("null ws", dict(ws=None, ws_n=1 << 30), saf.SAF_ERR_INVALID_ARG),
    ("short ws", dict(ws_n=1000), saf.SAF_ERR_INVALID_ARG),
])
def test_pattern_gradient_rejects(case, kw, status):
    assert pgrad(**kw) == status, saf.saf_last_error()


def test_pattern_gradient_without_replaced_heads_is_noop():
    assert pgrad(rep=_mask(0, 0, 0, 0), v=None, a=None, r=None, da=None, dr=None, ws=None) == saf.SAF_OK


def test_pattern_gradient_workspace():
    B, H, T = 8, 12, 4096
    n = saf.saf_attn_bwd_pattern_workspace_size(B, H, T, 64)
    # pattern, delta, per-(batch, head) da partials, dr partials per 32-key sub-block
    assert n >= saf.saf_pattern_size(H, T) + 2 * B * H * T * 4 + B * H * (T // 32) * T * 4
    assert saf.saf_attn_bwd_pattern_workspace_size(0, H, T, 64) == 0
    assert saf.saf_attn_bwd_pattern_workspace_size(B, H, T, 80) == SIZE_MAX


@pytest.mark.parametrize("case,H,T,steps,lr,ptr,n,status", [
    ("no heads", 0, 64, 10, 0.1, FAKE, 1 << 30, saf.SAF_ERR_INVALID_ARG),
    ("too many heads", 300, 64, 10, 0.1, FAKE, 1 << 30, saf.SAF_ERR_UNSUPPORTED),
    ("T too long", 2, 70000, 10, 0.1, FAKE, 1 << 30, saf.SAF_ERR_UNSUPPORTED),
    ("negative steps", 2, 64, -1, 0.1, FAKE, 1 << 30, saf.SAF_ERR_INVALID_ARG),
    ("zero lr", 2, 64, 10, 0.0, FAKE, 1 << 30, saf.SAF_ERR_INVALID_ARG),
    ("NaN lr", 2, 64, 10, float("nan"), FAKE, 1 << 30, saf.SAF_ERR_INVALID_ARG),
    ("null ahat", 2, 64, 10, 0.1, None, 1 << 30, saf.SAF_ERR_INVALID_ARG),
    ("short ws", 2, 64, 10, 0.1, FAKE, 1000, saf.SAF_ERR_INVALID_ARG),
])
def test_fit_rejects(case, H, T, steps, lr, ptr, n, status):
    st = saf.saf_fit_pattern(H, T, ptr, steps, lr, FAKE, FAKE, FAKE, None, FAKE, n, None)
    assert st == status, saf.saf_last_error()


def test_fit_workspace():
    n = saf.saf_fit_pattern_workspace_size(16, 8192)
    # fp64 state of 15 T values per head plus the partial sums of the marginal pass
    assert n >= 16 * 15 * 8192 * 8 + 16 * 128 * 8192 * 8
    assert saf.saf_fit_pattern_workspace_size(16, 0) == 0
    assert saf.saf_fit_pattern_workspace_size(0, 64) == SIZE_MAX
