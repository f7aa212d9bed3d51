"""Python binding of libsaf.so: the fused mixed-head SAF attention layer on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of libsaf.so.
PyTorch supplies device memory (outputs and workspaces are torch tensors on the inputs' device)
and the current HIP stream.  There is no CPU or PyTorch fallback: if the library is missing this
module raises at import time.

The entry points mirror include/saf.h (same names, same argument order for the raw calls):
  saf_attn_fwd / saf_attn_bwd / saf_calibrate   raw C-ABI calls (ctypes, integer pointers)
  fwd(q, k, v, replaced, a, r)  -> (o, lse)
  bwd(q, k, v, o, dout, lse, replaced, a, r) -> (dq, dk, dv)
  calibrate(q, k) -> (ahat, svar[, skl])
  select_heads(score, ratio, accepted) -> (replaced [L, H], n)
  bwd_pattern(v, o, dout, lse, replaced, a, r) -> (da, dr)   trained-pattern gradient
  fit_pattern(ahat, steps, lr) -> (a, r, kl, loss)            compact fit of target maps
[Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记" (§二.1 Eq.(1), §二.3 Eq.(3),
§二.4 for what the three calls compute).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsaf.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libsaf.so is not built (expected at %s); run `python fixed_pattern_mixed_amd/build.py` "
        "or __graft_entry__.build() first" % LIB_PATH)

# PyTorch provides the device memory and streams handed to the library, so the library must run on
# the same HIP runtime instance as PyTorch.  Importing torch first makes the dynamic loader bind
# libsaf.so's libamdhip64.so.7 dependency to the runtime torch already loaded; loading libsaf.so
# first would map a second, separate runtime, to which torch's stream handles mean nothing.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes()) > 1:
    raise ImportError("more than one HIP runtime is mapped into this process (%s); import torch "
                      "before anything loads libsaf.so" % ", ".join(_hip_runtimes()))

SAF_OK, SAF_ERR_INVALID_ARG, SAF_ERR_UNSUPPORTED, SAF_ERR_HIP = 0, 1, 2, 3
SAF_F32, SAF_BF16 = 0, 1

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

_lib.saf_attn_fwd_workspace_size.argtypes = [_i, _i, _i, _i]
_lib.saf_attn_fwd_workspace_size.restype = _sz
_lib.saf_attn_bwd_workspace_size.argtypes = [_i, _i, _i, _i]
_lib.saf_attn_bwd_workspace_size.restype = _sz
_lib.saf_attn_bwd_ds_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i]
_lib.saf_attn_bwd_ds_workspace_size.restype = _sz
_lib.saf_calibrate_workspace_size.argtypes = [_i, _i, _i, _i]
_lib.saf_calibrate_workspace_size.restype = _sz
_lib.saf_last_error.argtypes = []
_lib.saf_last_error.restype = ctypes.c_char_p
_lib.saf_pattern_size.argtypes = [_i, _i]
_lib.saf_pattern_size.restype = _sz
_lib.saf_pattern_prepare.argtypes = [_i, _vp, _vp, _vp, _i, _vp, _sz, _vp]
_lib.saf_pattern_prepare.restype = _i
_lib.saf_attn_fwd.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp,
                              ctypes.c_float, _vp, _vp, _vp, _sz, _vp]
_lib.saf_attn_fwd.restype = _i
_lib.saf_attn_bwd.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                              _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.saf_attn_bwd.restype = _i
_lib.saf_attn_bwd_noalloc.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _i, _vp, ctypes.c_float, _vp, _vp, _vp, _vp]
_lib.saf_attn_bwd_noalloc.restype = _i
_lib.saf_attn_fwd_gqa.argtypes = [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp,
                                  ctypes.c_float, _vp, _vp, _vp, _sz, _vp]
_lib.saf_attn_fwd_gqa.restype = _i
_lib.saf_attn_bwd_gqa.argtypes = [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _i, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.saf_attn_bwd_gqa.restype = _i
_lib.saf_calibrate.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp,
                               _sz, _vp]
_lib.saf_calibrate.restype = _i
_lib.saf_attn_bwd_pattern_workspace_size.argtypes = [_i, _i, _i, _i]
_lib.saf_attn_bwd_pattern_workspace_size.restype = _sz
_lib.saf_attn_bwd_pattern.argtypes = [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                      _vp, _vp, _vp, _vp, _sz, _vp]
_lib.saf_attn_bwd_pattern.restype = _i
_lib.saf_fit_pattern_workspace_size.argtypes = [_i, _i]
_lib.saf_fit_pattern_workspace_size.restype = _sz
_lib.saf_fit_pattern.argtypes = [_i, _i, _vp, _i, ctypes.c_double, _vp, _vp, _vp, _vp, _vp, _sz,
                                 _vp]
_lib.saf_fit_pattern.restype = _i
_lib.saf_set_backward_overlap.argtypes = [_i]
_lib.saf_set_backward_overlap.restype = _i
_lib.saf_select_heads.argtypes = [_i, _i, _vp, _vp, ctypes.c_double, _vp, ctypes.POINTER(_i)]
_lib.saf_select_heads.restype = _i

# raw entry points, same names as the C ABI
saf_attn_fwd = _lib.saf_attn_fwd
saf_attn_bwd = _lib.saf_attn_bwd
saf_attn_fwd_gqa = _lib.saf_attn_fwd_gqa
saf_attn_bwd_gqa = _lib.saf_attn_bwd_gqa
saf_attn_bwd_noalloc = _lib.saf_attn_bwd_noalloc
saf_calibrate = _lib.saf_calibrate
saf_select_heads = _lib.saf_select_heads
saf_set_backward_overlap = _lib.saf_set_backward_overlap
saf_fit_pattern = _lib.saf_fit_pattern
saf_fit_pattern_workspace_size = _lib.saf_fit_pattern_workspace_size
saf_attn_bwd_pattern = _lib.saf_attn_bwd_pattern
saf_attn_bwd_pattern_workspace_size = _lib.saf_attn_bwd_pattern_workspace_size
saf_attn_fwd_workspace_size = _lib.saf_attn_fwd_workspace_size
saf_attn_bwd_workspace_size = _lib.saf_attn_bwd_workspace_size
saf_attn_bwd_ds_workspace_size = _lib.saf_attn_bwd_ds_workspace_size
saf_calibrate_workspace_size = _lib.saf_calibrate_workspace_size
saf_pattern_size = _lib.saf_pattern_size
saf_pattern_prepare = _lib.saf_pattern_prepare


def saf_last_error() -> str:
    return _lib.saf_last_error().decode()


class SafError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed (status %d): %s" % (where, status, saf_last_error()))


def _check(status, where):
    if status != SAF_OK:
        raise SafError(status, where)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SAF_BF16
    if t.dtype == torch.float32:
        return SAF_F32
    raise TypeError("tensors must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _mask(replaced, H):
    if len(replaced) != H:
        raise ValueError("replaced must have one entry per head (%d)" % H)
    return (ctypes.c_uint8 * H)(*[1 if int(x) else 0 for x in replaced])


def _stream(dev):
    import torch
    return torch.cuda.current_stream(dev).cuda_stream


def _ws(nbytes, device):
    import torch
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _expect(t, name, shape, dtype, device):
    """Raise ValueError unless t has exactly this shape, dtype and device.  The C ABI takes plain
    pointers and cannot check sizes: a tensor of another shape or element size would be read or
    written out of its bounds."""
    if t is None:
        raise ValueError("%s is required" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _expect_pattern(a, r, H, T, device):
    """a, r: fp32 [H, pat_len] with pat_len >= T on the device (rows of replaced heads are read)."""
    import torch
    if a is None or r is None:
        raise ValueError("a and r are required when a head is replaced")
    if a.dim() != 2 or a.shape[0] != H or a.shape[1] < T:
        raise ValueError("a has shape %s, expected [%d, pat_len >= %d]" % (tuple(a.shape), H, T))
    _expect(a, "a", (H, a.shape[1]), torch.float32, device)
    _expect(r, "r", tuple(a.shape), torch.float32, device)


def _expect_prepared(pattern, H, pat_len, device):
    import torch
    if pattern is None:
        return
    need = saf_pattern_size(H, pat_len)
    if pattern.dtype != torch.uint8 or pattern.dim() != 1 or pattern.numel() < need:
        raise ValueError("pattern must be a uint8 buffer of at least %d bytes (prepare_pattern)" % need)
    if pattern.device != device:
        raise ValueError("pattern is on %s, expected %s" % (pattern.device, device))


def prepare_pattern(replaced, a, r):
    """Prepared pattern of the replaced heads (a, r: [H, pat_len] fp32 on the GPU), to pass as
    `pattern=` to fwd / bwd with the same replaced, a and r.  Returns a uint8 device tensor."""
    import torch
    if a is None or a.dim() != 2:
        raise ValueError("a must be [H, pat_len]")
    H, P = a.shape
    _expect_pattern(a, r, H, P, a.device)
    n = saf_pattern_size(H, P)
    buf = torch.empty(max(n, 1), dtype=torch.uint8, device=a.device)
    st = saf_pattern_prepare(H, _mask(replaced, H), _ptr(a), _ptr(r), P, _ptr(buf), n,
                             _stream(a.device))
    _check(st, "saf_pattern_prepare")
    return buf


def fwd(q, k, v, replaced, a=None, r=None, scale=None, out=None, lse=None, pattern=None):
    """Forward of the mixed layer.  q: [B, H, T, d], k, v: [B, Hkv, T, d] (bf16 or fp32, same
    dtype; Hkv divides H, Hkv < H for grouped key/value heads), replaced: H flags, a, r:
    [H, pat_len] fp32 on the GPU, pattern: optional prepare_pattern() result.  Returns (o, lse).
    q and k may be None when every head is replaced (they are never read then)."""
    import torch
    if v is None or v.dim() != 4:
        raise ValueError("v must be [B, Hkv, T, d]")
    B, Hkv, T, d = v.shape
    H = q.shape[1] if q is not None else len(replaced)
    dt = _dtype_code(v)
    if any(not x for x in replaced) or q is not None:
        _expect(q, "q", (B, H, T, d), v.dtype, v.device)
        _expect(k, "k", (B, Hkv, T, d), v.dtype, v.device)
    if any(replaced):
        _expect_pattern(a, r, H, T, v.device)
        _expect_prepared(pattern, H, a.shape[1], v.device)
    if out is not None:
        _expect(out, "out", (B, H, T, d), v.dtype, v.device)
    if lse is not None:
        _expect(lse, "lse", (B, H, T), torch.float32, v.device)
    o = torch.empty((B, H, T, d), dtype=v.dtype, device=v.device) if out is None else out
    lse = torch.empty((B, H, T), dtype=torch.float32, device=v.device) if lse is None else lse
    ws_n = saf_attn_fwd_workspace_size(B, H, T, d)
    ws = _ws(ws_n, v.device)
    pat_len = a.shape[-1] if a is not None else 0
    st = saf_attn_fwd_gqa(dt, B, H, Hkv, T, d, _ptr(q), _ptr(k), _ptr(v), _mask(replaced, H),
                          _ptr(a), _ptr(r), pat_len, _ptr(pattern),
                          0.0 if scale is None else float(scale), _ptr(o), _ptr(lse), _ptr(ws),
                          ws_n, _stream(v.device))
    _check(st, "saf_attn_fwd")
    return o, lse


# Largest extra backward workspace bwd() allocates to keep dS between the two backward kernels.
DS_WORKSPACE_MAX = 16 << 30


def bwd(q, k, v, o, dout, lse, replaced, a=None, r=None, scale=None, pattern=None, keep_ds=True):
    """Backward of the mixed layer.  Returns (dq [B, H, T, d], dk, dv [B, Hkv, T, d]); replaced
    heads get dq = 0 and add nothing to dk.  keep_ds: pass the workspace of
    saf_attn_bwd_ds_workspace_size where the library keeps the ordinary heads' dS between its two
    backward kernels (bf16, d = 128, Hkv = H) and the extra room is at most DS_WORKSPACE_MAX bytes;
    False: the smaller workspace, with which dQ forms S and dP again."""
    import torch
    if v is None or v.dim() != 4 or dout is None or dout.dim() != 4:
        raise ValueError("v must be [B, Hkv, T, d] and dout [B, H, T, d]")
    B, Hkv, T, d = v.shape
    H = dout.shape[1]
    dt = _dtype_code(v)
    _expect(dout, "dout", (B, H, T, d), v.dtype, v.device)
    if any(not x for x in replaced) or q is not None:
        _expect(q, "q", (B, H, T, d), v.dtype, v.device)
        _expect(k, "k", (B, Hkv, T, d), v.dtype, v.device)
    if any(not x for x in replaced) or o is not None:
        _expect(o, "o", (B, H, T, d), v.dtype, v.device)
    _expect(lse, "lse", (B, H, T), torch.float32, v.device)
    if any(replaced):
        _expect_pattern(a, r, H, T, v.device)
        _expect_prepared(pattern, H, a.shape[1], v.device)
    dq = torch.empty_like(dout)
    dk, dv = torch.empty_like(v), torch.empty_like(v)
    ws_n = saf_attn_bwd_workspace_size(B, H, T, d)
    if keep_ds:
        n_rep = sum(1 for x in replaced if int(x))
        big = saf_attn_bwd_ds_workspace_size(dt, B, H, Hkv, T, d, n_rep)
        if ws_n < big <= ws_n + DS_WORKSPACE_MAX:
            ws_n = big
    ws = _ws(ws_n, v.device)
    pat_len = a.shape[-1] if a is not None else 0
    st = saf_attn_bwd_gqa(dt, B, H, Hkv, T, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                          _ptr(lse), _mask(replaced, H), _ptr(a), _ptr(r), pat_len, _ptr(pattern),
                          0.0 if scale is None else float(scale), _ptr(dq), _ptr(dk), _ptr(dv),
                          _ptr(ws), ws_n, _stream(v.device))
    _check(st, "saf_attn_bwd")
    return dq, dk, dv


def bwd_pattern(v, o, dout, lse, replaced, a, r, pattern=None, da=None, dr=None):
    """Gradient of a trained pattern: returns (da, dr) [H, pat_len] fp32; rows of replaced heads
    written (summed over the batch), rows of ordinary heads zero (fresh tensors) or untouched."""
    import torch
    if v is None or v.dim() != 4:
        raise ValueError("v must be [B, H, T, d]")
    B, H, T, d = v.shape
    dt = _dtype_code(v)
    _expect(o, "o", (B, H, T, d), v.dtype, v.device)
    _expect(dout, "dout", (B, H, T, d), v.dtype, v.device)
    _expect(lse, "lse", (B, H, T), torch.float32, v.device)
    _expect_pattern(a, r, H, T, v.device)
    pat_len = a.shape[-1]
    _expect_prepared(pattern, H, pat_len, v.device)
    if da is not None:
        _expect(da, "da", (H, pat_len), torch.float32, v.device)
    if dr is not None:
        _expect(dr, "dr", (H, pat_len), torch.float32, v.device)
    da = torch.zeros_like(a) if da is None else da
    dr = torch.zeros_like(r) if dr is None else dr
    ws_n = saf_attn_bwd_pattern_workspace_size(B, H, T, d)
    ws = _ws(ws_n, v.device)
    st = saf_attn_bwd_pattern(dt, B, H, T, d, _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                              _mask(replaced, H), _ptr(a), _ptr(r), pat_len, _ptr(pattern),
                              _ptr(da), _ptr(dr), _ptr(ws), ws_n, _stream(v.device))
    _check(st, "saf_attn_bwd_pattern")
    return da, dr


def calibrate(q, k, scale=None, kl=False):
    """Calibration statistics over N sequences: q, k [N, H, T, d].  Returns (ahat [H, T, T] fp32,
    svar [H] fp64), plus skl [H] fp64 (the forward-KL score) when kl is True."""
    import torch
    if q is None or q.dim() != 4:
        raise ValueError("q must be [N, H, T, d]")
    N, H, T, d = q.shape
    dt = _dtype_code(q)
    _expect(k, "k", (N, H, T, d), q.dtype, q.device)
    ahat = torch.empty((H, T, T), dtype=torch.float32, device=q.device)
    svar = torch.empty((H,), dtype=torch.float64, device=q.device)
    skl = torch.empty((H,), dtype=torch.float64, device=q.device) if kl else None
    ws_n = saf_calibrate_workspace_size(N, H, T, d)
    ws = _ws(ws_n, q.device)
    st = saf_calibrate(dt, N, H, T, d, _ptr(q), _ptr(k), 0.0 if scale is None else float(scale),
                       _ptr(ahat), _ptr(svar), _ptr(skl) if kl else None, _ptr(ws), ws_n,
                       _stream(q.device))
    _check(st, "saf_calibrate")
    return (ahat, svar, skl) if kl else (ahat, svar)


def fit_pattern(ahat, steps=400, lr=0.1):
    """Compact fit of target maps ahat [H, T, T] fp32 (GPU).  Returns (a [H, T], r [H, T] fp32,
    kl [H] fp64 mean row KL, loss [H] fp64)."""
    import torch
    if ahat is None or ahat.dim() != 3 or ahat.shape[1] != ahat.shape[2]:
        raise ValueError("ahat must be [H, T, T]")
    if ahat.dtype != torch.float32:
        raise ValueError("ahat has dtype %s, expected torch.float32" % ahat.dtype)
    H, T, _ = ahat.shape
    a = torch.empty((H, T), dtype=torch.float32, device=ahat.device)
    r = torch.empty_like(a)
    kl = torch.empty((H,), dtype=torch.float64, device=ahat.device)
    loss = torch.empty_like(kl)
    ws_n = saf_fit_pattern_workspace_size(H, T)
    ws = _ws(ws_n, ahat.device)
    st = saf_fit_pattern(H, T, _ptr(ahat), int(steps), float(lr), _ptr(a), _ptr(r), _ptr(kl),
                         _ptr(loss), _ptr(ws), ws_n, _stream(ahat.device))
    _check(st, "saf_fit_pattern")
    return a, r, kl, loss


def select_heads(score, ratio, accepted=None):
    """Head selection over a model: score [L, H] (host), ratio r.  Returns (replaced [L, H] uint8
    numpy array, number selected).  Host-only library call (no GPU work)."""
    import numpy as np
    sc = np.ascontiguousarray(np.asarray(score, dtype=np.float64))
    L, H = sc.shape
    acc = None if accepted is None else np.ascontiguousarray(np.asarray(accepted, dtype=np.uint8))
    out = np.zeros((L, H), dtype=np.uint8)
    n = ctypes.c_int(0)
    st = saf_select_heads(L, H, sc.ctypes.data, None if acc is None else acc.ctypes.data,
                          float(ratio), out.ctypes.data, ctypes.byref(n))
    _check(st, "saf_select_heads")
    return out, n.value


# ------------------------------------------------------------------ per-kernel timing (profiling)
class SafKernelEvent(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("start", _vp), ("stop", _vp)]


_lib.saf_trace_begin.argtypes = [ctypes.POINTER(SafKernelEvent), _i]
_lib.saf_trace_begin.restype = _i
_lib.saf_trace_end.argtypes = []
_lib.saf_trace_end.restype = _i
saf_trace_begin = _lib.saf_trace_begin
saf_trace_end = _lib.saf_trace_end

# The HIP runtime torch loaded (same SONAME, so dlopen returns the instance already mapped).
_hip = ctypes.CDLL("libamdhip64.so.7")
_hip.hipEventCreate.argtypes = [ctypes.POINTER(_vp)]
_hip.hipEventCreate.restype = _i
_hip.hipEventDestroy.argtypes = [_vp]
_hip.hipEventDestroy.restype = _i
_hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
_hip.hipEventElapsedTime.restype = _i


class KernelTrace:
    """Times every kernel the library launches between begin() and end() with HIP events recorded
    on the launching stream (saf_trace_begin / saf_trace_end).  Accumulates per-kernel durations
    over many begin/end rounds; read them after the stream has completed."""

    def __init__(self, capacity=16):
        self.cap = capacity
        self.ev = (SafKernelEvent * capacity)()
        for e in self.ev:
            for f in ("start", "stop"):
                h = _vp()
                if _hip.hipEventCreate(ctypes.byref(h)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                setattr(e, f, h)
        self.samples = {}
        self._n = 0

    def begin(self):
        _check(saf_trace_begin(self.ev, self.cap), "saf_trace_begin")

    def end(self):
        """Stop recording; must be followed by a stream synchronisation before collect()."""
        self._n = saf_trace_end()

    def collect(self):
        ms = ctypes.c_float()
        for e in self.ev[:self._n]:
            if _hip.hipEventElapsedTime(ctypes.byref(ms), e.start, e.stop) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            self.samples.setdefault(e.name.decode(), []).append(ms.value)
        self._n = 0

    def summary(self):
        return {k: {"launches": len(v), "avg_ms": sum(v) / len(v), "total_ms": sum(v)}
                for k, v in self.samples.items()}

    def close(self):
        for e in self.ev:
            _hip.hipEventDestroy(e.start)
            _hip.hipEventDestroy(e.stop)
