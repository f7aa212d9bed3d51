"""fp64 CPU oracle for the mixed-head SAF attention layer (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this package.
The GPU product path never imports it and has no fallback to it.  The arithmetic lives in
``saf_oracle.c`` (plain loops in fp64, one (batch, head) slice at a time); this module only
marshals arrays and loops over heads.

Citations:
  [Notes]      the page "When Can Attention Heads Be Statically Defined?：中文精读笔记".
  [Paper page] the page "When Can Attention Heads Be Statically Defined?" (tables and captions).

What it computes:
  ordinary head   softmax_causal(s Q K^T) V, s = 1/sqrt(d) unless given     [Notes §一]
  replaced head   P(i,j) = exp(a[j] + r[i-j]) / Z(i), causal, then P V       [Notes §二.3, Eq.(3)]
  backward        ordinary: dq, dk, dv; replaced: dv = P^T dO, dq = dk = 0   [Notes §二.4]
  calibration     Ahat = mean_n A^(n), s_var = sum_n ||A^(n)-Ahat||_F^2 / ((N-1) T^2)
                                                                             [Notes §二.1, Eq.(1)]
  KL score        mean_n,i KL(A^(n)_i || Ahat_i) (the alternative selector)  [Notes §二.1]
  head selection  ascending score across layers, k = round(r L H)            [Notes §二.1]
  pattern grad    dL/da, dL/dr when a replaced head's pattern is trained     [Paper page] Table 14
  compact fit     Adam on the row-wise cross-entropy to Ahat                 [Notes §二.3]
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "saf_oracle.c")
_LIB = os.path.join(_HERE, "_saf_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def build(force: bool = False) -> str:
    """Compile the oracle library with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp,
                        "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Lib:
    """ctypes view of one compiled oracle library (the default one, or a test's variant)."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        lib.orc_head_fwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp,
                                     _dp, ctypes.c_double, ctypes.c_int, _ip, _dp, _dp]
        lib.orc_head_pattern.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp,
                                         _dp, ctypes.c_double, _dp]
        lib.orc_head_bwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp,
                                     _dp, _dp, ctypes.c_double, ctypes.c_int, _ip, _dp,
                                     ctypes.c_int, _ip, _dp, _dp]
        lib.orc_head_calibrate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp,
                                           ctypes.c_double, ctypes.c_int, _ip, _dp, _dp]
        lib.orc_calibrate_maps.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        lib.orc_head_kl_score.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp,
                                          ctypes.c_double, ctypes.c_int, _ip, _dp]
        lib.orc_kl_maps.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp]
        lib.orc_head_pattern_grad.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp,
                                              _dp, _dp]
        lib.orc_fit_loss_grad.argtypes = [ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.orc_fit_pattern.argtypes = [ctypes.c_int, _dp, ctypes.c_int, ctypes.c_double, _dp,
                                        _dp, _dp, _dp]
        lib.orc_num_threads.argtypes = []
        for f in (lib.orc_head_fwd, lib.orc_head_pattern, lib.orc_head_bwd,
                  lib.orc_head_calibrate, lib.orc_calibrate_maps, lib.orc_head_kl_score,
                  lib.orc_kl_maps, lib.orc_head_pattern_grad, lib.orc_fit_loss_grad,
                  lib.orc_fit_pattern, lib.orc_num_threads):
            f.restype = ctypes.c_int
        self.c = lib


_active = None


def _load():
    global _active
    if _active is None:
        build()
        _active = _Lib(_LIB)
    return _active.c


def use_library(path):
    """Point this module at another compiled copy of the oracle (the mutant tests use this to
    show that the pins reject a planted mistake).  Pass None to return to the default library."""
    global _active
    _active = None if path is None else _Lib(path)


def compile_source(src_text, out_path):
    """Compile C source text (a copy of the oracle, possibly altered by a test) to out_path."""
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", c_path, "-o",
                    out_path, "-lm"], check=True, capture_output=True)
    return out_path


def source_text():
    with open(_SRC) as f:
        return f.read()


def _f64(x):
    """Exact widening to a C-contiguous fp64 numpy array (bf16 / fp32 torch tensors included)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: widen on the CPU, exactly
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x):
    return None if x is None else x.ctypes.data_as(_dp)


def _rows(rows, T):
    rows = np.arange(T, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    return rows, rows.ctypes.data_as(_ip)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle rejected the arguments of " + what)


def num_threads():
    """Threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


# ------------------------------------------------------------------------------ one head slice
def head_fwd(kind, v, q=None, k=None, a=None, r=None, scale=None, rows=None):
    """Forward rows of one head.  kind 0 = ordinary (q, k), 1 = replaced (a, r).
    Returns (o [nrows, d], lse [nrows])."""
    lib = _load()
    v = _f64(v)
    T, d = v.shape
    q, k, a, r = _f64(q), _f64(k), _f64(a), _f64(r)
    if a is not None:
        a, r = a[:T].copy(), r[:T].copy()  # the pattern's prefix serves a shorter input
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows, rp = _rows(rows, T)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    _check(lib.orc_head_fwd(kind, T, d, _p(q), _p(k), _p(v), _p(a), _p(r), scale, len(rows), rp,
                            _p(o), _p(lse)), "head_fwd")
    return o, lse


def head_pattern(kind, T, q=None, k=None, a=None, r=None, scale=None):
    """Dense causal pattern [T, T] of one head (tiny T only)."""
    lib = _load()
    q, k, a, r = _f64(q), _f64(k), _f64(a), _f64(r)
    d = q.shape[1] if q is not None else 1
    if a is not None:
        a, r = a[:T].copy(), r[:T].copy()
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    P = np.zeros((T, T))
    _check(lib.orc_head_pattern(kind, T, d, _p(q), _p(k), _p(a), _p(r), scale, _p(P)),
           "head_pattern")
    return P


def head_bwd(kind, v, dout, q=None, k=None, a=None, r=None, scale=None, qrows=None, krows=None,
             want_dq=True, want_dk=True, want_dv=True):
    """Backward rows of one head.  Returns (dq [nq, d] or None, dk [nk, d] or None, dv or None)."""
    lib = _load()
    v, dout = _f64(v), _f64(dout)
    T, d = v.shape
    q, k, a, r = _f64(q), _f64(k), _f64(a), _f64(r)
    if a is not None:
        a, r = a[:T].copy(), r[:T].copy()
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    qrows, qp = _rows(qrows, T)
    krows, kp = _rows(krows, T)
    dq = np.zeros((len(qrows), d)) if want_dq else None
    dk = np.zeros((len(krows), d)) if want_dk else None
    dv = np.zeros((len(krows), d)) if want_dv else None
    _check(lib.orc_head_bwd(kind, T, d, _p(q), _p(k), _p(v), _p(dout), _p(a), _p(r), scale,
                            len(qrows), qp, _p(dq), len(krows), kp, _p(dk), _p(dv)), "head_bwd")
    return dq, dk, dv


def head_calibrate(q, k, scale=None, rows=None, want_ahat=True):
    """Calibration rows of one head from q, k [N, T, d].  Returns (ahat [nrows, T] or None,
    dev [nrows]) with dev the per-row sum over n and j of (A^(n) - Ahat)^2."""
    lib = _load()
    q, k = _f64(q), _f64(k)
    N, T, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows, rp = _rows(rows, T)
    ahat = np.zeros((len(rows), T)) if want_ahat else None
    dev = np.zeros(len(rows))
    _check(lib.orc_head_calibrate(N, T, d, _p(q), _p(k), scale, len(rows), rp, _p(ahat),
                                  _p(dev)), "head_calibrate")
    return ahat, dev


def calibrate_maps(maps):
    """Eq. (1) from dense maps [N, T, T].  Returns (ahat [T, T], s_var)."""
    lib = _load()
    maps = _f64(maps)
    N, T, _ = maps.shape
    ahat = np.zeros((T, T))
    sv = ctypes.c_double(0.0)
    _check(lib.orc_calibrate_maps(N, T, _p(maps), _p(ahat), ctypes.byref(sv)), "calibrate_maps")
    return ahat, sv.value


def head_kl_score(q, k, scale=None, rows=None):
    """Row-wise forward-KL terms of one head from q, k [N, T, d]: kl[x] = sum_n KL(A^(n)_i ||
    Ahat_i) for row i = rows[x]; the head's score is kl.sum() / (N T) over all rows."""
    lib = _load()
    q, k = _f64(q), _f64(k)
    N, T, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows, rp = _rows(rows, T)
    kl = np.zeros(len(rows))
    _check(lib.orc_head_kl_score(N, T, d, _p(q), _p(k), scale, len(rows), rp, _p(kl)),
           "head_kl_score")
    return kl


def kl_maps(maps):
    """Forward-KL score from dense maps [N, T, T]."""
    lib = _load()
    maps = _f64(maps)
    N, T, _ = maps.shape
    out = ctypes.c_double(0.0)
    _check(lib.orc_kl_maps(N, T, _p(maps), ctypes.byref(out)), "kl_maps")
    return out.value


def head_pattern_grad(v, dout, a, r):
    """dL/da, dL/dr [T] of one replaced-head slice (v, dout [T, d]; a, r at least T long)."""
    lib = _load()
    v, dout = _f64(v), _f64(dout)
    T, d = v.shape
    a, r = _f64(a)[:T].copy(), _f64(r)[:T].copy()
    da, dr = np.zeros(T), np.zeros(T)
    _check(lib.orc_head_pattern_grad(T, d, _p(v), _p(dout), _p(a), _p(r), _p(da), _p(dr)),
           "head_pattern_grad")
    return da, dr


def fit_loss_grad(ahat, a, r):
    """Mean row cross-entropy of the pattern (a, r) against ahat [T, T] and its gradient."""
    lib = _load()
    ahat = _f64(ahat)
    T = ahat.shape[0]
    a, r = _f64(a), _f64(r)
    ga, gr = np.zeros(T), np.zeros(T)
    loss = ctypes.c_double(0.0)
    _check(lib.orc_fit_loss_grad(T, _p(ahat), _p(a), _p(r), ctypes.byref(loss), _p(ga), _p(gr)),
           "fit_loss_grad")
    return loss.value, ga, gr


def fit_pattern(ahat, steps=400, lr=0.05):
    """Compact fit of one target pattern ahat [T, T].  Returns (a, r, loss, mean row KL)."""
    lib = _load()
    ahat = _f64(ahat)
    T = ahat.shape[0]
    a, r = np.zeros(T), np.zeros(T)
    loss, kl = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(lib.orc_fit_pattern(T, _p(ahat), int(steps), float(lr), _p(a), _p(r),
                               ctypes.byref(loss), ctypes.byref(kl)), "fit_pattern")
    return a, r, loss.value, kl.value


def select_heads(score, ratio, accepted=None):
    """Head selection ([Notes §二.1]): every head of every layer ranked by ascending score, ties
    by (layer, head); k = round(ratio * L * H) with halves to even (Python's round); the first k
    ranked heads that are accepted (all when accepted is None) are selected.  score [L, H].
    Returns (replaced [L, H] uint8, number selected)."""
    score = np.asarray(score, dtype=np.float64)
    L, H = score.shape
    k = round(ratio * L * H)
    ranked = sorted((float(score[l, h]), l, h) for l in range(L) for h in range(H))
    out = np.zeros((L, H), dtype=np.uint8)
    taken = 0
    for _, l, h in ranked:
        if taken == k:
            break
        if accepted is None or accepted[l][h]:
            out[l, h] = 1
            taken += 1
    return out, taken


# ------------------------------------------------------------------------------ whole layer
def _heads(B, H, heads):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def layer_fwd(q, k, v, replaced, a, r, scale=None, heads=None, rows=None):
    """Forward of the mixed layer, tensors [B, H, T, d]; replaced[h] = 1 for a fixed head.
    Returns {(b, h): (o, lse)} for the listed (b, h) slices (all when heads is None)."""
    B, H, T, d = v.shape
    out = {}
    for b, h in _heads(B, H, heads):
        if replaced[h]:
            out[(b, h)] = head_fwd(1, v[b, h], a=a[h], r=r[h], rows=rows)
        else:
            out[(b, h)] = head_fwd(0, v[b, h], q=q[b, h], k=k[b, h], scale=scale, rows=rows)
    return out


def layer_bwd(q, k, v, dout, replaced, a, r, scale=None, heads=None, qrows=None, krows=None):
    """Backward of the mixed layer.  Returns {(b, h): (dq, dk, dv)}."""
    B, H, T, d = v.shape
    out = {}
    for b, h in _heads(B, H, heads):
        if replaced[h]:
            out[(b, h)] = head_bwd(1, v[b, h], dout[b, h], a=a[h], r=r[h], qrows=qrows,
                                   krows=krows)
        else:
            out[(b, h)] = head_bwd(0, v[b, h], dout[b, h], q=q[b, h], k=k[b, h], scale=scale,
                                   qrows=qrows, krows=krows)
    return out


def layer_fwd_gqa(q, k, v, replaced, a, r, scale=None, heads=None, rows=None):
    """Forward with grouped key/value heads: q [B, H, T, d], k, v [B, Hkv, T, d]; query head h
    reads key/value head h // (H // Hkv) ([Notes §二.4]: a replaced head still reads the V it
    shares).  Returns {(b, h): (o, lse)}."""
    B, H = q.shape[0], q.shape[1]
    G = H // k.shape[1]
    out = {}
    for b, h in _heads(B, H, heads):
        hk = h // G
        if replaced[h]:
            out[(b, h)] = head_fwd(1, v[b, hk], a=a[h], r=r[h], rows=rows)
        else:
            out[(b, h)] = head_fwd(0, v[b, hk], q=q[b, h], k=k[b, hk], scale=scale, rows=rows)
    return out


def layer_bwd_gqa(q, k, v, dout, replaced, a, r, scale=None, batches=None, kv_heads=None,
                  qrows=None, krows=None):
    """Backward with grouped key/value heads.  dq per query head; dk, dv per key/value head, the
    sums over the query heads of its group (a replaced head adds to dv only).  Returns
    (dq {(b, h)}, dk {(b, hk)}, dv {(b, hk)}) for the listed batches and key/value heads."""
    B, H = q.shape[0], q.shape[1]
    Hkv = k.shape[1]
    G = H // Hkv
    dq, dk, dv = {}, {}, {}
    for b in (range(B) if batches is None else batches):
        for hk in (range(Hkv) if kv_heads is None else kv_heads):
            sk, sv = None, None
            for h in range(hk * G, (hk + 1) * G):
                if replaced[h]:
                    x = head_bwd(1, v[b, hk], dout[b, h], a=a[h], r=r[h], qrows=qrows, krows=krows)
                else:
                    x = head_bwd(0, v[b, hk], dout[b, h], q=q[b, h], k=k[b, hk], scale=scale,
                                 qrows=qrows, krows=krows)
                dq[(b, h)] = x[0]
                sk = x[1] if sk is None else sk + x[1]
                sv = x[2] if sv is None else sv + x[2]
            dk[(b, hk)], dv[(b, hk)] = sk, sv
    return dq, dk, dv


def pattern_grad(v, dout, replaced, a, r, heads=None):
    """dL/da, dL/dr of the replaced heads, summed over batch: {h: (da [T], dr [T])}."""
    B, H, T, d = v.shape
    out = {}
    for h in (range(H) if heads is None else heads):
        if not replaced[h]:
            continue
        da, dr = np.zeros(T), np.zeros(T)
        for b in range(B):
            x, y = head_pattern_grad(v[b, h], dout[b, h], a[h], r[h])
            da += x
            dr += y
        out[h] = (da, dr)
    return out


def kl_score(q, k, scale=None, heads=None):
    """Forward-KL score per head over N sequences, q, k [N, H, T, d]: {h: s_kl}."""
    N, H, T, d = q.shape
    return {h: float(head_kl_score(q[:, h], k[:, h], scale=scale).sum()) / (N * T)
            for h in (range(H) if heads is None else heads)}


def calibrate(q, k, scale=None, heads=None, rows=None):
    """Calibration over N sequences, q, k [N, H, T, d].  Returns {h: (ahat_rows, s_var or None)}:
    s_var is given only when every row is computed."""
    N, H, T, d = q.shape
    out = {}
    for h in (range(H) if heads is None else heads):
        ahat, dev = head_calibrate(q[:, h], k[:, h], scale=scale, rows=rows)
        sv = float(dev.sum()) / ((N - 1) * T * T) if rows is None else None
        out[h] = (ahat, sv)
    return out
