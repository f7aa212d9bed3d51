"""Helpers of the GPU parity tests: run the HIP path through the binding, the oracle on the same
inputs, and compare (normwise per head slice, as max|x - y| / max|y|)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
# Row log-normalisers: fp32 arithmetic, but on the bf16 path the normaliser is the sum of the
# probabilities after their rounding to bf16 (unit roundoff 2^-8: relative error <= 2^-8 per term,
# hence in the sum), so |d lse| <= log(1 + 2^-8) < 2^-8 there.
TOL_LSE = {torch.float32: 1e-4, torch.bfloat16: 2.0 ** -8}


def cpu64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def norm_err(got, ref, floor=0.0):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    den = max(float(np.abs(ref).max()), floor, 1e-300)
    return float(np.abs(got - ref).max()) / den


def rel_l2(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def sample_rows(T, n, seed=0):
    """n row indices of [0, T): always 0 and T-1, the rest drawn without replacement."""
    if T <= n:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], rest])).astype(np.int32)


def pick_heads(B, replaced, n_each=1):
    """A few (b, h) slices covering both head kinds and the first / last batch entries."""
    ords = [h for h, x in enumerate(replaced) if not x]
    reps = [h for h, x in enumerate(replaced) if x]
    out = []
    for i in range(n_each):
        if ords:
            out.append((0 if i % 2 == 0 else B - 1, ords[(i * 5) % len(ords)]))
        if reps:
            out.append((B - 1 if i % 2 == 0 else 0, reps[(i * 3) % len(reps)]))
    return sorted(set(out))


def check_fwd(x, o, lse, heads, rows, tol, what=""):
    """Compare o / lse of the listed (b, h) slices and rows with the oracle."""
    worst = 0.0
    rows = np.arange(x.v.shape[2], dtype=np.int32) if rows is None else rows
    G = len(x.replaced) // x.v.shape[1]  # query heads per key/value head (1 unless grouped)
    for b, h in heads:
        hk = h // G
        if x.replaced[h]:
            ro, rl = oracle.head_fwd(1, x.v[b, hk], a=x.a[h], r=x.r[h], rows=rows)
        else:
            ro, rl = oracle.head_fwd(0, x.v[b, hk], q=x.q[b, h], k=x.k[b, hk], rows=rows)
        idx = torch.as_tensor(rows, dtype=torch.long, device=o.device)
        e = norm_err(cpu64(o[b, h].index_select(0, idx)), ro)
        el = norm_err(cpu64(lse[b, h].index_select(0, idx)), rl, floor=1.0)
        assert e <= tol, "%s o[b=%d,h=%d] normwise error %.3e > %.1e" % (what, b, h, e, tol)
        tl = TOL_LSE[o.dtype]
        assert el <= tl, "%s lse[b=%d,h=%d] error %.3e > %.1e" % (what, b, h, el, tl)
        worst = max(worst, e)
    return worst


def check_bwd(x, dq, dk, dv, heads, qrows, krows, tol, what=""):
    worst = 0.0
    T = x.v.shape[2]
    qrows = np.arange(T, dtype=np.int32) if qrows is None else qrows
    krows = np.arange(T, dtype=np.int32) if krows is None else krows
    for b, h in heads:
        kind = 1 if x.replaced[h] else 0
        rq, rk, rv = oracle.head_bwd(kind, x.v[b, h], x.dout[b, h], q=x.q[b, h], k=x.k[b, h],
                                     a=x.a[h], r=x.r[h], qrows=qrows, krows=krows)
        iq = torch.as_tensor(qrows, dtype=torch.long, device=dq.device)
        ik = torch.as_tensor(krows, dtype=torch.long, device=dq.device)
        gq = cpu64(dq[b, h].index_select(0, iq))
        gk = cpu64(dk[b, h].index_select(0, ik))
        gv = cpu64(dv[b, h].index_select(0, ik))
        if kind == 1:
            assert np.all(gq == 0.0) and np.all(gk == 0.0), "%s replaced dq/dk must be 0" % what
        else:
            for name, g, r in (("dq", gq, rq), ("dk", gk, rk)):
                # At T = 1 an ordinary head's dq and dk vanish by cancellation (P = 1, so
                # dS = dP - delta = 0 exactly); the GPU's dP - delta is a rounding residue, and a
                # reference of exact zeros has no relative scale: compare on the inputs' unit scale.
                e = norm_err(g, r, floor=1.0 if np.abs(r).max() == 0.0 else 0.0)
                assert e <= tol, "%s %s[b=%d,h=%d] normwise error %.3e > %.1e" % (what, name, b, h, e, tol)
                worst = max(worst, e)
        e = norm_err(gv, rv)
        assert e <= tol, "%s dv[b=%d,h=%d] normwise error %.3e > %.1e" % (what, b, h, e, tol)
        worst = max(worst, e)
    return worst
