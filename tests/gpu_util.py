"""Helpers of the GPU parity tests: run the HIP path through the binding, the oracle on the same
inputs, and compare.

The comparison is row by row: an output row (a query row of O or dQ, a key row of dK or dV, a row
of the mean map) is judged on its own scale, max_j |x_ij - y_ij| / max_j |y_ij|, so that late rows,
whose entries are averages over thousands of keys and an order of magnitude smaller than the first
rows, are held to the same relative bound.  rel-L2 = ||x - y||_2 / ||y||_2 is asserted per (b, h)
slice as well, the second error measure of the pages' own kernel check ([Paper page] Table 28).
Row log-normalisers (lse) are bounded in absolute terms.  Three scales replace a row's own one
where the arithmetic fixes a different one:
  - a reference row of exact zeros is a structural zero of the method (an ordinary head's dQ at row
    0, where P = 1 and dS = 0; every row at T = 1): the GPU's value there is a rounding residue of
    dP - delta, measured on the inputs' unit scale (the test tensors are N(0, 1));
  - terms below 2^-126 (the smallest normal of fp32 and bf16) are flushed to zero on the GPU, so a
    row of T such terms is lost whole: rows are measured against at least the most those terms can
    add up to, T 2^-126 max|x| (|x| <= 16 for the N(0, 1) test tensors), divided by the tolerance;
  - dQ_i = s sum_j dS_ij K_j and dK_j = s sum_i dS_ij Q_i with dS = P o (dP - delta) sum terms
    that cancel (sum_j dS_ij = 0), and three roundings enter them: dS is rounded to bf16 (unit
    roundoff 2^-8) before the matrix product; the forward normalises each row by the sum of its
    probabilities as rounded for its P V product, which defines lse and O, while the backward
    re-forms P from lse unrounded; and delta_i = dO_i . O_i is taken from O as stored in the tensor
    type (as FlashAttention does).  Each error is at most a few unit roundoffs of the uncancelled
    terms, so a row with few terms (the first queries of dQ, the last keys of dK) can miss its own
    scale while the arithmetic is as exact as it can be.  A row that fails its own scale is judged
    again against its uncancelled scale, computed for that row from the oracle's P, dP and O:
    s max_c sum_j P_ij (|dP_ij| + |delta|_i) |K_jc| (dQ), s max_c sum_i P_ij (|dP_ij| + |delta|_i)
    |Q_ic| (dK), with |delta|_i = sum_e |dO_ie O_ie| (delta is itself a sum over the d channels
    of products with the rounded O).  Such a row enters the slice's rel-L2 with that scale as its
    norm.  The number of rows judged that way is reported.
With SAF_PARITY_REPORT set to a file path, every check appends one JSON line with the worst row
error and rel-L2 it saw (the figures quoted in the design notes come from such a report).
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
# Row log-normalisers, absolute: fp32 arithmetic, but on the bf16 path the normaliser is the sum of
# the probabilities after their rounding to bf16 (unit roundoff 2^-8: relative error <= 2^-8 per
# term, hence in the sum), so |d lse| <= log(1 + 2^-8) < 2^-8 there.
TOL_LSE = {torch.float32: 1e-4, torch.bfloat16: 2.0 ** -8}
UNIT_SCALE = 1.0  # scale of the N(0, 1) test tensors: the measure of a structurally zero row
FLUSH = 2.0 ** -126  # smallest normal fp32 / bf16 value; smaller terms are flushed on the GPU
X_MAX = 16.0  # bound on |x| of the N(0, 1) test tensors (at most 2^26 samples per tensor)


def flush_floor(T, tol):
    """Row scale below which a row's terms may all have been flushed (see the module notes)."""
    return FLUSH * T * X_MAX / tol


def cpu64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def row_err(got, ref, scale=None, floor=0.0):
    """Per-row error of 2-D arrays [rows, cols]: max_j |x - y| / max(max_j |y|, scale, floor) for
    each row (a row whose reference is exactly zero is measured against UNIT_SCALE)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return np.zeros(got.shape[:1])
    got, ref = got.reshape(got.shape[0], -1), ref.reshape(ref.shape[0], -1)
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den == 0.0, UNIT_SCALE, den)
    if scale is not None:
        den = np.maximum(den, np.asarray(scale, np.float64))
    return num / np.maximum(den, floor)


def vec_err(got, ref):
    """Normwise error of a whole vector (the pattern gradient of a head is one vector over
    positions): max |x - y| / max |y|."""
    return float(row_err(np.asarray(got)[None, :], np.asarray(ref)[None, :])[0])


def rel_l2(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else UNIT_SCALE))


class Worst:
    """Running worst errors of one test, reported at the end (and to SAF_PARITY_REPORT)."""

    def __init__(self, name):
        self.name = name
        self.row = 0.0
        self.l2 = 0.0
        self.lse = 0.0
        self.where = ""
        self.n_rows = 0
        self.n_rescaled = 0

    def add(self, got, ref, tol, what, scale=None, T=None, rows=None, rounding=None):
        """Check one slice: every row within tol (row scales as in the module notes; T, when
        given, is the number of terms a row sums, for the flush floor).  rounding(row numbers)
        gives the uncancelled scale of rows that fail their own scale (rows: the row number of
        each checked row)."""
        floor = flush_floor(T, tol) if T else 0.0
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        e = row_err(got, ref, scale, floor)
        bad = np.nonzero(e > tol)[0]
        r = rel_l2(got, ref)
        if bad.size and rounding is not None:
            rn = np.arange(len(e)) if rows is None else np.asarray(rows)
            sc = rounding(rn[bad])
            e = e.copy()
            e[bad] = row_err(got[bad], ref[bad], sc, floor)
            self.n_rescaled += int(bad.size)
            g2, r2 = got.reshape(len(e), -1), ref.reshape(len(e), -1)
            nrm2 = (r2 ** 2).sum(axis=1)
            nrm2[bad] = np.maximum(nrm2[bad], sc ** 2 * r2.shape[1])
            r = float(np.sqrt(((g2 - r2) ** 2).sum() / max(nrm2.sum(), 1e-300)))
        worst_i = int(np.argmax(e)) if e.size else 0
        worst = float(e.max()) if e.size else 0.0
        assert worst <= tol, "%s %s: row %d error %.3e > %.1e" % (self.name, what, worst_i, worst, tol)
        assert r <= tol, "%s %s: rel-L2 %.3e > %.1e" % (self.name, what, r, tol)
        self.n_rows += e.size
        if worst > self.row:
            self.row, self.where = worst, what
        self.l2 = max(self.l2, r)
        return worst

    def add_lse(self, got, ref, tol, what):
        got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        e = float(np.abs(got - ref).max()) if got.size else 0.0
        assert e <= tol, "%s %s: |d lse| %.3e > %.1e" % (self.name, what, e, tol)
        self.lse = max(self.lse, e)

    def report(self, **extra):
        line = {"test": self.name, "worst_row_err": self.row, "worst_rel_l2": self.l2,
                "worst_abs_lse": self.lse, "worst_at": self.where, "rows_checked": self.n_rows,
                "rows_on_rounding_scale": self.n_rescaled}
        line.update(extra)
        print("parity", json.dumps(line), flush=True)
        path = os.environ.get("SAF_PARITY_REPORT")
        if path:
            with open(path, "a") as f:
                f.write(json.dumps(line) + "\n")
        return line


def sample_rows(T, n, seed=0):
    """n row indices of [0, T): always 0 and T-1, the rest drawn without replacement."""
    if T <= n:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], rest])).astype(np.int32)


def all_heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


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


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy() if hasattr(t, "detach") else np.asarray(t, np.float64)


def dq_uncancelled_scale(q, k, v, dout, rows, scale=None):
    """s max_c sum_j P_ij (|dP_ij| + |delta_i|) |K_jc| for the listed query rows of one ordinary
    head (q, k, v, dout [T, d]), from the oracle's O and lse of those rows (module notes)."""
    o, lse = oracle.head_fwd(0, v, q=q, k=k, rows=rows, scale=scale)
    Q, K, V, G = _f64(q), _f64(k), _f64(v), _f64(dout)
    s = 1.0 / np.sqrt(Q.shape[1]) if scale is None else scale
    out = np.zeros(len(rows))
    for x, i in enumerate(rows):
        p = np.exp(s * (K[:i + 1] @ Q[i]) - lse[x])
        w = p * (np.abs(V[:i + 1] @ G[i]) + np.abs(G[i] * o[x]).sum())
        out[x] = s * (w @ np.abs(K[:i + 1])).max()
    return out


def dk_uncancelled_scale(q, k, v, dout, keys, scale=None):
    """s max_c sum_i P_ij (|dP_ij| + |delta_i|) |Q_ic| for the listed key rows of one ordinary
    head, from the oracle's O and lse of the query rows that see them (module notes)."""
    T = _f64(v).shape[0]
    j0 = int(min(keys))
    qrows = np.arange(j0, T, dtype=np.int32)
    o, lse = oracle.head_fwd(0, v, q=q, k=k, rows=qrows, scale=scale)
    Q, K, V, G = _f64(q), _f64(k), _f64(v), _f64(dout)
    s = 1.0 / np.sqrt(Q.shape[1]) if scale is None else scale
    delta = np.abs(G[j0:] * o).sum(axis=1)
    out = np.zeros(len(keys))
    for x, j in enumerate(keys):
        sl = slice(j - j0, T - j0)
        p = np.exp(s * (Q[j:] @ K[j]) - lse[sl])
        w = p * (np.abs(G[j:] @ V[j]) + delta[sl])
        out[x] = s * (w @ np.abs(Q[j:])).max()
    return out


def check_fwd(x, o, lse, heads, rows, tol, what="", worst=None):
    """Compare o / lse of the listed (b, h) slices and rows with the oracle, row by row.
    o, lse may be GPU or CPU tensors."""
    wr = Worst(what) if worst is None else worst
    T = x.v.shape[2]
    rows = np.arange(T, dtype=np.int32) if rows is None else rows
    G = len(x.replaced) // x.v.shape[1]  # query heads per key/value head (1 unless grouped)
    idx = torch.as_tensor(rows, dtype=torch.long, device=o.device)
    for b, h in heads:
        hk = h // G
        if x.replaced[h]:
            ro, rl = oracle.head_fwd(1, x.v[b, hk], a=x.a[h], r=x.r[h], rows=rows)
        else:
            ro, rl = oracle.head_fwd(0, x.v[b, hk], q=x.q[b, h], k=x.k[b, hk], rows=rows)
        wr.add(cpu64(o[b, h].index_select(0, idx)), ro, tol, "o[b=%d,h=%d]" % (b, h), T=T)
        wr.add_lse(cpu64(lse[b, h].index_select(0, idx)), rl, TOL_LSE[o.dtype],
                   "lse[b=%d,h=%d]" % (b, h))
    if worst is None:
        wr.report()
    return wr.row


def check_bwd(x, dq, dk, dv, heads, qrows, krows, tol, what="", worst=None):
    """Compare dq (query rows) and dk, dv (key rows) of the listed slices with the oracle, row by
    row; a replaced head's dq and dk must be exactly zero."""
    wr = Worst(what) if worst is None else worst
    T = x.v.shape[2]
    qrows = np.arange(T, dtype=np.int32) if qrows is None else qrows
    krows = np.arange(T, dtype=np.int32) if krows is None else krows
    iq = torch.as_tensor(qrows, dtype=torch.long, device=dq.device)
    ik = torch.as_tensor(krows, dtype=torch.long, device=dq.device)
    for b, h in heads:
        kind = 1 if x.replaced[h] else 0
        rq, rk, rv = oracle.head_bwd(kind, x.v[b, h], x.dout[b, h], q=x.q[b, h], k=x.k[b, h],
                                     a=x.a[h], r=x.r[h], qrows=qrows, krows=krows)
        gq = cpu64(dq[b, h].index_select(0, iq))
        gk = cpu64(dk[b, h].index_select(0, ik))
        gv = cpu64(dv[b, h].index_select(0, ik))
        if kind == 1:
            assert np.all(gq == 0.0) and np.all(gk == 0.0), "%s replaced dq/dk must be 0" % what
        else:
            args = (x.q[b, h], x.k[b, h], x.v[b, h], x.dout[b, h])
            wr.add(gq, rq, tol, "dq[b=%d,h=%d]" % (b, h), T=T, rows=qrows,
                   rounding=lambda r: dq_uncancelled_scale(*args, r))
            wr.add(gk, rk, tol, "dk[b=%d,h=%d]" % (b, h), T=T, rows=krows,
                   rounding=lambda r: dk_uncancelled_scale(*args, r))
        wr.add(gv, rv, tol, "dv[b=%d,h=%d]" % (b, h), T=T)
    if worst is None:
        wr.report()
    return wr.row
