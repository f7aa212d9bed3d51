"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each check raises AssertionError on failure.  They use only the oracle package and independent
means (golden fixtures worked by hand, closed forms, torch / numpy / scipy library routines in
float64, finite differences), never the GPU path.  test_oracle_pins.py runs them on the real oracle;
test_oracle_mutants.py runs them on copies of the oracle with a planted mistake and requires that
every mutant fails at least one of them.

Citations: [Notes] = the page "When Can Attention Heads Be Statically Defined?：中文精读笔记".
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse a fixture: 'key: v v v' lines, values as fractions 'p/q' or 'ln(x)'; '#' comments."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, vals = line.split(":", 1)
            toks = vals.split()
            out[key.strip()] = np.array([_tok(t) for t in toks], dtype=np.float64)
    return out


def _tok(t):
    if t.startswith("ln(") and t.endswith(")"):
        return math.log(float(Fraction(t[3:-1])))
    return float(Fraction(t))


def _rel(x, y):
    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    den = max(np.abs(y).max(), 1e-300)
    return np.abs(x - y).max() / den


def _sdpa(q, k, v, scale):
    """torch's causal attention in float64 on the CPU: a library routine, not the oracle."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64)[None, None] for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    return o[0, 0].numpy()


def _torch_maps(q, k, scale):
    """Dense causal softmax maps [N, T, T] by torch in float64 (library routine)."""
    tq, tk = torch.tensor(q, dtype=torch.float64), torch.tensor(k, dtype=torch.float64)
    s = scale * tq @ tk.transpose(-1, -2)
    T = q.shape[1]
    mask = torch.ones(T, T, dtype=torch.bool).triu(1)
    s = s.masked_fill(mask, float("-inf"))
    return torch.softmax(s, dim=-1).numpy()


# ------------------------------------------------------------------ Eq. (3) pattern ([Notes §二.3])
def check_pattern_invariants():
    rng = np.random.default_rng(11)
    for T, std in ((1, 1.0), (5, 0.5), (37, 1.0), (64, 3.0)):
        a, r = rng.normal(0, std, T), rng.normal(0, std, T)
        P = oracle.head_pattern(1, T, a=a, r=r)
        assert np.all(np.abs(P.sum(1) - 1.0) <= 1e-13), "rows of Eq.(3) must sum to 1"
        assert np.all(P[np.triu_indices(T, 1)] == 0.0), "future keys must carry zero weight"
        assert np.all(P >= 0.0)
        q, k = rng.normal(size=(T, 4)), rng.normal(size=(T, 4))
        P = oracle.head_pattern(0, T, q=q, k=k)
        assert np.all(np.abs(P.sum(1) - 1.0) <= 1e-13)
        assert np.all(P[np.triu_indices(T, 1)] == 0.0)


def check_eq3_worked():
    g = read_golden("eq3_worked_t3.txt")
    T = 3
    P = oracle.head_pattern(1, T, a=g["a"], r=g["r"])
    want = np.stack([g["P_row0"], g["P_row1"], g["P_row2"]])
    assert np.abs(P - want).max() <= 1e-15, P
    o, lz = oracle.head_fwd(1, g["v"][:, None], a=g["a"], r=g["r"])
    assert np.abs(o[:, 0] - g["o"]).max() <= 1e-14
    assert np.abs(lz - g["logZ"]).max() <= 1e-14
    dq, dk, dv = oracle.head_bwd(1, g["v"][:, None], g["dout"][:, None], a=g["a"], r=g["r"])
    assert np.abs(dv[:, 0] - g["dv"]).max() <= 1e-14
    assert np.all(dq == 0.0) and np.all(dk == 0.0)


def check_identity_pattern():
    """r[0] = 0 and r[delta >= 1] = -inf (or -1e4, which underflows to an exact 0) is the identity
    pattern: O = V and dV = dO exactly, whatever a holds."""
    rng = np.random.default_rng(12)
    T, d = 9, 3
    v, do = rng.normal(size=(T, d)), rng.normal(size=(T, d))
    a = rng.normal(size=T)
    for big in (-np.inf, -1e4):
        r = np.full(T, big)
        r[0] = 0.0
        o, lz = oracle.head_fwd(1, v, a=a, r=r)
        assert np.array_equal(o, v)
        assert np.allclose(lz, a, rtol=0, atol=1e-15)
        _, _, dv = oracle.head_bwd(1, v, do, a=a, r=r)
        assert np.array_equal(dv, do)


def check_uniform_prefix_mean():
    """a = r = 0 gives equal weights on the visible keys: O_i = mean of V_0..V_i; an ordinary head
    with Q = 0 gives the same."""
    rng = np.random.default_rng(13)
    T, d = 17, 5
    v = rng.normal(size=(T, d))
    want = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    o, lz = oracle.head_fwd(1, v, a=np.zeros(T), r=np.zeros(T))
    assert _rel(o, want) <= 1e-14
    assert np.abs(lz - np.log(np.arange(1, T + 1))).max() <= 1e-14
    o0, _ = oracle.head_fwd(0, v, q=np.zeros((T, d)), k=rng.normal(size=(T, d)))
    assert _rel(o0, want) <= 1e-14


def check_constant_r_and_constant_a():
    """r constant: row i is softmax(a[0..i]); a constant: row i is proportional to e^{r[i-j]}."""
    rng = np.random.default_rng(14)
    T = 12
    a, r = rng.normal(size=T), rng.normal(size=T)
    P = oracle.head_pattern(1, T, a=a, r=np.full(T, 0.7))
    for i in range(T):
        assert np.abs(P[i, :i + 1] - scipy.special.softmax(a[:i + 1])).max() <= 1e-15
    P = oracle.head_pattern(1, T, a=np.full(T, -1.3), r=r)
    for i in range(T):
        w = np.exp(r[i - np.arange(i + 1)])
        assert np.abs(P[i, :i + 1] - w / w.sum()).max() <= 1e-15


# ------------------------------------------------------------- ordinary head ([Notes §一])
def check_ordinary_vs_library():
    rng = np.random.default_rng(15)
    for T, d, scale in ((23, 8, None), (40, 16, 0.37), (1, 4, None)):
        q, k, v = (rng.normal(size=(T, d)) for _ in range(3))
        s = 1.0 / math.sqrt(d) if scale is None else scale
        o, lse = oracle.head_fwd(0, v, q=q, k=k, scale=scale)
        assert _rel(o, _sdpa(q, k, v, s)) <= 1e-13
        sc = torch.tensor(s * q @ k.T).masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1),
                                                    float("-inf"))
        assert np.abs(lse - torch.logsumexp(sc, -1).numpy()).max() <= 1e-13


def check_two_key_example():
    g = read_golden("softmax_two_keys.txt")
    o, lse = oracle.head_fwd(0, g["v"][:, None], q=g["q"][:, None], k=g["k"][:, None], scale=1.0)
    assert np.abs(o[:, 0] - g["o"]).max() <= 1e-15
    assert np.abs(lse - g["lse"]).max() <= 1e-15


def check_t1():
    """T = 1: the only key is the query's own, so O = V and dV = dO; dQ = dK = 0."""
    rng = np.random.default_rng(16)
    d = 6
    q, k, v, do = (rng.normal(size=(1, d)) for _ in range(4))
    for kind in (0, 1):
        o, _ = oracle.head_fwd(kind, v, q=q, k=k, a=rng.normal(size=1), r=rng.normal(size=1))
        assert np.array_equal(o, v)
        dq, dk, dv = oracle.head_bwd(kind, v, do, q=q, k=k, a=np.zeros(1), r=np.zeros(1))
        assert np.array_equal(dv, do)
        assert np.all(dq == 0.0) and np.all(dk == 0.0)


# ------------------------------------------------------------------------- backward ([Notes §二.4])
def _loss(kind, q, k, v, a, r, g, scale):
    o, _ = oracle.head_fwd(kind, v, q=q, k=k, a=a, r=r, scale=scale)
    return float((o * g).sum())


def check_backward_finite_differences():
    rng = np.random.default_rng(17)
    T, d, h = 7, 3, 1e-6
    q, k, v, g = (rng.normal(size=(T, d)) for _ in range(4))
    a, r = rng.normal(size=T), rng.normal(size=T)
    scale = 0.61
    for kind in (0, 1):
        dq, dk, dv = oracle.head_bwd(kind, v, g, q=q, k=k, a=a, r=r, scale=scale)
        names = ("q", "k", "v") if kind == 0 else ("v",)
        got = {"q": dq, "k": dk, "v": dv}
        for name in names:
            base = {"q": q, "k": k, "v": v}
            fd = np.zeros((T, d))
            for i in range(T):
                for c in range(d):
                    args = {n: x.copy() for n, x in base.items()}
                    args[name][i, c] += h
                    lp = _loss(kind, args["q"], args["k"], args["v"], a, r, g, scale)
                    args[name][i, c] -= 2 * h
                    lm = _loss(kind, args["q"], args["k"], args["v"], a, r, g, scale)
                    fd[i, c] = (lp - lm) / (2 * h)
            assert _rel(got[name], fd) <= 1e-7, (kind, name, _rel(got[name], fd))
        if kind == 1:
            assert np.all(dq == 0.0) and np.all(dk == 0.0)


def check_backward_vs_autograd():
    rng = np.random.default_rng(18)
    T, d = 19, 8
    q, k, v, g = (rng.normal(size=(T, d)) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None],
                                                         tv[None, None], is_causal=True)
    (o[0, 0] * torch.tensor(g)).sum().backward()
    dq, dk, dv = oracle.head_bwd(0, v, g, q=q, k=k)
    assert _rel(dq, tq.grad.numpy()) <= 1e-12
    assert _rel(dk, tk.grad.numpy()) <= 1e-12
    assert _rel(dv, tv.grad.numpy()) <= 1e-12


def check_backward_invariants():
    """Rows of P sum to 1, so sum_j dV_j = sum_i dO_i (both kinds); rows of dS sum to 0, so
    sum_j dK_j = 0 (ordinary)."""
    rng = np.random.default_rng(19)
    T, d = 33, 4
    q, k, v, g = (rng.normal(size=(T, d)) for _ in range(4))
    a, r = rng.normal(size=T), rng.normal(size=T)
    for kind in (0, 1):
        dq, dk, dv = oracle.head_bwd(kind, v, g, q=q, k=k, a=a, r=r)
        assert np.abs(dv.sum(0) - g.sum(0)).max() <= 1e-12
        assert np.abs(dk.sum(0)).max() <= 1e-12


# ------------------------------------------------------------ calibration ([Notes §二.1, Eq.(1)])
def check_eq1_golden():
    g = read_golden("eq1_n2_t2.txt")
    maps = np.stack([g["A1"].reshape(2, 2), g["A2"].reshape(2, 2)])
    ahat, sv = oracle.calibrate_maps(maps)
    assert np.abs(ahat.ravel() - g["ahat"]).max() <= 1e-15
    assert abs(sv - g["svar"][0]) <= 1e-15


def check_eq1_brute_force():
    rng = np.random.default_rng(20)
    N, T = 5, 6
    maps = np.zeros((N, T, T))
    for n in range(N):
        for i in range(T):
            maps[n, i, :i + 1] = rng.dirichlet(np.ones(i + 1))
    ahat, sv = oracle.calibrate_maps(maps)
    assert np.abs(ahat - maps.mean(0)).max() <= 1e-15
    assert abs(sv - np.var(maps, axis=0, ddof=1).mean()) <= 1e-15
    assert sv >= 0.0
    ahat, sv = oracle.calibrate_maps(np.stack([maps[0]] * 4))
    assert sv <= 1e-30 and np.abs(ahat - maps[0]).max() <= 1e-15


def check_calibrate_qk_route():
    """The streamed route (maps formed from Q, K row by row) equals Eq. (1) on dense maps built by
    torch, and the brute-force variance of numpy."""
    rng = np.random.default_rng(21)
    N, T, d = 4, 9, 5
    q, k = rng.normal(size=(N, T, d)), rng.normal(size=(N, T, d))
    maps = _torch_maps(q, k, 1.0 / math.sqrt(d))
    ahat, dev = oracle.head_calibrate(q, k)
    sv = dev.sum() / ((N - 1) * T * T)
    assert np.abs(ahat - maps.mean(0)).max() <= 1e-14
    assert abs(sv - np.var(maps, axis=0, ddof=1).mean()) <= 1e-14 * max(sv, 1e-300) + 1e-18
    ahat2, sv2 = oracle.calibrate_maps(maps)
    assert np.abs(ahat - ahat2).max() <= 1e-14 and abs(sv - sv2) <= 1e-14 * sv


def check_calibrate_q0():
    """Q = 0 for every sequence: every map is the uniform causal pattern, so s_var = 0 and
    Ahat(i,j) = 1/(i+1) below the diagonal."""
    rng = np.random.default_rng(22)
    N, T, d = 3, 8, 4
    ahat, dev = oracle.head_calibrate(np.zeros((N, T, d)), rng.normal(size=(N, T, d)))
    assert dev.sum() <= 1e-30
    want = np.tril(np.ones((T, T))) / np.arange(1, T + 1)[:, None]
    assert np.abs(ahat - want).max() <= 1e-15


def check_mean_optimality_identity():
    """Finite-sample form of the mean-optimality identity ([Notes §二.2], Appendix B.1): for any
    fixed P, (1/(N T^2)) sum_n ||A^(n) - P||^2 = ((N-1)/N) s_var + ||P - Ahat||^2 / T^2."""
    rng = np.random.default_rng(23)
    N, T, d = 6, 10, 3
    q, k = rng.normal(size=(N, T, d)), rng.normal(size=(N, T, d))
    maps = _torch_maps(q, k, 1.0 / math.sqrt(d))
    ahat, dev = oracle.head_calibrate(q, k)
    sv = dev.sum() / ((N - 1) * T * T)
    for _ in range(3):
        P = rng.random((T, T))
        lhs = ((maps - P) ** 2).sum() / (N * T * T)
        rhs = (N - 1) / N * sv + ((P - ahat) ** 2).sum() / (T * T)
        assert abs(lhs - rhs) <= 1e-13 * lhs


# ------------------------------------------------------------------- row sampling and causality
def check_row_subsets():
    rng = np.random.default_rng(24)
    T, d = 21, 4
    q, k, v, g = (rng.normal(size=(T, d)) for _ in range(4))
    a, r = rng.normal(size=T), rng.normal(size=T)
    rows = np.array([0, 5, 20, 7])
    for kind in (0, 1):
        of, lf = oracle.head_fwd(kind, v, q=q, k=k, a=a, r=r)
        os_, ls = oracle.head_fwd(kind, v, q=q, k=k, a=a, r=r, rows=rows)
        assert np.array_equal(of[rows], os_) and np.array_equal(lf[rows], ls)
        full = oracle.head_bwd(kind, v, g, q=q, k=k, a=a, r=r)
        sub = oracle.head_bwd(kind, v, g, q=q, k=k, a=a, r=r, qrows=rows, krows=rows)
        for x, y in zip(full, sub):
            assert np.array_equal(x[rows], y)
    N = 3
    qc, kc = rng.normal(size=(N, T, d)), rng.normal(size=(N, T, d))
    af, df = oracle.head_calibrate(qc, kc)
    as_, ds = oracle.head_calibrate(qc, kc, rows=rows)
    assert np.array_equal(af[rows], as_) and np.array_equal(df[rows], ds)


def check_causal_prefix():
    """Row i depends on positions <= i only: the first T1 rows at length T1 equal those at T2."""
    rng = np.random.default_rng(25)
    T1, T2, d = 11, 26, 4
    q, k, v, g = (rng.normal(size=(T2, d)) for _ in range(4))
    a, r = rng.normal(size=T2), rng.normal(size=T2)
    for kind in (0, 1):
        o1, l1 = oracle.head_fwd(kind, v[:T1], q=q[:T1], k=k[:T1], a=a, r=r)
        o2, l2 = oracle.head_fwd(kind, v, q=q, k=k, a=a, r=r)
        assert _rel(o1, o2[:T1]) <= 1e-15 and np.abs(l1 - l2[:T1]).max() <= 1e-14


# ------------------------------------------------ forward-KL selector and head selection ([Notes §二.1])
def check_kl_golden():
    g = read_golden("kl_n2_t2.txt")
    maps = np.stack([g["A1"].reshape(2, 2), g["A2"].reshape(2, 2)])
    assert abs(oracle.kl_maps(maps) * 4 - g["kl_sum"][0]) <= 1e-15


def check_kl_vs_library():
    """The streamed score equals KL by scipy (rel_entr) on dense maps built by torch, and the
    Jensen-gap form (1/T) sum_i [H(Ahat_i) - mean_n H(A^(n)_i)] with scipy's entropy."""
    import scipy.stats
    rng = np.random.default_rng(30)
    N, T, d = 4, 9, 5
    q, k = rng.normal(size=(N, T, d)), rng.normal(size=(N, T, d))
    maps = _torch_maps(q, k, 1.0 / math.sqrt(d))
    ahat = maps.mean(0)
    rows = oracle.head_kl_score(q, k)
    for i in range(T):
        want = sum(scipy.special.rel_entr(maps[n, i, :i + 1], ahat[i, :i + 1]).sum() for n in range(N))
        assert abs(rows[i] - want) <= 1e-13 * max(1.0, want)
    skl = rows.sum() / (N * T)
    jensen = np.mean([scipy.stats.entropy(ahat[i, :i + 1]) -
                      np.mean([scipy.stats.entropy(maps[n, i, :i + 1]) for n in range(N)])
                      for i in range(T)])
    assert abs(skl - jensen) <= 1e-13 and skl > 0.0
    assert abs(oracle.kl_maps(maps) - skl) <= 1e-14


def check_kl_special_cases():
    """Identical maps or Q = 0 (every map uniform) give a score of exactly 0."""
    rng = np.random.default_rng(31)
    N, T, d = 3, 7, 4
    q, k = rng.normal(size=(1, T, d)), rng.normal(size=(1, T, d))
    assert abs(oracle.head_kl_score(np.repeat(q, N, 0), np.repeat(k, N, 0)).sum()) <= 1e-14
    assert abs(oracle.head_kl_score(np.zeros((N, T, d)), rng.normal(size=(N, T, d))).sum()) <= 1e-14


def check_select_golden():
    g = read_golden("select_ties.txt")
    score = g["score"].reshape(2, 3)
    for key, ratio in (("sel_half", 0.5), ("sel_quarter", 0.25), ("sel_twelfth", 1 / 12)):
        sel, n = oracle.select_heads(score, ratio)
        assert np.array_equal(sel.ravel(), g[key].astype(np.uint8)) and n == int(g[key].sum())
    acc = g["accepted"].reshape(2, 3).astype(np.uint8)
    sel, n = oracle.select_heads(score, 0.5, accepted=acc)
    assert np.array_equal(sel.ravel(), g["sel_half_accepted"].astype(np.uint8)) and n == 3


def check_select_brute_force():
    """With distinct scores the selection is the unique k-subset of accepted heads of least total
    score (brute force over all subsets)."""
    import itertools
    rng = np.random.default_rng(32)
    L, H = 3, 4
    for trial in range(4):
        score = rng.random((L, H))
        acc = (rng.random((L, H)) < 0.75).astype(np.uint8) if trial % 2 else None
        heads = [(l, h) for l in range(L) for h in range(H) if acc is None or acc[l, h]]
        for ratio in (0.0, 0.1, 0.25, 0.5, 0.75, 1.0):
            k = min(round(ratio * L * H), len(heads))
            best = min(itertools.combinations(heads, k), key=lambda c: sum(score[x] for x in c))
            sel, n = oracle.select_heads(score, ratio, accepted=acc)
            assert n == k and set(zip(*np.nonzero(sel))) == set(best)


# ------------------------------------------- trainable pattern: dL/da, dL/dr ([Paper page] Table 14)
def _pattern_loss(v, g, a, r):
    o, _ = oracle.head_fwd(1, v, a=a, r=r)
    return float((o * g).sum())


def check_pattern_grad_finite_differences():
    rng = np.random.default_rng(40)
    T, d, h = 7, 3, 1e-6
    v, g = rng.normal(size=(T, d)), rng.normal(size=(T, d))
    a, r = rng.normal(size=T), rng.normal(size=T)
    da, dr = oracle.head_pattern_grad(v, g, a, r)
    for vec, grad in ((a, da), (r, dr)):
        for x in range(T):
            old = vec[x]
            vec[x] = old + h
            lp = _pattern_loss(v, g, a, r)
            vec[x] = old - h
            lm = _pattern_loss(v, g, a, r)
            vec[x] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[x]) <= 1e-7 * max(1.0, abs(fd))


def check_pattern_grad_vs_autograd():
    """torch autograd in float64 through a dense masked softmax (library routine)."""
    rng = np.random.default_rng(41)
    T, d = 10, 4
    v, g = rng.normal(size=(T, d)), rng.normal(size=(T, d))
    a, r = rng.normal(size=T), rng.normal(size=T)
    ta = torch.tensor(a, requires_grad=True)
    tr = torch.tensor(r, requires_grad=True)
    idx = torch.arange(T)
    dist = (idx[:, None] - idx[None, :]).clamp(min=0)
    logits = ta[None, :] + tr[dist]
    logits = logits.masked_fill(idx[None, :] > idx[:, None], float("-inf"))
    o = torch.softmax(logits, -1) @ torch.tensor(v)
    (o * torch.tensor(g)).sum().backward()
    da, dr = oracle.head_pattern_grad(v, g, a, r)
    assert _rel(da, ta.grad.numpy()) <= 1e-13 and _rel(dr, tr.grad.numpy()) <= 1e-13


def check_pattern_grad_invariants():
    """Shifting every a, every r, or (a(j) + b j, r(delta) + b delta) leaves each row's pattern
    unchanged (a constant per row cancels), so sum da = 0, sum dr = 0 and
    sum_j j da(j) + sum_delta delta dr(delta) = 0.  Equal value rows give zero gradient."""
    rng = np.random.default_rng(42)
    T, d = 12, 3
    v, g = rng.normal(size=(T, d)), rng.normal(size=(T, d))
    a, r = rng.normal(size=T), rng.normal(size=T)
    da, dr = oracle.head_pattern_grad(v, g, a, r)
    pos = np.arange(T)
    scale = np.abs(da).max() + np.abs(dr).max()
    assert abs(da.sum()) <= 1e-13 * scale and abs(dr.sum()) <= 1e-13 * scale
    assert abs(pos @ da + pos @ dr) <= 1e-12 * T * scale
    da0, dr0 = oracle.head_pattern_grad(np.tile(v[:1], (T, 1)), g, a, r)
    assert np.abs(da0).max() <= 1e-14 and np.abs(dr0).max() <= 1e-14


# ------------------------------------------------------------- compact fit of a, r ([Notes §二.3])
def _dense_pattern(a, r):
    """Eq. (3) pattern by scipy's softmax over masked logits (library routine)."""
    T = len(a)
    idx = np.arange(T)
    t = a[None, :] + r[np.clip(idx[:, None] - idx[None, :], 0, None)]
    t = np.where(idx[None, :] <= idx[:, None], t, -np.inf)
    return scipy.special.softmax(t, axis=1)


def _random_target(rng, T, normalise=True):
    M = np.zeros((T, T))
    for i in range(T):
        M[i, :i + 1] = rng.dirichlet(np.ones(i + 1))
    if not normalise:
        M *= rng.uniform(0.5, 2.0, size=(T, 1))
    return M


def check_fit_loss_vs_autograd():
    """L and its gradient against torch autograd (float64) of -(1/T) sum Ahat * log_softmax,
    with row-stochastic targets and with rows of other sums."""
    rng = np.random.default_rng(50)
    T = 9
    idx = torch.arange(T)
    dist = (idx[:, None] - idx[None, :]).clamp(min=0)
    mask = idx[None, :] > idx[:, None]
    for normalise in (True, False):
        M = _random_target(rng, T, normalise)
        a, r = rng.normal(size=T), rng.normal(size=T)
        ta = torch.tensor(a, requires_grad=True)
        tr = torch.tensor(r, requires_grad=True)
        lsm = torch.log_softmax((ta[None, :] + tr[dist]).masked_fill(mask, float("-inf")), -1)
        loss = -(torch.tensor(M) * lsm.masked_fill(mask, 0.0)).sum() / T
        loss.backward()
        L, ga, gr = oracle.fit_loss_grad(M, a, r)
        assert abs(L - loss.item()) <= 1e-13 * abs(L)
        assert _rel(ga, ta.grad.numpy()) <= 1e-12 and _rel(gr, tr.grad.numpy()) <= 1e-12


def check_fit_gauge():
    """L is unchanged by (a(j) + b j + c1, r(delta) + b delta + c2); the gradient sums vanish."""
    rng = np.random.default_rng(51)
    T = 11
    M = _random_target(rng, T)
    a, r = rng.normal(size=T), rng.normal(size=T)
    pos = np.arange(T)
    L0, ga, gr = oracle.fit_loss_grad(M, a, r)
    L1, _, _ = oracle.fit_loss_grad(M, a + 0.7 * pos + 1.3, r + 0.7 * pos - 2.1)
    assert abs(L1 - L0) <= 1e-12 * abs(L0)
    assert abs(ga.sum()) <= 1e-14 and abs(gr.sum()) <= 1e-14
    assert abs(pos @ ga + pos @ gr) <= 1e-13 * T


def check_fit_adam_vs_library():
    """25 steps of the fit equal torch.optim.Adam (float64, default moment rates) on the same loss
    written with torch's log_softmax."""
    rng = np.random.default_rng(52)
    T, steps, lr = 8, 25, 0.1
    M = _random_target(rng, T)
    idx = torch.arange(T)
    dist = (idx[:, None] - idx[None, :]).clamp(min=0)
    mask = idx[None, :] > idx[:, None]
    ta = torch.zeros(T, dtype=torch.float64, requires_grad=True)
    tr = torch.zeros(T, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([ta, tr], lr=lr)
    tm = torch.tensor(M)
    for _ in range(steps):
        opt.zero_grad()
        lsm = torch.log_softmax((ta[None, :] + tr[dist]).masked_fill(mask, float("-inf")), -1)
        (-(tm * lsm.masked_fill(mask, 0.0)).sum() / T).backward()
        opt.step()
    a, r, _, _ = oracle.fit_pattern(M, steps=steps, lr=lr)
    assert np.abs(a - ta.detach().numpy()).max() <= 1e-11
    assert np.abs(r - tr.detach().numpy()).max() <= 1e-11


def check_fit_recovers_eq3_and_matches_moments():
    """A target of the form of Eq. (3) is recovered (mean row KL ~ 0, same pattern); for any
    target the fitted pattern's column and diagonal sums equal the target's (the sufficient
    statistics of the notes: the optimum matches both marginals), and KL = L + (1/T) sum A ln A."""
    rng = np.random.default_rng(53)
    T = 24
    a0, r0 = rng.normal(size=T), np.r_[3.0, rng.normal(size=T - 1) * 0.5]
    P0 = _dense_pattern(a0, r0)
    a, r, L, kl = oracle.fit_pattern(P0, steps=400, lr=0.1)
    assert 0.0 <= kl + 1e-14 and kl <= 1e-8
    assert np.abs(_dense_pattern(a, r) - P0).max() <= 1e-4
    M = _random_target(rng, 16)
    a, r, L, kl = oracle.fit_pattern(M, steps=400, lr=0.1)
    P = _dense_pattern(a, r)
    T = 16
    col = lambda X: X.sum(0)
    diag = lambda X: np.array([np.trace(X, offset=-dl) for dl in range(T)])
    assert np.abs(col(P) - col(M)).max() <= 1e-6 and np.abs(diag(P) - diag(M)).max() <= 1e-6
    ent = (M[M > 0] * np.log(M[M > 0])).sum()
    assert abs(kl - (L + ent / T)) <= 1e-13 and kl > 0.0
    lsm = np.log(np.where(P > 0, P, 1.0))
    want_kl = np.mean([(M[i, :i + 1] * (np.log(M[i, :i + 1]) - lsm[i, :i + 1])).sum() for i in range(T)])
    assert abs(kl - want_kl) <= 1e-12


# ------------------------------------------------ grouped key/value heads ([Notes §二.4], GQA)
def check_gqa_identity_mapping():
    """With one query head per key/value head the grouped layer is the plain mixed layer."""
    rng = np.random.default_rng(60)
    B, H, T, d = 2, 3, 9, 4
    q, k, v, g = (rng.normal(size=(B, H, T, d)) for _ in range(4))
    a, r = rng.normal(size=(H, T)), rng.normal(size=(H, T))
    rep = [0, 1, 0]
    f1, f2 = oracle.layer_fwd(q, k, v, rep, a, r), oracle.layer_fwd_gqa(q, k, v, rep, a, r)
    for key in f1:
        assert np.array_equal(f1[key][0], f2[key][0]) and np.array_equal(f1[key][1], f2[key][1])
    b1 = oracle.layer_bwd(q, k, v, g, rep, a, r)
    dq, dk, dv = oracle.layer_bwd_gqa(q, k, v, g, rep, a, r)
    for key in b1:
        assert np.array_equal(b1[key][0], dq[key]) and np.array_equal(b1[key][1], dk[key])
        assert np.array_equal(b1[key][2], dv[key])


def check_gqa_finite_differences():
    """dk, dv of a shared key/value head are the derivatives of L = sum_h sum dO_h . O_h through
    every query head of the group (central differences), including a replaced head's share of dv;
    a group whose heads are all replaced has dk = 0."""
    rng = np.random.default_rng(61)
    B, H, Hkv, T, d, hstep = 1, 4, 2, 6, 3, 1e-6
    q, g = rng.normal(size=(B, H, T, d)), rng.normal(size=(B, H, T, d))
    k, v = rng.normal(size=(B, Hkv, T, d)), rng.normal(size=(B, Hkv, T, d))
    a, r = rng.normal(size=(H, T)), rng.normal(size=(H, T))
    rep = [0, 1, 1, 1]  # group 0: ordinary + replaced; group 1: replaced only

    def loss():
        out = oracle.layer_fwd_gqa(q, k, v, rep, a, r)
        return sum(float((out[(0, h)][0] * g[0, h]).sum()) for h in range(H))

    dq, dk, dv = oracle.layer_bwd_gqa(q, k, v, g, rep, a, r)
    for arr, grad in ((k, dk), (v, dv)):
        for hk in range(Hkv):
            for j in (0, 2, T - 1):
                for c in range(d):
                    old = arr[0, hk, j, c]
                    arr[0, hk, j, c] = old + hstep
                    lp = loss()
                    arr[0, hk, j, c] = old - hstep
                    lm = loss()
                    arr[0, hk, j, c] = old
                    fd = (lp - lm) / (2 * hstep)
                    assert abs(fd - grad[(0, hk)][j, c]) <= 1e-7 * max(1.0, abs(fd))
    assert np.abs(dk[(0, 1)]).max() == 0.0 and np.abs(dv[(0, 1)]).max() > 0.0


ALL_CHECKS = [
    check_pattern_invariants, check_eq3_worked, check_identity_pattern, check_uniform_prefix_mean,
    check_constant_r_and_constant_a, check_ordinary_vs_library, check_two_key_example, check_t1,
    check_backward_finite_differences, check_backward_vs_autograd, check_backward_invariants,
    check_eq1_golden, check_eq1_brute_force, check_calibrate_qk_route, check_calibrate_q0,
    check_mean_optimality_identity, check_row_subsets, check_causal_prefix,
    check_kl_golden, check_kl_vs_library, check_kl_special_cases, check_select_golden,
    check_select_brute_force, check_pattern_grad_finite_differences,
    check_pattern_grad_vs_autograd, check_pattern_grad_invariants, check_fit_loss_vs_autograd,
    check_fit_gauge, check_fit_adam_vs_library, check_fit_recovers_eq3_and_matches_moments,
    check_gqa_identity_mapping, check_gqa_finite_differences,
]
