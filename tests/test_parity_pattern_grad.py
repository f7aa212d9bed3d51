"""Gradient of a trained pattern (dL/da, dL/dr of the replaced heads, [Paper page] Table 14) on the
GPU through the C ABI, against the fp64 oracle (softmax chain rule over the Eq. (3) logits)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, cpu64, rel_l2, vec_err

pytestmark = pytest.mark.gpu


def _saf():
    import fixed_pattern_mixed_amd as saf
    return saf


def _run(x, g, rep, pat_extra=0):
    saf = _saf()
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    da, dr = saf.bwd_pattern(g.v, o, g.dout, lse, rep, g.a, g.r)
    torch.cuda.synchronize()
    return o, lse, da, dr


def _compare(x, rep, da, dr, tol, what):
    T = x.v.shape[2]
    ref = oracle.pattern_grad(x.v, x.dout, rep, x.a, x.r)
    gda, gdr = cpu64(da), cpu64(dr)
    for h, (rda, rdr) in ref.items():
        e1, e2 = vec_err(gda[h, :T], rda), vec_err(gdr[h, :T], rdr)
        l1, l2 = rel_l2(gda[h, :T], rda), rel_l2(gdr[h, :T], rdr)
        print("%s head %d: da err %.2e (rel-L2 %.2e), dr err %.2e (rel-L2 %.2e)"
              % (what, h, e1, l1, e2, l2), flush=True)
        assert max(e1, e2, l1, l2) <= tol, (what, h, e1, e2, l1, l2)
        assert np.all(gda[h, T:] == 0.0) and np.all(gdr[h, T:] == 0.0)
    for h in range(len(rep)):
        if not rep[h]:  # rows of ordinary heads are not touched (the binding passes zeros)
            assert np.all(gda[h] == 0.0) and np.all(gdr[h] == 0.0)


SMALL = [
    # B, H, T, d, dtype, R, placement, a/r std, extra pattern length
    (1, 4, 256, 64, torch.float32, 1, "interleaved", 1.0, 0),
    (2, 4, 200, 128, torch.float32, 2, "contiguous", 1.0, 37),
    (3, 2, 129, 64, torch.float32, 2, "all", 0.5, 0),
    (2, 4, 300, 64, torch.bfloat16, 2, "interleaved", 0.5, 0),
    (1, 4, 257, 128, torch.bfloat16, 1, "contiguous", 0.5, 5),
    (1, 12, 520, 64, torch.bfloat16, 6, "interleaved", 0.5, 0),
]


@pytest.mark.parametrize("B,H,T,d,dtype,R,placement,std,extra", SMALL,
                         ids=["B%dH%dT%dd%d-%s-R%d" % (c[0], c[1], c[2], c[3], str(c[4])[6:], c[5]) for c in SMALL])
def test_pattern_gradient_small_full_compare(B, H, T, d, dtype, R, placement, std, extra):
    rep = synth.replaced_mask(H, R, placement)
    x = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=std, seed=61 + T, pat_len=T + extra)
    g = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=std, seed=61 + T, pat_len=T + extra,
                           device="cuda")
    _, _, da, dr = _run(x, g, rep)
    _compare(x, rep, da, dr, TOL[dtype], "small")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pattern_gradient_exponential_form(dtype):
    """A wide-range pattern (the product form would underflow) takes the exponential form."""
    B, H, T, d = 2, 4, 257, 64
    rep = [0, 1, 0, 1]
    x = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=1.0, seed=15)
    x.a[1, T - 1] = 200.0
    x.a[3, 5] = 150.0
    x.r[3, 7] = -300.0
    g = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=1.0, seed=15, device="cuda")
    g.a.copy_(x.a)
    g.r.copy_(x.r)
    _, _, da, dr = _run(x, g, rep)
    _compare(x, rep, da, dr, TOL[dtype], "wide")


def test_pattern_gradient_t1_and_repeatable():
    """T = 1: each row has one entry of weight 1, so dT = G - delta = 0.  The result of a second
    call is bitwise equal to the first."""
    saf = _saf()
    rep = [0, 1, 1]
    g = synth.layer_inputs(2, 3, 1, 64, torch.float32, rep, ar_std=1.0, seed=3, device="cuda")
    _, _, da, dr = _run(None, g, rep)
    assert float(da.abs().max()) <= 1e-5 and float(dr.abs().max()) <= 1e-5
    g = synth.layer_inputs(2, 4, 700, 64, torch.bfloat16, [0, 1, 0, 1], ar_std=0.5, seed=4,
                           device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, [0, 1, 0, 1], g.a, g.r)
    d1 = saf.bwd_pattern(g.v, o, g.dout, lse, [0, 1, 0, 1], g.a, g.r)
    d2 = saf.bwd_pattern(g.v, o, g.dout, lse, [0, 1, 0, 1], g.a, g.r)
    torch.cuda.synchronize()
    assert torch.equal(d1[0], d2[0]) and torch.equal(d1[1], d2[1])


def test_pattern_gradient_full_size():
    """The 124M-shaped layer (B=8, H=12, T=4096, d=64, bf16, heads 3, 7, 11 replaced): the full
    da, dr of two replaced heads against the oracle, and the shift invariants (sum da and sum dr
    vanish up to the rounding of delta) for all."""
    saf = _saf()
    w = synth.WORKLOADS["l124m_t4096"]
    x = synth.workload_inputs(w)
    print("workload", w.name, flush=True)
    v, q, k, gd, a, r = (t.to("cuda") for t in (x.v, x.q, x.k, x.dout, x.a, x.r))
    o, lse = saf.fwd(q, k, v, x.replaced, a, r)
    da, dr = saf.bwd_pattern(v, o, gd, lse, x.replaced, a, r)
    torch.cuda.synchronize()
    gda, gdr = cpu64(da), cpu64(dr)
    reps = [h for h, z in enumerate(x.replaced) if z]
    ref = oracle.pattern_grad(x.v, x.dout, x.replaced, x.a, x.r, heads=[reps[0], reps[-1]])
    for h, (rda, rdr) in ref.items():
        e1, e2 = vec_err(gda[h], rda), vec_err(gdr[h], rdr)
        l1, l2 = rel_l2(gda[h], rda), rel_l2(gdr[h], rdr)
        print("full head %d: da err %.2e (rel-L2 %.2e), dr err %.2e (rel-L2 %.2e)"
              % (h, e1, l1, e2, l2), flush=True)
        assert max(e1, e2, l1, l2) <= TOL[torch.bfloat16]
    for h in reps:
        scale = np.abs(gda[h]).max() * np.sqrt(w.T)
        assert abs(gda[h].sum()) <= 1e-2 * scale and abs(gdr[h].sum()) <= 1e-2 * scale
