"""Backward of the mixed layer on the GPU (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import TOL, check_bwd, pick_heads, sample_rows

pytestmark = pytest.mark.gpu


def _saf():
    import fixed_pattern_mixed_amd as saf
    return saf


SMALL = [
    (1, 4, 256, 64, torch.float32, 1, "interleaved", 1.0),
    (1, 2, 1, 64, torch.float32, 1, "interleaved", 1.0),
    (2, 4, 17, 128, torch.float32, 2, "contiguous", 1.0),
    (1, 4, 300, 64, torch.float32, 4, "all", 3.0),
    (2, 3, 129, 128, torch.float32, 0, "interleaved", 0.5),
    (2, 4, 300, 64, torch.bfloat16, 2, "interleaved", 0.5),
    (1, 4, 257, 128, torch.bfloat16, 1, "contiguous", 0.5),
    (1, 12, 520, 64, torch.bfloat16, 6, "interleaved", 0.5),
]


@pytest.mark.parametrize("B,H,T,d,dtype,R,placement,std", SMALL,
                         ids=["B%dH%dT%dd%d-%s-R%d-%s" % (c[0], c[1], c[2], c[3], str(c[4])[6:], c[5], c[6]) for c in SMALL])
def test_backward_small_full_compare(B, H, T, d, dtype, R, placement, std):
    saf = _saf()
    rep = synth.replaced_mask(H, R, placement)
    x = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=std, seed=23 + T)
    g = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=std, seed=23 + T, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)]
    check_bwd(x, dq, dk, dv, heads, None, None, TOL[dtype], "small")


FULL = ["l124m_t4096", "l124m_t8192", "l1b_t8192"]


@pytest.mark.parametrize("name", FULL)
def test_backward_full_size_sampled(name):
    saf = _saf()
    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w)
    print("workload", name, flush=True)
    q, k, v, g, a, r = (t.to("cuda") for t in (x.q, x.k, x.v, x.dout, x.a, x.r))
    o, lse = saf.fwd(q, k, v, x.replaced, a, r)
    dq, dk, dv = saf.bwd(q, k, v, o, g, lse, x.replaced, a, r)
    torch.cuda.synchronize()
    rows = sample_rows(w.T, 24, seed=w.index + 7)
    heads = pick_heads(w.B, x.replaced, n_each=1)
    check_bwd(x, dq, dk, dv, heads, rows, rows, TOL[w.torch_dtype], name)
    # every replaced head of every batch entry: dq and dk are exactly zero
    for h, isrep in enumerate(x.replaced):
        if isrep:
            assert torch.count_nonzero(dq[:, h]) == 0 and torch.count_nonzero(dk[:, h]) == 0
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dv.float()).all()
