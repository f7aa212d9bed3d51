"""Forward of the mixed layer on the GPU (through the C ABI) against the fp64 oracle, row by row."""
import pytest
import torch

import synth
from gpu_util import TOL, Worst, all_heads, check_bwd, check_fwd, sample_rows

pytestmark = pytest.mark.gpu


def _saf():
    import fixed_pattern_mixed_amd as saf
    return saf


SMALL = [
    # B, H, T, d, dtype, n_replaced, placement, ar_std
    (1, 4, 256, 64, torch.float32, 1, "interleaved", 1.0),   # the tiny fp32 workload
    (1, 4, 1, 64, torch.float32, 1, "interleaved", 1.0),
    (2, 4, 17, 64, torch.float32, 2, "contiguous", 1.0),
    (1, 2, 257, 128, torch.float32, 1, "interleaved", 1.0),
    (1, 4, 300, 64, torch.float32, 4, "all", 3.0),            # all replaced, wide logits
    (2, 3, 129, 128, torch.float32, 0, "interleaved", 0.5),   # all ordinary
    (2, 4, 300, 64, torch.bfloat16, 2, "interleaved", 0.5),
    (1, 4, 255, 128, torch.bfloat16, 1, "contiguous", 0.5),
    (3, 2, 64, 64, torch.bfloat16, 2, "all", 0.5),
    (1, 12, 520, 64, torch.bfloat16, 3, "interleaved", 0.5),
]


@pytest.mark.parametrize("B,H,T,d,dtype,R,placement,std", SMALL,
                         ids=["B%dH%dT%dd%d-%s-R%d-%s" % (c[0], c[1], c[2], c[3], str(c[4])[6:], c[5], c[6]) for c in SMALL])
def test_forward_small_full_compare(B, H, T, d, dtype, R, placement, std):
    saf = _saf()
    rep = synth.replaced_mask(H, R, placement)
    x = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=std, seed=11 + T, backward=False)
    g = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=std, seed=11 + T, backward=False,
                           device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    torch.cuda.synchronize()
    check_fwd(x, o, lse, all_heads(B, H), None, TOL[dtype], "small")


# The forward cuts a (batch, head) into work items of 8, 4 or 2 waves (256, 128 or 64 queries): the
# widest whose grid still has 256 items.  The shapes below reach each width with a ragged last block.
def _waves(B, H, T):
    for w in (8, 4):
        if B * H * -(-T // (32 * w)) >= 256:
            return w
    return 2


WIDTHS = [
    # B, H, T, d, dtype, n_replaced
    (8, 8, 1000, 64, torch.bfloat16, 2),
    (8, 8, 1000, 128, torch.float32, 2),
    (2, 4, 4000, 64, torch.bfloat16, 1),
    (2, 4, 4000, 128, torch.float32, 2),
    (2, 4, 4000, 128, torch.bfloat16, 1),
    (1, 4, 2000, 64, torch.bfloat16, 1),
    (1, 4, 2000, 128, torch.bfloat16, 2),
    (1, 3, 1500, 64, torch.float32, 1),
]


@pytest.mark.parametrize("B,H,T,d,dtype,R", WIDTHS,
                         ids=["W%d-B%dH%dT%dd%d-%s" % (_waves(c[0], c[1], c[2]), c[0], c[1], c[2], c[3], str(c[4])[6:]) for c in WIDTHS])
def test_forward_each_work_item_width(B, H, T, d, dtype, R):
    saf = _saf()
    rep = synth.replaced_mask(H, R, "interleaved")
    x = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=0.5, seed=T + d, backward=False)
    g = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=0.5, seed=T + d, backward=False,
                           device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    torch.cuda.synchronize()
    rows = sample_rows(T, 64, seed=d)
    check_fwd(x, o, lse, all_heads(B, H), rows, TOL[dtype], "W%d" % _waves(B, H, T))


def run_workload_fwd(saf, w, x):
    """The forward exactly as the benchmark launches it: inputs resident on the GPU, the replaced
    heads' pattern prepared once and passed in.  Returns (o, lse) on the CPU."""
    q, k, v, a, r = (t.to("cuda") for t in (x.q, x.k, x.v, x.a, x.r))
    pat = saf.prepare_pattern(x.replaced, a, r) if any(x.replaced) else None
    o, lse = saf.fwd(q, k, v, x.replaced, a, r, pattern=pat)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


# Every forward workload of the benchmark table, compared in full (every row of every slice).
FULL = ["l124m_t4096", "l124m_t8192", "l1b_t8192", "prefill_b64_t4096", "prefill_b2_t16384"]


@pytest.mark.parametrize("name", FULL)
def test_forward_full_size_full_compare(name):
    saf = _saf()
    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w)
    print("workload", name, flush=True)
    o, lse = run_workload_fwd(saf, w, x)
    wr = Worst("fwd full " + name)
    check_fwd(x, o, lse, all_heads(w.B, w.H), None, TOL[w.torch_dtype], name, worst=wr)
    wr.report(workload=name)


# Launch-bound and grouped shapes: every slice on 64 sampled rows (rows 0 and T-1 included).
SAMPLED = ["prefill_b1_t4096"]


@pytest.mark.parametrize("name", SAMPLED)
def test_forward_full_size_sampled(name):
    saf = _saf()
    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w)
    print("workload", name, flush=True)
    o, lse = run_workload_fwd(saf, w, x)
    rows = sample_rows(w.T, 64, seed=w.index)
    wr = Worst("fwd sampled " + name)
    check_fwd(x, o, lse, all_heads(w.B, w.H), rows, TOL[w.torch_dtype], name, worst=wr)
    wr.report(workload=name)


# bf16 with 8-wave items (grids of at least 256 items).  At d = 128 a replaced head's item covers two
# query blocks (each wave one 32-query subtile in each); at d = 64, with a third or more of the heads
# replaced, the backward runs the replaced-only key blocks in a kernel of their own (bwd_dv_rep).
# Product form on a ragged length (the last query block pair reaches past T), and the exponential
# form (a pattern whose factorised weights underflow).
PAIRED = [
    # B, H, T, wide-range pattern, d, replaced heads (interleaved)
    (4, 16, 4000, False, 128, 4),
    (2, 16, 2048, True, 128, 4),
    (4, 8, 2100, False, 64, 4),
    (2, 16, 2304, True, 64, 16),
]


@pytest.mark.parametrize("B,H,T,wide,d,R", PAIRED,
                         ids=["B%dH%dT%d-d%d-R%d-%s" % (c[0], c[1], c[2], c[4], c[5], "exp" if c[3] else "prod") for c in PAIRED])
def test_replaced_items_covering_two_query_blocks(B, H, T, wide, d, R):
    saf = _saf()
    dtype = torch.bfloat16
    rep = synth.replaced_mask(H, R, "interleaved")
    x = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=0.5, seed=71 + T)
    if wide:  # one key preferred by 200 nats: exp(a - max a) is 0 in fp32 for every other key
        for h in range(H):
            if rep[h]:
                x.a[h, T - 1] = 200.0
    g = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=0.5, seed=71 + T, device="cuda")
    g.a.copy_(x.a)
    g.r.copy_(x.r)
    pat = saf.prepare_pattern(rep, g.a, g.r)
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r, pattern=pat)
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r, pattern=pat)
    torch.cuda.synchronize()
    print("B%d H%d T%d wide=%s" % (B, H, T, wide), flush=True)
    # every replaced slice and one ordinary slice per batch entry; rows of both query blocks of
    # every pair, the last ones included
    heads = sorted(set([(b, h) for b in range(B) for h in range(H) if rep[h]] + [(b, 0) for b in range(B)]))
    rows = sample_rows(T, 96, seed=T)
    wr = Worst("paired B%dH%dT%d" % (B, H, T))
    check_fwd(x, o, lse, heads, rows, TOL[dtype], "paired fwd", worst=wr)
    check_bwd(x, dq, dk, dv, [(b, h) for b in range(B) for h in range(H) if rep[h]], rows, rows,
              TOL[dtype], "paired bwd", worst=wr)
    wr.report()
