"""Forward of the mixed layer on the GPU (through the C ABI) against the fp64 oracle."""
import pytest
import torch

import synth
from gpu_util import TOL, check_fwd, pick_heads, sample_rows

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
    heads = [(b, h) for b in range(B) for h in range(H)]
    check_fwd(x, o, lse, heads, None, TOL[dtype], "small")


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
    rows = sample_rows(T, 48, seed=d)
    heads = pick_heads(B, rep, n_each=2)
    check_fwd(x, o, lse, heads, rows, TOL[dtype], "W%d" % _waves(B, H, T))


FULL = ["l124m_t4096", "l124m_t8192", "l1b_t8192", "prefill_b64_t4096", "prefill_b2_t16384",
        "prefill_b1_t4096"]


@pytest.mark.parametrize("name", FULL)
def test_forward_full_size_sampled(name):
    saf = _saf()
    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w)
    print("workload", name, flush=True)
    q, k, v, a, r = (t.to("cuda") for t in (x.q, x.k, x.v, x.a, x.r))
    o, lse = saf.fwd(q, k, v, x.replaced, a, r)
    torch.cuda.synchronize()
    rows = sample_rows(w.T, 40, seed=w.index)
    heads = pick_heads(w.B, x.replaced, n_each=2)
    check_fwd(x, o, lse, heads, rows, TOL[w.torch_dtype], name)
