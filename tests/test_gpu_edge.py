"""Edge cases of the mixed layer on the GPU: wide score ranges for the online softmax, what replaced
heads must never read, degenerate patterns, a pattern longer than the input, repeatability, and a
non-default stream."""
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, Worst, check_bwd, check_fwd, dq_uncancelled_scale, sample_rows

pytestmark = pytest.mark.gpu


def _saf():
    import fixed_pattern_mixed_amd as saf
    return saf


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("trend", ["rising", "falling", "spiky"])
def test_wide_score_ranges(dtype, trend):
    """Ordinary scores over a range of ~200 log2 units: the forward's lazily updated row maximum
    moves on almost every subtile (rising), is set by the first key (falling), or meets jumps whose
    probabilities overflow fp32 before the rescale (spiky); forward and backward must still match
    the oracle's softmax.  With rows this peaked, dS = P o (dP - delta) nearly cancels wherever P
    is close to 1, so many dQ and dK rows are judged on their uncancelled terms (gpu_util notes),
    and many dV rows sum terms that underflow fp32 (the flush floor)."""
    saf = _saf()
    T = 300
    x = synth.score_range_inputs(T, 64, dtype, trend)
    g = synth.score_range_inputs(T, 64, dtype, trend, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, g.replaced, g.a, g.r)
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, g.replaced, g.a, g.r)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    tol = TOL[dtype]
    check_fwd(x, o, lse, [(0, 0), (0, 1)], None, tol, trend)
    check_bwd(x, dq, dk, dv, [(0, 0), (0, 1)], None, None, tol, trend)


def test_maximum_length():
    """T = 65536, the largest length the library takes, one ordinary and one replaced head (bf16,
    d = 64): forward rows, dQ rows of the ordinary head and dV rows of the replaced head, sampled
    (always including the first and the last position), against the oracle."""
    saf = _saf()
    T = 65536
    rep = [False, True]
    x = synth.layer_inputs(1, 2, T, 64, torch.bfloat16, rep, ar_std=0.5, seed=65)
    g = synth.layer_inputs(1, 2, T, 64, torch.bfloat16, rep, ar_std=0.5, seed=65, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
    torch.cuda.synchronize()
    rows = sample_rows(T, 64, seed=7)
    check_fwd(x, o, lse, [(0, 0), (0, 1)], rows, TOL[torch.bfloat16], "T=65536")
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    idx = torch.as_tensor(rows, dtype=torch.long, device="cuda")
    rq, _, _ = oracle.head_bwd(0, x.v[0, 0], x.dout[0, 0], q=x.q[0, 0], k=x.k[0, 0], qrows=rows,
                               want_dk=False, want_dv=False)
    wr = Worst("T=65536")
    wr.add(f64(dq[0, 0].index_select(0, idx)), rq, TOL[torch.bfloat16], "dq", T=T, rows=rows,
           rounding=lambda r: dq_uncancelled_scale(x.q[0, 0], x.k[0, 0], x.v[0, 0], x.dout[0, 0], r))
    _, _, rv = oracle.head_bwd(1, x.v[0, 1], x.dout[0, 1], a=x.a[1], r=x.r[1], krows=rows,
                               want_dq=False, want_dk=False)
    wr.add(f64(dv[0, 1].index_select(0, idx)), rv, TOL[torch.bfloat16], "replaced dv", T=T)
    wr.report()
    assert torch.count_nonzero(dq[0, 1]) == 0 and torch.count_nonzero(dk[0, 1]) == 0


def test_maximum_length_with_stored_ds():
    """T = 65536 at bf16, d = 128, one ordinary and one replaced head: the backward keeps dS in
    its workspace (4.3 GB: element offsets past 2^31).  Sampled dQ rows of the ordinary head
    (always including the first and the last position) against the oracle, and dQ, dK, dV against
    the backward that forms S and dP again."""
    saf = _saf()
    T, d = 65536, 128
    rep = [False, True]
    x = synth.layer_inputs(1, 2, T, d, torch.bfloat16, rep, ar_std=0.5, seed=66)
    g = synth.layer_inputs(1, 2, T, d, torch.bfloat16, rep, ar_std=0.5, seed=66, device="cuda")
    assert saf.saf_attn_bwd_ds_workspace_size(saf.SAF_BF16, 1, 2, 2, T, d, 1) > (4 << 30)
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    tr = saf.KernelTrace(capacity=8)
    tr.begin()
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
    tr.end()
    torch.cuda.synchronize()
    tr.collect()
    assert "bwd_dq_ds" in tr.summary()
    tr.close()
    dq2, dk2, dv2 = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r, keep_ds=False)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    err = (dq.double() - dq2.double()).abs().amax(dim=-1)
    scale = dq2.double().abs().amax(dim=-1)
    assert bool(torch.all(err <= TOL[torch.bfloat16] * scale + 1e-30))
    rows = sample_rows(T, 64, seed=8)
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    idx = torch.as_tensor(rows, dtype=torch.long, device="cuda")
    rq, _, _ = oracle.head_bwd(0, x.v[0, 0], x.dout[0, 0], q=x.q[0, 0], k=x.k[0, 0], qrows=rows,
                               want_dk=False, want_dv=False)
    wr = Worst("T=65536 stored dS")
    wr.add(f64(dq[0, 0].index_select(0, idx)), rq, TOL[torch.bfloat16], "dq", T=T, rows=rows,
           rounding=lambda r: dq_uncancelled_scale(x.q[0, 0], x.k[0, 0], x.v[0, 0], x.dout[0, 0], r))
    wr.report()
    assert torch.count_nonzero(dq[0, 1]) == 0 and torch.count_nonzero(dk[0, 1]) == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_replaced_heads_never_read_q_k(dtype):
    saf = _saf()
    B, H, T, d = 2, 4, 190, 64
    rep = synth.replaced_mask(H, 2, "interleaved")
    g = synth.layer_inputs(B, H, T, d, dtype, rep, seed=3, device="cuda")
    o1, l1 = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    d1 = saf.bwd(g.q, g.k, g.v, o1, g.dout, l1, rep, g.a, g.r)
    q2, k2 = g.q.clone(), g.k.clone()
    for h in range(H):
        if rep[h]:
            q2[:, h] = float("nan")
            k2[:, h] = float("nan")
    o2, l2 = saf.fwd(q2, k2, g.v, rep, g.a, g.r)
    d2 = saf.bwd(q2, k2, g.v, o2, g.dout, l2, rep, g.a, g.r)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(d1, d2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("big", [float("-inf"), -1e4])
def test_identity_pattern_copies_v(dtype, big):
    """r[0] = 0 and r[delta >= 1] very negative: the fixed pattern is the identity, so O = V and
    dV = dO (to the parity tolerance; the oracle pins the exact statement)."""
    saf = _saf()
    B, H, T, d = 2, 2, 150, 128
    rep = [1, 1]
    x = synth.layer_inputs(B, H, T, d, dtype, rep, seed=4)
    x.r.fill_(big)
    x.r[:, 0] = 0.0
    g = synth.layer_inputs(B, H, T, d, dtype, rep, seed=4, device="cuda")
    g.r.copy_(x.r)
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)]
    check_fwd(x, o, lse, heads, None, TOL[dtype], "identity")
    check_bwd(x, dq, dk, dv, heads, None, None, TOL[dtype], "identity")
    assert float((o.float() - g.v.float()).abs().max()) <= TOL[dtype] * float(g.v.float().abs().max())


def test_pattern_longer_than_input_uses_prefix():
    saf = _saf()
    B, H, T, d = 1, 4, 100, 64
    rep = synth.replaced_mask(H, 2)
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, seed=6, device="cuda", pat_len=333)
    o1, l1 = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    o2, l2 = saf.fwd(g.q, g.k, g.v, rep, g.a[:, :T].contiguous(), g.r[:, :T].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# a quarter of the heads replaced (the replaced-only key/value heads in bwd_kv's second section), half
# replaced (bwd_dv_rep), and bf16 d = 128 on a grid of 8-wave items (paired replaced forward items)
REPEAT = [(2, 12, 700, 64, 3), (2, 12, 700, 64, 6), (2, 16, 2048, 128, 4), (1, 16, 1000, 128, 8)]


@pytest.mark.parametrize("B,H,T,d,R", REPEAT, ids=["B%dH%dT%dd%dR%d" % c for c in REPEAT])
def test_bitwise_repeatable(B, H, T, d, R):
    """Every output element is written by one work item and summed in a fixed order."""
    saf = _saf()
    rep = synth.replaced_mask(H, R)
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, seed=8, device="cuda")
    outs = []
    for _ in range(2):
        o, l = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
        outs.append((o, l) + saf.bwd(g.q, g.k, g.v, o, g.dout, l, rep, g.a, g.r))
    torch.cuda.synchronize()
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def test_non_default_stream():
    saf = _saf()
    B, H, T, d = 1, 4, 333, 128
    rep = synth.replaced_mask(H, 1)
    x = synth.layer_inputs(B, H, T, d, torch.float32, rep, seed=9)
    g = synth.layer_inputs(B, H, T, d, torch.float32, rep, seed=9, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
        dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
    s.synchronize()
    heads = [(0, h) for h in range(H)]
    check_fwd(x, o, lse, heads, None, TOL[torch.float32], "stream")
    check_bwd(x, dq, dk, dv, heads, None, None, TOL[torch.float32], "stream")


def test_empty_batch_is_noop():
    saf = _saf()
    g = synth.layer_inputs(0, 4, 64, 64, torch.bfloat16, [0, 0, 0, 1], seed=1, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, [0, 0, 0, 1], g.a, g.r)
    assert o.shape == (0, 4, 64, 64)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prepared_pattern_matches_call_prepared(dtype):
    saf = _saf()
    B, H, T, d = 2, 4, 300, 64
    rep = synth.replaced_mask(H, 2)
    g = synth.layer_inputs(B, H, T, d, dtype, rep, seed=12, device="cuda")
    pat = saf.prepare_pattern(rep, g.a, g.r)
    o1, l1 = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    o2, l2 = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r, pattern=pat)
    d1 = saf.bwd(g.q, g.k, g.v, o1, g.dout, l1, rep, g.a, g.r)
    d2 = saf.bwd(g.q, g.k, g.v, o2, g.dout, l2, rep, g.a, g.r, pattern=pat)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(d1, d2):
        assert torch.equal(x, y)


def test_pattern_prepared_longer_than_input():
    """A pattern prepared at its fitted length serves a shorter input (row i only sees <= i)."""
    saf = _saf()
    B, H, T, d, P = 1, 4, 100, 64, 333
    rep = synth.replaced_mask(H, 2)
    x = synth.layer_inputs(B, H, T, d, torch.float32, rep, seed=13, pat_len=P)
    g = synth.layer_inputs(B, H, T, d, torch.float32, rep, seed=13, device="cuda", pat_len=P)
    pat = saf.prepare_pattern(rep, g.a, g.r)
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r, pattern=pat)
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r, pattern=pat)
    torch.cuda.synchronize()
    heads = [(0, h) for h in range(H)]
    check_fwd(x, o, lse, heads, None, TOL[torch.float32], "prefix")
    check_bwd(x, dq, dk, dv, heads, None, None, TOL[torch.float32], "prefix")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_wide_range_pattern_uses_exponential_form(dtype):
    """A pattern whose factorised weights would underflow (one key preferred by 200 nats, so
    exp(a - max a) is 0 in fp32 for every other key) must still match the oracle: the kernels
    switch to exp(a[j] + r[i-j] - log Z(i)) for such a head."""
    saf = _saf()
    B, H, T, d = 1, 4, 257, 64
    rep = [0, 1, 0, 1]
    x = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=1.0, seed=14)
    x.a[1, T - 1] = 200.0
    x.a[3, 5] = 150.0
    x.r[3, 7] = -300.0
    g = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=1.0, seed=14, device="cuda")
    g.a.copy_(x.a)
    g.r.copy_(x.r)
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
    torch.cuda.synchronize()
    heads = [(0, h) for h in range(H)]
    check_fwd(x, o, lse, heads, None, TOL[dtype], "wide")
    check_bwd(x, dq, dk, dv, heads, None, None, TOL[dtype], "wide")


@pytest.mark.parametrize("overlap,d", [(0, 64), (1, 64), (0, 128)])
def test_graph_capture_of_forward_and_backward_replays_exactly(overlap, d):
    """fwd + bwd captured into a HIP graph (with overlap on, the backward forks its query-block
    kernel onto a side stream and joins back; at d = 128 the backward keeps dS in its workspace)
    replay to the bits of the eager calls, with eager work between replays."""
    saf = _saf()
    saf.saf_set_backward_overlap(overlap)
    B, H, T = 2, 4, 300
    rep = [0, 1, 0, 1]
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, seed=17, device="cuda")
    pat = saf.prepare_pattern(rep, g.a, g.r)
    o0, l0 = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r, pattern=pat)
    d0 = saf.bwd(g.q, g.k, g.v, o0, g.dout, l0, rep, g.a, g.r, pattern=pat)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):  # warm up on the capture stream
        o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r, pattern=pat)
        dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r, pattern=pat)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cs):
        o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r, pattern=pat)
        dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r, pattern=pat)
    for it in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(lse, l0), it
        assert torch.equal(dq, d0[0]) and torch.equal(dk, d0[1]) and torch.equal(dv, d0[2]), it
        saf.fwd(g.q, g.k, g.v, rep, g.a, g.r, pattern=pat)  # eager work between replays
        torch.cuda.synchronize()
    saf.saf_set_backward_overlap(0)


def test_backward_overlap_gives_the_same_bits():
    saf = _saf()
    B, H, T, d = 2, 6, 700, 64
    rep = [0, 1, 0, 0, 1, 0]
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, seed=19, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    serial = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
    saf.saf_set_backward_overlap(1)
    try:
        over = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
        torch.cuda.synchronize()
    finally:
        saf.saf_set_backward_overlap(0)
    for x, y in zip(serial, over):
        assert torch.equal(x, y)
