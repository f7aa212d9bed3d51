"""Backward of the mixed layer on the GPU (through the C ABI) against the fp64 oracle, row by row."""
import pytest
import torch

import synth
from gpu_util import TOL, Worst, all_heads, check_bwd

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
    # bf16 d = 64 with every head replaced: the replaced-only key/value kernel alone (wide-range
    # patterns: product and exponential forms), ragged T
    (1, 4, 300, 64, torch.bfloat16, 4, "all", 3.0),
    # bf16, half the heads replaced (the replaced-only key/value heads in bwd_dv_rep beside the
    # key-block kernel): one position, and a length shorter than one 256-key item at d = 128
    (1, 4, 1, 64, torch.bfloat16, 2, "interleaved", 0.5),
    (2, 4, 200, 128, torch.bfloat16, 2, "contiguous", 1.0),
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
    check_bwd(x, dq, dk, dv, all_heads(B, H), None, None, TOL[dtype], "small")


# Every fwd+bwd workload of the benchmark table, in the launch configuration the benchmark times
# (inputs resident on the GPU, the pattern prepared once and passed in), compared in full: every
# dQ row and every dK / dV row of every slice.
FULL = ["l124m_t4096", "l124m_t8192", "l1b_t8192"]


@pytest.mark.parametrize("name", FULL)
def test_backward_full_size_full_compare(name):
    saf = _saf()
    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w)
    print("workload", name, flush=True)
    q, k, v, g, a, r = (t.to("cuda") for t in (x.q, x.k, x.v, x.dout, x.a, x.r))
    pat = saf.prepare_pattern(x.replaced, a, r)
    o, lse = saf.fwd(q, k, v, x.replaced, a, r, pattern=pat)
    dq, dk, dv = saf.bwd(q, k, v, o, g, lse, x.replaced, a, r, pattern=pat)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    del q, k, v, g, o, lse
    wr = Worst("bwd full " + name)
    check_bwd(x, dq, dk, dv, all_heads(w.B, w.H), None, None, TOL[w.torch_dtype], name, worst=wr)
    wr.report(workload=name)


# bf16 at d = 128 the backward keeps dS in a larger workspace (bwd_kv stores it, bwd_dq_ds reads
# it) instead of forming S and dP a second time for dQ.  Both paths against each other: dK and dV
# come from the same key-block arithmetic (bitwise equal), dQ from the same bf16 dS summed in the
# same key order; each dQ row is held to the bf16 tolerance on its own scale.  The parity tests
# above and the full-size compare run the stored-dS path against the oracle.
DS_CASES = [
    (1, 4, 257, 1, "contiguous"),
    (2, 3, 97, 0, "interleaved"),
    (1, 2, 1, 1, "interleaved"),
    (2, 4, 520, 3, "contiguous"),
    (1, 16, 1000, 4, "interleaved"),
    (3, 2, 33, 0, "interleaved"),
]


@pytest.mark.parametrize("B,H,T,R,placement", DS_CASES,
                         ids=["B%dH%dT%d-R%d" % (c[0], c[1], c[2], c[3]) for c in DS_CASES])
def test_stored_ds_path_matches_the_recomputing_path(B, H, T, R, placement):
    saf = _saf()
    d = 128
    rep = synth.replaced_mask(H, R, placement)
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, ar_std=0.5, seed=71 + T, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    torch.cuda.synchronize()
    outs, names = [], []
    for keep in (True, False):
        tr = saf.KernelTrace(capacity=8)
        tr.begin()
        outs.append(saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r, keep_ds=keep))
        tr.end()
        torch.cuda.synchronize()
        tr.collect()
        names.append(set(tr.summary()))
        tr.close()
    assert "bwd_dq_ds" in names[0] and "bwd_dq" not in names[0], names[0]
    assert "bwd_dq" in names[1] and "bwd_dq_ds" not in names[1], names[1]
    (dq1, dk1, dv1), (dq2, dk2, dv2) = outs
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    x, y = dq1.double(), dq2.double()
    scale = y.abs().amax(dim=-1, keepdim=True)
    err = (x - y).abs().amax(dim=-1, keepdim=True)
    assert bool(torch.all(err <= TOL[torch.bfloat16] * scale + 1e-30)), float((err / scale.clamp_min(1e-30)).max())
    print("dQ bitwise equal between the paths:", torch.equal(dq1, dq2), flush=True)


# The stored-dS backward against the oracle, every row of every slice: with the pattern prepared
# once and passed in (the benchmark's launch configuration), with wide-range patterns (std 3: the
# exponential form on the replaced heads beside the stored dS of the ordinary ones), and with more
# heads and sequences than one 8-wave item covers.
DS_ORACLE = [
    (2, 4, 300, 1, "interleaved", 0.5, True),
    (1, 4, 257, 2, "contiguous", 3.0, False),
    (4, 8, 160, 2, "interleaved", 0.5, False),
    (1, 3, 640, 0, "interleaved", 0.5, False),
]


@pytest.mark.parametrize("B,H,T,R,placement,std,prepared", DS_ORACLE,
                         ids=["B%dH%dT%d-R%d-std%g%s" % (c[0], c[1], c[2], c[3], c[5], "-prep" if c[6] else "") for c in DS_ORACLE])
def test_stored_ds_backward_full_compare(B, H, T, R, placement, std, prepared):
    saf = _saf()
    d = 128
    rep = synth.replaced_mask(H, R, placement)
    x = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, ar_std=std, seed=91 + T)
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, ar_std=std, seed=91 + T, device="cuda")
    pat = saf.prepare_pattern(rep, g.a, g.r) if prepared and R else None
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r, pattern=pat)
    tr = saf.KernelTrace(capacity=8)
    tr.begin()
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r, pattern=pat)
    tr.end()
    torch.cuda.synchronize()
    tr.collect()
    assert "bwd_dq_ds" in tr.summary()
    tr.close()
    check_bwd(x, dq, dk, dv, all_heads(B, H), None, None, TOL[torch.bfloat16], "stored dS")


def test_stored_ds_needs_the_whole_room():
    """Through the C ABI: with ws_bytes one short of saf_attn_bwd_ds_workspace_size the backward
    takes the re-forming path (bwd_dq), with the full size the stored-dS path (bwd_dq_ds); the
    results agree (dK, dV bitwise, dQ row by row)."""
    saf = _saf()
    B, H, T, d = 2, 4, 300, 128
    rep = [0, 1, 0, 0]
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, seed=44, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    big = saf.saf_attn_bwd_ds_workspace_size(saf.SAF_BF16, B, H, H, T, d, sum(rep))
    assert big > saf.saf_attn_bwd_workspace_size(B, H, T, d)
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    outs, names = [], []
    for n in (big - 1, big):
        out = tuple(torch.full_like(g.q, float("nan")) for _ in range(3))
        tr = saf.KernelTrace(capacity=8)
        tr.begin()
        st = saf.saf_attn_bwd(saf.SAF_BF16, B, H, T, d, g.q.data_ptr(), g.k.data_ptr(), g.v.data_ptr(),
                              o.data_ptr(), g.dout.data_ptr(), lse.data_ptr(), saf._mask(rep, H),
                              g.a.data_ptr(), g.r.data_ptr(), T, None, 0.0, out[0].data_ptr(),
                              out[1].data_ptr(), out[2].data_ptr(), ws.data_ptr(), n,
                              torch.cuda.current_stream().cuda_stream)
        tr.end()
        assert st == saf.SAF_OK, saf.saf_last_error()
        torch.cuda.synchronize()
        tr.collect()
        names.append(set(tr.summary()))
        tr.close()
        outs.append(out)
    assert "bwd_dq" in names[0] and "bwd_dq_ds" not in names[0]
    assert "bwd_dq_ds" in names[1] and "bwd_dq" not in names[1]
    (dq1, dk1, dv1), (dq2, dk2, dv2) = outs
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    err = (dq1.double() - dq2.double()).abs().amax(dim=-1)
    assert bool(torch.all(err <= TOL[torch.bfloat16] * dq1.double().abs().amax(dim=-1) + 1e-30))


def test_binding_falls_back_beyond_its_cap(monkeypatch):
    """bwd() passes the smaller workspace when the stored dS would need more than
    DS_WORKSPACE_MAX bytes: the backward then forms S and dP again (bwd_dq), with the same dK, dV."""
    saf = _saf()
    B, H, T, d = 1, 4, 200, 128
    rep = [0, 1, 0, 0]
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, seed=45, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    outs, names = [], []
    for cap in (saf.DS_WORKSPACE_MAX, 1024):
        monkeypatch.setattr(saf, "DS_WORKSPACE_MAX", cap)
        tr = saf.KernelTrace(capacity=8)
        tr.begin()
        outs.append(saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r))
        tr.end()
        torch.cuda.synchronize()
        tr.collect()
        names.append(set(tr.summary()))
        tr.close()
    assert "bwd_dq_ds" in names[0] and "bwd_dq" in names[1] and "bwd_dq_ds" not in names[1]
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])
