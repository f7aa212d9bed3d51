"""Grouped key/value heads (GQA: several query heads share one key/value head; [Notes §二.4]) on
the GPU through the C ABI, against the oracle mapped over the groups."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, TOL_LSE, Worst, cpu64, dq_uncancelled_scale, sample_rows

pytestmark = pytest.mark.gpu


def _saf():
    import fixed_pattern_mixed_amd as saf
    return saf


def _compare(x, rep, o, lse, dq, dk, dv, tol, tol_lse, batches=None, kv_heads=None, rows=None,
             what=""):
    B, H = x.q.shape[:2]
    Hkv = x.k.shape[1]
    G = H // Hkv
    batches = range(B) if batches is None else batches
    kv_heads = range(Hkv) if kv_heads is None else kv_heads
    heads = [(b, h) for b in batches for hk in kv_heads for h in range(hk * G, (hk + 1) * G)]
    ridx = slice(None) if rows is None else rows
    ref = oracle.layer_fwd_gqa(x.q, x.k, x.v, rep, x.a, x.r, heads=heads, rows=rows)
    go, gl = cpu64(o), cpu64(lse)
    wr = Worst("gqa " + what)
    for (b, h), (ro, rl) in ref.items():
        wr.add(go[b, h][ridx], ro, tol, "o[b=%d,h=%d]" % (b, h), T=x.v.shape[2])
        wr.add_lse(gl[b, h][ridx], rl, tol_lse, "lse[b=%d,h=%d]" % (b, h))
    if dq is None:
        wr.report()
        return
    rq, rk, rv = oracle.layer_bwd_gqa(x.q, x.k, x.v, x.dout, rep, x.a, x.r, batches=batches,
                                      kv_heads=kv_heads, qrows=rows, krows=rows)
    gq, gk, gv = cpu64(dq), cpu64(dk), cpu64(dv)
    for (b, h), ref_q in rq.items():
        if rep[h]:
            assert np.all(gq[b, h][ridx] == 0.0), (what, "dq", b, h)
        else:
            # rows of exact zeros in the reference (row 0, where P = 1 and dS = 0) are measured
            # on the inputs' unit scale, rows with few keys that fail their own scale against
            # their uncancelled terms (gpu_util notes)
            T = x.v.shape[2]
            rws = np.arange(T, dtype=np.int32) if rows is None else rows
            args = (x.q[b, h], x.k[b, h // G], x.v[b, h // G], x.dout[b, h])
            wr.add(gq[b, h][ridx], ref_q, tol, "dq[b=%d,h=%d]" % (b, h), T=T, rows=rws,
                   rounding=lambda r, a=args: dq_uncancelled_scale(*a, r))
    for (b, hk), ref_k in rk.items():
        if all(rep[h] for h in range(hk * G, (hk + 1) * G)):  # every head replaced: exactly zero
            assert np.all(gk[b, hk][ridx] == 0.0), (what, "dk", b, hk)
        else:
            wr.add(gk[b, hk][ridx], ref_k, tol, "dk[b=%d,hk=%d]" % (b, hk), T=x.v.shape[2])
        wr.add(gv[b, hk][ridx], rv[(b, hk)], tol, "dv[b=%d,hk=%d]" % (b, hk), T=x.v.shape[2])
    wr.report()


SMALL = [
    # B, H, Hkv, T, d, dtype, replaced
    (2, 8, 2, 300, 64, torch.bfloat16, [0, 1, 0, 0, 1, 1, 1, 1]),
    (1, 4, 1, 257, 128, torch.float32, [0, 0, 1, 0]),
    (2, 6, 3, 200, 64, torch.float32, [1, 0, 0, 1, 1, 1]),
    (1, 8, 4, 129, 128, torch.bfloat16, [0, 0, 0, 0, 0, 0, 0, 0]),
    (1, 4, 2, 1, 64, torch.float32, [0, 1, 1, 0]),
    # bf16 d = 128 (the 8-wave key-block kernel): a group of ordinary and replaced heads, and a
    # group whose heads are all replaced (its replaced-only sweep, key factors in every entry)
    (1, 8, 2, 257, 128, torch.bfloat16, [0, 0, 0, 1, 1, 1, 1, 1]),
]


@pytest.mark.parametrize("B,H,Hkv,T,d,dtype,rep", SMALL,
                         ids=["B%dH%dkv%dT%dd%d-%s" % (c[0], c[1], c[2], c[3], c[4], str(c[5])[6:]) for c in SMALL])
def test_gqa_small_full_compare(B, H, Hkv, T, d, dtype, rep):
    saf = _saf()
    x = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=0.5, seed=71 + T, Hkv=Hkv)
    g = synth.layer_inputs(B, H, T, d, dtype, rep, ar_std=0.5, seed=71 + T, Hkv=Hkv, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    dq, dk, dv = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
    torch.cuda.synchronize()
    assert dk.shape == g.k.shape and dq.shape == g.q.shape
    _compare(x, rep, o, lse, dq, dk, dv, TOL[dtype], 1e-4 if dtype == torch.float32 else 2.0 ** -8,
             what="small")


def test_gqa_with_one_query_head_per_group_is_the_plain_layer():
    """saf_attn_fwd_gqa / saf_attn_bwd_gqa with Hkv = H give the bits of saf_attn_fwd / _bwd."""
    saf = _saf()
    B, H, T, d = 2, 4, 300, 64
    rep = [0, 1, 0, 1]
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, seed=5, device="cuda")
    o1, l1 = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)  # the binding calls the grouped entry point
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    n = saf.saf_attn_fwd_workspace_size(B, H, T, d)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    st = saf.saf_attn_fwd(saf.SAF_BF16, B, H, T, d, g.q.data_ptr(), g.k.data_ptr(), g.v.data_ptr(),
                          saf._mask(rep, H), g.a.data_ptr(), g.r.data_ptr(), T, None, 0.0,
                          o2.data_ptr(), l2.data_ptr(), ws.data_ptr(), n,
                          torch.cuda.current_stream().cuda_stream)
    assert st == saf.SAF_OK
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_plain_backward_export_matches_the_grouped_one(dtype):
    """saf_attn_bwd (no grouping argument), called directly through the C ABI, writes the bits of
    saf_attn_bwd_gqa with Hkv = H (what the binding calls), for a layer with both head kinds."""
    saf = _saf()
    B, H, T, d = 2, 4, 300, 128 if dtype == torch.float32 else 64
    rep = [0, 1, 0, 1]
    g = synth.layer_inputs(B, H, T, d, dtype, rep, seed=6, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    dq1, dk1, dv1 = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r)
    dq2, dk2, dv2 = (torch.full_like(g.q, float("nan")) for _ in range(3))
    n = saf.saf_attn_bwd_workspace_size(B, H, T, d)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    code = saf.SAF_BF16 if dtype == torch.bfloat16 else saf.SAF_F32
    st = saf.saf_attn_bwd(code, B, H, T, d, g.q.data_ptr(), g.k.data_ptr(), g.v.data_ptr(),
                          o.data_ptr(), g.dout.data_ptr(), lse.data_ptr(), saf._mask(rep, H),
                          g.a.data_ptr(), g.r.data_ptr(), T, None, 0.0, dq2.data_ptr(),
                          dk2.data_ptr(), dv2.data_ptr(), ws.data_ptr(), n,
                          torch.cuda.current_stream().cuda_stream)
    assert st == saf.SAF_OK, saf.saf_last_error()
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)


def test_gqa_rejects_groups_that_do_not_divide():
    saf = _saf()
    rep = (ctypes.c_uint8 * 6)(*[0] * 6)
    fake = 0x100000
    st = saf.saf_attn_fwd_gqa(saf.SAF_BF16, 1, 6, 4, 64, 64, fake, fake, fake, rep, fake, fake, 64,
                              None, 0.0, fake, fake, fake, 1 << 20, None)
    assert st == saf.SAF_ERR_INVALID_ARG and "Hkv" in saf.saf_last_error()


def test_gqa_full_size_sampled():
    """The Qwen3-4B-shaped grouped prefill (B=1, 32 query heads over 8 key/value heads, T=4096,
    d=128, bf16, one replaced head per group): forward on sampled rows of two groups, and the
    backward of one group (dq of its 4 query heads, dk and dv of the shared head) on sampled rows."""
    saf = _saf()
    w = synth.WORKLOADS["qwen4b_gqa_t4096"]
    rep = w.replaced()
    x = synth.layer_inputs(w.B, w.H, w.T, w.d, w.torch_dtype, rep, w.ar_std, synth.SEED0 + w.index,
                           backward=True, Hkv=w.Hkv)
    print("workload", w.name, flush=True)
    q, k, v, gd, a, r = (t.to("cuda") for t in (x.q, x.k, x.v, x.dout, x.a, x.r))
    o, lse = saf.fwd(q, k, v, rep, a, r)
    dq, dk, dv = saf.bwd(q, k, v, o, gd, lse, rep, a, r)
    torch.cuda.synchronize()
    rows = sample_rows(w.T, 64, seed=3)
    _compare(x, rep, o, lse, None, None, None, TOL[torch.bfloat16], TOL_LSE[torch.bfloat16],
             batches=[0], kv_heads=[0, w.Hkv - 1], rows=rows, what="full fwd")
    _compare(x, rep, o, lse, dq, dk, dv, TOL[torch.bfloat16], TOL_LSE[torch.bfloat16],
             batches=[0], kv_heads=[w.Hkv - 1], rows=rows, what="full bwd")
    assert torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
