"""saf_attn_bwd_noalloc, the backward for callers that cannot allocate (its workspace is a device
array owned by the library), through the C ABI: the bits of saf_attn_bwd with a caller workspace,
on consecutive calls with a smaller input second (the array keeps the previous call's contents),
with and without a prepared pattern, replayed from a HIP graph, and the rejection of shapes
whose workspace exceeds the array."""
import ctypes

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _saf():
    import fixed_pattern_mixed_amd as saf
    return saf


def _code(saf, dtype):
    return saf.SAF_BF16 if dtype == torch.bfloat16 else saf.SAF_F32


def _bwd_noalloc(saf, g, o, lse, rep, pattern, out, stream=None):
    B, H, T, d = g.q.shape
    dq, dk, dv = out
    st = saf.saf_attn_bwd_noalloc(
        _code(saf, g.q.dtype), B, H, T, d, g.q.data_ptr(), g.k.data_ptr(), g.v.data_ptr(),
        o.data_ptr(), g.dout.data_ptr(), lse.data_ptr(), saf._mask(rep, H), g.a.data_ptr(),
        g.r.data_ptr(), g.a.shape[1], None if pattern is None else pattern.data_ptr(), 0.0,
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
        torch.cuda.current_stream().cuda_stream if stream is None else stream)
    assert st == saf.SAF_OK, saf.saf_last_error()


CASES = [
    # B, H, T, d, dtype, replaced heads, prepared pattern
    (2, 8, 1000, 128, torch.bfloat16, 2, False),
    (1, 4, 300, 64, torch.bfloat16, 1, False),   # smaller than the call before
    (3, 12, 777, 64, torch.bfloat16, 3, True),
    (1, 4, 129, 128, torch.float32, 2, False),
]


def test_noalloc_backward_matches_the_workspace_call():
    saf = _saf()
    for B, H, T, d, dtype, R, prepared in CASES:
        print("case", B, H, T, d, dtype, R, prepared, flush=True)
        rep = synth.replaced_mask(H, R)
        g = synth.layer_inputs(B, H, T, d, dtype, rep, seed=T + d, device="cuda")
        pat = saf.prepare_pattern(rep, g.a, g.r) if prepared else None
        o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r, pattern=pat)
        # the workspace call with the same kernels (the no-allocation call never keeps dS)
        ref = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r, pattern=pat, keep_ds=False)
        got = tuple(torch.full_like(t, float("nan")) for t in ref)
        _bwd_noalloc(saf, g, o, lse, rep, pat, got)
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(x, y), (name, B, H, T, d, dtype)


def test_noalloc_backward_replays_from_a_graph():
    """Captured into a HIP graph (no allocation inside the capture), replays give the bits of the
    eager call, with other work on the device between replays."""
    saf = _saf()
    B, H, T, d = 2, 4, 500, 64
    rep = [0, 1, 0, 1]
    g = synth.layer_inputs(B, H, T, d, torch.bfloat16, rep, seed=41, device="cuda")
    o, lse = saf.fwd(g.q, g.k, g.v, rep, g.a, g.r)
    ref = saf.bwd(g.q, g.k, g.v, o, g.dout, lse, rep, g.a, g.r, keep_ds=False)
    out = tuple(torch.empty_like(t) for t in ref)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        _bwd_noalloc(saf, g, o, lse, rep, None, out, stream=cs.cuda_stream)
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cs):
        _bwd_noalloc(saf, g, o, lse, rep, None, out, stream=cs.cuda_stream)
    small = synth.layer_inputs(1, 2, 64, 64, torch.bfloat16, [0, 1], seed=42, device="cuda")
    for it in range(3):
        for t in out:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(out, ref):
            assert torch.equal(x, y), it
        # another call between replays overwrites the library's array
        so, sl = saf.fwd(small.q, small.k, small.v, [0, 1], small.a, small.r)
        _bwd_noalloc(saf, small, so, sl, [0, 1], None,
                     tuple(torch.empty_like(t) for t in (small.q, small.k, small.v)))
        torch.cuda.synchronize()


def test_noalloc_backward_rejects_shapes_beyond_its_array():
    """B*H*T*4 bytes of delta above 16 MiB: SAF_ERR_UNSUPPORTED, with a message naming the limit,
    before any HIP call (the pointers here are stand-ins that are never dereferenced)."""
    saf = _saf()
    fake = 0x100000
    H = 12
    rep = (ctypes.c_uint8 * H)(*([0] * H))
    st = saf.saf_attn_bwd_noalloc(saf.SAF_BF16, 64, H, 8192, 64, fake, fake, fake, fake, fake,
                                  fake, rep, fake, fake, 8192, None, 0.0, fake, fake, fake, None)
    assert st == saf.SAF_ERR_UNSUPPORTED
    assert "noalloc" in saf.saf_last_error() and str(16 << 20) in saf.saf_last_error()
