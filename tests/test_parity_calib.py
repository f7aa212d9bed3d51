"""Calibration statistics on the GPU (through the C ABI) against the fp64 oracle: the mean map
Ahat, the Eq. (1) variance score and the row-wise forward-KL score ([Notes §二.1]), plus the
mean-optimality identity checked on the GPU's own outputs."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, Worst, cpu64

pytestmark = pytest.mark.gpu


def _saf():
    import fixed_pattern_mixed_amd as saf
    return saf


SMALL = [
    # N, H, T, d, dtype
    (4, 2, 200, 64, torch.float32),
    (2, 1, 1, 64, torch.float32),
    (3, 2, 129, 128, torch.float32),
    (5, 3, 256, 64, torch.bfloat16),
    (8, 2, 1024, 128, torch.bfloat16),
    # bf16 edges of the fragment-order query copy: one row; one row past a 128-row tile
    (2, 1, 1, 64, torch.bfloat16),
    (3, 2, 130, 128, torch.bfloat16),
]


@pytest.mark.parametrize("N,H,T,d,dtype", SMALL,
                         ids=["N%dH%dT%dd%d-%s" % (c[0], c[1], c[2], c[3], str(c[4])[6:]) for c in SMALL])
def test_calibrate_full_compare(N, H, T, d, dtype):
    saf = _saf()
    q, k = synth.calib_inputs(N, H, T, d, dtype, seed=31 + T)
    ahat, svar, skl = saf.calibrate(q.cuda(), k.cuda(), kl=True)
    ahat2, svar2 = saf.calibrate(q.cuda(), k.cuda())
    torch.cuda.synchronize()
    # the KL score is an extra output: Ahat and s_var are the same with or without it
    assert torch.equal(ahat, ahat2) and torch.equal(svar, svar2)
    ga, gs, gk = cpu64(ahat), cpu64(svar), cpu64(skl)
    rk = oracle.kl_score(q, k)
    wr = Worst("calib small N%dH%dT%dd%d" % (N, H, T, d))
    for h in range(H):
        ra, dev = oracle.head_calibrate(q[:, h], k[:, h])
        rs = dev.sum() / ((N - 1) * T * T)
        wr.add(ga[h], ra, TOL[dtype], "ahat[h=%d]" % h)
        assert np.all(ga[h][np.triu_indices(T, 1)] == 0.0)
        if rs == 0.0:
            assert abs(gs[h]) <= 1e-12
        else:
            assert abs(gs[h] - rs) / rs <= TOL[dtype], (h, gs[h], rs)
        assert abs(gk[h] - rk[h]) <= TOL[dtype] * rk[h] + 1e-6, (h, gk[h], rk[h])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_calibrate_wide_score_ranges(dtype):
    """Three sequences whose scores span ~200 log2 units with different shapes along the keys (row
    maximum moving with the keys, set by the first key, isolated jumps past the fp32 exponent
    range): the row statistics and the streamed mean / variance must match the oracle."""
    saf = _saf()
    T = 300
    xs = [synth.score_range_inputs(T, 64, dtype, t) for t in ("rising", "falling", "spiky")]
    q = torch.cat([x.q[:, :1] for x in xs])  # [3, 1, T, d]: the ordinary head of each
    k = torch.cat([x.k[:, :1] for x in xs])
    ahat, svar, skl = saf.calibrate(q.cuda(), k.cuda(), kl=True)
    torch.cuda.synchronize()
    ga, gs, gk = cpu64(ahat), cpu64(svar), cpu64(skl)
    assert np.isfinite(ga).all() and np.isfinite(gs).all() and np.isfinite(gk).all()
    ra, dev = oracle.head_calibrate(q[:, 0], k[:, 0])
    rs = dev.sum() / (2 * T * T)
    rk = oracle.kl_score(q, k)
    Worst("calib wide").add(ga[0], ra, TOL[dtype], "ahat")
    assert abs(gs[0] - rs) / rs <= TOL[dtype], (gs[0], rs)
    assert abs(gk[0] - rk[0]) <= TOL[dtype] * rk[0] + 1e-6, (gk[0], rk[0])


def test_kl_score_identical_sequences_and_uniform_maps():
    """N copies of one sequence, or Q = 0 (every map uniform): s_var = 0 and s_kl = 0 up to
    rounding, at a size that spans many tiles (T = 1000, ragged)."""
    saf = _saf()
    N, H, T, d = 4, 2, 1000, 128
    q, k = synth.calib_inputs(1, H, T, d, torch.bfloat16, seed=77)
    q, k = q.expand(N, -1, -1, -1).contiguous(), k.expand(N, -1, -1, -1).contiguous()
    _, svar, skl = saf.calibrate(q.cuda(), k.cuda(), kl=True)
    torch.cuda.synchronize()
    assert float(svar.abs().max()) <= 1e-12
    assert float(skl.abs().max()) <= 1e-5
    _, svar, skl = saf.calibrate(torch.zeros_like(q).cuda(), k.cuda(), kl=True)
    torch.cuda.synchronize()
    assert float(svar.abs().max()) <= 1e-12 and float(skl.abs().max()) <= 1e-5


def test_mean_optimality_identity_on_gpu_outputs():
    """For any fixed P: (1/(N T^2)) sum_n ||A^(n) - P||^2 = ((N-1)/N) s_var + ||P - Ahat||^2/T^2
    ([Notes §二.2], Appendix B.1), with Ahat and s_var from the GPU and the maps from torch."""
    saf = _saf()
    N, H, T, d = 6, 2, 96, 64
    q, k = synth.calib_inputs(N, H, T, d, torch.float32, seed=5)
    ahat, svar = saf.calibrate(q.cuda(), k.cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for h in range(H):
        s = (q[:, h].double() @ k[:, h].double().transpose(-1, -2)) / math.sqrt(d)
        s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
        maps = torch.softmax(s, -1).numpy()
        P = rng.random((T, T))
        lhs = ((maps - P) ** 2).sum() / (N * T * T)
        rhs = (N - 1) / N * float(svar[h]) + ((P - cpu64(ahat[h])) ** 2).sum() / (T * T)
        assert abs(lhs - rhs) <= 1e-5 * lhs


def test_calibrate_full_size():
    """The 1B-shaped calibration (N=32, H=16, T=8192, d=128, bf16): for the first and the last head,
    every row of Ahat, s_var and the KL score against the oracle (rows formed in chunks, the
    deviation sums added up for s_var); for every head the properties that hold at any size (rows
    sum to 1, zeros above the diagonal, s_var and s_kl finite and >= 0)."""
    saf = _saf()
    w = synth.WORKLOADS["l1b_t8192"]
    N, H, T, d = w.calib_N, w.H, w.T, w.d
    q, k = synth.calib_inputs(N, H, T, d, torch.bfloat16)
    print("workload l1b_t8192 calibration", flush=True)
    ahat, svar, skl = saf.calibrate(q.cuda(), k.cuda(), kl=True)
    torch.cuda.synchronize()
    sums = ahat.double().sum(-1)
    assert torch.allclose(sums, torch.ones_like(sums), atol=1e-4)
    for h in range(H):
        assert torch.count_nonzero(torch.triu(ahat[h], 1)) == 0
    gs, gk = cpu64(svar), cpu64(skl)
    assert np.isfinite(gs).all() and (gs >= 0).all() and np.isfinite(gk).all() and (gk >= 0).all()
    wr = Worst("calib full l1b_t8192")
    tol = TOL[torch.bfloat16]
    for h in (0, H - 1):
        ga = ahat[h].cpu()
        dev_sum = 0.0
        for r0 in range(0, T, 1024):
            rows = np.arange(r0, min(T, r0 + 1024), dtype=np.int32)
            ra, dev = oracle.head_calibrate(q[:, h], k[:, h], rows=rows)
            dev_sum += float(dev.sum())
            wr.add(ga[r0:r0 + len(rows)].double().numpy(), ra, tol, "ahat[h=%d]" % h)
        rs = dev_sum / ((N - 1) * T * T)
        rk = float(oracle.head_kl_score(q[:, h], k[:, h]).sum()) / (N * T)
        print("head %d: s_var gpu %.6e oracle %.6e; s_kl gpu %.6e oracle %.6e"
              % (h, gs[h], rs, gk[h], rk), flush=True)
        assert abs(gs[h] - rs) <= tol * rs, (h, gs[h], rs)
        assert abs(gk[h] - rk) <= tol * rk, (h, gk[h], rk)
    wr.report(workload="l1b_t8192 calibration", svar_heads=[0, H - 1])
