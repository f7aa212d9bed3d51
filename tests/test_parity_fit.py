"""Compact fit of a, r to target maps ([Notes §二.3]) on the GPU through the C ABI, against the
fp64 oracle (Adam on the row-wise cross-entropy from a = r = 0)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import cpu64

pytestmark = pytest.mark.gpu


def _saf():
    import fixed_pattern_mixed_amd as saf
    return saf


def _dirichlet_targets(H, T, seed, conc=1.0):
    rng = np.random.default_rng(seed)
    M = np.zeros((H, T, T), dtype=np.float32)
    for h in range(H):
        for i in range(T):
            M[h, i, :i + 1] = rng.dirichlet(np.full(i + 1, conc))
    return M


def _eq3_target(a, r):
    T = len(a)
    idx = np.arange(T)
    t = a[None, :] + r[np.clip(idx[:, None] - idx[None, :], 0, None)]
    t = np.where(idx[None, :] <= idx[:, None], t, -np.inf)
    t = np.exp(t - t.max(1, keepdims=True))
    return t / t.sum(1, keepdims=True)


@pytest.mark.parametrize("H,T,steps,lr,conc", [(2, 200, 400, 0.1, 1.0), (3, 77, 250, 0.05, 0.3),
                                               (1, 300, 400, 0.1, 5.0)])
def test_fit_full_trajectory_matches_oracle(H, T, steps, lr, conc):
    """Same targets (fp32 values), same Adam trajectory: a, r, loss and KL agree with the oracle."""
    saf = _saf()
    M = _dirichlet_targets(H, T, seed=T + H, conc=conc)
    a, r, kl, loss = saf.fit_pattern(torch.from_numpy(M).cuda(), steps=steps, lr=lr)
    torch.cuda.synchronize()
    ga, gr, gk, gl = cpu64(a), cpu64(r), cpu64(kl), cpu64(loss)
    for h in range(H):
        ra, rr, rl, rk = oracle.fit_pattern(M[h], steps=steps, lr=lr)
        ea, er_ = np.abs(ga[h] - ra).max(), np.abs(gr[h] - rr).max()
        print("head %d: |da| %.2e |dr| %.2e loss %.12f/%.12f kl %.3e/%.3e"
              % (h, ea, er_, gl[h], rl, gk[h], rk), flush=True)
        # a, r are returned in fp32: rounding of |a| <= ~20 is ~1e-6
        assert ea <= 1e-5 and er_ <= 1e-5
        assert abs(gl[h] - rl) <= 1e-9 * abs(rl)
        # KL = L + (1/T) sum A ln A: the GPU's entropy term takes fp32 logarithms of the fp32
        # entries (relative error <= 2^-21 per term) and (1/T) sum |A ln A| <= ln T
        assert abs(gk[h] - rk) <= 1e-9 * abs(rk) + 2.0 ** -21 * np.log(T)


def test_fit_recovers_eq3_pattern_and_t1():
    """A target of the form of Eq. (3) is recovered (KL ~ 0); T = 1 gives a = r = 0 and KL = 0."""
    saf = _saf()
    rng = np.random.default_rng(5)
    T = 300
    P0 = _eq3_target(rng.normal(size=T), np.r_[3.0, rng.normal(size=T - 1) * 0.5])
    a, r, kl, _ = saf.fit_pattern(torch.from_numpy(P0[None].astype(np.float32)).cuda())
    one = torch.ones((2, 1, 1), dtype=torch.float32, device="cuda")
    a1, r1, kl1, _ = saf.fit_pattern(one)
    torch.cuda.synchronize()
    assert float(kl[0]) <= 1e-5, float(kl[0])
    assert float(a1.abs().max()) == 0.0 and float(r1.abs().max()) == 0.0
    assert float(kl1.abs().max()) <= 1e-12


def test_fit_on_calibration_output_large_T():
    """Targets from saf_calibrate (N=8 sequences, H=2, T=4096, d=64, bf16): the loss the GPU
    reports equals the oracle's loss at the GPU's fitted a, r (evaluated once, fp64), the fit
    improves on the uniform start, and KL = L + (1/T) sum A ln A."""
    saf = _saf()
    N, H, T, d = 8, 2, 4096, 64
    q, k = synth.calib_inputs(N, H, T, d, torch.bfloat16, seed=91)
    ahat, _ = saf.calibrate(q.cuda(), k.cuda())
    a, r, kl, loss = saf.fit_pattern(ahat)
    a0, r0, kl0, loss0 = saf.fit_pattern(ahat, steps=0)
    torch.cuda.synchronize()
    for h in range(H):
        A = cpu64(ahat[h])
        rl, _, _ = oracle.fit_loss_grad(A, cpu64(a[h]), cpu64(r[h]))
        rl0, _, _ = oracle.fit_loss_grad(A, np.zeros(T), np.zeros(T))
        ent = float((A[A > 0] * np.log(A[A > 0])).sum())
        print("head %d: loss %.9f oracle %.9f (start %.6f), kl %.4f" % (h, float(loss[h]), rl, rl0, float(kl[h])),
              flush=True)
        # the GPU's loss is at its fp64 parameters; the oracle's at their fp32 rounding
        assert abs(float(loss[h]) - rl) <= 1e-5 * abs(rl)
        assert abs(float(loss0[h]) - rl0) <= 1e-12 * abs(rl0)
        assert float(loss[h]) < float(loss0[h])
        assert abs(float(kl[h]) - (float(loss[h]) + ent / T)) <= 1e-6
