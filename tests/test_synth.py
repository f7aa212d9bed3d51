"""CPU checks of the seeded input generators: the shapes, seeds and value structure that the
parity tests and the benchmark rely on."""
import math

import pytest
import torch

import synth


def test_replaced_mask_placements():
    assert synth.replaced_mask(12, 3) == [0, 0, 0, 1] * 3
    assert synth.replaced_mask(4, 1) == [0, 0, 0, 1]
    assert synth.replaced_mask(12, 3, "contiguous") == [0] * 9 + [1] * 3
    assert synth.replaced_mask(5, 5, "all") == [1] * 5
    assert synth.replaced_mask(7, 0) == [0] * 7
    with pytest.raises(ValueError):
        synth.replaced_mask(12, 5)
    with pytest.raises(ValueError):
        synth.replaced_mask(12, 3, "random")


def test_workloads_are_consistent():
    for name, w in synth.WORKLOADS.items():
        assert w.name == name
        assert sum(w.replaced()) == w.n_replaced
        assert w.H % w.kv_heads == 0
        assert w.d in (64, 128) and w.T % 64 == 0
    seeds = [w.index for w in synth.WORKLOADS.values()]
    assert len(set(seeds)) == len(seeds)


def test_layer_inputs_seeded_and_shaped():
    x = synth.layer_inputs(2, 4, 96, 64, torch.bfloat16, [0, 1, 0, 1], Hkv=2)
    y = synth.layer_inputs(2, 4, 96, 64, torch.bfloat16, [0, 1, 0, 1], Hkv=2)
    assert x.q.shape == (2, 4, 96, 64) and x.k.shape == (2, 2, 96, 64)
    assert x.v.shape == x.k.shape and x.dout.shape == x.q.shape
    assert x.a.shape == (4, 96) and x.a.dtype == torch.float32 and x.q.dtype == torch.bfloat16
    for n in ("q", "k", "v", "dout", "a", "r"):
        assert torch.equal(getattr(x, n), getattr(y, n))
    z = synth.layer_inputs(2, 4, 96, 64, torch.bfloat16, [0, 1, 0, 1], seed=synth.SEED0 + 1)
    assert not torch.equal(x.q, z.q)
    assert synth.layer_inputs(1, 1, 64, 64, torch.float32, [0], backward=False).dout is None


@pytest.mark.parametrize("trend", ["rising", "falling", "spiky"])
def test_score_range_profile(trend):
    """With the 1/sqrt(64) scale every query row sees scores close to the promised c_j."""
    T = 300
    x = synth.score_range_inputs(T, 64, torch.float32, trend)
    assert x.q.shape == (1, 2, T, 64) and x.replaced == [False, True]
    s = (x.q[0, 0].double() @ x.k[0, 0].double().T) / math.sqrt(64)
    j = torch.arange(T, dtype=torch.float64)
    if trend == "rising":
        c = 150 * j / (T - 1)
    elif trend == "falling":
        c = 150 * (T - 1 - j) / (T - 1)
    else:
        c = torch.where(j % 37 == 5, 120.0, 0.0)
    # noise: the 8u.(0.05 n) and c_j u.(0.05 n) terms over sqrt(d), at most about 3 here
    assert (s - c[None, :]).abs().max() < 4.0
    if trend == "rising":
        assert (s.argmax(1) == T - 1).all()
    elif trend == "falling":
        assert (s.argmax(1) == 0).all()
    else:
        assert (s.argmax(1) % 37 == 5).all()
    with pytest.raises(ValueError):
        synth.score_range_inputs(T, 64, torch.float32, "flat")
