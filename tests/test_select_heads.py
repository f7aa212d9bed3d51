"""Head selection through the C ABI (host code, no GPU needed) against the oracle's definition
([Notes §二.1]: ascending score across all layers, k = round(r L H)); the oracle itself is pinned
by tests/golden/select_ties.txt and a brute-force search (oracle_pins.py)."""
import numpy as np
import pytest

import fixed_pattern_mixed_amd as saf
import oracle
from oracle_pins import read_golden


def test_golden_ties_and_rounding():
    g = read_golden("select_ties.txt")
    score = g["score"].reshape(2, 3)
    for key, ratio in (("sel_half", 0.5), ("sel_quarter", 0.25), ("sel_twelfth", 1 / 12)):
        sel, n = saf.select_heads(score, ratio)
        assert np.array_equal(sel.ravel(), g[key].astype(np.uint8)) and n == int(g[key].sum())
    sel, n = saf.select_heads(score, 0.5, accepted=g["accepted"].reshape(2, 3))
    assert np.array_equal(sel.ravel(), g["sel_half_accepted"].astype(np.uint8)) and n == 3


@pytest.mark.parametrize("seed", range(6))
def test_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    L, H = [(12, 12), (24, 16), (3, 5), (1, 1), (36, 32), (2, 7)][seed]
    score = rng.random((L, H))
    if seed % 2:  # ties: scores on a coarse grid
        score = np.round(score * 4) / 4
    acc = (rng.random((L, H)) < 0.8).astype(np.uint8) if seed % 3 == 0 else None
    for ratio in (0.0, 0.1, 0.25, 0.5, 0.75, 1.0, 1 / (2 * L * H), 3 / (2 * L * H)):
        if ratio > 1.0:
            continue
        got, n = saf.select_heads(score, ratio, accepted=acc)
        want, m = oracle.select_heads(score, ratio, accepted=acc)
        assert n == m and np.array_equal(got, want)


def test_rejects():
    ok = np.zeros((2, 2))
    for bad in (dict(ratio=-0.1), dict(ratio=1.5), dict(ratio=float("nan"))):
        with pytest.raises(saf.SafError):
            saf.select_heads(ok, **bad)
    with pytest.raises(saf.SafError):
        saf.select_heads(np.array([[0.0, float("nan")]]), 0.5)
