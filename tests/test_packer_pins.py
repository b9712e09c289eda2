"""Pins of the packer oracle (CPU only): invariants that define first-fit in arrival order, and
closed forms of the exponential moving average."""

import math

import numpy as np
import pytest

from oracle import packer as PK


def _queues(seed, n_cases=200):
    rng = np.random.default_rng(seed)
    for _ in range(n_cases):
        n = int(rng.integers(0, 40))
        lengths = rng.integers(1, 17, n)
        budget = int(rng.integers(0, 200))
        cap = int(rng.choice([0, 0, 1, 3, 8]))
        yield lengths, budget, cap


def test_first_fit_invariants():
    for lengths, budget, cap in _queues(1):
        out = PK.pack_first_fit(lengths, budget, cap)
        sel = out["selected"]
        # arrival order, within budget and cap, offsets are the exclusive prefix sum
        assert sel == sorted(sel) and len(set(sel)) == len(sel)
        assert out["rows"] == sum(int(lengths[r]) for r in sel) <= budget
        assert cap == 0 or len(sel) <= cap
        assert out["offsets"] == [0] + list(np.cumsum([int(lengths[r]) for r in sel]))
        # prefix property: each taken request fitted in what was left when it was reached
        used = 0
        for r in range(len(lengths)):
            if r in sel:
                assert used + lengths[r] <= budget
                used += int(lengths[r])
        # maximality: unless the request cap was reached, no request left behind fits in the leftover
        if not (cap and len(sel) == cap):
            left = budget - out["rows"]
            assert all(int(lengths[r]) > left for r in range(len(lengths)) if r not in sel)


def test_first_fit_worked_example():
    # budget 20: take 8 (8), skip 16 (24 > 20), take 5 (13), skip 9 (22), take 7 (20), skip 1 (21)
    out = PK.pack_first_fit([8, 16, 5, 9, 7, 1], 20)
    assert out["selected"] == [0, 2, 4]
    assert out["offsets"] == [0, 8, 13, 20]
    assert out["lengths"] == [8, 5, 7]
    out = PK.pack_first_fit([8, 16, 5, 9, 7, 1], 20, max_requests=2)
    assert out["selected"] == [0, 2]


def test_empty_and_zero_budget():
    assert PK.pack_first_fit([], 100)["selected"] == []
    assert PK.pack_first_fit([1, 2, 3], 0)["offsets"] == [0]
    with pytest.raises(ValueError):
        PK.pack_first_fit([3, 0], 10)


def test_ema_constant_observations_are_a_fixed_point():
    s = None
    for _ in range(20):
        s, b = PK.ema_update(s, 1234.0, 0.9)
        assert s == pytest.approx(1234.0, rel=1e-15) and b == 1234


@pytest.mark.parametrize("beta", [0.0, 0.5, 0.9, 0.99])
def test_ema_step_response_closed_form(beta):
    # after c0 for the first round then c1 forever: e_t = c1 + (c0 - c1) beta^t
    c0, c1 = 4000.0, 2500.0
    s, _ = PK.ema_update(None, c0, beta)
    for t in range(1, 30):
        s, b = PK.ema_update(s, c1, beta)
        exact = c1 + (c0 - c1) * beta ** t
        assert s == pytest.approx(exact, rel=1e-12)
        assert b == math.floor(s)


def test_ema_beta_zero_follows_the_last_observation():
    s = None
    for c in [10.7, 3.2, 99.9, 0.0]:
        s, b = PK.ema_update(s, c, 0.0)
        assert s == c and b == math.floor(c)
