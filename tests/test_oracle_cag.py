"""Pins of the oracle's chunk-aware growth schedule (Light Forcing §2.1).

Checked against: the closed-form beta of the linear (unclipped) case, the
two-chunk case where the FLOP match alone fixes s_1 = 2 s_target, the
constraint itself, the shape the page describes (chunk 0 dense, sparsity
growing with the chunk index, inside [0, s_max]), the limits of reachable
targets, and hand-computed frame budgets.
"""

import math

import pytest

from oracle import cag


def test_two_chunks_of_equal_cost():
    for st in (0.1, 0.2, 0.3):
        s, beta = cag.schedule([5.0, 5.0], st, 0.5, 0.9)
        assert s[0] == 0.0
        assert abs(s[1] - 2 * st) < 1e-12


def test_linear_case_matches_closed_form():
    cost = [float(i + 1) for i in range(12)]       # a cache that grows by one chunk each time
    st, sb, smax = 0.5, 0.8, 0.99
    s, beta = cag.schedule(cost, st, sb, smax)
    num = (1 - st) * sum(cost) - cost[0] - (1 - sb) * sum(cost[1:])
    den = sum(cag.alpha(i) * cost[i] for i in range(1, 12))
    assert abs(beta - num / den) < 1e-12 * abs(num / den)
    assert all(0.0 < x < smax for x in s[1:])       # no clipping happened
    for i in range(1, 12):
        assert abs(s[i] - (sb - beta / math.sqrt(i + 1))) < 1e-12


@pytest.mark.parametrize("st,sb,smax", [(0.6, 0.9, 0.95), (0.3, 0.2, 0.9), (0.75, 1.0, 0.85),
                                        (0.05, 0.6, 0.9)])
def test_constraint_and_shape(st, sb, smax):
    cost = [3.0 + (i % 4) for i in range(20)]
    s, beta = cag.schedule(cost, st, sb, smax)
    kept = sum((1 - si) * f for si, f in zip(s, cost))
    assert abs(kept - (1 - st) * sum(cost)) < 1e-12 * sum(cost)
    assert s[0] == 0.0
    assert all(0.0 <= x <= smax for x in s)
    if beta > 0:
        assert all(a <= b for a, b in zip(s[1:], s[2:]))   # later chunks are sparser


def test_zero_target_is_dense_and_limits_raise():
    s, _ = cag.schedule([1.0] * 6, 0.0, 0.5, 0.9)
    assert s[0] == 0.0 and all(0.0 <= x < 1e-12 for x in s)
    # at most 5/6 of the cost can go, at s_max on every later chunk
    with pytest.raises(ValueError):
        cag.schedule([1.0] * 6, 0.9 * 5 / 6 + 1e-3, 0.5, 0.9)
    s, _ = cag.schedule([1.0] * 6, 0.9 * 5 / 6 - 1e-9, 0.5, 0.9)
    assert all(abs(x - 0.9) < 1e-8 for x in s[1:])
    with pytest.raises(ValueError):
        cag.schedule([1.0, -1.0], 0.1, 0.5, 0.9)
    with pytest.raises(ValueError):
        cag.schedule([], 0.1, 0.5, 0.9)


def test_frame_budgets():
    assert cag.frame_budgets([0.5, 0.75, 0.99, 0.0, 0.3], [7, 2, 3, 9, 10]) == [4, 1, 1, 9, 7]
