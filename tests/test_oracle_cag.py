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


@pytest.mark.parametrize("n,sb,smax", [(2, 0.5, 0.9), (7, 0.8, 0.6), (60, 0.6, 0.95), (3, 0.0, 0.5)])
def test_bracket_clips_every_chunk_at_each_end(n, sb, smax):
    # The bisection's bracket: at its low end every later chunk sits at s_max,
    # at its high end every one at 0; chunk 0 is dense at both.
    lo, hi = cag.bracket(n, sb, smax)
    s_lo, s_hi = cag.sparsity_at(lo, n, sb, smax), cag.sparsity_at(hi, n, sb, smax)
    assert s_lo[0] == 0.0 and s_hi[0] == 0.0
    assert all(v == smax for v in s_lo[1:])
    assert all(v == 0.0 for v in s_hi[1:])


@pytest.mark.parametrize("beta", [0.0, 0.05, 0.3, 1.0, -0.2])
def test_sparsity_profile_is_monotone_and_bounded(beta):
    n, sb, smax = 40, 0.7, 0.85
    s = cag.sparsity_at(beta, n, sb, smax)
    assert s[0] == 0.0 and all(0.0 <= v <= smax for v in s)
    later = s[1:]
    if beta >= 0:   # the weight of beta falls with i, so later chunks are sparser, up to s_base
        assert all(a <= b for a, b in zip(later, later[1:]))
        assert all(v <= sb for v in later)
    else:           # a negative beta pushes early chunks above s_base instead
        assert all(a >= b for a, b in zip(later, later[1:]))
        assert all(v >= min(sb, smax) for v in later)
    if beta == 0.0:
        assert later == [min(sb, smax)] * (n - 1)


def test_kept_cost_endpoints_and_monotone_in_beta():
    cost = [4.0, 1.0, 2.0, 8.0, 16.0]
    assert cag.kept_cost([0.0] * 5, cost) == 31.0                       # dense: every cost kept
    assert cag.kept_cost([0.0, 0.5, 0.5, 0.5, 0.5], cost) == 4.0 + 13.5  # exact halves
    n, sb, smax = len(cost), 0.6, 0.9
    betas = [-1.0 + 0.05 * i for i in range(60)]
    kept = [cag.kept_cost(cag.sparsity_at(b, n, sb, smax), cost) for b in betas]
    assert all(a <= b for a, b in zip(kept, kept[1:]))
