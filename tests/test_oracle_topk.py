"""Pins of the oracle's frame pooling and top-k selection (Light Forcing §2.2;
Head Forcing methodology §2, memory heads).

Checked against: planted frames with a known order (exact small integers),
exact rational arithmetic (fractions.Fraction, whose conversion to float is
correctly rounded) for every pooled sum -- on random inputs and on cases where
every fixed summation order differs from the exact sum (cancellation, a
rounding tie, a tie broken by a term far below it, exponent spans beyond 53
bits) --, invariance under any reordering of the tokens, the ban on fused
multiply-add in the scores, ties, and scaling.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import topk


def test_planted_frames_rank_by_alignment():
    # every query token equals u; frame f's tokens all equal c_f·u
    D, P, Nq = 8, 5, 10
    u = np.arange(1, D + 1, dtype=np.float64)
    c = [3, -1, 7, 0, 5, 2, 7.5, -4]
    q = np.tile(u, (Nq, 1))
    k = np.concatenate([np.tile(cf * u, (P, 1)) for cf in c])
    frames, scores = topk.select_topk_frames(q, k, P, range(Nq), range(len(c)), 3)
    assert frames == [2, 4, 6]          # c = 7, 5, 7.5
    assert scores.tolist() == [Nq * P * cf * float(u @ u) for cf in c]


def _exact_scores(q, k, P, rows, cands):
    # exact rational sums: any summation order gives these values
    qs = [sum(Fraction(float(q[i, d])) for i in rows) for d in range(q.shape[1])]
    out = []
    for f in cands:
        ks = [sum(Fraction(float(k[f * P + p, d])) for p in range(P)) for d in range(q.shape[1])]
        out.append(sum(a * b for a, b in zip(qs, ks)))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_matches_exact_arithmetic_ranking(seed):
    rng = np.random.default_rng(seed)
    D, P, F, Nq, kk = 16, 6, 12, 12, 4
    q = rng.standard_normal((Nq, D)).astype(np.float32).astype(np.float64)
    k = rng.standard_normal((F * P, D)).astype(np.float32).astype(np.float64)
    frames, scores = topk.select_topk_frames(q, k, P, range(Nq), range(F), kk)
    exact = _exact_scores(q, k, P, range(Nq), range(F))
    order = sorted(range(F), key=lambda f: (-exact[f], f))
    # the float64 ranking equals the exact one whenever the cut is not a near tie
    gap = abs(exact[order[kk - 1]] - exact[order[kk]])
    assert gap > Fraction(1, 10**6)
    assert frames == sorted(order[:kk])
    for f in range(F):
        assert abs(scores[f] - float(exact[f])) <= 1e-9 * max(1.0, abs(float(exact[f])))
    # the pooled sums themselves are the correctly rounded exact sums
    qs = topk.pooled_query_sum(q, P)
    assert qs.tolist() == [_rn_exact(q[:, d]) for d in range(D)]
    ks = topk.pooled_key_sums(k, P, range(F))
    assert ks[3].tolist() == [_rn_exact(k[3 * P:4 * P, d]) for d in range(D)]


def _rn_exact(col) -> float:
    """The exact sum of float64 values rounded to the nearest float64 (ties to
    even): Fraction arithmetic is exact and int/int division in Python rounds
    correctly."""
    return float(sum(Fraction(float(x)) for x in col))


def test_pooled_sums_are_the_exact_sum_rounded_once():
    # 1e16 + 1 rounds back to 1e16 (spacing 2) in any sequential order: a
    # token-sequential sum gives 1, frames-then-total gives 0, the exact sum is 2
    q = np.array([[1e16], [1.0], [-1e16], [1.0]])
    assert topk.pooled_query_sum(q, 4).tolist() == [2.0]
    assert topk.pooled_query_sum(q, 2).tolist() == [2.0]
    assert topk.pooled_key_sums(np.vstack([q, [[5.0], [0.0], [0.0], [0.0]]]), 4,
                                [0, 1]).tolist() == [[2.0], [5.0]]
    with pytest.raises(ValueError):
        topk.pooled_query_sum(q, 3)


@pytest.mark.parametrize("col,expect", [
    ([1.0, 2.0**-53], 1.0),                               # an exact tie: to even
    ([1.0 + 2.0**-52, 2.0**-53], 1.0 + 2.0**-51),          # a tie: to even, upwards
    ([1.0, 2.0**-53, 2.0**-105], 1.0 + 2.0**-52),          # just above the tie
    ([2.0**-105, 2.0**-53, 1.0], 1.0 + 2.0**-52),          # the same, any order
    ([3e38, 1e-38, -3e38], 1e-38),                         # bf16/fp32 extremes cancel
    ([2.0**-149, 2.0**127, -(2.0**127)], 2.0**-149),       # fp32 subnormal survives
    ([-0.0, -0.0], 0.0),                                   # zero is +0
    ([0.1] * 10, 1.0),                                     # exact 10 * fl(0.1) rounds to 1
])
def test_pooled_sum_special_cases(col, expect):
    got = topk.exact_column_sums(np.array(col)[:, None])[0]
    assert got == expect and math.copysign(1.0, got) == math.copysign(1.0, expect)
    assert got == _rn_exact(col) + 0.0


@pytest.mark.parametrize("seed", range(8))
def test_pooled_sums_match_rational_arithmetic_in_any_order(seed):
    rng = np.random.default_rng(50 + seed)
    N, D = 64, 6
    # bf16-like values: 8 significant bits, exponents spread over 60 binades
    mant = rng.integers(128, 256, size=(N, D)) * rng.choice([-1, 1], size=(N, D))
    expo = rng.integers(-40, 20, size=(N, D))
    x = np.ldexp(mant.astype(np.float64), expo - 7)
    got = topk.exact_column_sums(x)
    assert got.tolist() == [_rn_exact(x[:, d]) for d in range(D)]
    perm = rng.permutation(N)
    assert topk.exact_column_sums(x[perm]).tobytes() == got.tobytes()


def test_scores_round_each_product_before_adding():
    # qsum·ksum = 1·(1 + 2^-26) + (-(1 + 2^-27))·(1 + 2^-27).  The second product is
    # -(1 + 2^-26 + 2^-54): rounded alone it cancels the first term exactly (0.0);
    # a fused multiply-add would keep -2^-54.
    qsum = np.array([1.0, -(1 + 2.0**-27)])
    ksum = np.array([[1 + 2.0**-26, 1 + 2.0**-27]])
    assert topk.frame_scores(qsum, ksum).tolist() == [0.0]


def test_scores_sum_sequentially_in_d():
    qsum = np.array([1e16, 1.0, -1e16, 1.0])
    ksum = np.ones((1, 4))
    assert topk.frame_scores(qsum, ksum).tolist() == [1.0]


def test_ties_go_to_the_earlier_frame():
    D, P = 4, 3
    q = np.ones((3, D))
    base = np.ones((P, D))
    k = np.concatenate([base * 2, base, base * 2, base * 2, base])
    frames, _ = topk.select_topk_frames(q, k, P, range(3), range(5), 2)
    assert frames == [0, 2]


def test_positive_scaling_of_queries_keeps_the_selection():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((12, 8))
    k = rng.standard_normal((8 * 4, 8))
    a, _ = topk.select_topk_frames(q, k, 4, range(12), range(8), 3)
    b, _ = topk.select_topk_frames(q * 4.0, k, 4, range(12), range(8), 3)
    assert a == b


def test_candidate_subset_and_errors():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 4))
    k = rng.standard_normal((6 * 2, 4))
    frames, scores = topk.select_topk_frames(q, k, 2, range(4), [1, 3, 4], 3)
    assert frames == [1, 3, 4] and scores.shape == (3,)
    with pytest.raises(ValueError):
        topk.select_topk_frames(q, k, 2, range(4), [1, 3], 3)
    with pytest.raises(ValueError):
        topk.select_topk_frames(q, k, 2, range(3), [1, 3], 1)
    with pytest.raises(ValueError):
        topk.rank_topk(np.array([1.0, np.nan]), [0, 1], 1)
