"""Pins of the oracle's LSE merge (ISPA §2 item 1, §3 item 2: partial attentions
over disjoint key sets combine exactly through their log-sum-exp)."""

import math

import numpy as np

from oracle import attention as att
from oracle import merge


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sets(lists):
    cap = max(1, max(len(a) for a in lists))
    idx = np.full((1, 1, len(lists), cap), -1, np.int32)
    cnt = np.zeros((1, 1, len(lists)), np.int32)
    for t, a in enumerate(lists):
        idx[0, 0, t, :len(a)] = a
        cnt[0, 0, t] = len(a)
    return idx, cnt


def test_merge_of_disjoint_split_equals_attention_over_union():
    T, P, D = 6, 5, 8
    q, k, v = (_rand((1, 1, T * P, D), s) for s in (1, 2, 3))
    part_a = [[0, 5], [1], [2, 3], [0], [], [4]]
    part_b = [[1, 2], [0, 4], [5], [1, 2, 3], [0, 1], []]
    union = [sorted(a + b) for a, b in zip(part_a, part_b)]
    oa, la = att.sparse_frame_attention(q, k, v, *_sets(part_a), P)
    ob, lb = att.sparse_frame_attention(q, k, v, *_sets(part_b), P)
    ou, lu = att.sparse_frame_attention(q, k, v, *_sets(union), P)
    om, lm = merge.merge_lse(oa, la, ob, lb)
    np.testing.assert_allclose(om, ou, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lm, lu, atol=1e-12, rtol=0)


def test_equal_lse_closed_form():
    o1, o2 = _rand((4, 3), 4), _rand((4, 3), 5)
    l = np.array([0.0, -3.5, 12.25, 700.0])
    o, lse = merge.merge_lse(o1, l, o2, l)
    np.testing.assert_allclose(o, (o1 + o2) / 2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, l + math.log(2.0), atol=1e-12, rtol=0)


def test_weights_follow_softmax_of_lse():
    # L1 = ln 3, L2 = ln 1: the merged output is 3/4 O1 + 1/4 O2, L = ln 4.
    o1, o2 = np.array([[4.0, 0.0]]), np.array([[0.0, 8.0]])
    o, lse = merge.merge_lse(o1, np.array([math.log(3.0)]), o2, np.array([0.0]))
    np.testing.assert_allclose(o, [[3.0, 2.0]], atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, [math.log(4.0)], atol=1e-14, rtol=0)


def test_empty_branches():
    o1, o2 = _rand((3, 2), 6), _rand((3, 2), 7)
    l1 = np.array([-np.inf, 1.0, -np.inf])
    l2 = np.array([2.0, -np.inf, -np.inf])
    o, lse = merge.merge_lse(o1, l1, o2, l2)
    np.testing.assert_array_equal(o[0], o2[0])
    np.testing.assert_array_equal(o[1], o1[1])
    np.testing.assert_array_equal(o[2], [0.0, 0.0])
    assert lse.tolist() == [2.0, 1.0, -np.inf]


def test_commutative_and_associative():
    o = [_rand((5, 4), s) for s in (8, 9, 10)]
    l = [_rand((5,), s) * 10 for s in (11, 12, 13)]
    a = merge.merge_lse(o[0], l[0], o[1], l[1])
    b = merge.merge_lse(o[1], l[1], o[0], l[0])
    np.testing.assert_allclose(a[0], b[0], atol=1e-13, rtol=0)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13, rtol=0)
    left = merge.merge_lse(*merge.merge_lse(o[0], l[0], o[1], l[1]), o[2], l[2])
    right = merge.merge_lse(o[0], l[0], *merge.merge_lse(o[1], l[1], o[2], l[2]))
    np.testing.assert_allclose(left[0], right[0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(left[1], right[1], atol=1e-12, rtol=0)


def test_large_lse_gap_does_not_overflow():
    o1, o2 = np.array([[1.0]]), np.array([[5.0]])
    o, lse = merge.merge_lse(o1, np.array([1000.0]), o2, np.array([-1000.0]))
    assert o[0, 0] == 1.0 and lse[0] == 1000.0
