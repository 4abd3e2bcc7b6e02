"""Pins of the oracle's frame-sparse attention.

Each check compares against something other than the oracle's own formula:
torch's fp64 scaled-dot-product attention and logsumexp on the special cases
that reduce to dense attention (the FULL set; A(t) = {t}, the intra-frame
branch of ARL2 §2.1), closed forms (zero queries, a single key), a pure-Python
brute force with math.exp / math.fsum, and invariances the definition implies.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import frame_sets as fs


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v):
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v))
    d = q.shape[-1]
    s = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) / math.sqrt(d)
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


def _sets(lists, B=1, H=1):
    """idx/cnt arrays from per-(b,h,t) python lists."""
    Tq = len(lists)
    cap = max(1, max(len(a) for a in lists))
    idx = np.full((B, H, Tq, cap), -1, np.int32)
    cnt = np.zeros((B, H, Tq), np.int32)
    for b in range(B):
        for h in range(H):
            for t, a in enumerate(lists):
                idx[b, h, t, :len(a)] = a
                cnt[b, h, t] = len(a)
    return idx, cnt


def test_full_set_is_dense_attention():
    B, H, T, P, D = 1, 2, 3, 16, 32
    q, k, v = (_rand((B, H, T * P, D), s) for s in (1, 2, 3))
    idx, cnt = _sets([list(range(T))] * T, B, H)
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, P)
    o_ref, lse_ref = _sdpa(q, k, v)
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)
    o2, lse2 = att.dense_attention(q, k, v)
    np.testing.assert_allclose(o2, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse2, lse_ref, atol=1e-12, rtol=0)


def test_own_frame_only_is_per_frame_dense_attention():
    # ARL2 §2.1: bidirectional softmax within each frame, i.e. A(t) = {t}.
    B, H, T, P, D = 1, 2, 4, 8, 16
    q, k, v = (_rand((B, H, T * P, D), s) for s in (4, 5, 6))
    idx, cnt = _sets([[t] for t in range(T)], B, H)
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, P)
    for t in range(T):
        sl = slice(t * P, (t + 1) * P)
        o_ref, lse_ref = _sdpa(q[:, :, sl], k[:, :, sl], v[:, :, sl])
        np.testing.assert_allclose(o[:, :, sl], o_ref, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[:, :, sl], lse_ref, atol=1e-12, rtol=0)


def test_zero_query_gives_mean_of_attended_values_and_log_count():
    B, H, T, P, D = 1, 1, 5, 6, 8
    q = np.zeros((B, H, T * P, D))
    k, v = _rand((B, H, T * P, D), 7), _rand((B, H, T * P, D), 8)
    lists = [[0], [0, 1], [1, 3, 4], [2], [0, 1, 2, 3, 4]]
    idx, cnt = _sets(lists)
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, P)
    for t, a in enumerate(lists):
        rows = np.concatenate([np.arange(f * P, (f + 1) * P) for f in a])
        mean_v = v[0, 0, rows].mean(axis=0)
        for p in range(P):
            np.testing.assert_allclose(o[0, 0, t * P + p], mean_v, atol=1e-13, rtol=0)
            assert lse[0, 0, t * P + p] == pytest.approx(math.log(len(a) * P), abs=1e-14)


def test_single_attended_key_returns_its_value_and_score():
    # P = 1 and |A(t)| = 1: softmax over one key has probability 1.
    D = 8
    q, k, v = (_rand((1, 1, 3, D), s) for s in (9, 10, 11))
    idx, cnt = _sets([[2], [0], [1]])
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, 1)
    for t, f in enumerate([2, 0, 1]):
        np.testing.assert_array_equal(o[0, 0, t], v[0, 0, f])
        assert lse[0, 0, t] == pytest.approx(q[0, 0, t] @ k[0, 0, f] / math.sqrt(D), abs=1e-15)


def _brute(q, k, v, lists, P, scale):
    """Pure-Python attention with math.exp / math.fsum, one row at a time."""
    B, H, Nq, D = q.shape
    O = np.zeros_like(q)
    L = np.zeros(q.shape[:3])
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                frames = lists[i // P]
                keys = [j for j in range(k.shape[2]) if j // P in frames]
                if not keys:
                    L[b, h, i] = -math.inf
                    continue
                sc = [scale * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(D))
                      for j in keys]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                z = math.fsum(w)
                L[b, h, i] = mx + math.log(z)
                for d in range(v.shape[3]):
                    O[b, h, i, d] = math.fsum(wj * v[b, h, j, d] for wj, j in zip(w, keys)) / z
    return O, L


def test_brute_force_tiny_sink_window():
    # Shape of the tiny fp32 workload, scaled down: T=4, sink + causal window.
    B, H, T, P, D = 1, 2, 4, 4, 8
    q, k, v = (_rand((B, H, T * P, D), s) for s in (12, 13, 14))
    pol = dict(kind=fs.SINK_WINDOW, n_sink=1, window=2, budget=0, t_per=1, step=0,
               topk=0, n_recent=0, lo=0, hi=-1)
    idx, cnt = fs.build([pol, pol], B, T, T)
    lists = [list(idx[0, 0, t, :cnt[0, 0, t]]) for t in range(T)]
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, P)
    o_ref, lse_ref = _brute(q, k, v, lists, P, 1 / math.sqrt(D))
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_brute_force_scattered_lists_and_outliers():
    B, H, T, P, D = 1, 1, 6, 3, 8
    q, k, v = (_rand((B, H, T * P, D), s, 3.0) for s in (15, 16, 17))
    lists = [[0, 5], [1], [0, 2, 4], [], [3, 4, 5], [0, 1, 2, 3, 4, 5]]
    idx, cnt = _sets(lists)
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, P, scale=0.3)
    o_ref, lse_ref = _brute(q, k, v, lists, P, 0.3)
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)
    # the empty set: O = 0, LSE = -inf
    assert np.all(o[0, 0, 3 * P:4 * P] == 0)
    assert np.all(lse[0, 0, 3 * P:4 * P] == -np.inf)


def test_unattended_frames_do_not_matter():
    B, H, T, P, D = 1, 1, 5, 4, 8
    q, k, v = (_rand((B, H, T * P, D), s) for s in (18, 19, 20))
    lists = [[0, 1], [1, 2], [0, 4], [3], [1, 3]]
    idx, cnt = _sets(lists)
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, P)
    k2, v2 = k.copy(), v.copy()
    # frame 2 is attended only by t=1; change it and only rows of t=1 may move
    k2[0, 0, 2 * P:3 * P] += 5.0
    v2[0, 0, 2 * P:3 * P] -= 7.0
    o2, lse2 = att.sparse_frame_attention(q, k2, v2, idx, cnt, P)
    for t in range(T):
        sl = slice(t * P, (t + 1) * P)
        if t == 1:
            assert not np.allclose(o[0, 0, sl], o2[0, 0, sl])
        else:
            np.testing.assert_array_equal(o[0, 0, sl], o2[0, 0, sl])
            np.testing.assert_array_equal(lse[0, 0, sl], lse2[0, 0, sl])


def test_key_permutation_inside_a_frame_leaves_output_unchanged():
    B, H, T, P, D = 1, 1, 3, 8, 8
    q, k, v = (_rand((B, H, T * P, D), s) for s in (21, 22, 23))
    lists = [[0, 2], [1], [0, 1, 2]]
    idx, cnt = _sets(lists)
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, P)
    perm = np.arange(T * P)
    perm[P:2 * P] = perm[P:2 * P][::-1]
    o2, lse2 = att.sparse_frame_attention(q, k[:, :, perm], v[:, :, perm], idx, cnt, P)
    np.testing.assert_allclose(o, o2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, lse2, atol=1e-13, rtol=0)


def test_row_subset_equals_full_evaluation():
    B, H, T, P, D = 1, 2, 4, 5, 8
    q, k, v = (_rand((B, H, T * P, D), s) for s in (24, 25, 26))
    idx, cnt = _sets([[0], [0, 1], [2, 3], [1, 3]], B, H)
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, P)
    rows = np.array([0, 4, 5, 13, 19])
    o_s, lse_s = att.sparse_frame_attention(q, k, v, idx, cnt, P, rows=rows)
    # BLAS may round a different row count differently in the last bit
    np.testing.assert_allclose(o_s, o[:, :, rows], atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse_s, lse[:, :, rows], atol=1e-14, rtol=0)


def test_shift_of_all_scores_moves_only_lse():
    # Adding one vector u to every key shifts every score of row i by
    # scale·q_i·u: O is unchanged and LSE moves by exactly that amount.
    B, H, T, P, D = 1, 1, 3, 4, 8
    q, k, v = (_rand((B, H, T * P, D), s) for s in (27, 28, 29))
    u = _rand((D,), 30)
    idx, cnt = _sets([[0, 1], [2], [0, 1, 2]])
    o, lse = att.sparse_frame_attention(q, k, v, idx, cnt, P)
    o2, lse2 = att.sparse_frame_attention(q, k + u, v, idx, cnt, P)
    np.testing.assert_allclose(o, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose((lse2 - lse)[0, 0], (q[0, 0] @ u) / math.sqrt(D), atol=1e-12, rtol=0)
