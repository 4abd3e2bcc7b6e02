"""Pins of the oracle's per-head frame-level RoPE re-encoding (Head Forcing §3).

Checked against: torch's own float32 -> bfloat16 rounding and hand-worked ties
and a double-rounding case for the final rounding; closed-form angles,
composition, norm preservation and shift invariance of the rotation; the
special cases where re-encoding changes nothing (a contiguous frame set gives
the same attention as the true positions; rot = 0 is the identity); and
hand-computed ranks for a set with gaps.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, rope


def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(rope.round_to_bf16(x.astype(np.float64)), ref)


def test_bf16_rounding_ties_and_edges():
    e = 2.0 ** -8
    vals = [1 + e, 1 + 3 * e, -(1 + e), -(1 + 3 * e), 0.0, -0.0, 3.4e38, -3.4e38, math.inf]
    out = rope.round_to_bf16(np.array(vals))
    assert out.tolist() == [1.0, 1 + 4 * e, -1.0, -(1 + 4 * e), 0.0, -0.0, math.inf, -math.inf,
                            math.inf]
    assert math.copysign(1.0, out[5]) == -1.0
    # a float64 value just above a tie rounds up; going through float32 first
    # would land exactly on the tie and round to even (down)
    x = 1 + e + 2.0 ** -40
    assert rope.round_to_bf16(np.array([x]))[0] == 1 + 2 * e
    assert torch.tensor([np.float32(x)]).to(torch.bfloat16).item() == 1.0


def test_frequencies():
    th = rope.frequencies(8, 10000.0)
    assert th[0] == 1.0 and len(th) == 4
    np.testing.assert_allclose(th, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    assert rope.frequencies(0).size == 0
    with pytest.raises(ValueError):
        rope.frequencies(3)


def test_rotation_closed_forms():
    x = np.array([[1.0, 0.0, 7.0, -3.0]])
    # pair 0 has theta 1: a quarter turn moves (1, 0) to (0, 1); channels past rot stay
    y = rope.rotate(x, math.pi / 2, 2)
    np.testing.assert_allclose(y[0, :2], [0.0, 1.0], atol=1e-16)
    assert y[0, 2:].tolist() == [7.0, -3.0]
    y = rope.rotate(np.array([[2.0, 0.0]]), math.pi / 3, 2)
    np.testing.assert_allclose(y[0], [1.0, math.sqrt(3.0)], rtol=1e-15)
    assert (rope.rotate(x, 0.0, 4) == x).all()


def test_rotation_group_properties():
    rng = np.random.default_rng(1)
    D, rot = 16, 12
    q = rng.standard_normal((5, D))
    k = rng.standard_normal((5, D))
    a, b, c = 3.0, 11.0, 40.0
    # composition and norm of each pair
    np.testing.assert_allclose(rope.rotate(rope.rotate(q, a, rot), b, rot),
                               rope.rotate(q, a + b, rot), atol=1e-12)
    r = rope.rotate(q, a, rot)
    np.testing.assert_allclose(r[:, 0:rot:2] ** 2 + r[:, 1:rot:2] ** 2,
                               q[:, 0:rot:2] ** 2 + q[:, 1:rot:2] ** 2, rtol=1e-13)
    # scores depend only on the position difference
    s1 = (rope.rotate(q, a, rot) * rope.rotate(k, b, rot)).sum(1)
    s2 = (rope.rotate(q, a + c, rot) * rope.rotate(k, b + c, rot)).sum(1)
    np.testing.assert_allclose(s1, s2, atol=1e-12)


def test_ranks_close_the_gaps():
    frames = [0, 5, 6, 9]
    assert [rope.new_position(frames, f) for f in (0, 5, 6, 9)] == [0, 1, 2, 3]
    assert rope.new_position(frames, 7) == 3 and rope.new_position(frames, 10) == 4
    rng = np.random.default_rng(2)
    P, D = 3, 4
    q = rng.standard_normal((2 * P, D))   # query frames are KV frames 6 and 7
    k = rng.standard_normal((10 * P, D))
    qn, kn = rope.reencode(q, k, P, frames, offset=6, rot=2, dtype="f64")
    np.testing.assert_allclose(qn[:P], rope.rotate(q[:P], 2, 2), rtol=0, atol=0)
    np.testing.assert_allclose(qn[P:], rope.rotate(q[P:], 3, 2), rtol=0, atol=0)
    np.testing.assert_allclose(kn[5 * P:6 * P], rope.rotate(k[5 * P:6 * P], 1, 2), atol=0)
    assert (kn[P:5 * P] == k[P:5 * P]).all()        # frames outside the set are unchanged


def test_contiguous_set_gives_true_position_attention():
    # frames 4..8, queries in frames 7 and 8 (offset 7): the ranks are the true
    # frame indices minus 4, so the attention equals the one with true positions
    rng = np.random.default_rng(3)
    P, D, rot, Tk = 4, 8, 6, 9
    frames = list(range(4, 9))
    q = rng.standard_normal((2 * P, D))
    k = rng.standard_normal((Tk * P, D))
    v = rng.standard_normal((Tk * P, D))
    qn, kn = rope.reencode(q, k, P, frames, offset=7, rot=rot, dtype="f64")
    qt = rope.rotate(q, np.repeat([7.0, 8.0], P), rot)
    kt = rope.rotate(k, np.repeat(np.arange(Tk, dtype=float), P), rot)
    idx = np.array([[[frames, frames]]], dtype=np.int32)
    cnt = np.array([[[5, 5]]], dtype=np.int32)
    o1, l1 = attention.sparse_frame_attention(qn[None, None], kn[None, None], v[None, None], idx,
                                              cnt, P)
    o2, l2 = attention.sparse_frame_attention(qt[None, None], kt[None, None], v[None, None], idx,
                                              cnt, P)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_gapped_set_differs_from_true_positions():
    rng = np.random.default_rng(4)
    P, D, rot = 2, 4, 4
    frames = [0, 6, 7]
    q = rng.standard_normal((P, D))
    k = rng.standard_normal((8 * P, D))
    qn, kn = rope.reencode(q, k, P, frames, offset=7, rot=rot, dtype="f64")
    # query frame 7 sits at rank 2, key frame 0 at rank 0: distance 2, not 7
    s = qn[0] @ kn[0]
    np.testing.assert_allclose(s, rope.rotate(q[:1], 2, rot)[0] @ k[0], rtol=1e-13)
    assert abs(s - rope.rotate(q[:1], 7, rot)[0] @ k[0]) > 1e-6


def test_rot_zero_and_rounding_of_results():
    rng = np.random.default_rng(5)
    q = torch.randn(6, 8, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    k = torch.randn(12, 8, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    qf, kf = q.double().numpy(), k.double().numpy()
    qn, kn = rope.reencode(qf, kf, 3, [0, 2, 3], offset=2, rot=0)
    assert (qn == qf).all() and (kn == kf).all()
    qn, kn = rope.reencode(qf, kf, 3, [0, 2, 3], offset=2, rot=8)
    # results are bfloat16 values
    assert (torch.from_numpy(qn).to(torch.bfloat16).double().numpy() == qn).all()
    qf32, _ = rope.reencode(rng.standard_normal((6, 8)), rng.standard_normal((12, 8)), 3, [1],
                            offset=0, rot=4, dtype="f32")
    assert (qf32.astype(np.float32).astype(np.float64) == qf32).all()
