"""Pins of the oracle's two-level (frame, then block) selection (Light Forcing
§2.2 hierarchical sparse attention).

Checked against: hand-computed lists on planted scores (integers, exact), exact
rational arithmetic on random inputs, the hierarchical summation order, the
special cases that reduce to the frame-level memory selection (blocks as large
as frames) and to dense causal attention (everything selected), and the
block-unit form of frame-level policies.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import attention, frame_sets, hsa, topk


def test_block_and_frame_sums_are_exact_sums_of_tokens():
    # blocks of 2: 1e16 + 1 and -1e16 + 1 are ties that round to even (+-1e16);
    # the frame sum is the exact sum of its 4 tokens, 2 -- not the sum of the
    # rounded block sums (0) nor any sequential order (1)
    x = np.array([[1e16], [1.0], [-1e16], [1.0]])
    assert hsa.block_sums(x, 2).tolist() == [[1e16], [-1e16]]
    assert hsa.block_sums(x, 4).tolist() == [[2.0]]
    with pytest.raises(ValueError):
        hsa.block_sums(x, 3)


def _planted():
    # D = 2, frames of P = 6 tokens in nb = 3 blocks of Bs = 2; query block sum (1, 0).
    # Per-block key sums (channel 0) chosen so that frame 1 has the best single block
    # but a poor frame total, and frames 3 and 0 win level 1.
    per_block = {
        0: [4, 3, 2],      # frame total 9
        1: [50, -40, -8],  # frame total 2, holds the best block (50)
        2: [1, 1, 1],      # 3
        3: [5, 5, 6],      # 16
        4: [0, 0, 0],      # 0
        5: [0, 0, 0],      # recent frame
    }
    kblocks = np.zeros((6 * 3, 2))
    for f, vals in per_block.items():
        for i, v in enumerate(vals):
            kblocks[f * 3 + i, 0] = v
            kblocks[f * 3 + i, 1] = 7 * f + i   # channel 1 is ignored by the query
    kframes = kblocks.reshape(6, 3, 2).sum(axis=1)    # small integers: exact
    return kblocks, kframes


def test_planted_two_level_selection():
    kblocks, kframes = _planted()
    q = np.array([1.0, 0.0])
    blocks, frames = hsa.select_blocks(q, kblocks, kframes, nb=3, e=5, n_recent=1, kf=2, kb=4)
    assert frames == [0, 3]                      # totals 16 and 9 beat 3, 2, 0
    # blocks of frames 0 and 3 by score: 11 (6), 9 (5), 10 (5), 0 (4), 1 (3), 2 (2)
    # -> 9, 10, 11 and 0, the tie 9/10 going to the lower index; then frame 5's blocks
    assert blocks == [0, 9, 10, 11, 15, 16, 17]
    # block 3 (score 50) is never a candidate: its frame lost at level 1
    assert 3 not in blocks


def test_planted_selection_with_more_recent_frames():
    kblocks, kframes = _planted()
    q = np.array([1.0, 0.0])
    blocks, frames = hsa.select_blocks(q, kblocks, kframes, nb=3, e=5, n_recent=3, kf=1, kb=2)
    # candidates 0..2; frame 0 (9) wins; its blocks 0 (4), 1 (3)
    assert frames == [0]
    assert blocks == [0, 1] + list(range(9, 18))


def _exact_dot(a, b):
    return sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b))


@pytest.mark.parametrize("seed", range(5))
def test_matches_exact_arithmetic(seed):
    rng = np.random.default_rng(100 + seed)
    D, Bs, nb, F = 8, 3, 4, 9
    P = Bs * nb
    qtok = rng.standard_normal((Bs, D)).astype(np.float32)
    ktok = rng.standard_normal((F * P, D)).astype(np.float32)
    e, n_recent, kf, kb = F - 1, 2, 3, 5
    qsum = hsa.block_sums(qtok, Bs)[0]
    kbl = hsa.block_sums(ktok, Bs)
    kfr = hsa.block_sums(ktok, P)
    blocks, frames = hsa.select_blocks(qsum, kbl, kfr, nb, e, n_recent, kf, kb)
    # exact sums over tokens (any order), exact scores
    qx = [sum(Fraction(float(qtok[p, d])) for p in range(Bs)) for d in range(D)]
    kx = [[sum(Fraction(float(ktok[b * Bs + p, d])) for p in range(Bs)) for d in range(D)]
          for b in range(F * nb)]
    cands = range(e - n_recent + 1)
    fscore = {f: sum(qx[d] * sum(kx[f * nb + i][d] for i in range(nb)) for d in range(D))
              for f in cands}
    order = sorted(cands, key=lambda f: (-fscore[f], f))
    assert abs(fscore[order[kf - 1]] - fscore[order[kf]]) > Fraction(1, 10**6)
    assert frames == sorted(order[:kf])
    cb = [f * nb + i for f in frames for i in range(nb)]
    bscore = {b: sum(qx[d] * kx[b][d] for d in range(D)) for b in cb}
    border = sorted(cb, key=lambda b: (-bscore[b], b))
    assert abs(bscore[border[kb - 1]] - bscore[border[kb]]) > Fraction(1, 10**6)
    recent = list(range((e - n_recent + 1) * nb, (e + 1) * nb))
    assert blocks == sorted(border[:kb]) + recent


def test_blocks_as_large_as_frames_reduce_to_memory_selection():
    rng = np.random.default_rng(5)
    D, P, F = 8, 5, 10
    q = rng.standard_normal((P, D))            # one query frame = one query block
    k = rng.standard_normal((F * P, D))
    e, n_recent, kf = F - 1, 3, 4
    blocks, frames = hsa.select_blocks(hsa.block_sums(q, P)[0], hsa.block_sums(k, P),
                                       hsa.block_sums(k, P), 1, e, n_recent, kf, kf)
    ref, _ = topk.select_topk_frames(q, k, P, range(P), frame_sets.memory_candidates(n_recent, e),
                                     kf)
    assert frames == ref
    assert blocks == frame_sets.memory(ref, n_recent, e)


def test_selecting_everything_is_dense_causal_attention():
    rng = np.random.default_rng(6)
    D, Bs, nb, Tk, chunk = 8, 4, 3, 6, 2
    P = Bs * nb
    Tq, offset = 2, Tk - 2                     # one chunk: query frames are KV frames 4, 5
    q = rng.standard_normal((Tq * P, D))
    k = rng.standard_normal((Tk * P, D))
    v = rng.standard_normal((Tk * P, D))
    n_recent = 2
    n_cand = Tk - n_recent
    lists = hsa.hsa_lists(q, k, P, Bs, offset, chunk, n_recent, kf=n_cand, kb=n_cand * nb)
    assert all(a == list(range(Tk * nb)) for a in lists)
    idx = np.array(lists, dtype=np.int32)[None, None]
    cnt = np.full((1, 1, len(lists)), Tk * nb, dtype=np.int32)
    o, lse = attention.sparse_frame_attention(q[None, None], k[None, None], v[None, None], idx,
                                              cnt, Bs)
    od, lsed = attention.dense_attention(q[None, None], k[None, None], v[None, None])
    np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, rtol=1e-12, atol=1e-12)


def test_query_blocks_of_one_chunk_share_the_history_end():
    rng = np.random.default_rng(7)
    D, Bs, nb, Tk = 4, 2, 2, 8
    P = Bs * nb
    q = rng.standard_normal((3 * P, D))        # three query frames, chunk of 3
    k = rng.standard_normal((Tk * P, D))
    lists = hsa.hsa_lists(q, k, P, Bs, offset=Tk - 3, chunk=3, n_recent=3, kf=2, kb=3)
    assert len(lists) == 3 * nb
    for a in lists:
        assert a[-3 * nb:] == list(range((Tk - 3) * nb, Tk * nb))   # the chunk itself
        assert len(a) == 3 + 3 * nb and all(b < (Tk - 3) * nb for b in a[:3])


def test_budget_errors():
    kblocks, kframes = _planted()
    q = np.array([1.0, 0.0])
    with pytest.raises(ValueError):
        hsa.select_blocks(q, kblocks, kframes, nb=3, e=5, n_recent=1, kf=6, kb=1)  # 5 cands
    with pytest.raises(ValueError):
        hsa.select_blocks(q, kblocks, kframes, nb=3, e=5, n_recent=1, kf=1, kb=4)  # 3 blocks
    with pytest.raises(ValueError):
        hsa.select_blocks(q, kblocks, kframes, nb=3, e=1, n_recent=3, kf=1, kb=1)


@pytest.mark.parametrize("n_sink,window", [(0, 6), (3, 6), (1, 2)])
def test_block_unit_policies_expand_frame_lists(n_sink, window):
    nb, Tq, Tk, offset, chunk = 4, 3, 12, 9, 3
    pol = dict(kind=frame_sets.SINK_WINDOW, n_sink=n_sink, window=window)
    idx_f, cnt_f = frame_sets.build([pol], 1, Tq, Tk, offset, chunk)
    bpol = hsa.scale_policy_to_blocks(pol, nb)
    idx_b, cnt_b = frame_sets.build([bpol], 1, Tq * nb, Tk * nb, offset * nb, chunk * nb)
    for j in range(Tq * nb):
        frames = idx_f[0, 0, j // nb, :cnt_f[0, 0, j // nb]]
        expect = [f * nb + i for f in frames for i in range(nb)]
        assert idx_b[0, 0, j, :cnt_b[0, 0, j]].tolist() == expect
    rng_pol = hsa.scale_policy_to_blocks(dict(kind=frame_sets.RANGE, lo=2, hi=4), nb)
    assert (rng_pol["lo"], rng_pol["hi"]) == (8, 19)
    with pytest.raises(ValueError):
        hsa.scale_policy_to_blocks(dict(kind=frame_sets.MEMORY, topk=2, n_recent=1), nb)
