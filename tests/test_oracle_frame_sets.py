"""Pins of the oracle's frame sets against the pages' stated properties and
hand-worked cases (tests/golden/frame_sets.txt)."""

import os

import pytest

from oracle import frame_sets as fs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "frame_sets.txt")


def _parse_frames(text):
    out = []
    for item in text.split(","):
        item = item.strip()
        if "-" in item:
            a, b = item.split("-")
            out.extend(range(int(a), int(b) + 1))
        else:
            out.append(int(item))
    return out


def _golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split(":")
            parts = lhs.split()
            kind, kv = parts[0], dict(p.split("=") for p in parts[1:])
            cases.append((kind, kv, _parse_frames(rhs)))
    return cases


@pytest.mark.parametrize("kind,kv,expected", _golden_cases())
def test_golden_hand_worked(kind, kv, expected):
    if kind == "lvsa":
        got = fs.lvsa(int(kv["T"]), int(kv["C"]), int(kv["W"]), int(kv["T_per"]),
                      int(kv["s"]), int(kv["t"]))
    elif kind == "sink_window":
        got = fs.sink_window(int(kv["n_sink"]), int(kv["w"]), int(kv["e"]))
    elif kind == "memory":
        got = fs.memory(_parse_frames(kv["selected"]), int(kv["n_recent"]), int(kv["e"]))
    else:
        raise AssertionError(kind)
    assert got == expected


def _anchors_seen_by_all(T, C, W, T_per, s):
    """Frames present in A_s(t) for every t: for a long video these are exactly
    the anchors, since windows of distant query frames do not overlap."""
    common = set(range(T))
    for t in range(T):
        common &= set(fs.lvsa(T, C, W, T_per, s, t))
    return common


@pytest.mark.parametrize("T,C,W,T_per", [(42, 21, 7, 6), (126, 33, 11, 8), (60, 12, 5, 4),
                                         (37, 9, 3, 5)])
def test_each_frame_is_anchor_exactly_once_per_period(T, C, W, T_per):
    # LVSA §2 item 1: over T_per consecutive steps each frame is an anchor exactly once.
    for s0 in (0, 3):
        count = {f: 0 for f in range(T)}
        for s in range(s0, s0 + T_per):
            for f in _anchors_seen_by_all(T, C, W, T_per, s):
                count[f] += 1
        assert all(c == 1 for c in count.values()), count


@pytest.mark.parametrize("T,C,W,T_per,S", [(42, 21, 7, 6, 6), (126, 33, 11, 8, 8)])
def test_budget_met_exactly_on_the_workloads(T, C, W, T_per, S):
    # LVSA §2 item 2: the widened window keeps |A(t)| at the budget C.
    for s in range(S):
        for t in range(T):
            a = fs.lvsa(T, C, W, T_per, s, t)
            assert len(a) == C
            assert a == sorted(set(a)) and 0 <= a[0] and a[-1] < T


def _lvsa_by_interval(T, C, W, T_per, s, t):
    """Independent closed form of the same reading: the k nearest frames to t
    (ties to the past, shifted inward at the ends) form the interval
    [lo, lo + L - 1] with lo = clamp(t - floor(L/2), 0, T - L); take the
    shortest L >= min(W, T) whose union with the anchors reaches min(C, T)."""
    G = {f for f in range(T) if f % T_per == s % T_per}
    L = min(W, T)
    while True:
        lo = min(max(t - L // 2, 0), T - L)
        A = G | set(range(lo, lo + L))
        if len(A) >= min(C, T) or L == T:
            return sorted(A), G
        L += 1


def test_matches_interval_closed_form_small_sweep():
    for T in range(1, 19):
        for T_per in range(1, 7):
            for W in range(1, 8):
                for C in range(1, 20):
                    for s in range(T_per):
                        for t in range(T):
                            a = fs.lvsa(T, C, W, T_per, s, t)
                            b, G = _lvsa_by_interval(T, C, W, T_per, s, t)
                            assert a == b, (T, C, W, T_per, s, t)
                            assert G <= set(a) and t in a
                            assert len(a) >= min(C, T)


def test_window_of_even_width_leans_to_the_past():
    a = fs.lvsa(10, 4, 4, 100, 0, 5)
    assert a == [0, 3, 4, 5, 6]


def test_window_shifts_inward_at_the_ends():
    assert fs.lvsa(30, 5, 5, 1000, 0, 0) == [0, 1, 2, 3, 4]
    assert fs.lvsa(30, 5, 5, 1000, 0, 29) == [0, 25, 26, 27, 28, 29]


def test_build_pads_with_minus_one_and_counts():
    pols = [dict(kind=fs.SINK_WINDOW, n_sink=1, window=2, budget=0, t_per=1, step=0,
                 topk=0, n_recent=0, lo=0, hi=-1)] * 2
    idx, cnt = fs.build(pols, B=1, Tq=4, Tk=4)
    assert idx.shape == (1, 2, 4, 3)
    assert cnt.tolist() == [[[1, 2, 3, 3], [1, 2, 3, 3]]]
    assert idx[0, 0].tolist() == [[0, -1, -1], [0, 1, -1], [0, 1, 2], [0, 2, 3]]


def test_chunk_mode_shares_one_set_per_chunk():
    pol = dict(kind=fs.SINK_WINDOW, n_sink=3, window=6, budget=0, t_per=1, step=0,
               topk=0, n_recent=0, lo=0, hi=-1)
    idx, cnt = fs.build([pol], B=1, Tq=3, Tk=60, offset=57, chunk=3)
    for tq in range(3):
        assert idx[0, 0, tq, :cnt[0, 0, tq]].tolist() == [0, 1, 2, 54, 55, 56, 57, 58, 59]


def test_memory_candidates_exclude_recent():
    assert fs.memory_candidates(3, 59) == list(range(57))


def test_range_and_full():
    assert fs.frame_range(1, 45, 49) == list(range(1, 46))
    assert fs.frame_range(-3, 100, 5) == [0, 1, 2, 3, 4]
    assert fs.full(4) == [0, 1, 2, 3]


@pytest.mark.parametrize("offset,chunk", [(0, 1), (57, 3), (5, 4), (0, 7)])
def test_chunk_last_frame_is_the_chunks_last_kv_frame(offset, chunk):
    # A chunk covers query frames [c*chunk, (c+1)*chunk), i.e. KV frames
    # offset + c*chunk .. offset + (c+1)*chunk - 1; every member maps to the last.
    for tq in range(4 * chunk):
        e = fs.chunk_last_frame(tq, chunk, offset)
        assert 0 <= e - (offset + tq) < chunk
        assert (e - offset + 1) % chunk == 0
        first = tq - tq % chunk
        assert all(fs.chunk_last_frame(u, chunk, offset) == e for u in range(first, first + chunk))
    # the AR workload: query frames 0..2 at KV frames 57..59 form one chunk ending at 59
    if (offset, chunk) == (57, 3):
        assert [fs.chunk_last_frame(t, 3, 57) for t in range(3)] == [59, 59, 59]
