"""Oracle: per-head frame sets A(t) (integer only, plain Python).

TEST INFRASTRUCTURE -- imported only by tests, the smoke check and the CPU
baseline of the benchmark.  Shares no code with the library.

A frame set is the sorted list of KV frame indices that every query token of
query frame t attends to.  Policies:

FULL         every KV frame.
LVSA         rotating global anchors united with a local window that widens
             until the set reaches the budget C
             [LVSA page, §2 core mechanism: A(t) = G ∪ W(t); item 1 rotating
             global anchors shifted by s mod T_per at denoising step s; item 2
             expanded adaptive window keeping |A(t)| near the budget C].
SINK_WINDOW  the first n_sink frames (attention sink / anchor frames) united
             with the w most recent frames up to the end of the query's chunk
             [Head Forcing, methodology §2: local heads keep the current block
             and its nearest frames, anchor heads add the first latent frames;
             ISPA §2 item 1: local stream = current frame + sink].
MEMORY       top-k frames chosen by pooled scores united with the n_recent
             most recent frames (fast memory)
             [Head Forcing, methodology §2, memory heads (fast memory);
             Light Forcing §2.2 step 1, frame selection per query block].
RANGE        every frame in [lo, hi] (an explicit history branch, e.g. the
             history half of ISPA's decomposable attention).

Readings where the pages leave a step open (each listed in the design notes):
  * anchors at step s are the frames f with f mod T_per == s mod T_per;
  * the local window is the W frames nearest to t, ties going to the earlier
    frame, shifted inward at the ends of the video;
  * widening: the window keeps growing nearest-first until |G ∪ W| reaches
    min(C, T); it never shrinks below W and no anchor is ever dropped, so if
    G ∪ W is already larger than C it is kept as is;
  * in chunked (autoregressive) mode every query frame of a chunk shares the
    set built for the last KV frame e of that chunk.
"""

from __future__ import annotations

import numpy as np

FULL, LVSA, SINK_WINDOW, MEMORY, RANGE = 0, 1, 2, 3, 4


def lvsa(T: int, C: int, W: int, T_per: int, s: int, t: int) -> list[int]:
    """LVSA frame set A_s(t) for query frame t of a T-frame video at step s.

    [LVSA page, §2 core mechanism, items 1 and 2.]
    """
    r = s % T_per
    # rotating global anchors G_s: one residue class of the T_per-periodic grid
    anchors = {f for f in range(T) if f % T_per == r}
    # frames ordered by distance to t, the earlier frame first on ties
    by_distance = sorted(range(T), key=lambda f: (abs(f - t), f))
    k = min(W, T)
    target = min(C, T)
    while len(anchors | set(by_distance[:k])) < target:
        k += 1
    return sorted(anchors | set(by_distance[:k]))


def chunk_last_frame(tq: int, chunk: int, offset: int) -> int:
    """KV index of the last frame of the chunk that query frame tq belongs to.

    Query frame tq sits at KV frame offset + tq; chunks are `chunk` query
    frames long and a chunk attends up to and including its own last frame.
    """
    return offset + (tq // chunk + 1) * chunk - 1


def sink_window(n_sink: int, w: int, e: int) -> list[int]:
    """Sink frames {0..n_sink-1} united with the w frames ending at e.

    [Head Forcing, methodology §2, local and anchor heads.]
    """
    sink = set(range(n_sink))
    window = set(range(max(0, e - w + 1), e + 1))
    return sorted(sink | window)


def memory_candidates(n_recent: int, e: int) -> list[int]:
    """Frames a memory head may select from: everything before the recent frames."""
    return list(range(0, max(0, e - n_recent + 1)))


def memory(selected: list[int], n_recent: int, e: int) -> list[int]:
    """Top-k selected frames united with the n_recent frames ending at e.

    [Head Forcing, methodology §2, memory heads: fast memory of recent frames;
    Light Forcing §2.2 step 1 for the selected frames.]
    """
    recent = set(range(max(0, e - n_recent + 1), e + 1))
    return sorted(set(int(f) for f in selected) | recent)


def frame_range(lo: int, hi: int, Tk: int) -> list[int]:
    """Every frame f with lo <= f <= hi, clipped to [0, Tk)."""
    return list(range(max(0, lo), min(hi, Tk - 1) + 1))


def full(Tk: int) -> list[int]:
    """Every KV frame: ordinary dense attention."""
    return list(range(Tk))


def frame_set_for(policy: dict, Tq: int, Tk: int, offset: int, chunk: int, tq: int,
                  selected=None) -> list[int]:
    """Frame set of one query frame under one head's policy.

    policy keys: kind, n_sink, window, budget, t_per, step, topk, n_recent, lo, hi.
    `selected` holds the top-k frames of this query frame's group (MEMORY only).
    Every set is a subset of the existing frames {0..Tk-1} [LVSA §2: A(t)
    replaces the full set {0, ..., T-1}], so a sink longer than the cache is cut.
    """
    kind = policy["kind"]
    if kind == FULL:
        frames = full(Tk)
    elif kind == LVSA:
        frames = lvsa(Tk, policy["budget"], policy["window"], policy["t_per"],
                      policy["step"], offset + tq)
    else:
        e = chunk_last_frame(tq, chunk, offset)
        if kind == SINK_WINDOW:
            frames = sink_window(policy["n_sink"], policy["window"], e)
        elif kind == MEMORY:
            frames = memory(selected, policy["n_recent"], e)
        elif kind == RANGE:
            frames = frame_range(policy["lo"], policy["hi"], Tk)
        else:
            raise ValueError(f"unknown policy kind {kind}")
    return [f for f in frames if 0 <= f < Tk]


def build(policies: list[dict], B: int, Tq: int, Tk: int, offset: int = 0,
          chunk: int = 1, selected=None, cap: int | None = None):
    """Frame sets of every (b, h, tq) as padded arrays.

    Returns (idx int32 [B,H,Tq,cap], cnt int32 [B,H,Tq]); entries of idx past
    cnt are -1.  `selected[b][h][g]` lists the chosen frames of query group
    g = tq // chunk for MEMORY heads.
    """
    H = len(policies)
    sets = []
    for b in range(B):
        for h in range(H):
            for tq in range(Tq):
                sel = None
                if policies[h]["kind"] == MEMORY:
                    sel = selected[b][h][tq // chunk]
                sets.append(frame_set_for(policies[h], Tq, Tk, offset, chunk, tq, sel))
    need = max((len(a) for a in sets), default=0)
    if cap is None:
        cap = max(need, 1)
    if need > cap:
        raise ValueError(f"frame set of {need} frames exceeds capacity {cap}")
    idx = np.full((B, H, Tq, cap), -1, dtype=np.int32)
    cnt = np.zeros((B, H, Tq), dtype=np.int32)
    n = 0
    for b in range(B):
        for h in range(H):
            for tq in range(Tq):
                a = sets[n]
                n += 1
                idx[b, h, tq, :len(a)] = a
                cnt[b, h, tq] = len(a)
    return idx, cnt
