"""Oracle: frame mean-pooling and top-k frame selection for memory heads.

TEST INFRASTRUCTURE -- imported only by tests, the smoke check and the CPU
baseline of the benchmark.  Shares no code with the library.

[Light Forcing page, §2.2 hierarchical sparse attention: query and key tokens
are compressed by mean pooling to frame granularity, and for each query block
the most relevant history frames are picked with the frame-level keys.
Head Forcing, methodology §2: memory heads keep selected frames besides the
fast memory of recent frames.]

Readings (the pages fix neither the arithmetic nor the tie rule):
  * pooling is kept as float64 sums; a mean differs from the sum by a positive
    factor, so the ranking is the same under exact arithmetic and no division
    enters the bits;
  * qf[t,d]   = Σ_p Q[t·P + p, d]: queries are compressed to frame
                granularity first, like the keys, added one at a time in
                ascending p;
  * qsum[d]   = Σ_t qf[t, d] over the frames of the query group, added one at
                a time in ascending frame order (in exact arithmetic: the sum
                over all of the group's tokens);
  * ksum[f,d] = Σ_p K[f·P + p, d], added one at a time in ascending p;
  * score[f]  = Σ_d qsum[d] · ksum[f, d], each product rounded to float64 and
                then added one at a time in ascending d (no fused multiply-add);
  * frames are ranked by (score descending, frame index ascending) and the
    first k are returned in ascending frame order.
Because the order of every floating-point operation is fixed, any correct
implementation of these steps gives the same bits, hence the same frames.
"""

from __future__ import annotations

import numpy as np


def pooled_query_sum(q_tokens: np.ndarray, P: int) -> np.ndarray:
    """qsum[d] of a query group given as whole frames of P tokens (q_tokens [F·P, D]):
    each frame summed sequentially over its tokens, then the frame sums added
    sequentially in frame order (all in float64)."""
    q = np.asarray(q_tokens, dtype=np.float64)
    if q.shape[0] % P:
        raise ValueError("a query group is made of whole frames")
    acc = np.zeros(q.shape[1], dtype=np.float64)
    for f in range(q.shape[0] // P):
        frame = np.zeros(q.shape[1], dtype=np.float64)
        for p in range(P):
            frame = frame + q[f * P + p]
        acc = acc + frame
    return acc


def pooled_key_sums(k_tokens: np.ndarray, P: int, frames) -> np.ndarray:
    """ksum[f, d] for the listed frames: float64 sums sequential in p."""
    k = np.asarray(k_tokens)
    frames = np.asarray(list(frames), dtype=np.int64)
    acc = np.zeros((frames.size, k.shape[1]), dtype=np.float64)
    for p in range(P):
        acc = acc + k[frames * P + p].astype(np.float64)
    return acc


def frame_scores(qsum: np.ndarray, ksum: np.ndarray) -> np.ndarray:
    """score[f] = Σ_d qsum[d]·ksum[f,d]: rounded products added sequentially in d."""
    acc = np.zeros(ksum.shape[0], dtype=np.float64)
    for d in range(qsum.shape[0]):
        prod = qsum[d] * ksum[:, d]
        acc = acc + prod
    return acc


def rank_topk(scores: np.ndarray, frames, k: int) -> list[int]:
    """The k best frames by (score descending, index ascending), sorted ascending."""
    frames = [int(f) for f in frames]
    if k > len(frames):
        raise ValueError(f"k={k} exceeds the {len(frames)} candidate frames")
    if not np.all(np.isfinite(scores)):
        raise ValueError("non-finite frame score")
    order = sorted(range(len(frames)), key=lambda i: (-scores[i], frames[i]))
    return sorted(frames[i] for i in order[:k])


def select_topk_frames(q_bh: np.ndarray, k_bh: np.ndarray, P: int, q_rows,
                       cand_frames, k: int):
    """Top-k frames of one (b, h, query group).

    q_bh [Nq, D], k_bh [Nk, D]; q_rows are the token indices of the query
    group's frames (whole frames, in order); cand_frames the KV frames that may
    be chosen.
    Returns (sorted frames, scores of every candidate).
    """
    qsum = pooled_query_sum(np.asarray(q_bh)[np.asarray(q_rows)], P)
    ksum = pooled_key_sums(k_bh, P, cand_frames)
    scores = frame_scores(qsum, ksum)
    return rank_topk(scores, cand_frames, k), scores
