"""Oracle: frame mean-pooling and top-k frame selection for memory heads.

TEST INFRASTRUCTURE -- imported only by tests, the smoke check and the CPU
baseline of the benchmark.  Shares no code with the library.

[Light Forcing page, §2.2 hierarchical sparse attention: query and key tokens
are compressed by mean pooling to frame granularity, and for each query block
the most relevant history frames are picked with the frame-level keys.
Head Forcing, methodology §2: memory heads keep selected frames besides the
fast memory of recent frames.]

Readings (the pages fix neither the arithmetic nor the tie rule):
  * "mean pooling" of a set of tokens is taken as their sum per channel: a
    mean differs from the sum by a positive factor, so the ranking is the
    same and no division enters the bits;
  * each pooled sum is the EXACT sum of its (float64-widened) tokens, rounded
    once to the nearest float64, ties to even -- the plain definition of a sum
    that does not depend on any order of summation:
      qsum[d]   = RN(sum of Q[i, d] over every token i of the query group),
      ksum[f,d] = RN(sum of K[f*P + p, d] over p = 0..P-1);
    computed with math.fsum, which returns exactly that rounded value;
  * score[f]  = sum over d of qsum[d] * ksum[f, d], each product rounded to
    float64 and then added one at a time in ascending d (no fused
    multiply-add): a fixed, plain evaluation of a length-D dot product;
  * frames are ranked by (score descending, frame index ascending) and the
    first k are returned in ascending frame order.
Every result has one definition, so any correct implementation gives the same
bits, hence the same frames.
"""

from __future__ import annotations

import math

import numpy as np


def exact_column_sums(x: np.ndarray) -> np.ndarray:
    """[N, D] -> [D]: each column's exact sum, rounded once to float64."""
    x = np.asarray(x, dtype=np.float64)
    # + 0.0: an exact sum of zero is +0.0 whatever the signs of the zero terms
    return np.array([math.fsum(col) + 0.0 for col in x.T.tolist()], dtype=np.float64)


def pooled_query_sum(q_tokens: np.ndarray, P: int) -> np.ndarray:
    """qsum[d] of a query group given as whole frames of P tokens (q_tokens
    [F*P, D]): the exact sum over all of the group's tokens, rounded once."""
    q = np.asarray(q_tokens, dtype=np.float64)
    if q.shape[0] % P:
        raise ValueError("a query group is made of whole frames")
    return exact_column_sums(q)


def pooled_key_sums(k_tokens: np.ndarray, P: int, frames) -> np.ndarray:
    """ksum[f, d] for the listed frames: each frame's exact sum, rounded once."""
    k = np.asarray(k_tokens)
    frames = [int(f) for f in frames]
    out = np.zeros((len(frames), k.shape[1]), dtype=np.float64)
    for i, f in enumerate(frames):
        out[i] = exact_column_sums(k[f * P:(f + 1) * P])
    return out


def frame_scores(qsum: np.ndarray, ksum: np.ndarray) -> np.ndarray:
    """score[f] = sum_d qsum[d]*ksum[f,d]: rounded products added sequentially in d."""
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
                       cand_frames, k: int, ksum: np.ndarray | None = None):
    """Top-k frames of one (b, h, query group).

    q_bh [Nq, D], k_bh [Nk, D]; q_rows are the token indices of the query
    group's frames (whole frames, in order); cand_frames the KV frames that may
    be chosen.  ksum, if given, holds the pooled key sums of cand_frames (as
    pooled_key_sums returns them), so callers that select repeatedly from the
    same frames pool them once.
    Returns (sorted frames, scores of every candidate).
    """
    qsum = pooled_query_sum(np.asarray(q_bh)[np.asarray(q_rows)], P)
    if ksum is None:
        ksum = pooled_key_sums(k_bh, P, cand_frames)
    scores = frame_scores(qsum, ksum)
    return rank_topk(scores, cand_frames, k), scores
