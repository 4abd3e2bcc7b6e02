"""Oracle: softmax attention restricted to the frames of A(t), in float64.

TEST INFRASTRUCTURE -- imported only by tests, the smoke check and the CPU
baseline of the benchmark.  Shares no code with the library.

Definition followed [LVSA page, §2 core mechanism: query frame t attends only
to the frames of A(t) instead of all T frames; complexity paragraph: cost per
query is C·P·d; ISPA §2 item 1: the kernel keeps the log-sum-exp state so that
partial results can be merged afterwards]:

  token n of frame f is n = f·P + p (frame-major, P tokens per frame);
  M[i, j] = 1  iff  floor(j / P) is in A(floor(i / P));
  S = scale · Q Kᵀ with scale = 1/sqrt(D), and S[i, j] = -inf where M is 0;
  LSE_i = m_i + ln Σ_j exp(S_ij - m_i),   m_i = max_j S_ij   (natural log);
  O_i   = Σ_j exp(S_ij - LSE_i) V_j;
  a row with no attended key has O = 0 and LSE = -inf.

Everything is computed in float64 after an exact cast of the inputs.  The mask
is built explicitly; the exponentials of masked entries are exactly zero, so
the sums are taken over the columns the mask keeps (np.flatnonzero), which is
the same value as summing the full masked row.
"""

from __future__ import annotations

import math

import numpy as np


def token_mask(frames, Tk: int, P: int) -> np.ndarray:
    """Boolean key mask [Tk·P]: key j is kept iff its frame floor(j/P) is listed."""
    keep_frame = np.zeros(Tk, dtype=bool)
    for f in frames:
        keep_frame[int(f)] = True
    return np.repeat(keep_frame, P)


def attend_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                scale: float):
    """Masked softmax attention of some query rows against one head's keys.

    q_rows [R, D]; k, v [Nk, D]; mask [Nk] bool.  Returns (O [R, D], LSE [R]).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, D = q_rows.shape
    cols = np.flatnonzero(mask)
    if cols.size == 0:
        return np.zeros((R, v.shape[1]), dtype=np.float64), np.full(R, -np.inf)
    kk = np.asarray(k[cols], dtype=np.float64)
    vv = np.asarray(v[cols], dtype=np.float64)
    s = (q_rows @ kk.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(l[:, 0])
    o = (e / l) @ vv
    return o, lse


def sparse_frame_attention(q, k, v, idx, cnt, P: int, scale: float | None = None,
                           rows=None):
    """Frame-sparse attention for every (b, h) and query row.

    q [B,H,Nq,D], k/v [B,H,Nk,D] (any real dtype; cast exactly to float64);
    idx [B,H,Tq,cap] int, cnt [B,H,Tq] int: A(t) = idx[b,h,t,:cnt[b,h,t]].
    rows: optional sorted array of query-token indices to evaluate (the same
    for every (b, h)); the outputs then have Nq replaced by len(rows).

    Returns (O float64 [B,H,R,D], LSE float64 [B,H,R]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if Nq % P or Nk % P:
        raise ValueError("token counts must be whole frames")
    Tk = Nk // P
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((B, H, rows.size, v.shape[3]), dtype=np.float64)
    LSE = np.full((B, H, rows.size), -np.inf, dtype=np.float64)
    row_frame = rows // P
    for b in range(B):
        for h in range(H):
            for t in np.unique(row_frame):
                sel = np.flatnonzero(row_frame == t)
                frames = idx[b, h, t, :cnt[b, h, t]]
                mask = token_mask(frames, Tk, P)
                o, lse = attend_rows(q[b, h, rows[sel]], k[b, h], v[b, h], mask, scale)
                O[b, h, sel] = o
                LSE[b, h, sel] = lse
    return O, LSE


def dense_attention(q, k, v, scale: float | None = None):
    """Ordinary attention over every key (the FULL frame set), float64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, Nq, D = q.shape
    Nk = np.asarray(k).shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = np.zeros((B, H, Nq, np.asarray(v).shape[3]))
    LSE = np.zeros((B, H, Nq))
    mask = np.ones(Nk, dtype=bool)
    for b in range(B):
        for h in range(H):
            O[b, h], LSE[b, h] = attend_rows(q[b, h], k[b, h], v[b, h], mask, scale)
    return O, LSE
