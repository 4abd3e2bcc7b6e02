"""Oracle: per-head frame-level RoPE re-encoding of an assembled KV cache.

TEST INFRASTRUCTURE -- imported only by tests, the smoke check and the CPU
baseline of the benchmark.  Shares no code with the library.

[Head Forcing page, §3 per-head RoPE re-encoding: keys are cached with the
spatial rotary encoding only; when a head's cache is assembled, the
frame-level (temporal) positions are encoded again for that head alone, so
that query-key relative positions stay inside the range seen in training
however long the generation runs.]

Readings (the page fixes neither the channel layout, the frequencies nor the
new positions):
  * the temporal rotation acts on the first `rot` channels of a head (rot
    even, 0 <= rot <= D) as rot/2 interleaved pairs (2i, 2i+1); the other
    channels (the spatial part, already encoded when cached) are unchanged;
  * pair i turns by the angle pos * theta_i with theta_i = base^(-2i/rot)
    (the usual rotary frequencies, base 10000 unless stated);
  * a head's new position of KV frame f is its rank in the head's sorted
    frame set A, i.e. the number of frames of A before f; a query frame takes
    the same rank of its own KV frame (offset + tq), so the assembled frames
    sit at consecutive positions and the gaps of the set are closed;
  * the rotation is computed in float64 (each product rounded, no fused
    multiply-add) and rounded once to the storage type: round to nearest,
    ties to even, for bfloat16 and for float32.
"""

from __future__ import annotations

import numpy as np


def frequencies(rot: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base^(-2i/rot) for i < rot/2, float64."""
    if rot % 2 or rot < 0:
        raise ValueError("rot must be even and non-negative")
    return np.array([base ** ((-2.0 * i) / rot) for i in range(rot // 2)], dtype=np.float64)


def rotate(x: np.ndarray, pos, rot: int, base: float = 10000.0) -> np.ndarray:
    """x [N, D] float64 with pair i of row n turned by pos[n] * theta_i."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    pos = np.broadcast_to(np.asarray(pos, dtype=np.float64), (x.shape[0],))
    for i, th in enumerate(frequencies(rot, base)):
        ang = pos * th
        c = np.cos(ang)
        s = np.sin(ang)
        a = x[:, 2 * i]
        b = x[:, 2 * i + 1]
        out[:, 2 * i] = a * c - b * s
        out[:, 2 * i + 1] = a * s + b * c
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> the nearest bfloat16 value (ties to even), as float64.

    bfloat16 keeps 8 significant bits: the value is scaled so that its
    significand has 8 integer bits, rounded half to even, and scaled back
    (exact power-of-two scalings).  Below the normal range the spacing is
    2^-133; beyond the largest finite value the result is infinite."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                          # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                     # subnormal bf16: fixed spacing 2^-133
    with np.errstate(invalid="ignore", over="ignore"):
        q = np.rint(np.ldexp(x, 8 - e))         # 8 significant bits, ties to even
        r = np.ldexp(q, e - 8)
        big = np.abs(r) > 3.3895313892515355e38  # past the largest finite bfloat16
    return np.where(big, np.copysign(np.inf, x), r)


def new_position(frames_sorted, f: int) -> int:
    """Rank of frame f in the head's set: how many listed frames come before it."""
    return int(sum(1 for g in frames_sorted if g < f))


def reencode(q_bh: np.ndarray, k_bh: np.ndarray, P: int, frames, offset: int, rot: int,
             base: float = 10000.0, dtype: str = "bf16"):
    """Re-encoded (q', k') of one head for its frame set `frames`.

    Query token n (query frame tq = n // P, KV frame offset + tq) turns by the
    rank of offset + tq; key rows of listed frame f turn by the rank of f.
    Key rows of frames outside the set are returned unchanged (the attention
    over this set never reads them).  Values are float64 holding values of the
    storage type ("bf16" or "f32"; "f64" skips the final rounding)."""
    frames = sorted(int(f) for f in frames)
    q = np.asarray(q_bh, dtype=np.float64)
    k = np.asarray(k_bh, dtype=np.float64)
    qpos = np.array([new_position(frames, offset + n // P) for n in range(q.shape[0])])
    qn = rotate(q, qpos, rot, base)
    kn = k.copy()
    for r, f in enumerate(frames):
        kn[f * P:(f + 1) * P] = rotate(k[f * P:(f + 1) * P], r, rot, base)
    if dtype == "bf16":
        return round_to_bf16(qn), round_to_bf16(kn)
    if dtype == "f32":
        return qn.astype(np.float32).astype(np.float64), kn.astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return qn, kn
    raise ValueError(f"unknown dtype {dtype}")
