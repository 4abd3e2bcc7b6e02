"""Oracle: chunk-aware growth (CAG) of the sparsity ratio across the chunks of
an autoregressive rollout.

TEST INFRASTRUCTURE -- imported only by tests, the smoke check and the CPU
baseline of the benchmark.  Shares no code with the library.

[Light Forcing page, §2.1 chunk-aware growth: the first chunk is attended
densely and later chunks, which inherit structure from the clean chunks
before them, are made progressively sparser; the sparsity of chunk i is
s_i = s_base - alpha_i * beta, alpha_i following the noise level (in
proportion to 1/sqrt(T)), with beta set so that the total attention FLOPs
equal those of a target sparsity.]

Readings (the page leaves alpha_i, s_base and the matching open):
  * chunk 0 is dense: s_0 = 0;
  * alpha_i = 1/sqrt(i + 1) for chunk i >= 1 (the 1/sqrt law in the chunk
    count; decreasing in i, so beta > 0 makes later chunks sparser);
  * s_i = clip(s_base - alpha_i * beta, 0, s_max) for i >= 1;
  * F_i is chunk i's dense attention cost (given); the matching condition is
    sum_i (1 - s_i) F_i = (1 - s_target) sum_i F_i, sums taken in ascending i;
  * the kept cost is non-decreasing in beta, so beta is the smallest value of
    a fixed bisection (200 halvings of a bracket that clips every s_i at
    s_max at one end and at 0 at the other) whose kept cost reaches the
    target; the schedule is then evaluated at that beta;
  * a chunk with c candidate frames keeps k_i = floor((1 - s_i) * c + 1/2)
    of them, at least 1 and at most c (all of it float64).
"""

from __future__ import annotations

import math


def alpha(i: int) -> float:
    return 1.0 / math.sqrt(i + 1.0)


def sparsity_at(beta: float, n: int, s_base: float, s_max: float) -> list[float]:
    s = [0.0]
    for i in range(1, n):
        v = s_base - alpha(i) * beta
        s.append(min(s_max, max(0.0, v)))
    return s


def kept_cost(s, cost) -> float:
    acc = 0.0
    for si, fi in zip(s, cost):
        acc = acc + (1.0 - si) * fi
    return acc


def bracket(n: int, s_base: float, s_max: float):
    """beta_lo clips every s_i (i >= 1) at s_max, beta_hi clips every one at 0."""
    r2, rn = math.sqrt(2.0), math.sqrt(float(n))
    d = s_base - s_max
    lo = min(d * r2, d * rn) - 1.0
    hi = max(s_base * r2, s_base * rn, 0.0) + 1.0
    return lo, hi


def schedule(cost, s_target: float, s_base: float, s_max: float):
    """(sparsity per chunk, beta).  Raises ValueError if no beta reaches the target."""
    n = len(cost)
    if n < 1 or any(not (f > 0.0) for f in cost):
        raise ValueError("need at least one chunk and positive costs")
    if not (0.0 <= s_target < 1.0 and 0.0 <= s_max < 1.0 and 0.0 <= s_base <= 1.0):
        raise ValueError("ratios out of range")
    total = 0.0
    for f in cost:
        total = total + f
    target = (1.0 - s_target) * total
    lo, hi = bracket(n, s_base, s_max)
    if kept_cost(sparsity_at(lo, n, s_base, s_max), cost) > target or \
            kept_cost(sparsity_at(hi, n, s_base, s_max), cost) < target:
        raise ValueError("the target sparsity cannot be reached")
    for _ in range(200):
        mid = lo + (hi - lo) * 0.5
        if mid <= lo or mid >= hi:
            break
        if kept_cost(sparsity_at(mid, n, s_base, s_max), cost) >= target:
            hi = mid
        else:
            lo = mid
    return sparsity_at(hi, n, s_base, s_max), hi


def frame_budgets(s, candidates) -> list[int]:
    """k_i = floor((1 - s_i) * c_i + 1/2), clipped to [1, c_i] (c_i >= 1)."""
    out = []
    for si, c in zip(s, candidates):
        k = math.floor((1.0 - si) * c + 0.5)
        out.append(max(1, min(int(c), k)))
    return out
