"""Oracle: exact merge of two partial attentions through their LSE, float64.

TEST INFRASTRUCTURE -- imported only by tests, the smoke check and the CPU
baseline of the benchmark.  Shares no code with the library.

[ISPA page, §2 item 1 and §3 item 2: decomposable attention splits the keys
into a local and a history branch, each tracked with its log-sum-exp state,
and merges them afterwards with online-softmax algebra.]

For partial results (O1, L1) over key set K1 and (O2, L2) over a disjoint K2:
  M = max(L1, L2);  L = M + ln(exp(L1 - M) + exp(L2 - M));
  O = exp(L1 - L) · O1 + exp(L2 - L) · O2.
A branch with L = -inf (no keys) contributes nothing; if both are -inf the
result is O = 0, L = -inf.
"""

from __future__ import annotations

import numpy as np


def merge_lse(o1, lse1, o2, lse2):
    """Merge two partials row by row.  o* [..., D], lse* [...]; returns (O, L)."""
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    l1 = np.asarray(lse1, dtype=np.float64)
    l2 = np.asarray(lse2, dtype=np.float64)
    out_o = np.zeros(np.broadcast_shapes(o1.shape, o2.shape))
    out_l = np.full(np.broadcast_shapes(l1.shape, l2.shape), -np.inf)
    it = np.ndindex(out_l.shape)
    for ix in it:
        a, b = l1[ix], l2[ix]
        if a == -np.inf and b == -np.inf:
            continue  # O = 0, L = -inf
        if b == -np.inf:
            out_o[ix], out_l[ix] = o1[ix], a
            continue
        if a == -np.inf:
            out_o[ix], out_l[ix] = o2[ix], b
            continue
        m = max(a, b)
        lse = m + np.log(np.exp(a - m) + np.exp(b - m))
        out_l[ix] = lse
        out_o[ix] = np.exp(a - lse) * o1[ix] + np.exp(b - lse) * o2[ix]
    return out_o, out_l
