"""Reference oracle for frame-block-sparse softmax attention (TEST INFRASTRUCTURE).

This package is a plain, slow, obviously-correct CPU implementation of what the
library computes, written in numpy float64 (integers for the frame sets).  It
exists only to check the HIP path: the only code that may import it is the test
suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py``.  The library itself never imports, links or calls anything here,
and this package imports nothing from the library.

Modules
-------
frame_sets  per-head frame sets A(t): LVSA rotating anchors + widened window,
            sink/local window, memory (top-k + recent), range, full.
attention   attention over the frames of A(t), by an explicit token mask, in
            float64; returns O and the natural-log LSE per query row.
merge       exact LSE merge of two partial attentions over disjoint key sets.
topk        frame mean-pooling (as float64 sums in a fixed sequential order)
            and frame ranking for memory heads.

Sources (the pages this follows; each function cites its passage):
  * LVSA, training-free sparse attention for long video diffusion -- §2 core
    mechanism (A(t) = G ∪ W(t), rotating anchors, widened window, budget C),
    complexity paragraph.
  * Light Forcing -- §2.2 hierarchical sparse attention (mean-pooled tokens,
    frame selection per query block).
  * ISPA (instance-specific parametric absorption) -- §2 dual-stream warmup,
    decomposable attention merged through LSE.
  * Head Forcing -- methodology §2, per-head KV sets (local, anchor, memory
    with fast memory of recent frames).
  * ARL2 -- §2.1, intra-frame bidirectional softmax (A(t) = {t}).

Every function is pinned by CPU tests against facts that do not come from this
package (closed forms, library routines on special cases, brute force, the
invariants the pages state); see tests/test_oracle_*.py.
"""

from . import attention, frame_sets, merge, topk  # noqa: F401
