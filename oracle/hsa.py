"""Oracle: two-level (frame, then block) selection of hierarchical sparse
attention.

TEST INFRASTRUCTURE -- imported only by tests, the smoke check and the CPU
baseline of the benchmark.  Shares no code with the library.

[Light Forcing page, §2.2 hierarchical sparse attention: query and key tokens
are compressed by mean pooling to both block and frame granularity; for each
query block a few relevant history frames are retrieved with frame-level
keys, then the critical blocks inside those frames are found with block-level
keys; attention runs over the selected (frame, block) pairs only, at a cost
that does not grow with the number of history frames.]

Readings (the page fixes neither the sizes nor the arithmetic):
  * a block is `Bs` consecutive tokens inside a frame (P is a multiple of Bs,
    nb = P / Bs blocks per frame); query blocks and key blocks have the same
    size, and global block index = frame * nb + block-in-frame;
  * pooling is kept as float64 sums, as for the frame-level top-k: a block sum
    is the exact sum of its Bs tokens and a frame sum the exact sum of its P
    tokens, each rounded once to float64 (the coarse level is not built from
    rounded fine sums, so no order of summation enters either);
  * scores are dot products of a query block sum with a frame sum (level 1) or
    a block sum (level 2), each product rounded, added in ascending channel
    order; ranking is (score descending, index ascending), as in topk.py;
  * the history a query block chooses from is the same as a memory head's
    (Head Forcing methodology §2): with e the last KV frame of the query
    block's chunk, the n_recent frames e-n_recent+1..e are attended whole and
    the candidates are the frames 0..e-n_recent;
  * level 1 keeps the kf best candidate frames, level 2 the kb best blocks
    among all blocks of those kf frames (one budget per query block, so the
    attended size is fixed: kb blocks plus the recent frames);
  * A(j) = selected blocks united with every block of the recent frames,
    sorted ascending, in block units.
"""

from __future__ import annotations

import numpy as np

from . import frame_sets, topk


def block_sums(tokens: np.ndarray, Bs: int) -> np.ndarray:
    """[N, D] tokens -> [N/Bs, D]: each block's exact sum, rounded once to float64."""
    x = np.asarray(tokens, dtype=np.float64)
    if x.shape[0] % Bs:
        raise ValueError("tokens do not split into whole blocks")
    return np.stack([topk.exact_column_sums(x[i:i + Bs]) for i in range(0, x.shape[0], Bs)]) \
        if x.shape[0] else np.zeros((0, x.shape[1]))


def select_blocks(qblock_sum: np.ndarray, kblocks: np.ndarray, kframes: np.ndarray, nb: int,
                  e: int, n_recent: int, kf: int, kb: int):
    """Block set of one query block.

    qblock_sum [D]: the query block's sum.  kblocks [>= (e+1)*nb, D] and
    kframes [>= e+1, D]: key block sums and key frame sums of the head (frame
    f's blocks are f*nb .. f*nb+nb-1).  Returns (sorted block list, selected
    frames).
    """
    first_recent = e - n_recent + 1
    if n_recent < 0 or first_recent < 0:
        raise ValueError("recent frames reach before frame 0")
    cands = list(range(first_recent))
    frames = topk.rank_topk(topk.frame_scores(qblock_sum, kframes[:first_recent]), cands, kf)
    cand_blocks = [f * nb + i for f in frames for i in range(nb)]
    bscores = topk.frame_scores(qblock_sum, kblocks[cand_blocks])
    blocks = topk.rank_topk(bscores, cand_blocks, kb)
    recent = list(range(first_recent * nb, (e + 1) * nb))
    return sorted(blocks + recent), frames


def hsa_lists(q_bh: np.ndarray, k_bh: np.ndarray, P: int, Bs: int, offset: int, chunk: int,
              n_recent: int, kf: int, kb: int):
    """Block lists of every query block of one head.

    q_bh [Tq*P, D], k_bh [Tk*P, D].  Query block j lies in query frame
    tq = j*Bs // P, which sits in the chunk ending at KV frame
    e = offset + (tq//chunk + 1)*chunk - 1.  Returns a list of sorted lists.
    """
    if P % Bs:
        raise ValueError("P must be a multiple of the block size")
    nb = P // Bs
    qb = block_sums(q_bh, Bs)
    kbs = block_sums(k_bh, Bs)
    kfs = block_sums(k_bh, P)
    out = []
    for j in range(qb.shape[0]):
        tq = j * Bs // P
        e = frame_sets.chunk_last_frame(tq, chunk, offset)
        blocks, _ = select_blocks(qb[j], kbs, kfs, nb, e, n_recent, kf, kb)
        out.append(blocks)
    return out


def scale_policy_to_blocks(pol: dict, nb: int) -> dict:
    """A frame-level SINK_WINDOW or RANGE policy written in block units (every
    frame becomes its nb blocks), for heads that keep whole frames next to HSA
    heads in one block-unit list set."""
    p = dict(pol)
    if p["kind"] == frame_sets.SINK_WINDOW:
        p["n_sink"] *= nb
        p["window"] *= nb
    elif p["kind"] == frame_sets.RANGE:
        p["lo"] = p["lo"] * nb
        p["hi"] = p["hi"] * nb + nb - 1
    elif p["kind"] != frame_sets.FULL:
        raise ValueError("only FULL, SINK_WINDOW and RANGE scale to block units")
    return p
