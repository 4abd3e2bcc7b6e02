"""Non-finite inputs on the device paths: the selection kernels still write
exactly k entries per row and nothing past their outputs (a NaN score ranks
below every number), and a value beyond the float16 range in a frame a row
does not attend never reaches that row's output (the float16 copy of V
saturates at +-65504)."""

import numpy as np
import pytest
import torch

import frame_sparse_attention_amd as fsa

from _parity import assert_close, oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = -777


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _guarded(shape, guard=4096):
    """A tensor view of `shape` at the front of a larger int32 buffer whose tail
    holds a sentinel, so writes past the view are seen."""
    n = int(np.prod(shape))
    buf = torch.full((n + guard,), SENTINEL, dtype=torch.int32, device=DEV)
    return buf, buf[:n].view(*shape)


@pytest.mark.parametrize("F", [40, 1500])   # rank path, and the argmax rounds past 1024
def test_topk_with_nan_scores_keeps_exactly_k(F):
    B, H, P, D, k = 1, 2, 4, 64, 8
    g = torch.Generator().manual_seed(11)
    q = torch.randn((B, H, 2 * P, D), generator=g).to(torch.bfloat16)
    kk = torch.randn((B, H, F * P, D), generator=g).to(torch.bfloat16)
    q[0, 0, 1, 3] = float("inf")             # head 0: inf * 0-ish sums -> NaN / inf scores
    q[0, 0, 2, 3] = float("-inf")            # inf - inf = NaN in the pooled query
    kk[0, 1, 5 * P + 2, 7] = float("nan")    # head 1: one NaN key frame
    buf, out = _guarded((B, H, 1, k))
    _say(f"top-k with non-finite inputs, {F} candidates")
    fsa.select_topk_frames(q.to(DEV), kk.to(DEV), P, 0, H, 2, 0, F, k, out=out)
    torch.cuda.synchronize()
    assert (buf[out.numel():] == SENTINEL).all(), "top-k wrote past its output"
    rows = out.cpu().numpy().reshape(-1, k)
    for r in rows:
        assert np.all((r >= 0) & (r < F)), r
        assert np.all(np.diff(r) > 0), r          # k distinct frames, ascending


def test_hsa_with_nan_scores_keeps_exactly_kb():
    B, H, Tq, Tk, P, block, D = 1, 2, 2, 9, 12, 4, 64
    offset, chunk, n_recent, kf, kb = 7, 2, 2, 3, 5
    nb = P // block
    g = torch.Generator().manual_seed(12)
    q = torch.randn((B, H, Tq * P, D), generator=g).to(torch.bfloat16)
    kk = torch.randn((B, H, Tk * P, D), generator=g).to(torch.bfloat16)
    q[0, 0, :block, 0] = float("nan")        # every score of head 0's first query block
    kk[0, 1, 3 * P, 1] = float("inf")
    kk[0, 1, 3 * P + 1, 1] = float("-inf")   # frame 3 of head 1 pools to NaN
    cap = kb + n_recent * nb
    G = Tq * P // block
    buf, idx = _guarded((B, H, G, cap))
    cnt = torch.zeros((B, H, G), dtype=torch.int32, device=DEV)
    _say("HSA selection with non-finite inputs")
    fsa.select_hsa_blocks(q.to(DEV), kk.to(DEV), P, block, 0, H, n_recent, kf, kb, offset,
                          chunk, idx=idx, cnt=cnt)
    torch.cuda.synchronize()
    assert (buf[idx.numel():] == SENTINEL).all(), "HSA selection wrote past its output"
    assert (cnt.cpu() == cap).all()
    rows = idx.cpu().numpy().reshape(-1, cap)
    for r in rows:
        assert np.all(np.diff(r) > 0), r
        assert np.all((r >= 0) & (r < Tk * nb)), r


@pytest.mark.parametrize("P", [100, 1560])
def test_large_value_outside_the_set_does_not_reach_the_row(P):
    # frame 2 holds a value of 1e5 (beyond float16) and sits right after frame 1;
    # frame 1's rows attend {0, 1} only.  Their 64-key tiles run past the end of
    # frame 1 into frame 2 (probability exactly 0 there): their output stays
    # finite and equal to the oracle's.
    B, H, T, D = 1, 1, 3, 128
    g = torch.Generator().manual_seed(13)
    q, k, v = (torch.randn((B, H, T * P, D), generator=g).to(torch.bfloat16) for _ in range(3))
    v[0, 0, 2 * P + 1, 5] = 1e5
    v[0, 0, 2 * P + 3, 6] = -3e38
    idx = torch.tensor([[[[0, 1], [0, 1], [1, 2]]]], dtype=torch.int32)
    cnt = torch.tensor([[[2, 2, 2]]], dtype=torch.int32)
    _say(f"value beyond float16 next to the frame set, P={P}")
    o, lse = fsa.sparse_frame_attn(q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV), cnt.to(DEV), P)
    torch.cuda.synchronize()
    rows = np.arange(0, 2 * P)                       # query frames 0 and 1: set {0, 1}
    assert torch.isfinite(o[0, 0, :2 * P]).all()
    o_ref, l_ref = oracle_rows(q, k, v, idx, cnt, P, rows)
    assert_close(o[:, :, rows].cpu().numpy(), lse[:, :, rows].cpu().numpy(), o_ref, l_ref,
                 "bf16", f"rows beside a 1e5 value, P={P}")
