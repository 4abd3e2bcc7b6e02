"""GPU parity of attention with each frame list cut into parts whose partials
are merged through their LSE: every split count gives the oracle's result
within the bf16 tolerance, including parts left empty by short lists."""

import numpy as np
import pytest
import torch

import frame_sparse_attention_amd as fsa
import workloads as wl
from oracle import frame_sets as ofs
from oracle import topk as otopk

from _parity import assert_close, oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("splits,D", [(1, 128), (2, 128), (3, 128), (7, 128), (16, 128),
                                      (0, 128), (3, 64), (16, 64)])
def test_split_counts_small(splits, D):
    # 3 heads: a 1-frame list (most parts empty), a 4-frame window, all 9 frames;
    # splits = 0 takes the library's default plan
    w = wl.Workload("split_small", 70, 1, 3, D, 3, 9, 40, "bf16",
                    [wl.policy(wl.SINK_WINDOW, n_sink=0, window=1),
                     wl.policy(wl.SINK_WINDOW, n_sink=1, window=3),
                     wl.policy(wl.FULL)], offset=6, chunk=1)
    _say(f"split attention, {splits} parts, D={D}")
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    idx, cnt = fsa.build_frame_sets(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk, device=DEV)
    o, lse = fsa.sparse_frame_attn_split(qd, kd, fsa.prepare_values(vd), idx, cnt, w.P, splits)
    torch.cuda.synchronize()
    oidx, ocnt = ofs.build(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk, cap=idx.shape[3])
    rows = np.arange(w.Nq)
    o_ref, l_ref = oracle_rows(q, k, v, oidx, ocnt, w.P, rows)
    assert_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16",
                 f"split small, {splits} parts, D={D}")


def test_split_ar_chunk_four_parts():
    w = wl.ar_chunk()
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    S = 4
    _say(f"{w.name}: split attention, {S} parts")
    sel = fsa.select_topk_frames(qd, kd, w.P, 8, 12, 3, 0, 57, 8)
    cap = fsa.frame_set_capacity(w.policies, w.Tq, w.Tk, w.offset, w.chunk)
    idx, cnt = fsa.build_frame_sets(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk, sel, cap, DEV)
    prep = fsa.prepare_values(vd)
    o, lse = fsa.sparse_frame_attn_split(qd, kd, prep, idx, cnt, w.P, S)
    o1, l1 = fsa.sparse_frame_attn_prepared(qd, kd, prep, idx, cnt, w.P)
    torch.cuda.synchronize()
    sel_lists = [[[[]] for _ in range(12)]]
    for h in range(8, 12):
        f, _ = otopk.select_topk_frames(q[0, h].float().numpy(), k[0, h].float().numpy(), w.P,
                                        np.arange(w.Nq), range(57), 8)
        sel_lists[0][h] = [f]
    oidx, ocnt = ofs.build(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk, sel_lists, cap=cap)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    rows = np.array(sorted(set([0, 127, 128, 1559, 1560, 4679] +
                               np.random.default_rng(11).integers(0, w.Nq, 60).tolist())))
    o_ref, l_ref = oracle_rows(q, k, v, oidx, ocnt, w.P, rows)
    assert_close(o[:, :, rows].cpu().numpy(), lse[:, :, rows].cpu().numpy(), o_ref, l_ref,
                 "bf16", f"{w.name} split into {S} parts")
    # against the one-part result on every row
    print(f"[parity] split vs one part: max|dO|={float((o - o1).abs().max()):.3e} "
          f"max|dLSE|={float((lse - l1).abs().max()):.3e}", flush=True)
    assert float((o - o1).abs().max()) < 1e-3 and float((lse - l1).abs().max()) < 1e-4
