"""A chunk-aware-growth rollout on the device (Light Forcing §2.1: the first
chunk dense, later chunks sparser, the budgets matched to a target cost;
Head Forcing methodology §2: local, anchor and memory heads).

20 chunks of 3 frames run into a KV cache that grows by one chunk per step.
The library's schedule gives each chunk's frame budget k_i; the memory heads'
top-k_i frames are picked on the device from the chunk's queries and the
cached history, every head's frame set is built on the device, and the
attention runs on the cache.  The same rollout through the oracle
(oracle/cag.py -> oracle/topk.py -> oracle/frame_sets.py) must give the same
budgets and the same lists bit for bit, and O/LSE must match the oracle on
sampled rows of every chunk."""

import numpy as np
import pytest
import torch

import frame_sparse_attention_amd as fsa
import workloads as wl
from oracle import attention as oatt
from oracle import cag as ocag
from oracle import frame_sets as ofs
from oracle import topk as otopk

from _parity import assert_close, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def test_cag_rollout_matches_oracle_rollout():
    w = wl.ar_rollout()
    r = w.rollout
    n, c, P = r["n_chunks"], w.chunk, w.P
    mem_heads = [h for h, p in enumerate(w.policies) if p["kind"] == wl.MEMORY]
    h0, h1 = mem_heads[0], mem_heads[-1] + 1
    assert mem_heads == list(range(h0, h1))
    shapes = [wl.rollout_chunk(w, i) for i in range(n)]
    cost = [float(s["dense_frame_pairs"]) for s in shapes]
    cand = [max(1, s["candidates"]) for s in shapes]

    # the schedule: library (host) against the oracle, bit for bit
    sp, bud, beta = fsa.cag_schedule(cost, r["s_target"], r["s_base"], r["s_max"], cand)
    osp, obeta = ocag.schedule(cost, r["s_target"], r["s_base"], r["s_max"])
    obud = ocag.frame_budgets(osp, cand)
    assert beta == obeta and sp.tolist() == osp and bud.tolist() == obud
    _say(f"{w.name}: budgets {bud.tolist()}")

    _say(f"{w.name}: generating inputs")
    q, k, v = wl.make_qkv(w)
    qd, kd = q.to(DEV), k.to(DEV)
    prep = fsa.prepare_values(v.to(DEV))       # the cache's values, converted once
    k64 = {h: k[0, h].double().numpy() for h in range(w.H)}
    v64 = {h: v[0, h].double().numpy() for h in range(w.H)}
    # the oracle's pooled key frames, computed once: every chunk chooses among a
    # prefix of the same history
    ksum = {h: otopk.pooled_key_sums(k64[h], P, range(shapes[-1]["candidates"]))
            for h in mem_heads}
    scale = 1.0 / np.sqrt(w.D)
    for i, s in enumerate(shapes):
        off, cached, k_i = s["offset"], s["cached"], int(bud[i])
        pols = wl.rollout_policies(w, i, k_i)
        rows_q = slice(off * P, (off + c) * P)
        q_i = qd[:, :, rows_q].contiguous()
        _say(f"chunk {i}: cache {cached} frames, k_i = {k_i}")
        sel = None
        if i > 0:
            sel = fsa.select_topk_frames(q_i, kd, P, h0, h1, c, 0, s["candidates"], k_i)
        idx, cnt = fsa.build_frame_sets(pols, w.B, c, cached, off, c, sel, device=DEV)
        o, lse = fsa.sparse_frame_attn_prepared(q_i, kd, prep, idx, cnt, P)
        torch.cuda.synchronize()

        # the oracle rollout: its own top-k, its own lists
        osel = None
        if i > 0:
            osel = [[[[]] for _ in range(w.H)]]
            for h in mem_heads:
                f, _ = otopk.select_topk_frames(q[0, h].float().numpy(), k64[h], P,
                                                np.arange(rows_q.start, rows_q.stop),
                                                range(s["candidates"]), k_i,
                                                ksum=ksum[h][:s["candidates"]])
                osel[0][h] = [f]
        oidx, ocnt = ofs.build(pols, w.B, c, cached, off, c, osel, cap=idx.shape[3])
        np.testing.assert_array_equal(cnt.cpu().numpy(), ocnt)
        np.testing.assert_array_equal(idx.cpu().numpy(), oidx)

        # attention on sampled rows of each of the chunk's frames, every head
        rows = sample_rows(P, range(c), 6, seed=i)
        o_ref = np.zeros((1, w.H, rows.size, w.D))
        l_ref = np.zeros((1, w.H, rows.size))
        for h in range(w.H):
            qh = q[0, h, rows_q].double().numpy()[rows]
            mask = oatt.token_mask(oidx[0, h, 0, :ocnt[0, h, 0]], w.Tk, P)
            o_ref[0, h], l_ref[0, h] = oatt.attend_rows(qh, k64[h], v64[h], mask, scale)
        assert_close(o[:, :, rows].cpu().numpy(), lse[:, :, rows].cpu().numpy(), o_ref, l_ref,
                     "bf16", f"{w.name} chunk {i} ({rows.size} rows x {w.H} heads)")
