"""GPU parity of the two-level (frame, then block) selection and of attention
over the chosen blocks (Light Forcing §2.2 hierarchical sparse attention):
block lists bit-exact against the oracle, O and LSE within the bf16 / fp32
tolerances on the same lists."""

import numpy as np
import pytest
import torch

import frame_sparse_attention_amd as fsa
import workloads as wl
from oracle import frame_sets as ofs
from oracle import hsa as ohsa

from _parity import TOL, assert_close, oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _oracle_hsa_rows(q, k, P, block, offset, chunk, heads, n_recent, kf, kb):
    """Oracle block lists {(b, h): [list per query block]} for the given heads."""
    out = {}
    for b in range(q.shape[0]):
        for h in heads:
            out[(b, h)] = ohsa.hsa_lists(q[b, h].float().numpy(), k[b, h].float().numpy(), P,
                                         block, offset, chunk, n_recent, kf, kb)
    return out


def _check_lists(idx, cnt, ref, cap):
    idx = idx.cpu().numpy()
    cnt = cnt.cpu().numpy()
    for (b, h), lists in ref.items():
        for j, a in enumerate(lists):
            assert cnt[b, h, j] == len(a), (b, h, j)
            row = idx[b, h, j]
            assert row[:len(a)].tolist() == a, (b, h, j)
            assert (row[len(a):] == -1).all(), (b, h, j)


CASES = [
    # (dtype, B, H, D, Tq, Tk, P, block, offset, chunk, h_begin, h_end, n_recent, kf, kb)
    ("f32", 1, 2, 64, 2, 9, 12, 4, 7, 2, 0, 2, 2, 3, 5),        # one chunk of 2 frames
    ("f32", 2, 3, 64, 4, 10, 12, 3, 6, 2, 1, 3, 1, 2, 8),       # two chunks, later e differs
    ("bf16", 1, 2, 128, 3, 12, 20, 5, 9, 3, 0, 2, 3, 4, 16),    # kb = kf * nb: whole frames
    ("bf16", 1, 2, 128, 2, 8, 16, 8, 6, 2, 0, 2, 0, 6, 1),      # no recent frames, kb = 1
    ("bf16", 1, 1, 128, 1, 6, 24, 24, 5, 1, 0, 1, 2, 4, 4),     # blocks as large as frames
    ("bf16", 1, 2, 128, 2, 7, 16, 4, 5, 2, 0, 2, 2, 2, 0),      # kb = 0: recent frames only
    ("bf16", 1, 1, 64, 1, 40, 128, 2, 39, 1, 0, 1, 1, 20, 300),  # 1280 candidate blocks
    ("bf16", 1, 1, 64, 1, 1100, 2, 2, 1099, 1, 0, 1, 1, 1030, 9),  # 1098 candidate frames
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_select_hsa_blocks_bit_exact(case):
    dt, B, H, D, Tq, Tk, P, block, offset, chunk, h0, h1, n_recent, kf, kb = case
    _say(f"select_hsa_blocks {case}")
    w = wl.Workload("hsa_case", 40 + CASES.index(case), B, H, D, Tq, Tk, P, dt, [])
    q = wl.make_tensor(w, 0)
    k = wl.make_tensor(w, 1)
    idx, cnt = fsa.select_hsa_blocks(q.to(DEV), k.to(DEV), P, block, h0, h1, n_recent, kf, kb,
                                     offset, chunk)
    torch.cuda.synchronize()
    ref = _oracle_hsa_rows(q, k, P, block, offset, chunk, range(h0, h1), n_recent, kf, kb)
    _check_lists(idx, cnt, ref, idx.shape[3])
    # rows of heads outside the range are untouched
    other = [h for h in range(H) if not h0 <= h < h1]
    if other:
        assert (idx[:, other].cpu() == -1).all() and (cnt[:, other].cpu() == 0).all()


def _hsa_workload_lists(w, q, k):
    """Device lists for every head of a block-level workload: frame windows in
    block units from the device builder, memory heads from the selection."""
    nb = w.P // w.block
    bpol = wl.block_policies(w)
    mem = [h for h, p in enumerate(w.policies) if p["kind"] == wl.MEMORY]
    h0, h1 = mem[0], mem[-1] + 1
    assert mem == list(range(h0, h1))
    n_recent, kf = w.policies[h0]["n_recent"], w.policies[h0]["topk"]
    Tqb, Tkb = w.Tq * nb, w.Tk * nb
    cap = max(fsa.frame_set_capacity(bpol, Tqb, Tkb, w.offset * nb, w.chunk * nb),
              w.topk_blocks + n_recent * nb)
    idx, cnt = fsa.build_frame_sets(bpol, w.B, Tqb, Tkb, w.offset * nb, w.chunk * nb, None, cap,
                                    DEV)
    fsa.select_hsa_blocks(q, k, w.P, w.block, h0, h1, n_recent, kf, w.topk_blocks, w.offset,
                          w.chunk, idx=idx, cnt=cnt)
    return idx, cnt, (h0, h1, n_recent, kf)


def test_ar_chunk_hsa_lists_and_attention():
    w = wl.ar_chunk_hsa()
    nb = w.P // w.block
    _say(f"{w.name}: inputs")
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    _say(f"{w.name}: lists")
    idx, cnt, (h0, h1, n_recent, kf) = _hsa_workload_lists(w, qd, kd)
    torch.cuda.synchronize()
    # memory heads: two-level selection against the oracle
    ref = _oracle_hsa_rows(q, k, w.P, w.block, w.offset, w.chunk, range(h0, h1), n_recent, kf,
                           w.topk_blocks)
    _check_lists(idx, cnt, ref, idx.shape[3])
    # other heads: the frame windows of the oracle, written in blocks
    cap = idx.shape[3]
    for h in range(w.H):
        if h0 <= h < h1:
            continue
        bp = ohsa.scale_policy_to_blocks(w.policies[h], nb)
        oi, oc = ofs.build([bp], w.B, w.Tq * nb, w.Tk * nb, w.offset * nb, w.chunk * nb, cap=cap)
        np.testing.assert_array_equal(idx[:, h:h + 1].cpu().numpy(), oi)
        np.testing.assert_array_equal(cnt[:, h:h + 1].cpu().numpy(), oc)
    assert cnt[0, h0:h1].cpu().unique().tolist() == [w.topk_blocks + n_recent * nb]
    # attention over the chosen blocks ("frames" of `block` tokens)
    _say(f"{w.name}: attention")
    prep = fsa.prepare_values(vd)
    o, lse = fsa.sparse_frame_attn_prepared(qd, kd, prep, idx, cnt, w.block)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.array(sorted(set([0, 119, 120, 4559, 4679] + rng.integers(0, w.Nq, 40).tolist())))
    o_ref, l_ref = oracle_rows(q, k, v, idx, cnt, w.block, rows)
    assert_close(o[:, :, rows].cpu().numpy(), lse[:, :, rows].cpu().numpy(), o_ref, l_ref,
                 "bf16", f"{w.name} sampled rows, all heads")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_hsa_attention_small_all_rows(dt):
    # every row of a small case with ragged blocks: 3 query frames in one chunk,
    # blocks of 8 tokens in frames of 40, a 10-frame cache
    D = 64 if dt == "f32" else 128
    w = wl.Workload("hsa_small", 50, 1, 3, D, 3, 10, 40, dt,
                    [wl.policy(wl.SINK_WINDOW, n_sink=1, window=3),
                     wl.policy(wl.MEMORY, topk=3, n_recent=3),
                     wl.policy(wl.MEMORY, topk=3, n_recent=3)],
                    offset=7, chunk=3, q_group=3, block=8, topk_blocks=7)
    _say(f"hsa small attention {dt}")
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    idx, cnt, (h0, h1, n_recent, kf) = _hsa_workload_lists(w, qd, kd)
    if dt == "bf16":
        o, lse = fsa.sparse_frame_attn_prepared(qd, kd, fsa.prepare_values(vd), idx, cnt, w.block)
    else:
        o, lse = fsa.sparse_frame_attn(qd, kd, vd, idx, cnt, w.block)
    torch.cuda.synchronize()
    ref = _oracle_hsa_rows(q, k, w.P, w.block, w.offset, w.chunk, range(h0, h1), n_recent, kf,
                           w.topk_blocks)
    _check_lists(idx, cnt, ref, idx.shape[3])
    rows = np.arange(w.Nq)
    o_ref, l_ref = oracle_rows(q, k, v, idx, cnt, w.block, rows)
    assert_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, dt, f"hsa small {dt} all rows")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_select_hsa_blocks_exact_sums_of_wide_spread_values(dtype):
    # block and frame sums are exact sums of tokens rounded once; values spread
    # over ~2^200 with planted opposites make the device sum them exactly
    B, H, D, Tq, Tk, P, block = 1, 2, 64, 2, 9, 12, 4
    offset, chunk, n_recent, kf, kb = 7, 2, 2, 3, 5
    g = torch.Generator().manual_seed(32)

    def spread(n):
        m = torch.randint(128, 256, (B, H, n, D), generator=g).float()
        e = torch.randint(-100, 100, (B, H, n, D), generator=g).float()
        s = torch.randint(0, 2, (B, H, n, D), generator=g).float() * 2 - 1
        x = s * m * torch.exp2(e - 7)
        x[:, :, 1::3] = -x[:, :, 0::3][:, :, : x[:, :, 1::3].shape[2]]
        return x.to(dtype)

    q, k = spread(Tq * P), spread(Tk * P)
    _say(f"select_hsa_blocks over wide-spread values ({dtype})")
    idx, cnt = fsa.select_hsa_blocks(q.to(DEV), k.to(DEV), P, block, 0, H, n_recent, kf, kb,
                                     offset, chunk)
    torch.cuda.synchronize()
    ref = _oracle_hsa_rows(q, k, P, block, offset, chunk, range(H), n_recent, kf, kb)
    _check_lists(idx, cnt, ref, idx.shape[3])
