"""GPU parity of the sparse frame attention against the oracle, element by
element, on sizes the oracle finishes in seconds: several query tiles and key
tiles, ragged tails (P not a multiple of the 128-row / 64-key tiles or of the
8-key chunks), D = 64 and 128, and the degenerate frame sets (empty, one
frame, the own frame only, all frames, scattered lists, malformed entries)."""

import numpy as np
import pytest
import torch

import frame_sparse_attention_amd as fsa
import workloads as wl
from oracle import attention as oatt
from oracle import frame_sets as ofs

from _parity import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _rand(shape, dtype, seed, outliers=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g)
    if outliers:
        ch = torch.randperm(shape[-1], generator=g)[:outliers]
        x[..., ch] *= 8.0
    return x.to(dtype).contiguous()


def _lists_to_arrays(lists, B, H):
    """lists[b][h][t] -> padded idx/cnt int32 tensors."""
    Tq = len(lists[0][0])
    cap = max(1, max(len(a) for lb in lists for lh in lb for a in lh))
    idx = np.full((B, H, Tq, cap), -1, np.int32)
    cnt = np.zeros((B, H, Tq), np.int32)
    for b in range(B):
        for h in range(H):
            for t, a in enumerate(lists[b][h]):
                idx[b, h, t, :len(a)] = a
                cnt[b, h, t] = len(a)
    return torch.from_numpy(idx), torch.from_numpy(cnt)


def _run_and_check(q, k, v, idx, cnt, P, kind, what, scale=None):
    _say(what)
    o, lse = fsa.sparse_frame_attn(q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV), cnt.to(DEV),
                                   P, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oatt.sparse_frame_attention(q.float().numpy(), k.float().numpy(),
                                               v.float().numpy(), idx.numpy(), cnt.numpy(), P,
                                               scale=scale)
    return assert_close(o.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, kind, what)


def test_tiny_f32_workload_in_full():
    w = wl.tiny_f32()
    q, k, v = wl.make_qkv(w)
    idx, cnt = fsa.build_frame_sets(w.policies, w.B, w.Tq, w.Tk, device=DEV)
    oidx, ocnt = ofs.build(w.policies, w.B, w.Tq, w.Tk, cap=idx.shape[3])
    assert np.array_equal(idx.cpu().numpy(), oidx) and np.array_equal(cnt.cpu().numpy(), ocnt)
    _run_and_check(q, k, v, idx.cpu(), cnt.cpu(), w.P, "f32", "tiny fp32 workload")


@pytest.mark.parametrize("D,P", [(64, 13), (128, 16), (128, 70)])
def test_f32_ragged_and_scattered(D, P):
    B, H, T = 1, 2, 5
    q, k, v = (_rand((B, H, T * P, D), torch.float32, s) for s in (1, 2, 3))
    lists = [[[[0], [0, 2, 4], [], [1, 2, 3, 4], [3]], [[4], [0, 1], [2], [0, 1, 2, 3, 4], []]]]
    idx, cnt = _lists_to_arrays(lists, B, H)
    _run_and_check(q, k, v, idx, cnt, P, "f32", f"fp32 D={D} P={P}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("P", [1, 5, 8, 13, 64, 100, 130, 200])
def test_bf16_shapes_and_lists(D, P):
    B, H, T = 1, 2, 6
    q, k, v = (_rand((B, H, T * P, D), torch.bfloat16, s, outliers=4) for s in (4, 5, 6))
    lists = [[[[0], [0, 1, 2, 3, 4, 5], [1, 3, 5], [3], [], [0, 2, 3, 4]],
              [[5], [4, 5], [0, 5], [2, 3], [1], [0, 1, 2, 3, 4, 5]]]]
    idx, cnt = _lists_to_arrays(lists, B, H)
    _run_and_check(q, k, v, idx, cnt, P, "bf16", f"bf16 D={D} P={P}")


@pytest.mark.parametrize("s", range(6))
def test_bf16_lvsa_shrunk(s):
    # LVSA policy of the 42-frame workload (C=21, W=7, T_per=6, outliers x8) on
    # fewer heads and a ragged P=200: every step of the anchor rotation.
    w = wl.lvsa_shaped(s).shrunk(H=2, P=200)
    q, k, v = wl.make_qkv(w)
    idx, cnt = fsa.build_frame_sets(w.policies[:2], w.B, w.Tq, w.Tk, device=DEV)
    _run_and_check(q, k, v, idx.cpu(), cnt.cpu(), w.P, "bf16", f"lvsa T=42 P=200 step {s}")


def test_bf16_own_frame_only_and_full():
    # ARL2 §2.1 intra-frame branch: A(t) = {t}; and the FULL set (dense attention)
    B, H, T, P, D = 1, 2, 4, 150, 128
    q, k, v = (_rand((B, H, T * P, D), torch.bfloat16, s) for s in (7, 8, 9))
    own = [[[[t] for t in range(T)] for _ in range(H)]]
    idx, cnt = _lists_to_arrays(own, B, H)
    _run_and_check(q, k, v, idx, cnt, P, "bf16", "own frame only")
    full = [[[list(range(T)) for _ in range(T)] for _ in range(H)]]
    idx, cnt = _lists_to_arrays(full, B, H)
    _run_and_check(q, k, v, idx, cnt, P, "bf16", "full set")


def test_bf16_explicit_scale_and_batch():
    B, H, T, P, D = 2, 3, 3, 40, 64
    q, k, v = (_rand((B, H, T * P, D), torch.bfloat16, s) for s in (10, 11, 12))
    lists = [[[[0, 1], [2], [0, 2]] for _ in range(H)] for _ in range(B)]
    lists[1][2] = [[1], [0, 1, 2], []]
    idx, cnt = _lists_to_arrays(lists, B, H)
    _run_and_check(q, k, v, idx, cnt, P, "bf16", "scale 0.05, batch 2", scale=0.05)


def test_malformed_entries_are_skipped_not_read():
    # entries outside [0, Tk) are skipped and cnt is clamped to cap: the result
    # equals attention over the valid entries only
    B, H, T, P, D = 1, 1, 3, 24, 128
    q, k, v = (_rand((B, H, T * P, D), torch.bfloat16, s) for s in (13, 14, 15))
    idx = torch.tensor([[[[0, 99, 2], [-5, 1, 7], [2, 1000, -1]]]], dtype=torch.int32)
    cnt = torch.tensor([[[3, 3, 9]]], dtype=torch.int32)
    good = [[[[0, 2], [1], [2]]]]
    gidx, gcnt = _lists_to_arrays(good, B, H)
    _say("malformed entries")
    o, lse = fsa.sparse_frame_attn(q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV), cnt.to(DEV), P)
    o2, lse2 = fsa.sparse_frame_attn(q.to(DEV), k.to(DEV), v.to(DEV), gidx.to(DEV),
                                     gcnt.to(DEV), P)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("D", [64, 128])
def test_neighbouring_frames_with_unrelated_lists(D):
    # P = 150 (a 128-row tile and a 22-row tail per frame): neighbouring query
    # frames whose lists are disjoint, empty, identical, subset / superset or
    # interleaved, on heads of different kinds; every row against the oracle.
    B, H, T, P = 1, 4, 5, 150
    q, k, v = (_rand((B, H, T * P, D), torch.bfloat16, s, outliers=2) for s in (71, 72, 73))
    lists = [[[[0], [3], [], [1, 2, 3, 4], [2]],           # disjoint, empty, superset, subset
              [[0, 1], [0, 1], [0, 1], [4], [0, 2, 4]],    # identical, then disjoint, interleaved
              [[1, 3], [0, 2, 4], [1, 3], [0, 2, 4], []],  # interleaved, last frame empty
              [[4], [3, 4], [2, 3, 4], [1, 2, 3, 4], [0, 1, 2, 3, 4]]]]
    idx, cnt = _lists_to_arrays(lists, B, H)
    _run_and_check(q, k, v, idx, cnt, P, "bf16", f"neighbouring frames' lists D={D}")
    # out-of-range entries are skipped: the result equals the lists without them
    bad = idx.clone()
    bad[0, 0, 1, 1] = 99                     # frame 1: [3, 99]
    cnt_bad = cnt.clone()
    cnt_bad[0, 0, 1] = 2
    bad[0, 2, 2, 2] = -7                     # frame 2 of head 2: [1, 3, -7]
    cnt_bad[0, 2, 2] = 3
    _say(f"neighbouring lists with out-of-range entries D={D}")
    o1, l1 = fsa.sparse_frame_attn(q.to(DEV), k.to(DEV), v.to(DEV), bad.to(DEV),
                                   cnt_bad.to(DEV), P)
    o2, l2 = fsa.sparse_frame_attn(q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV), cnt.to(DEV), P)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_sets_give_zero_and_minus_inf():
    B, H, T, P, D = 1, 2, 2, 33, 128
    q, k, v = (_rand((B, H, T * P, D), torch.bfloat16, s) for s in (16, 17, 18))
    idx = torch.full((B, H, T, 2), -1, dtype=torch.int32)
    cnt = torch.zeros((B, H, T), dtype=torch.int32)
    _say("empty sets")
    o, lse = fsa.sparse_frame_attn(q.to(DEV), k.to(DEV), v.to(DEV), idx.to(DEV), cnt.to(DEV), P)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(lse == -float("inf"))


def test_zero_queries_closed_form():
    # Q = 0: every attended key has score 0, so O is the mean of the attended V
    # rows and LSE = ln(|A|·P) exactly
    B, H, T, P, D = 1, 1, 4, 96, 128
    q = torch.zeros(B, H, T * P, D, dtype=torch.bfloat16)
    k, v = (_rand((B, H, T * P, D), torch.bfloat16, s) for s in (19, 20))
    lists = [[[[0], [0, 1], [1, 2, 3], [0, 1, 2, 3]]]]
    idx, cnt = _lists_to_arrays(lists, B, H)
    _run_and_check(q, k, v, idx, cnt, P, "bf16", "zero queries")


@pytest.mark.parametrize("Nk,D", [(1, 64), (13, 128), (64, 128), (100, 64), (1560, 128)])
def test_prepare_values_layout(Nk, D):
    # prepared V = float16, key-chunked transposed [B*H][ceil(Nk/8)][D][8], zero past Nk
    B, H = 1, 3
    v = _rand((B, H, Nk, D), torch.bfloat16, 31, outliers=2)
    _say(f"prepare_values Nk={Nk} D={D}")
    prep = fsa.prepare_values(v.to(DEV))
    torch.cuda.synchronize()
    NkC = -(-Nk // 8)
    got = prep.view(torch.float16)[:B * H * NkC * D * 8].view(B * H, NkC, D, 8).cpu()
    ref = torch.zeros(B * H, NkC * 8, D, dtype=torch.float16)
    ref[:, :Nk] = v.reshape(B * H, Nk, D).to(torch.float16)
    ref = ref.view(B * H, NkC, 8, D).permute(0, 1, 3, 2)
    assert torch.equal(got, ref)


def test_prepared_path_equals_one_call():
    w = wl.lvsa_shaped(4).shrunk(H=2, P=136)
    q, k, v = (t.to(DEV) for t in wl.make_qkv(w))
    idx, cnt = fsa.build_frame_sets(w.policies[:2], w.B, w.Tq, w.Tk, device=DEV)
    _say("prepared vs one call")
    o1, l1 = fsa.sparse_frame_attn(q, k, v, idx, cnt, w.P)
    prep = fsa.prepare_values(v)
    o2, l2 = fsa.sparse_frame_attn_prepared(q, k, prep, idx, cnt, w.P)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("D,P", [(64, 40), (128, 150)])
def test_dual_pass_edges(D, P):
    # one pass over A then B: O_A = attention over A, O_AB = attention over A ∪ B
    B, H, T = 1, 2, 5
    q, k, v = (_rand((B, H, T * P, D), torch.bfloat16, s, outliers=2) for s in (41, 42, 43))
    la = [[[0], [], [1, 3], [], [0, 2, 4]], [[4], [2], [], [0, 1, 2, 3, 4], []]]
    lb = [[[1, 2], [0, 4], [], [], [1, 3]], [[0, 1], [], [3], [], []]]
    ia, ca = _lists_to_arrays([la], B, H)
    ib, cb = _lists_to_arrays([lb], B, H)
    lu = [[[sorted(a + b) for a, b in zip(la[h], lb[h])] for h in range(H)]]
    iu, cu = _lists_to_arrays(lu, B, H)
    prep = fsa.prepare_values(v.to(DEV))
    _say(f"dual pass D={D} P={P}")
    oa, la_, oab, lab = fsa.sparse_frame_attn_dual(q.to(DEV), k.to(DEV), prep, ia.to(DEV),
                                                    ca.to(DEV), ib.to(DEV), cb.to(DEV), P)
    o1, l1 = fsa.sparse_frame_attn_prepared(q.to(DEV), k.to(DEV), prep, ia.to(DEV), ca.to(DEV), P)
    torch.cuda.synchronize()
    assert torch.equal(oa, o1) and torch.equal(la_, l1)   # A's state is the single-list result
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    ra = oatt.sparse_frame_attention(qn, kn, vn, ia.numpy(), ca.numpy(), P)
    ru = oatt.sparse_frame_attention(qn, kn, vn, iu.numpy(), cu.numpy(), P)
    assert_close(oa.cpu().numpy(), la_.cpu().numpy(), *ra, "bf16", f"dual O_A D={D}")
    assert_close(oab.cpu().numpy(), lab.cpu().numpy(), *ru, "bf16", f"dual O_AB D={D}")


@pytest.mark.parametrize("B,H,widths", [(1, 5, [0, 3, 1, 5, 2]), (2, 3, [4, 0, 2, 1, 5, 3]),
                                         (1, 4, [2, 2, 2, 2]),
                                         (2, 32, [(7 * i) % 6 for i in range(64)])])
def test_small_grids_visit_heads_in_cost_order(B, H, widths):
    # Grids this small reorder the heads by cost inside the kernel (heaviest,
    # lightest, second heaviest, ...; equal costs keep the plain order).  Head
    # (b, h) lists the frames [t - w, t] of query frame t with its own width w,
    # so the heads' costs differ; every row of every head is checked.  The last
    # case has 64 heads, the largest count that is reordered (384 blocks).
    P, T, D = 40, 6, 128
    q, k, v = (_rand((B, H, T * P, D), torch.bfloat16, s, outliers=2) for s in (61, 62, 63))
    lists = [[[list(range(max(0, t - widths[b * H + h]), t + 1)) for t in range(T)]
              for h in range(H)] for b in range(B)]
    idx, cnt = _lists_to_arrays(lists, B, H)
    _run_and_check(q, k, v, idx, cnt, P, "bf16", f"heads in cost order, B={B} H={H}")
    # the dual pass takes list B into the cost: A = the own frame, B = the rest
    la = [[[[t] for t in range(T)] for _ in range(H)] for _ in range(B)]
    lb = [[[a[:-1] for a in lists[b][h]] for h in range(H)] for b in range(B)]
    ia, ca = _lists_to_arrays(la, B, H)
    ib, cb = _lists_to_arrays(lb, B, H)
    prep = fsa.prepare_values(v.to(DEV))
    oa, l_a, oab, l_ab = fsa.sparse_frame_attn_dual(q.to(DEV), k.to(DEV), prep, ia.to(DEV),
                                                     ca.to(DEV), ib.to(DEV), cb.to(DEV), P)
    torch.cuda.synchronize()
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    ra = oatt.sparse_frame_attention(qn, kn, vn, ia.numpy(), ca.numpy(), P)
    ru = oatt.sparse_frame_attention(qn, kn, vn, idx.numpy(), cnt.numpy(), P)
    assert_close(oa.cpu().numpy(), l_a.cpu().numpy(), *ra, "bf16", f"cost order dual O_A B={B}")
    assert_close(oab.cpu().numpy(), l_ab.cpu().numpy(), *ru, "bf16", f"cost order dual O_AB B={B}")


@pytest.mark.parametrize("B,H,T,P", [(1, 1, 257, 8), (2, 4, 64, 16), (1, 4, 25, 300),
                                     (1, 10, 17, 260)])
def test_grids_resident_at_once_pair_heavy_with_light(B, H, T, P):
    # Grids of 257 to 512 blocks (one per query tile) are resident at once, two
    # per CU; with lists of unequal cost the kernel ranks the blocks and puts
    # heavy ones on CUs of their own or next to light ones.  The cases take the
    # ends of that range (257 and 512 blocks of one tile) and frames of three
    # query tiles (300 and 510 blocks, the last tile ragged); frame t lists
    # [t - w, t] with a seeded width w in 0..5 per (b, h, t).  Every row is
    # checked against the oracle.
    D = 128
    rng = np.random.default_rng(B * 1000 + H * 100 + T)
    q, k, v = (_rand((B, H, T * P, D), torch.bfloat16, s, outliers=2) for s in (81, 82, 83))
    lists = [[[list(range(max(0, t - int(rng.integers(0, 6))), t + 1)) for t in range(T)]
              for _ in range(H)] for _ in range(B)]
    idx, cnt = _lists_to_arrays(lists, B, H)
    blocks = B * H * T * -(-P // 128)
    assert 256 < blocks <= 512
    _run_and_check(q, k, v, idx, cnt, P, "bf16", f"resident grid of {blocks} blocks, P={P}")


@pytest.mark.parametrize("kind,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_maximum_list_length_and_run_count(kind, D):
    # lists at the capacity limit (FSA_MAX_CAP = 1024 entries), a list of 512
    # one-frame runs (every other frame), a long random list, and one frame:
    # frames of P = 3 tokens in a 1100-frame cache, 2 query frames
    P, Tq, Tk = 3, 4, 1100
    rng = np.random.default_rng(12)
    lists = [[[list(range(1024)),
               list(range(0, 1024, 2)),
               sorted(rng.choice(Tk, 1000, replace=False).tolist()),
               [Tk - 1]]]]
    idx, cnt = _lists_to_arrays(lists, 1, 1)
    assert idx.shape[3] == 1024
    dt = torch.bfloat16 if kind == "bf16" else torch.float32
    q = _rand((1, 1, Tq * P, D), dt, 21)
    k = _rand((1, 1, Tk * P, D), dt, 22)
    v = _rand((1, 1, Tk * P, D), dt, 23)
    _run_and_check(q, k, v, idx, cnt, P, kind, f"{kind} D={D} 1024-entry lists, 512 runs")
