"""GPU parity: device frame-set construction and top-k frame selection must
equal the oracle bit for bit; the LSE merge must match it within fp32 noise."""

import numpy as np
import pytest
import torch

import frame_sparse_attention_amd as fsa
import workloads as wl
from oracle import frame_sets as ofs
from oracle import merge as omerge
from oracle import topk as otopk

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _device_vs_oracle(policies, B, Tq, Tk, offset, chunk, sel=None):
    cap = fsa.frame_set_capacity(policies, Tq, Tk, offset, chunk)
    sel_dev = torch.from_numpy(sel).to(DEV) if sel is not None else None
    idx, cnt = fsa.build_frame_sets(policies, B, Tq, Tk, offset, chunk, sel_dev, cap, DEV)
    torch.cuda.synchronize()
    sel_lists = None
    if sel is not None:
        sel_lists = [[[[f for f in sel[b, h, g, :policies[h]["topk"]] if 0 <= f < Tk]
                       for g in range(sel.shape[2])] for h in range(len(policies))]
                     for b in range(B)]
    oidx, ocnt = ofs.build(policies, B, Tq, Tk, offset, chunk, sel_lists, cap=cap)
    np.testing.assert_array_equal(cnt.cpu().numpy(), ocnt)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)


@pytest.mark.parametrize("make", [wl.tiny_f32, wl.lvsa_shaped, wl.ar_chunk, wl.decomposable,
                                  wl.long_video])
def test_device_frame_sets_bit_exact(make):
    w = make()
    for s in range(w.steps):
        ws = w.with_step(s)
        _say(f"frame sets {w.name} step {s}")
        sel = None
        if any(p["kind"] == wl.MEMORY for p in ws.policies):
            rng = np.random.default_rng(s)
            sel = np.stack([np.stack([rng.choice(57, 8, replace=False)[None]
                                      for _ in range(ws.H)])]).astype(np.int32)
        _device_vs_oracle(ws.policies, ws.B, ws.Tq, ws.Tk, ws.offset, ws.chunk, sel)
        for name, pols in ws.branches.items():
            _device_vs_oracle(pols, ws.B, ws.Tq, ws.Tk, ws.offset, ws.chunk)


def test_device_frame_sets_sweep_with_bad_selections():
    rng = np.random.default_rng(1)
    for Tk in (1, 5, 17):
        for chunk in (1, 3):
            offset = max(0, Tk - 2 * chunk)
            Tq = ((Tk - offset) // chunk) * chunk
            if Tq == 0:
                continue
            pols = [wl.policy(wl.SINK_WINDOW, n_sink=ns, window=w) for ns in (0, 2) for w in (1, 4)]
            pols += [wl.policy(wl.MEMORY, topk=3, n_recent=nr) for nr in (0, 2)]
            pols += [wl.policy(wl.LVSA, window=3, budget=6, t_per=4, step=s) for s in range(4)]
            pols += [wl.policy(wl.RANGE, lo=1, hi=Tk + 3), wl.policy(wl.FULL)]
            sel = rng.integers(-3, Tk + 3, size=(2, len(pols), Tq // chunk, 3)).astype(np.int32)
            _say(f"frame set sweep Tk={Tk} chunk={chunk}")
            _device_vs_oracle(pols, 2, Tq, Tk, offset, chunk, sel)


def _oracle_topk(q, k, P, h_begin, h_end, q_group, c0, c1, kk):
    B, H, Nq, D = q.shape
    G = Nq // (q_group * P)
    frames = np.full((B, H, G, kk), -1, np.int32)
    scores = np.full((B, H, G, c1 - c0), np.nan)
    for b in range(B):
        for h in range(h_begin, h_end):
            qh = q[b, h].float().numpy()
            kh = k[b, h].float().numpy()
            for g in range(G):
                rows = np.arange(g * q_group * P, (g + 1) * q_group * P)
                f, s = otopk.select_topk_frames(qh, kh, P, rows, range(c0, c1), kk)
                frames[b, h, g] = f
                scores[b, h, g] = s
    return frames, scores


def test_topk_ar_chunk_bit_exact():
    # Memory heads 8-11 of the AR-chunk workload: pool the 3-frame query chunk and
    # every cache frame 0..56, keep the best 8.
    w = wl.ar_chunk()
    q, k, _ = wl.make_qkv(w)
    _say("top-k ar_chunk full size")
    frames, scores = fsa.select_topk_frames(q.to(DEV), k.to(DEV), w.P, 8, 12, 3, 0, 57, 8,
                                            return_scores=True)
    torch.cuda.synchronize()
    of, os_ = _oracle_topk(q, k, w.P, 8, 12, 3, 0, 57, 8)
    np.testing.assert_array_equal(frames.cpu().numpy(), of)
    got = scores.cpu().numpy()[:, 8:12]
    assert np.array_equal(got, os_[:, 8:12]), "fp64 scores differ in some bit"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_topk_small_groups_and_candidate_windows(dtype):
    g = torch.Generator().manual_seed(11)
    B, H, P, D = 2, 3, 7, 64
    q = torch.randn(B, H, 4 * P, D, generator=g).to(dtype)
    k = torch.randn(B, H, 20 * P, D, generator=g).to(dtype)
    for q_group, c0, c1, kk in ((1, 0, 20, 5), (2, 3, 17, 14), (4, 10, 11, 1)):
        _say(f"top-k small {dtype} q_group={q_group} cand=[{c0},{c1}) k={kk}")
        frames, scores = fsa.select_topk_frames(q.to(DEV), k.to(DEV), P, 0, H, q_group, c0, c1,
                                                kk, return_scores=True)
        torch.cuda.synchronize()
        of, os_ = _oracle_topk(q, k, P, 0, H, q_group, c0, c1, kk)
        np.testing.assert_array_equal(frames.cpu().numpy(), of)
        assert np.array_equal(scores.cpu().numpy(), os_)


def test_topk_planted_ties_pick_earlier_frame():
    P, D = 4, 64
    q = torch.ones(1, 1, P, D)
    base = torch.ones(P, D)
    mult = [1, 3, 2, 3, 3, 0.5, 2, 3]       # frames 1, 3, 4, 7 tie at the top
    k = torch.cat([base * m for m in mult])[None, None].contiguous()
    _say("top-k planted ties")
    frames = fsa.select_topk_frames(q.to(DEV), k.to(DEV), P, 0, 1, 1, 0, 8, 3)
    torch.cuda.synchronize()
    assert frames.cpu().numpy().ravel().tolist() == [1, 3, 4]


def test_memory_heads_assembled_on_device():
    # top-k output feeds the device builder directly (no host round trip)
    w = wl.ar_chunk()
    q, k, _ = wl.make_qkv(w)
    _say("memory heads: top-k -> build_frame_sets")
    sel = fsa.select_topk_frames(q.to(DEV), k.to(DEV), w.P, 8, 12, 3, 0, 57, 8)
    idx, cnt = fsa.build_frame_sets(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk, sel,
                                    device=DEV)
    torch.cuda.synchronize()
    of, _ = _oracle_topk(q, k, w.P, 8, 12, 3, 0, 57, 8)
    sel_lists = [[[list(of[0, h, 0])] if h >= 8 else [[]] for h in range(12)]]
    oidx, ocnt = ofs.build(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk, sel_lists,
                           cap=idx.shape[3])
    np.testing.assert_array_equal(cnt.cpu().numpy(), ocnt)
    np.testing.assert_array_equal(idx.cpu().numpy(), oidx)
    assert cnt[0, :, 0].tolist() == [6] * 4 + [9] * 4 + [11] * 4


@pytest.mark.parametrize("rows,D", [(1, 1), (37, 64), (56160, 128), (1000, 300)])
def test_merge_lse_matches_oracle(rows, D):
    g = torch.Generator().manual_seed(rows)
    o1 = torch.randn(rows, D, generator=g)
    o2 = torch.randn(rows, D, generator=g)
    l1 = torch.randn(rows, generator=g) * 20
    l2 = torch.randn(rows, generator=g) * 20
    if rows >= 4:
        l1[0] = -float("inf")
        l2[1] = -float("inf")
        l1[2] = l2[2] = -float("inf")
        l1[3] = 80.0
        l2[3] = -80.0
    # the operand of a zero weight may hold anything: NaN and inf there must
    # not reach the output (the oracle gets the clean values, which carry no weight)
    o1_dev, o2_dev = o1.clone(), o2.clone()
    if rows >= 4:
        o1_dev[0] = float("nan")
        o2_dev[1] = float("inf")
        o1_dev[2] = float("nan")
        o2_dev[2] = -float("inf")
    _say(f"merge rows={rows} D={D}")
    o, lse = fsa.merge_lse(o1_dev.to(DEV), l1.to(DEV), o2_dev.to(DEV), l2.to(DEV))
    torch.cuda.synchronize()
    n = min(rows, 3000)
    oo, ol = omerge.merge_lse(o1[:n].double().numpy(), l1[:n].double().numpy(),
                              o2[:n].double().numpy(), l2[:n].double().numpy())
    got_o = o[:n].cpu().double().numpy()
    got_l = lse[:n].cpu().double().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ol))
    fin = np.isfinite(ol)
    assert np.max(np.abs(got_l[fin] - ol[fin])) <= 1e-5
    assert np.max(np.abs(got_o - oo)) <= 1e-5


def test_merge_in_place():
    g = torch.Generator().manual_seed(5)
    o1, o2 = torch.randn(64, 128, generator=g), torch.randn(64, 128, generator=g)
    l1, l2 = torch.randn(64, generator=g), torch.randn(64, generator=g)
    ref_o, ref_l = fsa.merge_lse(o1.to(DEV), l1.to(DEV), o2.to(DEV), l2.to(DEV))
    a, la = o1.to(DEV), l1.to(DEV)
    _say("merge in place")
    fsa.merge_lse(a, la, o2.to(DEV), l2.to(DEV), out=a, out_lse=la)
    torch.cuda.synchronize()
    assert torch.equal(a, ref_o) and torch.equal(la, ref_l)


@pytest.mark.parametrize("n_cand,kk", [(1024, 64), (1025, 7), (3000, 40)])
def test_topk_many_candidates(n_cand, kk):
    # at most 1024 candidates the k best are taken by rank, beyond that by
    # rounds of a wavefront argmax: both must give the oracle's frames
    g = torch.Generator().manual_seed(n_cand)
    B, H, P, D = 1, 2, 2, 64
    q = torch.randn(B, H, 2 * P, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, n_cand * P, D, generator=g).to(torch.bfloat16)
    _say(f"top-k over {n_cand} candidates, k={kk}")
    frames = fsa.select_topk_frames(q.to(DEV), k.to(DEV), P, 0, H, 2, 0, n_cand, kk)
    torch.cuda.synchronize()
    of, _ = _oracle_topk(q, k, P, 0, H, 2, 0, n_cand, kk)
    np.testing.assert_array_equal(frames.cpu().numpy(), of)


@pytest.mark.parametrize("dtype,D,P", [
    (torch.float32, 128, 300),   # 16-byte loads of 4 floats, 3 pieces per frame
    (torch.float32, 64, 500),    # 16 rows per step, 4 pieces of 125 rows
    (torch.bfloat16, 64, 700),   # 16-byte loads of 8 bf16, 32 rows per step
    (torch.bfloat16, 128, 100),  # one piece per frame, 2 pieces per query group
    (torch.bfloat16, 96, 90),    # 12 units per row: 21 rows per step, 4 threads idle
    (torch.float32, 200, 40),    # 50 units per row, 5 rows per step
    (torch.bfloat16, 60, 33),    # 120-byte rows: element-wise loads
    (torch.float32, 30, 129),    # 120-byte rows: element-wise loads, 2 pieces per frame
])
def test_topk_pooling_paths(dtype, D, P):
    g = torch.Generator().manual_seed(D * 1000 + P)
    B, H = 1, 2
    q = (torch.randn(B, H, 2 * P, D, generator=g) * 3).to(dtype)
    k = (torch.randn(B, H, 12 * P, D, generator=g) * 3).to(dtype)
    _say(f"top-k pooling path {dtype} D={D} P={P}")
    frames, scores = fsa.select_topk_frames(q.to(DEV), k.to(DEV), P, 0, H, 2, 0, 12, 4,
                                            return_scores=True)
    torch.cuda.synchronize()
    of, os_ = _oracle_topk(q, k, P, 0, H, 2, 0, 12, 4)
    np.testing.assert_array_equal(frames.cpu().numpy(), of)
    assert np.array_equal(scores.cpu().numpy(), os_)


def _wide_spread(shape, g, binades=200):
    """bf16-exact values whose exponents spread over `binades` binades, with
    exact opposites planted, so pooled segments fail the cheap exactness test
    and are summed exactly on the device."""
    m = torch.randint(128, 256, shape, generator=g).float()
    e = torch.randint(-binades // 2, binades // 2, shape, generator=g).float()
    s = torch.randint(0, 2, shape, generator=g).float() * 2 - 1
    x = s * m * torch.exp2(e - 7)
    x[..., 1::5, :] = -x[..., 0::5, :][..., : x[..., 1::5, :].shape[-2], :]
    return x


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_topk_exact_sums_of_wide_spread_values(dtype):
    # every pooled sum is the exact sum rounded once: the device's exact path
    # (segments spanning ~2^200) must give the oracle's bits
    g = torch.Generator().manual_seed(31)
    B, H, P, D = 1, 2, 40, 64
    q = _wide_spread((B, H, 2 * P, D), g).to(dtype)
    k = _wide_spread((B, H, 9 * P, D), g).to(dtype)
    k[0, 0, 3 * P:4 * P] = q[0, 0, :P]          # a frame that matches the query well
    _say(f"top-k over wide-spread values ({dtype})")
    frames, scores = fsa.select_topk_frames(q.to(DEV), k.to(DEV), P, 0, H, 2, 0, 9, 3,
                                            return_scores=True)
    torch.cuda.synchronize()
    of, os_ = _oracle_topk(q, k, P, 0, H, 2, 0, 9, 3)
    np.testing.assert_array_equal(frames.cpu().numpy(), of)
    assert np.array_equal(scores.cpu().numpy(), os_), "fp64 scores differ in some bit"


def test_topk_pooling_is_exact_not_sequential():
    # one key frame whose tokens are 2^100, 1, -2^100, 1 per channel: any
    # sequential float64 order loses the ones; the exact sum is 2
    P, D = 4, 64
    q = torch.ones(1, 1, P, D)
    k = torch.zeros(1, 1, 3 * P, D)
    k[0, 0, 0] = 2.0**100
    k[0, 0, 1] = 1.0
    k[0, 0, 2] = -(2.0**100)
    k[0, 0, 3] = 1.0                 # frame 0: exact sum 2 per channel
    k[0, 0, P:2 * P] = 0.25          # frame 1: sum 1 per channel
    k[0, 0, 2 * P:] = 0.125          # frame 2: sum 0.5 per channel
    _say("top-k: cancellation inside one frame")
    for dtype in (torch.float32, torch.bfloat16):
        frames, scores = fsa.select_topk_frames(q.to(dtype).to(DEV), k.to(dtype).to(DEV), P, 0,
                                                1, 1, 0, 3, 1, return_scores=True)
        torch.cuda.synchronize()
        assert frames.cpu().numpy().ravel().tolist() == [0]
        assert scores.cpu().numpy().ravel().tolist() == [4.0 * 2 * D, 4.0 * D, 4.0 * 0.5 * D]
