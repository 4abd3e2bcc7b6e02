"""GPU parity of the per-head frame-level RoPE re-encoding (Head Forcing §3)
and of attention over the re-encoded cache.

The re-encoding rounds a float64 rotation once to the storage type on both
sides, so the results agree bit for bit unless the float64 cos / sin / pow of
the two math libraries differ by an ulp right at a rounding boundary; the bar
is therefore: every element within one unit in the last place of the storage
type, and at most one element in a million not bit-identical.  Attention over
the re-encoded tensors is then held to the usual bf16 / fp32 tolerances."""

import numpy as np
import pytest
import torch

import frame_sparse_attention_amd as fsa
import workloads as wl
from oracle import frame_sets as ofs
from oracle import rope as orope
from oracle import topk as otopk

from _parity import assert_close, oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _ulps(a: np.ndarray, b: np.ndarray, dt: str) -> np.ndarray:
    """Distance in units in the last place of the storage type (finite values)."""
    if dt == "bf16":
        ia = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64)
        ib = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64)
        ia = np.where(ia < 0, -(ia & 0x7FFF), ia)
        ib = np.where(ib < 0, -(ib & 0x7FFF), ib)
    else:
        ia = a.astype(np.float32).view(np.int32).astype(np.int64)
        ib = b.astype(np.float32).view(np.int32).astype(np.int64)
        ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
        ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def _compare(got, ref, dt, what):
    got = got.astype(np.float64)
    d = _ulps(got, ref, dt)
    n_diff = int((d > 0).sum())
    print(f"[parity] {what}: {got.size} elements, {n_diff} not bit-identical, max {int(d.max())}"
          f" ulp", flush=True)
    assert int(d.max()) <= 1, what
    assert n_diff <= max(1, got.size // 1_000_000), what


def _oracle_reencode(q, k, idx, cnt, P, offset, rot, base, dt):
    B, H = q.shape[:2]
    qo = np.zeros(q.shape)
    ko = np.zeros(k.shape)
    for b in range(B):
        for h in range(H):
            frames = idx[b, h, :cnt[b, h]].tolist()
            qo[b, h], ko[b, h] = orope.reencode(q[b, h].double().numpy(), k[b, h].double().numpy(),
                                                P, frames, offset, rot, base, dt)
    return qo, ko


SMALL = [
    # (dtype, B, H, D, Tq, Tk, P, offset, rot)
    ("f32", 1, 3, 64, 2, 9, 10, 7, 64),
    ("f32", 2, 2, 64, 3, 6, 4, 3, 10),
    ("bf16", 1, 3, 128, 2, 12, 24, 10, 42),
    ("bf16", 1, 2, 128, 1, 5, 16, 4, 0),
    ("bf16", 2, 2, 128, 3, 8, 20, 5, 128),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"case{i}" for i in range(len(SMALL))])
def test_rope_reencode_small(case):
    dt, B, H, D, Tq, Tk, P, offset, rot = case
    _say(f"rope_reencode {case}")
    w = wl.Workload("rope_case", 60 + SMALL.index(case), B, H, D, Tq, Tk, P, dt, [])
    q, k = wl.make_tensor(w, 0), wl.make_tensor(w, 1)
    rng = np.random.default_rng(SMALL.index(case))
    cap = Tk
    idx = np.full((B, H, cap), -1, np.int32)
    cnt = np.zeros((B, H), np.int32)
    for b in range(B):
        for h in range(H):
            if h == H - 1 and b == 0:
                continue                           # one head with an empty set
            n = int(rng.integers(1, Tk + 1))
            frames = np.sort(rng.choice(Tk, n, replace=False))
            idx[b, h, :n] = frames
            cnt[b, h] = n
    qd, kd = q.to(DEV), k.to(DEV)
    qo, ko = fsa.rope_reencode(qd, kd, torch.from_numpy(idx).to(DEV),
                               torch.from_numpy(cnt).to(DEV), P, rot, 10000.0, offset)
    torch.cuda.synchronize()
    qr, kr = _oracle_reencode(q, k, idx, cnt, P, offset, rot, 10000.0, dt)
    _compare(qo.double().cpu().numpy(), qr, dt, f"q' {case}")
    _compare(ko.double().cpu().numpy(), kr, dt, f"k' {case}")
    if rot == 0:
        assert torch.equal(qo.cpu(), q) and torch.equal(ko.cpu(), k)
    # in place gives the same bits
    q2, k2 = qd.clone(), kd.clone()
    fsa.rope_reencode(q2, k2, torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV), P,
                      rot, 10000.0, offset, q_out=q2, k_out=k2)
    assert torch.equal(q2, qo) and torch.equal(k2, ko)


def test_ar_chunk_rope_reencode_and_attention():
    w = wl.ar_chunk_rope()
    _say(f"{w.name}: inputs")
    q, k, v = wl.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    _say(f"{w.name}: lists")
    sel = fsa.select_topk_frames(qd, kd, w.P, 8, 12, 3, 0, 57, 8)
    cap = fsa.frame_set_capacity(w.policies, w.Tq, w.Tk, w.offset, w.chunk)
    idx, cnt = fsa.build_frame_sets(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk, sel, cap, DEV)
    # the chunk's query frames share one set per head
    idx_h, cnt_h = idx[:, :, 0].contiguous(), cnt[:, :, 0].contiguous()
    _say(f"{w.name}: re-encode")
    qo, ko = fsa.rope_reencode(qd, kd, idx_h, cnt_h, w.P, w.rope_dims, w.rope_base, w.offset)
    _say(f"{w.name}: attention")
    o, lse = fsa.sparse_frame_attn_prepared(qo, ko, fsa.prepare_values(vd), idx, cnt, w.P)
    torch.cuda.synchronize()
    # oracle: its own frame sets, its own re-encoding
    sel_lists = [[[[]] for _ in range(12)]]
    for h in range(8, 12):
        f, _ = otopk.select_topk_frames(q[0, h].float().numpy(), k[0, h].float().numpy(), w.P,
                                        np.arange(w.Nq), range(57), 8)
        sel_lists[0][h] = [f]
    oidx, ocnt = ofs.build(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk, sel_lists, cap=cap)
    assert np.array_equal(idx.cpu().numpy(), oidx) and np.array_equal(cnt.cpu().numpy(), ocnt)
    qr, kr = _oracle_reencode(q, k, oidx[:, :, 0], ocnt[:, :, 0], w.P, w.offset, w.rope_dims,
                              w.rope_base, "bf16")
    _compare(qo.double().cpu().numpy(), qr, "bf16", f"{w.name} q'")
    listed = np.zeros((w.B, w.H, w.Nk), bool)
    for h in range(w.H):
        for f in oidx[0, h, 0, :ocnt[0, h, 0]]:
            listed[0, h, f * w.P:(f + 1) * w.P] = True
    _compare(ko.double().cpu().numpy()[listed], kr[listed], "bf16", f"{w.name} k' listed frames")
    rows = np.array(sorted(set([0, 127, 128, 1559, 1560, 4679] +
                               np.random.default_rng(8).integers(0, w.Nq, 40).tolist())))
    qr_t = torch.from_numpy(qr).to(torch.bfloat16)
    kr_t = torch.from_numpy(kr).to(torch.bfloat16)
    o_ref, l_ref = oracle_rows(qr_t, kr_t, v, oidx, ocnt, w.P, rows)
    assert_close(o[:, :, rows].cpu().numpy(), lse[:, :, rows].cpu().numpy(), o_ref, l_ref, "bf16",
                 f"{w.name} attention on the re-encoded cache")


def test_rope_reencode_extreme_values():
    # bf16 inputs at the ends of the range: results that overflow, that fall in
    # the subnormal range, zeros of both signs; every rounding path is taken
    _say("rope_reencode extreme values")
    B, H, D, P, Tq, Tk = 1, 1, 64, 8, 1, 4
    rng = np.random.default_rng(9)
    mags = np.array([3.3895313892515355e38, 3.0e38, 1.7e38, 1e-38, 1.2e-38, 9.2e-41, 3e-39,
                     0.0, 1.0, 65504.0], dtype=np.float64)
    def draw(n):
        x = rng.choice(mags, size=(n, D)) * rng.choice([-1.0, 1.0], size=(n, D))
        return torch.from_numpy(x).to(torch.bfloat16)
    q = draw(Tq * P)[None, None].contiguous()
    k = draw(Tk * P)[None, None].contiguous()
    idx = np.array([[[0, 1, 3]]], np.int32)
    cnt = np.array([[3]], np.int32)
    qo, ko = fsa.rope_reencode(q.to(DEV), k.to(DEV), torch.from_numpy(idx).to(DEV),
                               torch.from_numpy(cnt).to(DEV), P, D, 7.0, 3)
    torch.cuda.synchronize()
    qr, kr = _oracle_reencode(q, k, idx, cnt, P, 3, D, 7.0, "bf16")
    for got, ref, what in ((qo, qr, "q'"), (ko, kr, "k'")):
        g = got.double().cpu().numpy()
        both_inf = np.isinf(g) & np.isinf(ref) & (np.sign(g) == np.sign(ref))
        fin = np.isfinite(g) & np.isfinite(ref)
        assert (both_inf | fin).all(), f"{what}: infinities differ"
        _compare(g[fin], ref[fin], "bf16", f"extreme values {what}")
