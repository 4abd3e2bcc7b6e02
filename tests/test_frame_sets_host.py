"""The library's frame-set construction (host entry point, the same routine the
device kernel runs) against the oracle, bit for bit, plus capacity bounds and
the list validator."""

import numpy as np
import pytest

import frame_sparse_attention_amd as fsa
import workloads as wl
from oracle import frame_sets as ofs


def _compare(policies, B, Tq, Tk, offset=0, chunk=1, selected=None):
    cap = fsa.frame_set_capacity(policies, Tq, Tk, offset, chunk)
    idx, cnt = fsa.build_frame_sets_host(policies, B, Tq, Tk, offset, chunk, selected, cap)
    sel_lists = None
    if selected is not None:
        # the library skips selected entries outside [0, Tk); the oracle only
        # ever sees frames that exist
        sel_lists = [[[[f for f in selected[b, h, g, :policies[h]["topk"]] if 0 <= f < Tk]
                       for g in range(selected.shape[2])] for h in range(len(policies))]
                     for b in range(B)]
    oidx, ocnt = ofs.build(policies, B, Tq, Tk, offset, chunk, sel_lists, cap=cap)
    np.testing.assert_array_equal(cnt, ocnt)
    np.testing.assert_array_equal(idx, oidx)
    fsa.validate_frame_sets(idx, cnt, Tk)
    return idx, cnt


@pytest.mark.parametrize("make", [wl.tiny_f32, wl.lvsa_shaped, wl.long_video, wl.ar_chunk,
                                  wl.decomposable])
def test_workload_frame_sets_match_oracle(make):
    w = make()
    steps = range(w.steps)
    for s in steps:
        ws = w.with_step(s)
        sel = None
        if any(p["kind"] == wl.MEMORY for p in ws.policies):
            rng = np.random.default_rng(s)
            sel = np.stack([np.stack([np.sort(rng.choice(57, 8, replace=False))[None]
                                      for _ in range(ws.H)])]).astype(np.int32)
        _compare(ws.policies, ws.B, ws.Tq, ws.Tk, ws.offset, ws.chunk, sel)
        for pols in ws.branches.values():
            _compare(pols, ws.B, ws.Tq, ws.Tk, ws.offset, ws.chunk)


def test_lvsa_exhaustive_small():
    for T in range(1, 25):
        for T_per in range(1, 8):
            for W in range(0, 9):
                for C in range(0, 27, 2):
                    pols = [wl.policy(wl.LVSA, window=W, budget=C, t_per=T_per, step=s)
                            for s in range(T_per + 1)]
                    _compare(pols, 1, T, T)


def test_sink_window_memory_range_sweep():
    rng = np.random.default_rng(0)
    for Tk in (1, 3, 8, 20):
        for chunk in (1, 2, 4):
            for offset in range(0, Tk):
                Tq = ((Tk - offset) // chunk) * chunk
                if Tq == 0:
                    continue
                pols = [wl.policy(wl.SINK_WINDOW, n_sink=ns, window=w)
                        for ns in (0, 1, 3) for w in (0, 1, 2, 5)]
                pols += [wl.policy(wl.RANGE, lo=lo, hi=hi) for lo, hi in
                         ((0, Tk - 1), (1, 2), (-3, Tk + 4), (5, 2))]
                pols += [wl.policy(wl.FULL)]
                pols += [wl.policy(wl.MEMORY, topk=kk, n_recent=nr) for kk in (0, 1, 3)
                         for nr in (0, 2)]
                G = Tq // chunk
                sel = rng.integers(-2, Tk + 2, size=(2, len(pols), G, 3)).astype(np.int32)
                _compare(pols, 2, Tq, Tk, offset, chunk, sel)


def test_capacity_is_exact_on_the_workloads():
    assert fsa.frame_set_capacity(wl.lvsa_shaped().policies, 42, 42) == 21
    assert fsa.frame_set_capacity(wl.long_video().policies, 126, 126) == 33
    w = wl.ar_chunk()
    assert fsa.frame_set_capacity(w.policies, w.Tq, w.Tk, w.offset, w.chunk) == 11
    assert fsa.frame_set_capacity(wl.tiny_f32().policies, 4, 4) == 3


def test_validator_flags_bad_lists():
    idx = np.array([[[[0, 2, -1], [1, 1, -1], [3, 2, -1], [0, 9, -1], [0, -1, -1]]]],
                   dtype=np.int32)
    cnt = np.array([[[2, 2, 2, 2, 4]]], dtype=np.int32)
    for t, msg in ((1, "not above"), (2, "not above"), (3, "outside"), (4, "cnt=4")):
        i = idx[:, :, [0, t]].copy()
        c = cnt[:, :, [0, t]].copy()
        with pytest.raises(fsa.FsaError, match=msg):
            fsa.validate_frame_sets(i, c, 5)
    fsa.validate_frame_sets(idx[:, :, :1], cnt[:, :, :1], 5)


@pytest.mark.parametrize("make", [wl.ar_chunk_hsa])
def test_block_unit_frame_windows_match_oracle(make):
    # the frame windows of the non-memory heads, written in block units, from the
    # library's builder against the oracle's own scaling of the same policies
    from oracle import hsa as ohsa
    w = make()
    nb = w.P // w.block
    bpol = wl.block_policies(w)
    Tqb, Tkb, ob, cb = w.Tq * nb, w.Tk * nb, w.offset * nb, w.chunk * nb
    cap = fsa.frame_set_capacity(bpol, Tqb, Tkb, ob, cb)
    idx, cnt = fsa.build_frame_sets_host(bpol, w.B, Tqb, Tkb, ob, cb, None, cap)
    for h, p in enumerate(w.policies):
        if p["kind"] == wl.MEMORY:
            continue
        oidx, ocnt = ofs.build([ohsa.scale_policy_to_blocks(p, nb)], w.B, Tqb, Tkb, ob, cb,
                               cap=cap)
        np.testing.assert_array_equal(idx[:, h:h + 1], oidx)
        np.testing.assert_array_equal(cnt[:, h:h + 1], ocnt)
        # and every query block sees whole frames: the frame list times nb
        fidx, fcnt = ofs.build([p], w.B, w.Tq, w.Tk, w.offset, w.chunk)
        frames = fidx[0, 0, 0, :fcnt[0, 0, 0]]
        assert idx[0, h, 0, :cnt[0, h, 0]].tolist() == [f * nb + i for f in frames
                                                        for i in range(nb)]
