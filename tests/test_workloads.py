"""The seeded input generators: determinism, dtype, shapes, outlier channels,
and the frame-set sizes each workload is meant to have."""

import torch

import workloads as wl
from oracle import frame_sets as fs


def test_generation_is_deterministic_and_rounded_to_bf16():
    w = wl.lvsa_shaped().shrunk(H=2, Tq=3, Tk=3, P=20)
    a = wl.make_qkv(w)
    b = wl.make_qkv(w)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 2, 60, 128)
        assert torch.equal(x, y)
    # q, k, v and heads draw from different streams
    assert not torch.equal(a[0], a[1])
    assert not torch.equal(a[0][0, 0], a[0][0, 1])


def test_outlier_channels_are_scaled():
    w = wl.lvsa_shaped().shrunk(H=1, Tq=4, Tk=4, P=500)
    ch = wl.outlier_channels(w)
    assert len(ch) == 4
    q = wl.make_tensor(w, 0).float()[0, 0]
    std = q.std(dim=0)
    others = [d for d in range(w.D) if d not in ch]
    assert std[ch].min() > 6.0 and std[others].max() < 1.3


def test_head_subset_matches_full_tensor():
    w = wl.ar_chunk().shrunk(P=8)
    full = wl.make_tensor(w, 1)
    sub = wl.make_tensor(w, 1, heads=[3, 7])
    assert torch.equal(sub[0, 0], full[0, 3]) and torch.equal(sub[0, 1], full[0, 7])


def test_frame_set_sizes_of_each_workload():
    w = wl.tiny_f32()
    _, cnt = fs.build(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk)
    assert cnt[0, 0].tolist() == [1, 2, 3, 3]
    for s in range(6):
        w = wl.lvsa_shaped(s)
        _, cnt = fs.build(w.policies[:1], w.B, w.Tq, w.Tk, w.offset, w.chunk)
        assert (cnt == 21).all()
    w = wl.ar_chunk()
    sel = [[[list(range(8))] for _ in range(12)]]
    _, cnt = fs.build(w.policies, w.B, w.Tq, w.Tk, w.offset, w.chunk, selected=sel)
    assert cnt[0, :, 0].tolist() == [6] * 4 + [9] * 4 + [11] * 4
    w = wl.decomposable()
    sizes = {}
    for name, pols in w.branches.items():
        _, cnt = fs.build(pols, w.B, w.Tq, w.Tk, w.offset, w.chunk)
        sizes[name] = set(cnt.ravel().tolist())
    assert sizes == {"A": {4}, "B": {45}, "U": {49}}
    w = wl.long_video(3)
    _, cnt = fs.build(w.policies[:1], w.B, w.Tq, w.Tk, w.offset, w.chunk)
    assert (cnt == 33).all()


def test_rollout_chunks_grow_the_cache():
    w = wl.ar_rollout()
    shapes = [wl.rollout_chunk(w, i) for i in range(w.rollout["n_chunks"])]
    assert [s["cached"] for s in shapes] == list(range(3, 61, 3))
    assert shapes[-1]["candidates"] == 57 and shapes[0]["candidates"] == 0
    assert [s["dense_frame_pairs"] for s in shapes[:3]] == [9, 18, 27]
    # first chunk dense on every head; later memory heads keep k_i + 3 recent frames
    for h, p in enumerate(wl.rollout_policies(w, 0, 1)):
        _, cnt = fs.build([p], 1, 3, 3, 0, 3)
        assert (cnt == 3).all(), h
    pols = wl.rollout_policies(w, 7, 5)
    assert [p["topk"] for p in pols[8:]] == [5] * 4
    sel = [[[[0, 2, 4, 6, 8]]]]
    _, cnt = fs.build(pols[8:9], 1, 3, 24, 21, 3, sel)
    assert (cnt == 8).all()
