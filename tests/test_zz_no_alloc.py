"""The allocation-free top-k entry point (fsa_select_topk_frames_noalloc),
called through the C ABI, against the workspace entry point
(fsa_select_topk_frames) on the same inputs: frames and float64 scores equal
bit for bit, on two calls in a row (the second on a smaller input, so it runs
on scratch still holding the first call's sums), and inputs beyond the static
scratch are refused before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import frame_sparse_attention_amd as fsa
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _both(q, k, P, h0, h1, q_group, c0, c1, topk):
    """(frames, scores) from the workspace entry point and from the
    allocation-free one, each into its own pre-filled outputs."""
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    G = Nq // (q_group * P)
    ref_f, ref_s = fsa.select_topk_frames(q, k, P, h0, h1, q_group, c0, c1, topk,
                                          return_scores=True)
    out = torch.full((B, H, G, topk), -1, dtype=torch.int32, device=DEV)
    sc = torch.full((B, H, G, c1 - c0), float("nan"), dtype=torch.float64, device=DEV)
    st = fsa._lib.fsa_select_topk_frames_noalloc(
        q.data_ptr(), k.data_ptr(), fsa._dtype_code(q), B, H, Nq, Nk, D, P, h0, h1, q_group,
        c0, c1, topk, out.data_ptr(), sc.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, fsa.last_error()
    torch.cuda.synchronize()
    return ref_f, ref_s, out, sc


def _assert_same(ref_f, ref_s, out, sc, h0, h1, what):
    assert torch.equal(out, ref_f), what
    # scores of the selected heads equal bit for bit; other heads untouched (NaN)
    a = ref_s[:, h0:h1].cpu().numpy().view(np.int64)
    b = sc[:, h0:h1].cpu().numpy().view(np.int64)
    assert np.array_equal(a, b), what
    rest = torch.cat([sc[:, :h0], sc[:, h1:]], dim=1)
    assert torch.isnan(rest).all(), what
    _say(f"{what}: frames and scores equal")


def test_noalloc_matches_workspace_entry_point_twice():
    w = wl.ar_chunk()
    q, k, _ = wl.make_qkv(w)
    qd, kd = q.to(DEV), k.to(DEV)
    _say(f"{w.name}: memory heads 8-11, 57 candidates, top-8")
    _assert_same(*_both(qd, kd, w.P, 8, 12, 3, 0, 57, 8), 8, 12, "first call (AR chunk)")
    # second call: a smaller input, on scratch that still holds the first call's sums
    g = torch.Generator().manual_seed(21)
    P = 40
    q2 = torch.randn((1, 3, 2 * P, 64), generator=g).to(torch.bfloat16).to(DEV)
    k2 = torch.randn((1, 3, 20 * P, 64), generator=g).to(torch.bfloat16).to(DEV)
    _say("second call: H3 D64 P40, candidates 5..19, top-3")
    _assert_same(*_both(q2, k2, P, 1, 3, 1, 5, 19, 3), 1, 3, "second call (smaller)")


def test_noalloc_near_the_scratch_limit_and_beyond():
    # 24 heads x (126 + 126) pooled sums of 128 float64, plus one 64-row piece
    # per group and frame (128 float64 partials + 2 keys): 12.4 MB of the 16 MiB
    B, H, T, P, D = 1, 24, 126, 64, 128
    g = torch.Generator(device=DEV).manual_seed(22)
    q = torch.randn((B, H, T * P, D), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((B, H, T * P, D), generator=g, device=DEV).to(torch.bfloat16)
    _say("24 heads x 126 frames, top-16")
    _assert_same(*_both(q, k, P, 0, H, 1, 0, T, 16), 0, H, "large call")
    # a call whose pooled sums exceed the scratch is refused before any launch
    Nq = 4096 * P
    st = fsa._lib.fsa_select_topk_frames_noalloc(
        q.data_ptr(), k.data_ptr(), fsa.BF16, B, H, Nq, T * P, D, P, 0, H, 1, 0, T, 4,
        ctypes.c_void_p(16), None, torch.cuda.current_stream().cuda_stream)
    assert st == 4 and "scratch" in fsa.last_error()
