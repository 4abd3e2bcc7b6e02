"""The Python binding rejects tensors a device call cannot take -- host
tensors, tensors on different devices, wrong dtypes or shapes -- before any
library function runs, so no kernel is ever launched with a host pointer or a
short output buffer.  CPU only: the library is replaced by a stub that fails
if it is reached."""

import numpy as np
import pytest
import torch

import frame_sparse_attention_amd as fsa


@pytest.fixture
def no_library(monkeypatch):
    def unreachable():
        raise AssertionError("the library was called before the arguments were checked")
    monkeypatch.setattr(fsa, "_load", unreachable)


def _qkv(dtype=torch.bfloat16, B=1, H=2, T=3, P=8, D=64):
    return tuple(torch.zeros((B, H, T * P, D), dtype=dtype) for _ in range(3))


def _lists(B=1, H=2, T=3, cap=2):
    return torch.zeros((B, H, T, cap), dtype=torch.int32), torch.ones((B, H, T), dtype=torch.int32)


@pytest.mark.parametrize("call", [
    lambda q, k, v, i, c: fsa.sparse_frame_attn(q, k, v, i, c, 8),
    lambda q, k, v, i, c: fsa.sparse_frame_attn_prepared(q, k, torch.zeros(16, dtype=torch.uint8),
                                                         i, c, 8),
    lambda q, k, v, i, c: fsa.sparse_frame_attn_split(q, k, torch.zeros(16, dtype=torch.uint8),
                                                      i, c, 8, 2),
    lambda q, k, v, i, c: fsa.sparse_frame_attn_dual(q, k, torch.zeros(16, dtype=torch.uint8),
                                                     i, c, i, c, 8),
    lambda q, k, v, i, c: fsa.prepare_values(v),
    lambda q, k, v, i, c: fsa.select_topk_frames(q, k, 8, 0, 2, 1, 0, 2, 1),
    lambda q, k, v, i, c: fsa.select_hsa_blocks(q, k, 8, 4, 0, 2, 1, 1, 1),
    lambda q, k, v, i, c: fsa.rope_reencode(q, k, i[:, :, 0].contiguous(),
                                            c[:, :, 0].contiguous(), 8, 8),
    lambda q, k, v, i, c: fsa.merge_lse(q.float(), q.float()[..., 0].contiguous(), q.float(),
                                        q.float()[..., 0].contiguous()),
    lambda q, k, v, i, c: fsa.build_frame_sets([dict(kind=fsa.FULL)] * 2, 1, 3, 3,
                                               device="cpu"),
])
def test_host_tensors_are_rejected_before_the_library(no_library, call):
    q, k, v = _qkv()
    idx, cnt = _lists()
    with pytest.raises(ValueError, match="cpu|GPU"):
        call(q, k, v, idx, cnt)


class _FakeCuda:
    """Just enough of a tensor to pass the device check: the shape and dtype
    checks behind it are then exercised without a GPU."""

    def __init__(self, t, index=0):
        self._t = t
        self.device = torch.device("cuda", index)

    def __getattr__(self, name):
        return getattr(self._t, name)


def test_expect_checks_dtype_and_exact_shape():
    t = torch.zeros((2, 3), dtype=torch.int32)
    fsa._expect(t, "t", torch.int32, (2, 3))
    fsa._expect(None, "absent", torch.int32, (9,))
    with pytest.raises(TypeError, match="t must be torch.float32"):
        fsa._expect(t, "t", torch.float32)
    with pytest.raises(ValueError, match=r"shape \(2, 4\)"):
        fsa._expect(t, "t", torch.int32, (2, 4))


def test_on_gpu_device_rules(monkeypatch):
    a = _FakeCuda(torch.zeros(4))
    b = _FakeCuda(torch.zeros(4), index=1)
    monkeypatch.setattr(torch, "is_tensor", lambda x: True)
    assert fsa._on_gpu(a=a, none=None) == torch.device("cuda", 0)
    with pytest.raises(ValueError, match="b is on cuda:1"):
        fsa._on_gpu(a=a, b=b)
    with pytest.raises(ValueError, match="no GPU tensor"):
        fsa._on_gpu(x=None)
    nc = _FakeCuda(torch.zeros(4, 4).t())
    with pytest.raises(ValueError, match="contiguous"):
        fsa._on_gpu(nc=nc)


def test_list_and_output_shapes():
    B, H, T, P, D = 1, 2, 3, 8, 64
    q, k, _ = _qkv()
    assert fsa._qk_shapes(q, k) == (B, H, T * P, T * P, D)
    with pytest.raises(TypeError):
        fsa._qk_shapes(q, k.float())
    with pytest.raises(ValueError):
        fsa._qk_shapes(q, k[:, :1].contiguous())
    idx, cnt = _lists()
    assert fsa._lists(idx, cnt, B, H, T) == 2
    with pytest.raises(ValueError, match="cnt"):
        fsa._lists(idx, cnt[:, :, :2].contiguous(), B, H, T)
    with pytest.raises(TypeError, match="idx"):
        fsa._lists(idx.long(), cnt, B, H, T)
    with pytest.raises(ValueError):
        fsa._lists(idx, cnt, B, H, T + 1)
    bad_out = torch.zeros((B, H, T * P, D), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="out must be torch.float32"):
        fsa._outputs(torch.device("cpu"), B, H, T * P, D, bad_out, None)
    short_lse = torch.zeros((B, H, T * P - 1), dtype=torch.float32)
    with pytest.raises(ValueError, match="out_lse"):
        fsa._outputs(torch.device("cpu"), B, H, T * P, D, None, short_lse)
    with pytest.raises(ValueError):
        fsa._frames(25, 8)


def test_host_builder_checks_selected_shape(no_library):
    sel = np.zeros((1, 2, 5, 1), dtype=np.int32)
    with pytest.raises(ValueError, match="selected"):
        fsa.build_frame_sets_host([dict(kind=fsa.MEMORY, topk=1)] * 2, 1, 3, 3, 0, 3,
                                  selected=sel, cap=4)
