"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and every host-side argument check returns the documented status
and message before anything is launched."""

import ctypes
import os
import re

import pytest

import frame_sparse_attention_amd as fsa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "fsa.h")
lib = fsa._lib

BAD = ctypes.c_void_p(16)   # never dereferenced: validation fails first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 21, names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(fsa.EXPORTED)


def test_abi_version_and_error_text():
    assert fsa.abi_version() == 1
    st = lib.fsa_merge_lse(BAD, BAD, BAD, BAD, -1, 4, BAD, BAD, None)
    assert st == 1 and "rows" in fsa.last_error()
    # a later successful call clears the text
    assert lib.fsa_merge_lse(BAD, BAD, BAD, BAD, 0, 4, BAD, BAD, None) == 0
    assert fsa.last_error() == ""


def _attn(**kw):
    a = dict(q=BAD, k=BAD, v=BAD, dt=1, B=1, H=2, Nq=64, Nk=64, D=128, P=16, idx=BAD, cnt=BAD,
             cap=4, scale=0.0, o=BAD, lse=BAD, ws=BAD, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.fsa_sparse_frame_attn(a["q"], a["k"], a["v"], a["dt"], a["B"], a["H"], a["Nq"],
                                     a["Nk"], a["D"], a["P"], a["idx"], a["cnt"], a["cap"],
                                     a["scale"], a["o"], a["lse"], a["ws"], a["ws_bytes"],
                                     a["stream"])


@pytest.mark.parametrize("kw,status,text", [
    (dict(dt=7), 3, "dtype"),
    (dict(D=96), 3, "head_dim"),
    (dict(B=-1), 1, "negative"),
    (dict(P=0), 2, "P=0"),
    (dict(Nq=60), 2, "Nq=60"),
    (dict(Nk=70), 2, "Nk=70"),
    (dict(cap=0), 4, "cap=0"),
    (dict(cap=5000), 4, "cap=5000"),
    (dict(q=None), 1, "null"),
    (dict(k=None), 1, "k or v"),
    (dict(ws_bytes=10), 4, "workspace"),
    (dict(ws=None), 1, "workspace is NULL"),
    (dict(scale=float("inf")), 1, "scale"),
    (dict(q=ctypes.c_void_p(24)), 1, "16-byte aligned"),
    (dict(ws=ctypes.c_void_p(40)), 1, "16-byte aligned"),
])
def test_attention_argument_errors(kw, status, text):
    assert _attn(**kw) == status
    assert text in fsa.last_error()


def test_attention_empty_problem_is_ok_without_gpu():
    assert _attn(Nq=0) == 0
    assert _attn(B=0) == 0


def test_prepared_entry_points_argument_errors():
    assert lib.fsa_prepare_values(BAD, 0, 1, 2, 64, 128, BAD, 1 << 40, None) == 3
    assert "bf16 only" in fsa.last_error()
    assert lib.fsa_prepare_values(BAD, 1, 1, 2, 64, 128, BAD, 100, None) == 4
    assert "prepared buffer" in fsa.last_error()
    assert lib.fsa_prepare_values(BAD, 1, 1, 2, 0, 128, None, 0, None) == 0
    st = lib.fsa_sparse_frame_attn_prepared(BAD, BAD, BAD, 0, 1, 2, 64, 64, 128, 16, BAD, BAD, 4,
                                            0.0, BAD, BAD, 1 << 40, None)
    assert st == 3 and "bf16 only" in fsa.last_error()
    st = lib.fsa_sparse_frame_attn_prepared(BAD, BAD, BAD, 1, 1, 2, 64, 64, 128, 16, BAD, BAD, 4,
                                            0.0, BAD, BAD, 8, None)
    assert st == 4 and "prepared buffer" in fsa.last_error()


def test_workspace_size_queries():
    n = ctypes.c_size_t()
    assert lib.fsa_sparse_frame_attn_workspace_size(1, 1, 12, 65520, 128, ctypes.byref(n)) == 0
    assert n.value == 12 * (65520 // 8) * 128 * 8 * 2
    assert lib.fsa_sparse_frame_attn_workspace_size(1, 1, 1, 13, 64, ctypes.byref(n)) == 0
    assert n.value == 2 * 64 * 8 * 2          # Nk rounded up to whole 8-key chunks
    assert lib.fsa_sparse_frame_attn_workspace_size(0, 1, 1, 13, 64, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.fsa_sparse_frame_attn_workspace_size(0, 1, 1, 13, 80, ctypes.byref(n)) == 3
    assert lib.fsa_select_topk_workspace_size(1, 12, 4680, 128, 1560, 3, 0, 57,
                                              ctypes.byref(n)) == 0
    # pooled sums of 12 query groups and 12 x 57 frames, then the pieces of at
    # most 128 rows (37 per 4680-row group, 13 per 1560-row frame): 128 float64
    # partial sums and 2 uint32 magnitude keys each; every array 256-byte aligned
    a = lambda x: -(-x // 256) * 256
    gp, fp = 12 * 37, 12 * 57 * 13
    assert n.value == (a(12 * 128 * 8) + a(12 * 57 * 128 * 8) + a(gp * 128 * 8) + a(gp * 8)
                       + a(fp * 128 * 8) + a(fp * 8))


def _topk(**kw):
    a = dict(q=BAD, kp=BAD, dt=1, B=1, H=12, Nq=4680, Nk=93600, D=128, P=1560, h0=8, h1=12, qg=3,
             c0=0, c1=57, k=8, out=BAD, scores=None, ws=BAD, ws_bytes=1 << 40)
    a.update(kw)
    return lib.fsa_select_topk_frames(a["q"], a["kp"], a["dt"], a["B"], a["H"], a["Nq"], a["Nk"],
                                      a["D"], a["P"], a["h0"], a["h1"], a["qg"], a["c0"], a["c1"],
                                      a["k"], a["out"], a["scores"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,text", [
    (dict(k=9, c1=8), 1, "exceeds"),
    (dict(k=0), 1, "topk=0"),
    (dict(k=65, c1=60), 1, "topk=65"),
    (dict(c1=61), 1, "exceed Tk"),
    (dict(c0=5, c1=5), 1, "empty"),
    (dict(h0=10, h1=13), 1, "head range"),
    (dict(qg=2), 2, "q_group"),
    (dict(dt=5), 3, "dtype"),
    (dict(ws_bytes=8), 4, "workspace"),
    (dict(out=None), 1, "null"),
])
def test_topk_argument_errors(kw, status, text):
    assert _topk(**kw) == status
    assert text in fsa.last_error()


def test_merge_argument_errors():
    assert lib.fsa_merge_lse(BAD, BAD, BAD, BAD, 5, 0, BAD, BAD, None) == 1
    assert "D=0" in fsa.last_error()
    assert lib.fsa_merge_lse(None, BAD, BAD, BAD, 5, 4, BAD, BAD, None) == 1
    assert "null" in fsa.last_error()


def test_build_frame_sets_argument_errors():
    pol = [dict(kind=fsa.LVSA, window=7, budget=21, t_per=6)]
    with pytest.raises(fsa.FsaError, match="cap"):
        fsa.build_frame_sets_host(pol, 1, 42, 42, cap=20)
    with pytest.raises(fsa.FsaError, match="t_per"):
        fsa.build_frame_sets_host([dict(kind=fsa.LVSA, window=7, budget=21, t_per=0)], 1, 4, 4)
    with pytest.raises(fsa.FsaError, match="chunk"):
        fsa.build_frame_sets_host([dict(kind=fsa.FULL)], 1, 4, 4, chunk=3)
    with pytest.raises(fsa.FsaError, match="MEMORY"):
        fsa.build_frame_sets_host([dict(kind=fsa.MEMORY, topk=2, n_recent=1)], 1, 3, 10,
                                  offset=7, chunk=3)
    with pytest.raises(fsa.FsaError, match="kind"):
        fsa.build_frame_sets_host([dict(kind=9)], 1, 4, 4)
    with pytest.raises(fsa.FsaError, match="exceed"):
        fsa.build_frame_sets_host([dict(kind=fsa.SINK_WINDOW, window=2)], 1, 4, 4, offset=1)
    with pytest.raises(fsa.FsaError, match="H=65"):
        fsa.build_frame_sets_host([dict(kind=fsa.FULL)] * 65, 1, 4, 4)


def test_missing_library_fails_loudly_on_first_call(monkeypatch, tmp_path):
    # the binding has no fallback: without libfsa.so the first call raises
    monkeypatch.setattr(fsa, "LIB_PATH", str(tmp_path / "libfsa.so"))
    monkeypatch.setattr(fsa, "_LIB", None)
    with pytest.raises(ImportError, match="libfsa.so is missing"):
        fsa.abi_version()


def test_build_module_imports_without_the_library():
    import importlib
    mod = importlib.import_module("frame_sparse_attention_amd.build")
    assert mod.ARCH == "gfx950" and "attn_bf16.hip" in mod.SOURCES


def _hsa(**kw):
    # the AR chunk with block-level memory heads: 3 query frames of 1560 tokens,
    # a 60-frame cache, blocks of 120 tokens (13 per frame)
    a = dict(q=BAD, k=BAD, dt=1, B=1, H=12, Nq=4680, Nk=93600, D=128, P=1560, block=120,
             offset=57, chunk=3, h_begin=8, h_end=12, n_recent=3, kf=8, kb=52, cap=91,
             idx=BAD, cnt=BAD, ws=BAD, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.fsa_select_hsa_blocks(a["q"], a["k"], a["dt"], a["B"], a["H"], a["Nq"], a["Nk"],
                                     a["D"], a["P"], a["block"], a["offset"], a["chunk"],
                                     a["h_begin"], a["h_end"], a["n_recent"], a["kf"], a["kb"],
                                     a["cap"], a["idx"], a["cnt"], a["ws"], a["ws_bytes"],
                                     a["stream"])


@pytest.mark.parametrize("kw,status,text", [
    (dict(dt=5), 3, "dtype"),
    (dict(D=300), 2, "D=300"),
    (dict(block=7), 2, "multiple of block"),
    (dict(Nq=4000), 2, "Nq=4000"),
    (dict(chunk=0), 1, "chunk=0"),
    (dict(offset=58), 1, "beyond"),
    (dict(n_recent=61), 1, "before KV frame 0"),
    (dict(n_recent=-1), 1, "n_recent=-1"),
    (dict(h_begin=9, h_end=8), 1, "head range"),
    (dict(kf=0), 1, "topk_frames=0"),
    (dict(kf=58), 1, "topk_frames=58"),
    (dict(kb=105), 1, "topk_blocks=105"),
    (dict(kb=-1), 1, "topk_blocks=-1"),
    (dict(cap=90), 4, "cap=90"),
    (dict(cap=2000, kb=52), 4, "cap=2000"),
    (dict(q=None), 1, "null"),
    (dict(ws_bytes=1000), 4, "workspace"),
])
def test_select_hsa_argument_checks(kw, status, text):
    assert _hsa(**kw) == status
    assert text in fsa.last_error()


def test_select_hsa_workspace_size_and_empty_calls():
    n = ctypes.c_size_t(0)
    assert lib.fsa_select_hsa_workspace_size(1, 12, 4680, 93600, 128, 1560, 120, 57, 3, 8, 12,
                                             3, ctypes.byref(n)) == 0
    # 4 heads x (39 query blocks + 57*13 key blocks + 57 frames) x 128 doubles of
    # sums, then one piece per 120-token block (39 + 741 per head): 128 float64
    # partial sums and 2 uint32 magnitude keys each; arrays 256-byte aligned
    a = lambda x: -(-x // 256) * 256
    qp, kp = 4 * 39, 4 * 57 * 13
    assert n.value == (a(qp * 1024) + a(kp * 1024) + a(4 * 57 * 1024) + a(qp * 1024) + a(qp * 8)
                       + a(kp * 1024) + a(kp * 8))
    # nothing to do: no heads, or no batch
    assert _hsa(h_begin=8, h_end=8) == 0
    assert _hsa(B=0) == 0


def _rope(**kw):
    a = dict(q=BAD, k=BAD, dt=1, B=1, H=12, Nq=4680, Nk=93600, D=128, P=1560, idx=BAD, cnt=BAD,
             cap=11, offset=57, rot=42, base=10000.0, qo=BAD, ko=BAD, stream=None)
    a.update(kw)
    return lib.fsa_rope_reencode(a["q"], a["k"], a["dt"], a["B"], a["H"], a["Nq"], a["Nk"],
                                 a["D"], a["P"], a["idx"], a["cnt"], a["cap"], a["offset"],
                                 a["rot"], a["base"], a["qo"], a["ko"], a["stream"])


@pytest.mark.parametrize("kw,status,text", [
    (dict(dt=2), 3, "dtype"),
    (dict(D=100), 2, "D=100"),
    (dict(D=264), 2, "D=264"),
    (dict(P=0), 2, "P=0"),
    (dict(Nk=93601), 2, "Nk=93601"),
    (dict(rot=43), 1, "rot=43"),
    (dict(rot=130), 1, "rot=130"),
    (dict(base=0.0), 1, "base"),
    (dict(base=float("inf")), 1, "base"),
    (dict(cap=0), 4, "cap=0"),
    (dict(offset=-1), 1, "q_kv_offset=-1"),
    (dict(ko=None), 1, "null"),
    (dict(qo=ctypes.c_void_p(24)), 1, "aligned"),
    (dict(H=-1), 1, "negative"),
])
def test_rope_argument_checks(kw, status, text):
    assert _rope(**kw) == status
    assert text in fsa.last_error()


def test_rope_nothing_to_do():
    assert _rope(B=0) == 0 and _rope(H=0) == 0


def test_split_plan():
    n = ctypes.c_int32(0)
    nb = ctypes.c_size_t(0)
    # 42 frames x 13 query tiles x 12 heads fill the chip: no split
    assert lib.fsa_attn_split_plan(1, 12, 65520, 128, 1560, 0, ctypes.byref(n),
                                   ctypes.byref(nb)) == 0
    assert n.value == 1 and nb.value == 0
    # a 3-frame chunk: 468 blocks fill the CUs -> one part
    assert lib.fsa_attn_split_plan(1, 12, 4680, 128, 1560, 0, ctypes.byref(n),
                                   ctypes.byref(nb)) == 0
    assert n.value == 1 and nb.value == 0
    # one 1560-token frame of 4 heads: 52 blocks -> 10 parts capped at 8
    assert lib.fsa_attn_split_plan(1, 4, 1560, 128, 1560, 0, ctypes.byref(n),
                                   ctypes.byref(nb)) == 0
    assert n.value == 8 and nb.value == 8 * 4 * 1560 * 129 * 4
    assert lib.fsa_attn_split_plan(1, 12, 4680, 128, 1560, 3, ctypes.byref(n),
                                   ctypes.byref(nb)) == 0
    assert n.value == 3
    assert lib.fsa_attn_split_plan(1, 12, 4680, 128, 1560, 17, ctypes.byref(n),
                                   ctypes.byref(nb)) == 1
    assert lib.fsa_attn_split_plan(1, 12, 4680, 96, 1560, 2, ctypes.byref(n),
                                   ctypes.byref(nb)) == 3


@pytest.mark.parametrize("splits,ws_bytes,status,text", [
    (0, 1 << 40, 1, "splits=0"),
    (17, 1 << 40, 1, "splits=17"),
    (4, 1000, 4, "workspace"),
])
def test_split_attention_argument_checks(splits, ws_bytes, status, text):
    st = lib.fsa_sparse_frame_attn_prepared_split(BAD, BAD, BAD, 1, 1, 2, 64, 64, 128, 16, BAD,
                                                  BAD, 4, 0.0, splits, BAD, BAD, 1 << 40, BAD,
                                                  ws_bytes, None)
    assert st == status and text in fsa.last_error()


def test_noalloc_topk_refuses_inputs_beyond_its_scratch_without_a_gpu():
    # 12 heads x (4096 + 57) pooled sums of 128 float64 alone are 51 MB > 16 MiB: FSA_E_CAPACITY
    # before the scratch address is looked up or anything is launched
    st = lib.fsa_select_topk_frames_noalloc(BAD, BAD, 1, 1, 12, 4096 * 16, 60 * 16, 128, 16,
                                            0, 12, 1, 0, 57, 8, BAD, None, None)
    assert st == 4 and "scratch" in fsa.last_error()
    assert fsa.NOALLOC_SCRATCH_BYTES == 16 << 20
    # argument errors come first, as in the workspace entry point
    st = lib.fsa_select_topk_frames_noalloc(BAD, BAD, 1, 1, 12, 4680, 93600, 128, 1560, 0, 12,
                                            3, 0, 57, 0, BAD, None, None)
    assert st == 1 and "topk" in fsa.last_error()
