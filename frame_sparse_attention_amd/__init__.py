"""Python binding of libfsa (frame-block-sparse softmax attention on MI355X).

A thin ctypes layer over the C ABI declared in include/fsa.h: it checks that
every tensor handed to a device call is a contiguous tensor on the inputs' GPU
with the dtype and shape the call expects (before anything is launched),
allocates outputs and workspaces with torch on that device, passes raw
pointers and torch's current HIP stream, and turns a non-OK status into
FsaError.  Every computation happens in the library's HIP
kernels; there is no fallback.  The first library call raises ImportError
when libfsa.so has not been built (python -m frame_sparse_attention_amd.build);
the library is loaded lazily so that the build script in this package can
run before it exists.

Functions (same names as the C entry points, without the fsa_ prefix):
  frame_set_capacity, build_frame_sets, build_frame_sets_host,
  validate_frame_sets, select_topk_frames, sparse_frame_attn, prepare_values,
  sparse_frame_attn_prepared, sparse_frame_attn_dual, merge_lse,
  plus the workspace-size queries, abi_version and last_error.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfsa.so")

FULL, LVSA, SINK_WINDOW, MEMORY, RANGE = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
MAX_HEADS = 64
MAX_CAP = 1024

STATUS_NAMES = {0: "FSA_OK", 1: "FSA_E_ARG", 2: "FSA_E_SHAPE", 3: "FSA_E_DTYPE",
                4: "FSA_E_CAPACITY", 5: "FSA_E_LIST", 6: "FSA_E_HIP"}


class FsaError(RuntimeError):
    """A libfsa call returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class HeadPolicy(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("kind", "n_sink", "window", "budget", "t_per", "step", "topk", "n_recent",
                 "lo", "hi")]


_i32, _i64, _f32, _sz, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t,
                              ctypes.c_void_p)
_pi32 = ctypes.POINTER(ctypes.c_int32)
_psz = ctypes.POINTER(ctypes.c_size_t)
_ppol = ctypes.POINTER(HeadPolicy)

_SIGS = {
    "fsa_abi_version": (_i32, []),
    "fsa_last_error": (ctypes.c_char_p, []),
    "fsa_frame_set_capacity": (_i32, [_i32, _ppol, _i32, _i32, _i32, _i32, _pi32]),
    "fsa_build_frame_sets": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _ppol, _vp, _i32, _i32,
                                    _vp, _vp, _vp]),
    "fsa_build_frame_sets_host": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _ppol, _vp, _i32,
                                         _i32, _vp, _vp]),
    "fsa_validate_frame_sets": (_i32, [_i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "fsa_select_topk_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                              _psz]),
    "fsa_select_topk_frames": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "fsa_select_topk_frames_noalloc": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                              _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp,
                                              _vp, _vp]),
    "fsa_select_hsa_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                             _i32, _i32, _i32, _i32, _psz]),
    "fsa_select_hsa_blocks": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                     _vp, _sz, _vp]),
    "fsa_cag_schedule": (_i32, [_i32, _vp, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                _vp, _vp, _vp, _vp]),
    "fsa_rope_reencode": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                 _i32, _i32, _i32, ctypes.c_double, _vp, _vp, _vp]),
    "fsa_sparse_frame_attn_workspace_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _psz]),
    "fsa_sparse_frame_attn": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _vp, _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "fsa_prepare_values": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "fsa_sparse_frame_attn_prepared": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                              _i32, _vp, _vp, _i32, _f32, _vp, _vp, _sz, _vp]),
    "fsa_attn_split_plan": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _pi32, _psz]),
    "fsa_sparse_frame_attn_prepared_split": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                    _i32, _i32, _vp, _vp, _i32, _f32, _i32, _vp,
                                                    _vp, _sz, _vp, _sz, _vp]),
    "fsa_sparse_frame_attn_dual_prepared": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                   _i32, _i32, _vp, _vp, _i32, _vp, _vp, _i32,
                                                   _f32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "fsa_merge_lse": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp]),
}
EXPORTED = tuple(_SIGS)
_LIB = None


def _load() -> ctypes.CDLL:
    """The loaded libfsa.so (loaded on first use, so that the build script in
    this package can run before the library exists).  Raises ImportError if
    it has not been built: there is no fallback."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m frame_sparse_attention_amd.build` (needs ROCm hipcc)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def __getattr__(name):
    if name == "_lib":
        return _load()
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


def abi_version() -> int:
    return int(_load().fsa_abi_version())


def last_error() -> str:
    return _load().fsa_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise FsaError(status, last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _policies(policies) -> ctypes.Array:
    arr = (HeadPolicy * max(1, len(policies)))()
    for i, p in enumerate(policies):
        for name, _ in HeadPolicy._fields_:
            setattr(arr[i], name, int(p.get(name, 0 if name != "t_per" else 1)))
    return arr


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _on_gpu(**named) -> torch.device:
    """Checks the tensors handed to a device call: each one given (None is
    skipped) must be a contiguous torch tensor on one and the same GPU.
    Returns that device.  Raises before any pointer reaches a kernel."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not torch.is_tensor(t):
            raise TypeError(f"{name} must be a torch tensor, not {type(t).__name__}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} is on {t.device}: the kernels read and write GPU memory "
                             "only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if dev is None:
        raise ValueError("no GPU tensor given")
    return dev


def _expect(t, name: str, dtype=None, shape=None) -> None:
    """Dtype and exact shape of a tensor (None: not given, nothing to check)."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _qk_shapes(q: torch.Tensor, k: torch.Tensor):
    """(B, H, Nq, Nk, D) of q [B,H,Nq,D] and k [B,H,Nk,D] of one dtype."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, D]")
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    _expect(k, "k", q.dtype, (B, H, Nk, D))
    _dtype_code(q)
    return B, H, Nq, Nk, D


def _lists(idx, cnt, B: int, H: int, rows: int, name: str = "idx"):
    """Frame lists idx int32 [B, H, rows, cap] and cnt int32 [B, H, rows]; returns cap."""
    if idx.dim() != 4:
        raise ValueError(f"{name} must be [B, H, {rows}, cap]")
    _expect(idx, name, torch.int32, (B, H, rows, idx.shape[3]))
    _expect(cnt, "cnt" if name == "idx" else name.replace("idx", "cnt"), torch.int32,
            (B, H, rows))
    return idx.shape[3]


def _outputs(dev, B: int, H: int, Nq: int, D: int, out, out_lse):
    """O float32 [B,H,Nq,D] and LSE float32 [B,H,Nq]: the given ones (checked) or new."""
    _expect(out, "out", torch.float32, (B, H, Nq, D))
    _expect(out_lse, "out_lse", torch.float32, (B, H, Nq))
    o = out if out is not None else torch.empty((B, H, Nq, D), dtype=torch.float32, device=dev)
    lse = out_lse if out_lse is not None else torch.empty((B, H, Nq), dtype=torch.float32,
                                                          device=dev)
    return o, lse


def _frames(N: int, P: int) -> int:
    if P <= 0 or N % P:
        raise ValueError(f"N={N} is not a positive multiple of P={P}")
    return N // P


# ----------------------------------------------------------------------------- frame sets
def frame_set_capacity(policies, Tq: int, Tk: int, offset: int = 0, chunk: int = 1) -> int:
    """Smallest cap that holds every frame set the policies can produce."""
    out = ctypes.c_int32(0)
    _check(_load().fsa_frame_set_capacity(len(policies), _policies(policies), Tq, Tk, offset,
                                          chunk, ctypes.byref(out)))
    return out.value


def build_frame_sets(policies, B: int, Tq: int, Tk: int, offset: int = 0, chunk: int = 1,
                     selected: torch.Tensor | None = None, cap: int | None = None,
                     device="cuda"):
    """Frame sets of every (b, h, tq) on the device: (idx [B,H,Tq,cap], cnt [B,H,Tq]) int32.

    selected: device int32 [B, H, Tq // chunk, k] frames chosen per query group
    (read for MEMORY heads only)."""
    H = len(policies)
    device = torch.device(device)
    if device.type != "cuda":
        raise ValueError(f"device {device}: frame sets are built by a GPU kernel "
                         "(build_frame_sets_host builds them on the CPU)")
    if cap is None:
        cap = frame_set_capacity(policies, Tq, Tk, offset, chunk)
    topk_k = 0
    if selected is not None:
        if selected.dim() != 4 or chunk <= 0:
            raise ValueError("selected must be int32 [B, H, Tq // chunk, k]")
        device = _on_gpu(selected=selected)
        _expect(selected, "selected", torch.int32, (B, H, Tq // chunk, selected.shape[3]))
        topk_k = selected.shape[3]
    idx = torch.empty((B, H, Tq, cap), dtype=torch.int32, device=device)
    cnt = torch.empty((B, H, Tq), dtype=torch.int32, device=device)
    _check(_load().fsa_build_frame_sets(B, H, Tq, Tk, offset, chunk, _policies(policies),
                                        _ptr(selected), topk_k, cap, _ptr(idx), _ptr(cnt),
                                        _stream(idx.device)))
    return idx, cnt


def build_frame_sets_host(policies, B: int, Tq: int, Tk: int, offset: int = 0, chunk: int = 1,
                          selected: np.ndarray | None = None, cap: int | None = None):
    """The same construction on host arrays (numpy int32)."""
    H = len(policies)
    if cap is None:
        cap = frame_set_capacity(policies, Tq, Tk, offset, chunk)
    idx = np.empty((B, H, Tq, cap), dtype=np.int32)
    cnt = np.empty((B, H, Tq), dtype=np.int32)
    topk_k = 0
    if selected is not None:
        if torch.is_tensor(selected):
            selected = selected.cpu().numpy()
        selected = np.ascontiguousarray(selected, dtype=np.int32)
        if selected.ndim != 4 or chunk <= 0 or selected.shape[:3] != (B, H, Tq // chunk):
            raise ValueError("selected must be int32 [B, H, Tq // chunk, k]")
        topk_k = selected.shape[3]
    _check(_load().fsa_build_frame_sets_host(B, H, Tq, Tk, offset, chunk, _policies(policies),
                                             _ptr(selected), topk_k, cap, _ptr(idx), _ptr(cnt)))
    return idx, cnt


def validate_frame_sets(idx, cnt, Tk: int) -> None:
    """Raises FsaError (FSA_E_LIST) unless every list is sorted, unique and in range."""
    idx = np.ascontiguousarray(idx.cpu().numpy() if torch.is_tensor(idx) else idx, dtype=np.int32)
    cnt = np.ascontiguousarray(cnt.cpu().numpy() if torch.is_tensor(cnt) else cnt, dtype=np.int32)
    if idx.ndim != 4 or cnt.shape != idx.shape[:3]:
        raise ValueError("idx must be [B, H, Tq, cap] and cnt [B, H, Tq]")
    B, H, Tq, cap = idx.shape
    _check(_load().fsa_validate_frame_sets(B, H, Tq, Tk, cap, _ptr(idx), _ptr(cnt)))


# ----------------------------------------------------------------------------- top-k
def select_topk_workspace_size(B: int, H: int, Nq: int, D: int, P: int, q_group: int,
                               cand_begin: int, cand_end: int) -> int:
    nbytes = ctypes.c_size_t(0)
    _check(_load().fsa_select_topk_workspace_size(B, H, Nq, D, P, q_group, cand_begin, cand_end,
                                                  ctypes.byref(nbytes)))
    return nbytes.value


def _topk_outputs(dev, B, H, G, topk, F, out, return_scores):
    _expect(out, "out", torch.int32, (B, H, G, topk))
    if out is None:
        out = torch.full((B, H, G, topk), -1, dtype=torch.int32, device=dev)
    scores = None
    if return_scores:
        scores = torch.full((B, H, G, F), float("nan"), dtype=torch.float64, device=dev)
    return out, scores


def select_topk_frames(q: torch.Tensor, k: torch.Tensor, P: int, h_begin: int, h_end: int,
                       q_group: int, cand_begin: int, cand_end: int, topk: int,
                       return_scores: bool = False, out: torch.Tensor | None = None):
    """Top-k frames by pooled Q.K per (b, h in [h_begin, h_end), query group).

    Returns int32 [B, H, G, topk] (rows of other heads are -1, or left as in
    `out`), and float64 scores [B, H, G, cand_end - cand_begin] when asked."""
    dev = _on_gpu(q=q, k=k, out=out)
    B, H, Nq, Nk, D = _qk_shapes(q, k)
    G = Nq // (q_group * P) if q_group * P > 0 else 0
    out, scores = _topk_outputs(dev, B, H, G, topk, cand_end - cand_begin, out, return_scores)
    nbytes = select_topk_workspace_size(B, H, Nq, D, P, q_group, cand_begin, cand_end)
    ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device=dev)
    _check(_load().fsa_select_topk_frames(_ptr(q), _ptr(k), _dtype_code(q), B, H, Nq, Nk, D, P,
                                          h_begin, h_end, q_group, cand_begin, cand_end, topk,
                                          _ptr(out), _ptr(scores), _ptr(ws), nbytes,
                                          _stream(dev)))
    return (out, scores) if return_scores else out


NOALLOC_SCRATCH_BYTES = 16 << 20


def select_topk_frames_noalloc(q: torch.Tensor, k: torch.Tensor, P: int, h_begin: int,
                               h_end: int, q_group: int, cand_begin: int, cand_end: int,
                               topk: int, out: torch.Tensor, scores: torch.Tensor | None = None):
    """select_topk_frames through the allocation-free entry point: the caller
    passes the output (int32 [B, H, G, topk], and optionally float64 scores
    [B, H, G, cand_end - cand_begin]); the pooled sums use the library's
    static device scratch (at most NOALLOC_SCRATCH_BYTES), and nothing is
    allocated, here or in the library.  Returns out."""
    dev = _on_gpu(q=q, k=k, out=out, scores=scores)
    B, H, Nq, Nk, D = _qk_shapes(q, k)
    G = Nq // (q_group * P) if q_group * P > 0 else 0
    _expect(out, "out", torch.int32, (B, H, G, topk))
    _expect(scores, "scores", torch.float64, (B, H, G, cand_end - cand_begin))
    _check(_load().fsa_select_topk_frames_noalloc(
        _ptr(q), _ptr(k), _dtype_code(q), B, H, Nq, Nk, D, P, h_begin, h_end, q_group,
        cand_begin, cand_end, topk, _ptr(out), _ptr(scores), _stream(dev)))
    return out


def select_hsa_blocks(q: torch.Tensor, k: torch.Tensor, P: int, block: int, h_begin: int,
                      h_end: int, n_recent: int, topk_frames: int, topk_blocks: int,
                      offset: int = 0, chunk: int = 1, cap: int | None = None,
                      idx: torch.Tensor | None = None, cnt: torch.Tensor | None = None):
    """Two-level (frame, then block) selection for heads [h_begin, h_end).

    Writes block-unit lists (block index = frame * (P // block) + block in
    frame) into idx [B, H, Nq // block, cap] and cnt [B, H, Nq // block]
    (allocated with -1 / 0 when not given; rows of other heads are left as
    they are) and returns (idx, cnt).  Attend with P = block."""
    dev = _on_gpu(q=q, k=k, idx=idx, cnt=cnt)
    B, H, Nq, Nk, D = _qk_shapes(q, k)
    if block <= 0:
        raise ValueError("block must be positive")
    nb = P // block if P % block == 0 else 0
    if cap is None:
        cap = topk_blocks + n_recent * nb if idx is None else idx.shape[3]
    G = Nq // block
    if idx is None:
        idx = torch.full((B, H, G, cap), -1, dtype=torch.int32, device=dev)
    if cnt is None:
        cnt = torch.zeros((B, H, G), dtype=torch.int32, device=dev)
    _expect(idx, "idx", torch.int32, (B, H, G, cap))
    _expect(cnt, "cnt", torch.int32, (B, H, G))
    nbytes = ctypes.c_size_t(0)
    _check(_load().fsa_select_hsa_workspace_size(B, H, Nq, Nk, D, P, block, offset, chunk,
                                                 h_begin, h_end, n_recent, ctypes.byref(nbytes)))
    ws = torch.empty(max(1, nbytes.value), dtype=torch.uint8, device=dev)
    _check(_load().fsa_select_hsa_blocks(_ptr(q), _ptr(k), _dtype_code(q), B, H, Nq, Nk, D, P,
                                         block, offset, chunk, h_begin, h_end, n_recent,
                                         topk_frames, topk_blocks, cap, _ptr(idx), _ptr(cnt),
                                         _ptr(ws), nbytes.value, _stream(dev)))
    return idx, cnt


def cag_schedule(cost, s_target: float, s_base: float, s_max: float, candidates=None):
    """Per-chunk sparsity s_i (chunk 0 dense, later chunks sparser) matching the
    total cost to a target sparsity; returns (sparsity float64 array, budgets
    int32 array or None, beta).  Host only."""
    cost = np.ascontiguousarray(cost, dtype=np.float64)
    n = cost.shape[0]
    sp = np.empty(n, dtype=np.float64)
    bud = None
    cand = None
    if candidates is not None:
        cand = np.ascontiguousarray(candidates, dtype=np.int32)
        if cand.shape != (n,):
            raise ValueError("candidates must have one entry per chunk")
        bud = np.empty(n, dtype=np.int32)
    beta = ctypes.c_double(0.0)
    _check(_load().fsa_cag_schedule(n, _ptr(cost), float(s_target), float(s_base), float(s_max),
                                    _ptr(cand), _ptr(sp), _ptr(bud), ctypes.byref(beta)))
    return sp, bud, beta.value


def rope_reencode(q: torch.Tensor, k: torch.Tensor, idx: torch.Tensor, cnt: torch.Tensor,
                  P: int, rot: int, base: float = 10000.0, offset: int = 0,
                  q_out: torch.Tensor | None = None, k_out: torch.Tensor | None = None):
    """Per-head frame-level rotary re-encoding for one frame set per (b, h):
    idx int32 [B, H, cap], cnt int32 [B, H].  Returns (q_out, k_out); q_out has
    every row written, k_out only the rows of listed frames (a fresh k_out
    starts as a copy of k).  Either output may be its input (in place)."""
    _on_gpu(q=q, k=k, idx=idx, cnt=cnt, q_out=q_out, k_out=k_out)
    B, H, Nq, Nk, D = _qk_shapes(q, k)
    if idx.dim() != 3:
        raise ValueError("idx must be [B, H, cap] and cnt [B, H]")
    _expect(idx, "idx", torch.int32, (B, H, idx.shape[2]))
    _expect(cnt, "cnt", torch.int32, (B, H))
    _expect(q_out, "q_out", q.dtype, q.shape)
    _expect(k_out, "k_out", k.dtype, k.shape)
    if q_out is None:
        q_out = torch.empty_like(q)
    if k_out is None:
        k_out = k.clone()
    _check(_load().fsa_rope_reencode(_ptr(q), _ptr(k), _dtype_code(q), B, H, Nq, Nk, D, P,
                                     _ptr(idx), _ptr(cnt), idx.shape[2], offset, rot,
                                     float(base), _ptr(q_out), _ptr(k_out), _stream(q.device)))
    return q_out, k_out


# ----------------------------------------------------------------------------- attention
def sparse_frame_attn_workspace_size(dtype, B: int, H: int, Nk: int, D: int) -> int:
    code = dtype if isinstance(dtype, int) else (BF16 if dtype == torch.bfloat16 else F32)
    out = ctypes.c_size_t(0)
    _check(_load().fsa_sparse_frame_attn_workspace_size(code, B, H, Nk, D, ctypes.byref(out)))
    return out.value


def sparse_frame_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                      cnt: torch.Tensor, P: int, scale: float | None = None,
                      workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                      out_lse: torch.Tensor | None = None):
    """Frame-sparse attention: returns (O float32 [B,H,Nq,D], LSE float32 [B,H,Nq])."""
    dev = _on_gpu(q=q, k=k, v=v, idx=idx, cnt=cnt, workspace=workspace, out=out,
                  out_lse=out_lse)
    B, H, Nq, Nk, D = _qk_shapes(q, k)
    _expect(v, "v", q.dtype, (B, H, Nk, D))
    cap = _lists(idx, cnt, B, H, _frames(Nq, P))
    dt = _dtype_code(q)
    o, lse = _outputs(dev, B, H, Nq, D, out, out_lse)
    need = sparse_frame_attn_workspace_size(dt, B, H, Nk, D)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(_load().fsa_sparse_frame_attn(_ptr(q), _ptr(k), _ptr(v), dt, B, H, Nq, Nk, D, P,
                                         _ptr(idx), _ptr(cnt), cap,
                                         float(scale) if scale is not None else 0.0, _ptr(o),
                                         _ptr(lse), _ptr(workspace), _nbytes(workspace),
                                         _stream(dev)))
    return o, lse


def prepare_values(v: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 V [B,H,Nk,D] -> the float16 key-chunked transposed copy the attention
    reads (a uint8 buffer of sparse_frame_attn_workspace_size bytes)."""
    dev = _on_gpu(v=v, out=out)
    if v.dim() != 4:
        raise ValueError("v must be [B, H, Nk, D]")
    B, H, Nk, D = v.shape
    need = sparse_frame_attn_workspace_size(_dtype_code(v), B, H, Nk, D)
    if out is None:
        out = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
    _check(_load().fsa_prepare_values(_ptr(v), _dtype_code(v), B, H, Nk, D, _ptr(out),
                                      _nbytes(out), _stream(dev)))
    return out


def sparse_frame_attn_prepared(q: torch.Tensor, k: torch.Tensor, prepared: torch.Tensor,
                               idx: torch.Tensor, cnt: torch.Tensor, P: int,
                               scale: float | None = None, out: torch.Tensor | None = None,
                               out_lse: torch.Tensor | None = None):
    """Attention reading values already converted by prepare_values."""
    dev = _on_gpu(q=q, k=k, prepared=prepared, idx=idx, cnt=cnt, out=out, out_lse=out_lse)
    B, H, Nq, Nk, D = _qk_shapes(q, k)
    cap = _lists(idx, cnt, B, H, _frames(Nq, P))
    o, lse = _outputs(dev, B, H, Nq, D, out, out_lse)
    _check(_load().fsa_sparse_frame_attn_prepared(
        _ptr(q), _ptr(k), _ptr(prepared), _dtype_code(q), B, H, Nq, Nk, D, P, _ptr(idx),
        _ptr(cnt), cap, float(scale) if scale is not None else 0.0, _ptr(o), _ptr(lse),
        _nbytes(prepared), _stream(dev)))
    return o, lse


def attn_split_plan(B: int, H: int, Nq: int, D: int, P: int, splits: int = 0):
    """(split count, workspace bytes) for the split attention; splits <= 0
    lets the library choose from the grid size."""
    n = ctypes.c_int32(0)
    nbytes = ctypes.c_size_t(0)
    _check(_load().fsa_attn_split_plan(B, H, Nq, D, P, splits, ctypes.byref(n),
                                       ctypes.byref(nbytes)))
    return n.value, nbytes.value


def sparse_frame_attn_split(q: torch.Tensor, k: torch.Tensor, prepared: torch.Tensor,
                            idx: torch.Tensor, cnt: torch.Tensor, P: int, splits: int = 0,
                            scale: float | None = None, workspace: torch.Tensor | None = None,
                            out: torch.Tensor | None = None, out_lse: torch.Tensor | None = None):
    """Attention with each frame list cut into `splits` parts (0: the library's
    choice for the grid) whose partials are merged through their LSE."""
    dev = _on_gpu(q=q, k=k, prepared=prepared, idx=idx, cnt=cnt, workspace=workspace, out=out,
                  out_lse=out_lse)
    B, H, Nq, Nk, D = _qk_shapes(q, k)
    cap = _lists(idx, cnt, B, H, _frames(Nq, P))
    S, nbytes = attn_split_plan(B, H, Nq, D, P, splits)
    o, lse = _outputs(dev, B, H, Nq, D, out, out_lse)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(_load().fsa_sparse_frame_attn_prepared_split(
        _ptr(q), _ptr(k), _ptr(prepared), _dtype_code(q), B, H, Nq, Nk, D, P, _ptr(idx),
        _ptr(cnt), cap, 0.0 if scale is None else float(scale), S, _ptr(o), _ptr(lse),
        _nbytes(prepared), _ptr(workspace), _nbytes(workspace), _stream(dev)))
    return o, lse


def sparse_frame_attn_dual(q: torch.Tensor, k: torch.Tensor, prepared: torch.Tensor,
                           idx_a: torch.Tensor, cnt_a: torch.Tensor, idx_b: torch.Tensor,
                           cnt_b: torch.Tensor, P: int, scale: float | None = None):
    """One pass over frame lists A then B: returns (O_A, LSE_A, O_AB, LSE_AB),
    attention over A alone and over A and B together (disjoint lists)."""
    dev = _on_gpu(q=q, k=k, prepared=prepared, idx_a=idx_a, cnt_a=cnt_a, idx_b=idx_b,
                  cnt_b=cnt_b)
    B, H, Nq, Nk, D = _qk_shapes(q, k)
    Tq = _frames(Nq, P)
    cap_a = _lists(idx_a, cnt_a, B, H, Tq, "idx_a")
    cap_b = _lists(idx_b, cnt_b, B, H, Tq, "idx_b")
    outs = [torch.empty((B, H, Nq, D), dtype=torch.float32, device=dev) for _ in range(2)]
    lses = [torch.empty((B, H, Nq), dtype=torch.float32, device=dev) for _ in range(2)]
    _check(_load().fsa_sparse_frame_attn_dual_prepared(
        _ptr(q), _ptr(k), _ptr(prepared), _dtype_code(q), B, H, Nq, Nk, D, P, _ptr(idx_a),
        _ptr(cnt_a), cap_a, _ptr(idx_b), _ptr(cnt_b), cap_b,
        float(scale) if scale is not None else 0.0, _ptr(outs[0]), _ptr(lses[0]), _ptr(outs[1]),
        _ptr(lses[1]), _nbytes(prepared), _stream(dev)))
    return outs[0], lses[0], outs[1], lses[1]


def merge_lse(o1: torch.Tensor, lse1: torch.Tensor, o2: torch.Tensor, lse2: torch.Tensor,
              out: torch.Tensor | None = None, out_lse: torch.Tensor | None = None):
    """Exact LSE merge of two partial attentions (float32); returns (O, LSE)."""
    _on_gpu(o1=o1, lse1=lse1, o2=o2, lse2=lse2, out=out, out_lse=out_lse)
    if o1.dim() < 1 or o1.shape[:-1] != lse1.shape:
        raise ValueError("o1 must be [..., D] and lse1 the matching [...]")
    _expect(o1, "o1", torch.float32)
    _expect(lse1, "lse1", torch.float32)
    _expect(o2, "o2", torch.float32, o1.shape)
    _expect(lse2, "lse2", torch.float32, lse1.shape)
    _expect(out, "out", torch.float32, o1.shape)
    _expect(out_lse, "out_lse", torch.float32, lse1.shape)
    D = o1.shape[-1]
    rows = lse1.numel()
    o = out if out is not None else torch.empty_like(o1)
    lse = out_lse if out_lse is not None else torch.empty_like(lse1)
    _check(_load().fsa_merge_lse(_ptr(o1), _ptr(lse1), _ptr(o2), _ptr(lse2), rows, D, _ptr(o),
                                 _ptr(lse), _stream(o1.device)))
    return o, lse
