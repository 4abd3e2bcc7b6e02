"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check.

This module only describes shapes and policies and draws seeded random inputs;
it holds none of the attention arithmetic, imports neither the library nor the
oracle, and both of those may be fed from it.

The pages measure on real video models (Wan 2.1 / 2.2, HunyuanVideo 1.5, Self
Forcing, LongLive, Krea) and quality suites (VBench, VQeval).  None of those is
available, so seeded Gaussian inputs of the same shapes stand in for them:
latent frames of P tokens (a 30x52 or 60x60 latent grid), 12 or 24 heads of
width 128, frame sets of the sizes the pages describe.

Recipe: for config seed c, tensor j in (q=0, k=1, v=2) and head h, a CPU
``torch.Generator`` seeded with ``c*1_000_003 + j*1009 + h`` draws float32
N(0, 1) values of shape [Ntokens, D]; optional outlier channels (chosen once per
config with seed c) are multiplied by a factor; bf16 configs then round to
nearest-even bfloat16.  The oracle receives the same bits widened exactly.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np
import torch

# policy kinds (integers shared by the frame-set descriptions below)
FULL, LVSA, SINK_WINDOW, MEMORY, RANGE = 0, 1, 2, 3, 4


def policy(kind, n_sink=0, window=0, budget=0, t_per=1, step=0, topk=0, n_recent=0,
           lo=0, hi=-1) -> dict:
    """One head's frame-set policy as a plain dict of integers."""
    return dict(kind=kind, n_sink=n_sink, window=window, budget=budget, t_per=t_per,
                step=step, topk=topk, n_recent=n_recent, lo=lo, hi=hi)


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    H: int
    D: int
    Tq: int
    Tk: int
    P: int
    dtype: str                     # "f32" or "bf16"
    policies: list                 # one dict per head
    offset: int = 0                # KV frame index of query frame 0
    chunk: int = 1                 # query frames sharing one frame set
    steps: int = 1                 # denoising steps (LVSA rotation)
    outliers: int = 0              # number of outlier channels
    outlier_scale: float = 8.0
    q_group: int = 1               # query frames pooled together (memory heads)
    branches: dict = field(default_factory=dict)   # extra named policy lists
    # two-level (frame, then block) selection for the MEMORY heads: tokens per
    # block and blocks kept per query block; 0 = frame-level lists only
    block: int = 0
    topk_blocks: int = 0
    # per-head frame-level rotary re-encoding of the assembled cache: rotated
    # leading channels (0 = none) and the frequency base
    rope_dims: int = 0
    rope_base: float = 10000.0
    # autoregressive rollout driven by the chunk-aware growth schedule: number
    # of chunks, schedule parameters (target sparsity, s_base, s_max) and the
    # memory heads' recent frames; empty = no rollout
    rollout: dict = field(default_factory=dict)

    @property
    def Nq(self) -> int:
        return self.Tq * self.P

    @property
    def Nk(self) -> int:
        return self.Tk * self.P

    def with_step(self, s: int) -> "Workload":
        """Same workload with every LVSA head moved to denoising step s."""
        pols = [dict(p, step=s) if p["kind"] == LVSA else dict(p) for p in self.policies]
        return dataclasses.replace(self, policies=pols)

    def shrunk(self, **kw) -> "Workload":
        """A copy with some sizes replaced (for oracle-sized parity runs)."""
        return dataclasses.replace(self, **kw)


def tiny_f32() -> Workload:
    """B=1, H=2, D=64, T=4 frames x P=16 tokens, fp32; A(t) = {0} ∪ {t-1, t}."""
    pol = policy(SINK_WINDOW, n_sink=1, window=2)
    return Workload("tiny_f32", 1, 1, 2, 64, 4, 4, 16, "f32", [pol, pol])


def lvsa_shaped(step: int = 0) -> Workload:
    """H=12, D=128, T=42 latent frames x 1560 tokens, bf16 with 4 outlier channels x8;
    LVSA budget C=21, window W=7, anchors every T_per=6 frames, steps s=0..5."""
    pol = policy(LVSA, window=7, budget=21, t_per=6, step=step)
    return Workload("lvsa_T42_P1560_H12", 2, 1, 12, 128, 42, 42, 1560, "bf16",
                    [dict(pol) for _ in range(12)], steps=6, outliers=4)


def ar_chunk() -> Workload:
    """Query chunk of 3 frames (4680 tokens) against a 60-frame KV cache, H=12;
    heads 0-3 local (last 6 frames), 4-7 anchor (frames 0-2 + last 6),
    8-11 memory (top-8 frames of 0..56 by pooled Q·K + the last 3)."""
    local = policy(SINK_WINDOW, n_sink=0, window=6)
    anchor = policy(SINK_WINDOW, n_sink=3, window=6)
    mem = policy(MEMORY, topk=8, n_recent=3)
    pols = [dict(local) for _ in range(4)] + [dict(anchor) for _ in range(4)] + \
        [dict(mem) for _ in range(4)]
    return Workload("ar_chunk_3x1560_cache60", 3, 1, 12, 128, 3, 60, 1560, "bf16", pols,
                    offset=57, chunk=3, q_group=3)


def ar_chunk_hsa() -> Workload:
    """The AR chunk workload (same tensors) with hierarchical selection on the
    memory heads: per 120-token query block, the 8 best of frames 0..56 by
    frame-pooled scores, then the 52 best 120-token blocks inside those frames
    by block-pooled scores, plus the last 3 frames whole.  Lists are in block
    units (13 blocks per 1560-token frame); heads 0-7 keep their frame windows
    written in blocks."""
    w = ar_chunk()
    return dataclasses.replace(w, name="ar_chunk_hsa_3x1560_cache60_blk120", block=120,
                               topk_blocks=52)


def ar_chunk_rope() -> Workload:
    """The AR chunk workload (same tensors and frame sets) with each head's
    assembled cache re-encoded: the first 42 of 128 channels (a third of the
    pairs, the temporal part) turn by the frame's rank in the head's set,
    frequencies 10000^(-2i/42)."""
    w = ar_chunk()
    return dataclasses.replace(w, name="ar_chunk_rope_3x1560_cache60_rot42", rope_dims=42)


def ar_rollout() -> Workload:
    """Autoregressive rollout of 20 chunks of 3 frames x 1560 tokens, H=12, D=128,
    into a KV cache that grows by one chunk per step up to the 60 frames of the
    AR chunk workload.  Chunk i's queries are frames 3i..3i+2; it attends frames
    0..3i+2 through the AR chunk's per-head sets: heads 0-3 local (last 6
    frames), 4-7 anchor (frames 0-2 + last 6), 8-11 memory (the k_i best of the
    history frames 0..3i-1 by pooled Q.K, plus the last 3).  k_i comes from the
    chunk-aware growth schedule (target sparsity 0.6, s_base 0.9, s_max 0.95)
    over the chunks' dense costs; chunk 0 is attended densely."""
    w = ar_chunk()
    return dataclasses.replace(
        w, name="ar_rollout_20x3x1560_cache60", seed=6, Tq=60, Tk=60, offset=0,
        rollout=dict(n_chunks=20, s_target=0.6, s_base=0.9, s_max=0.95, n_recent=3))


def rollout_chunk(w: Workload, i: int) -> dict:
    """Shape of chunk i of a rollout workload: its first query frame (= the KV
    frame offset of its queries), the frames cached when it runs, its dense
    cost in attended frame pairs (query frames x cached frames), and the
    history frames a memory head chooses from (those before the recent ones)."""
    c = w.chunk
    offset = i * c
    cached = offset + c
    return dict(offset=offset, cached=cached, dense_frame_pairs=c * cached,
                candidates=cached - w.rollout["n_recent"])


def rollout_policies(w: Workload, i: int, k_i: int) -> list:
    """Per-head policies of chunk i with the memory heads keeping k_i selected
    frames; the first chunk, with no history yet, is dense (FULL) on the
    memory heads, as the schedule attends the first chunk densely."""
    out = []
    for p in w.policies:
        p = dict(p)
        if p["kind"] == MEMORY:
            p = policy(FULL) if i == 0 else dict(p, topk=k_i, n_recent=w.rollout["n_recent"])
        out.append(p)
    return out


def block_policies(w: Workload) -> list:
    """The heads' policies in block units for a workload with `block` set: every
    frame count of a SINK_WINDOW / RANGE head is multiplied by the blocks per
    frame; a MEMORY head gets a window over its recent frames as a placeholder
    (its rows are written by the two-level selection)."""
    nb = w.P // w.block
    out = []
    for p in w.policies:
        p = dict(p)
        if p["kind"] == SINK_WINDOW:
            p.update(n_sink=p["n_sink"] * nb, window=p["window"] * nb)
        elif p["kind"] == RANGE:
            p.update(lo=p["lo"] * nb, hi=p["hi"] * nb + nb - 1)
        elif p["kind"] == MEMORY:
            p = policy(SINK_WINDOW, n_sink=0, window=p["n_recent"] * nb)
        elif p["kind"] != FULL:
            raise ValueError("policy kind has no block-unit form")
        out.append(p)
    return out


def decomposable() -> Workload:
    """Query chunk 3 x 1560 tokens, KV frames 0 = sink, 1..45 = history, 46..48 =
    current chunk; branch A = current chunk + sink, branch B = history; the merge of
    both is compared with one pass over all 49 frames."""
    a = policy(SINK_WINDOW, n_sink=1, window=3)
    b = policy(RANGE, lo=1, hi=45)
    u = policy(FULL)
    return Workload("decomposable_3x1560_kv49", 4, 1, 12, 128, 3, 49, 1560, "bf16",
                    [dict(u) for _ in range(12)], offset=46, chunk=3,
                    branches={"A": [dict(a) for _ in range(12)],
                              "B": [dict(b) for _ in range(12)],
                              "U": [dict(u) for _ in range(12)]})


def long_video(step: int = 0) -> Workload:
    """H=24, D=128, T=126 latent frames x 3600 tokens (60x60 grid), bf16;
    LVSA budget C=33, window W=11, T_per=8 rotating anchors, 8 denoising steps."""
    pol = policy(LVSA, window=11, budget=33, t_per=8, step=step)
    return Workload("lvsa_T126_P3600_H24", 5, 1, 24, 128, 126, 126, 3600, "bf16",
                    [dict(pol) for _ in range(24)], steps=8)


ALL = {w().name: w for w in (tiny_f32, lvsa_shaped, ar_chunk, ar_chunk_hsa, ar_chunk_rope,
                              ar_rollout, decomposable, long_video)}


def _seed(cfg_seed: int, tensor: int, head: int) -> int:
    return cfg_seed * 1_000_003 + tensor * 1009 + head


def outlier_channels(w: Workload) -> list[int]:
    if w.outliers == 0:
        return []
    g = torch.Generator().manual_seed(w.seed)
    return sorted(torch.randperm(w.D, generator=g)[: w.outliers].tolist())


def head_tensor(w: Workload, tensor: int, b: int, h: int) -> torch.Tensor:
    """One head's [N, D] tensor (tensor 0 = Q, 1 = K, 2 = V), in the workload dtype."""
    n = w.Nq if tensor == 0 else w.Nk
    g = torch.Generator().manual_seed(_seed(w.seed, tensor, b * w.H + h))
    x = torch.randn(n, w.D, generator=g, dtype=torch.float32)
    ch = outlier_channels(w)
    if ch:
        x[:, ch] *= w.outlier_scale
    return x.to(torch.bfloat16) if w.dtype == "bf16" else x


def make_tensor(w: Workload, tensor: int, heads=None) -> torch.Tensor:
    """Full [B, H', N, D] CPU tensor for the chosen heads (default: all)."""
    heads = range(w.H) if heads is None else list(heads)
    return torch.stack([torch.stack([head_tensor(w, tensor, b, h) for h in heads])
                        for b in range(w.B)])


def make_qkv(w: Workload, heads=None):
    """(q, k, v) CPU tensors [B, H', N, D] in the workload dtype."""
    return tuple(make_tensor(w, j, heads) for j in range(3))


def to_numpy64(x: torch.Tensor) -> np.ndarray:
    """Exact widening of a CPU float tensor (bf16 or fp32) to a float64 array."""
    return x.detach().to("cpu").to(torch.float64).numpy()
