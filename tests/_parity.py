"""Helpers shared by the GPU parity tests: tolerances, row sampling and the
oracle evaluated head by head on the rows being checked."""

from __future__ import annotations

import numpy as np
import torch

from oracle import attention as oatt

# Tolerances fixed for this method: bf16 inputs with fp32 accumulation
# max|dO| <= 1e-2 and max|dLSE| <= 1e-3; fp32 inputs 1e-5 for both.
TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-5, 1e-5)}


def sample_rows(P: int, frames, per_frame: int = 8, seed: int = 0) -> np.ndarray:
    """Token indices to check: rows at tile edges of each listed query frame
    (0, 31, 32, 127, 128, P-1) plus random ones."""
    rng = np.random.default_rng(seed)
    rows = []
    for t in frames:
        edge = [p for p in (0, 31, 32, 127, 128, P - 1) if 0 <= p < P]
        extra = rng.integers(0, P, size=max(0, per_frame - len(edge))).tolist()
        rows.extend(t * P + p for p in set(edge + extra))
    return np.array(sorted(set(rows)), dtype=np.int64)


def oracle_rows(q, k, v, idx, cnt, P, rows, heads=None, scale=None):
    """Oracle O, LSE [B, H', R(, D)] for the given query rows, one head at a time
    (q/k/v are CPU torch tensors; idx/cnt numpy or CPU tensors)."""
    idx = idx.cpu().numpy() if torch.is_tensor(idx) else idx
    cnt = cnt.cpu().numpy() if torch.is_tensor(cnt) else cnt
    B, H = q.shape[:2]
    heads = range(H) if heads is None else list(heads)
    O = np.zeros((B, len(heads), len(rows), q.shape[3]))
    L = np.zeros((B, len(heads), len(rows)))
    for b in range(B):
        for i, h in enumerate(heads):
            qh = q[b:b + 1, h:h + 1].float().numpy()
            kh = k[b:b + 1, h:h + 1].float().numpy()
            vh = v[b:b + 1, h:h + 1].float().numpy()
            o, lse = oatt.sparse_frame_attention(qh, kh, vh, idx[b:b + 1, h:h + 1],
                                                 cnt[b:b + 1, h:h + 1], P, scale=scale, rows=rows)
            O[b, i], L[b, i] = o[0, 0], lse[0, 0]
    return O, L


def oracle_whole_frames(q, k, v, idx, cnt, P, b, h, frames, threads=8, scale=None):
    """Oracle O [len(frames)*P, D] and LSE [len(frames)*P] of every row of the
    given query frames of head (b, h): the oracle's own masked attention,
    frame by frame, with the frames spread over a thread pool (numpy releases
    the interpreter lock in its BLAS and elementwise kernels)."""
    from concurrent.futures import ThreadPoolExecutor

    idx = idx.cpu().numpy() if torch.is_tensor(idx) else idx
    cnt = cnt.cpu().numpy() if torch.is_tensor(cnt) else cnt
    k64 = k[b, h].double().numpy()
    v64 = v[b, h].double().numpy()
    Tk = k64.shape[0] // P
    scale = 1.0 / np.sqrt(q.shape[3]) if scale is None else scale

    def one(t):
        mask = oatt.token_mask(idx[b, h, t, :cnt[b, h, t]], Tk, P)
        return oatt.attend_rows(q[b, h, t * P:(t + 1) * P].double().numpy(), k64, v64, mask,
                                scale)

    with ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(one, list(frames)))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def assert_close(o, lse, o_ref, lse_ref, kind: str, what: str = ""):
    """max|dO| and max|dLSE| within the tolerance; -inf LSE must match exactly."""
    to, tl = TOL[kind]
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    ninf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf_ref), f"{what}: -inf LSE pattern differs"
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    do = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    fin = ~ninf_ref
    dl = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    print(f"[parity] {what}: max|dO|={do:.3e} (tol {to:g}) max|dLSE|={dl:.3e} (tol {tl:g})",
          flush=True)
    assert do <= to, f"{what}: max|dO| = {do:.3e} > {to:g}"
    assert dl <= tl, f"{what}: max|dLSE| = {dl:.3e} > {tl:g}"
    return do, dl
