"""The library's chunk-aware growth schedule (host code) against the oracle,
bit for bit: the same float64 operations in the same order give the same
sparsities, the same beta and the same frame budgets."""

import numpy as np
import pytest

import frame_sparse_attention_amd as fsa
from oracle import cag as ocag


@pytest.mark.parametrize("seed", range(12))
def test_schedule_bit_exact(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 80))
    kind = seed % 3
    if kind == 0:
        cost = np.arange(1, n + 1, dtype=np.float64)           # a cache growing by one chunk
    elif kind == 1:
        cost = np.full(n, 7.5)                                  # a rolling cache of fixed size
    else:
        cost = rng.uniform(0.5, 4.0, n)
    s_max = float(rng.uniform(0.5, 0.98))
    s_base = float(rng.uniform(0.0, 1.0))
    reach = s_max * (cost[1:].sum() / cost.sum()) if n > 1 else 0.0
    s_target = float(rng.uniform(0.0, 0.95 * reach)) if reach > 0 else 0.0
    cand = rng.integers(1, 200, n).astype(np.int32)
    sp, bud, beta = fsa.cag_schedule(cost, s_target, s_base, s_max, cand)
    osp, obeta = ocag.schedule(cost.tolist(), s_target, s_base, s_max)
    assert beta == obeta
    assert sp.tolist() == osp
    assert bud.tolist() == ocag.frame_budgets(osp, cand.tolist())


def test_ar_rollout_budgets():
    # 20 chunks of 3 frames into a growing cache; memory heads choose among the
    # history frames, 8 of them at chunk 1 ... fewer as the rollout gets sparser
    n = 20
    cost = np.array([3.0 * (3 * (i + 1)) for i in range(n)])
    cand = np.array([max(1, 3 * i) for i in range(n)], dtype=np.int32)
    sp, bud, beta = fsa.cag_schedule(cost, 0.6, 0.9, 0.95, cand)
    osp, obeta = ocag.schedule(cost.tolist(), 0.6, 0.9, 0.95)
    assert sp.tolist() == osp and beta == obeta
    assert bud.tolist() == ocag.frame_budgets(osp, cand.tolist())
    assert sp[0] == 0.0 and bud[0] == cand[0] and (np.diff(sp[1:]) >= 0).all()


@pytest.mark.parametrize("args,text", [
    (dict(cost=[]), "n_chunks=0"),
    (dict(cost=[1.0, 0.0]), "cost[1]"),
    (dict(cost=[1.0, np.inf]), "cost[1]"),
    (dict(s_target=1.0), "ratios"),
    (dict(s_max=-0.1), "ratios"),
    (dict(s_base=1.5), "ratios"),
    (dict(s_target=0.9), "cannot be reached"),
    (dict(candidates=[3, 0, 2]), "candidates[1]"),
])
def test_schedule_errors(args, text):
    a = dict(cost=[1.0, 1.0, 1.0], s_target=0.3, s_base=0.5, s_max=0.8, candidates=None)
    a.update(args)
    with pytest.raises(fsa.FsaError) as e:
        fsa.cag_schedule(a["cost"], a["s_target"], a["s_base"], a["s_max"], a["candidates"])
    assert text in str(e.value)
