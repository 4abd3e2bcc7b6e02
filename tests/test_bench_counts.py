"""The benchmark's issued-work count (bench.issued_mfma), on the CPU.

The bench line reports the MFMA instructions the attention kernel issues for
the timed lists beside the algorithmic flop.  The count follows the kernel's
walk: runs of consecutive listed frames, each started on the 8-key boundary at
or below its first key and cut into 64-key tiles, walked by every wavefront
whose first row lies inside the query frame.  It is pinned here to small cases
counted by hand and to the hardware: rocprofv3's SQ_INSTS_MFMA per attention
launch on the LVSA step-0 lists (H12, 42 frames x 1560 tokens, D 128).
"""
import bench
import workloads as wl
from oracle import frame_sets as ofs


def test_tiles_of_runs_hand_counted():
    # one run of three 1560-token frames: keys [0, 4680) -> ceil(4680 / 64) = 74 tiles
    assert bench._tiles_of_runs([0, 1, 2], 1560, 64) == 74
    # two one-frame runs: frame 0 -> 25 tiles; frame 2 starts at key 3120 (a multiple of 8) -> 25
    assert bench._tiles_of_runs([0, 2], 1560, 64) == 50
    # P = 100: frame 1 covers keys [100, 200) and starts at key 96 -> 104 keys -> 2 tiles
    assert bench._tiles_of_runs([1], 100, 64) == 2
    # frames 1 and 2 form one run: keys from 96 to 300 -> 204 keys -> 4 tiles
    assert bench._tiles_of_runs([1, 2], 100, 64) == 4
    assert bench._tiles_of_runs([], 1560, 64) == 0


def test_issued_mfma_hand_counted():
    import numpy as np
    # one list of one 64-token frame, P = 64, D = 128: 2 wavefronts (rows 0-31, 32-63),
    # 1 tile each: per tile 2 x 8 Q.K^T + 4 x 4 P.V MFMAs, plus the Q.K^T of one tile past
    # the last -> 2 x (32 + 16) = 96
    idx = np.array([[[[0]]]], dtype=np.int32)
    cnt = np.array([[[1]]], dtype=np.int32)
    assert bench.issued_mfma(idx, cnt, 64, 128) == 96
    # an empty list issues nothing
    assert bench.issued_mfma(idx, np.zeros_like(cnt), 64, 128) == 0


def test_issued_mfma_matches_the_hardware_counter():
    # SQ_INSTS_MFMA per attention launch, rocprofv3 --pmc, LVSA step 0 (the
    # figure in profiles/lvsa_T42_P1560_H12.counters.txt)
    w = wl.lvsa_shaped(0)
    idx, cnt = ofs.build(w.policies, w.B, w.Tq, w.Tk)
    assert bench.issued_mfma(idx, cnt, w.P, w.D) == 407385216
