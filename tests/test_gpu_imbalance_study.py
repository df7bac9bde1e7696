"""The imbalance-score study against the oracle.

The study routes seeded router scores on the GPU both ways (grouped top-K' over
M groups, and a global top-K over one group), counts rows per device group with
the permutation kernel and reports IS = (max load - min load) / T (TechWalker
page, section 一).  Here the group loads and scores it computes are compared,
exactly, with the oracle's grouped and global top-K on the same scores, and the
grouped router's score must be zero in every trial."""
import numpy as np
import pytest

import imbalance_study as study
from oracle import moge_oracle as O
from tests.gpu_util import say

CASES = [(64, 8, 8, 16), (64, 8, 8, 1000), (64, 4, 8, 257), (128, 16, 32, 300),
         (256, 16, 16, 4096)]


@pytest.mark.gpu
@pytest.mark.parametrize("dist", ["iid", "zipf"])
@pytest.mark.parametrize("N,M,K,T", CASES)
def test_study_loads_match_oracle(lib, dist, N, M, K, T):
    r = study.Router(lib, N, M, K, T)
    for trial in range(3):
        scores = study.draw_scores(T, N, 1000 * trial + T, dist)
        say("imbalance study", dist, N, M, K, T, trial)
        import torch
        s = torch.from_numpy(scores).cuda()
        for m in (M, 1):
            got = r.group_loads(s, m)
            want = O.group_loads_of(O.group_topk(scores, m, K // m), N, M)
            np.testing.assert_array_equal(got, want, err_msg=f"groups={m} trial={trial}")
        grp, glb, peak = r.imbalance(scores, with_peak=True)
        loads = O.group_loads_of(O.global_topk(scores, K), N, M)
        assert grp == 0.0
        assert glb == O.imbalance_score(loads, T)
        assert peak == float(loads.max()) * M / (T * K)
