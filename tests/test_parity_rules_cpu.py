"""The vectorised route rule used by the full-shape GPU tests agrees with the per-row rule (CPU)."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import check_selection_row, check_selection_rows  # noqa: E402


def test_vectorised_route_rule_matches_per_row_rule():
    rng = np.random.default_rng(0)
    M, K = 200, 20
    S = rng.standard_normal((300, M))
    S[:50] = np.round(S[:50], 1)  # rows with many exact ties
    idx = np.stack([np.sort(np.lexsort((np.arange(M), -r))[:K]) for r in S])
    idx[60] = np.sort(np.lexsort((np.arange(M), -S[60]))[1:K + 1])  # drops the best block
    idx[61, 3] = idx[61, 2]  # a repeated block
    idx[62, 0] = -1  # out of range
    idx[63] = idx[63][::-1]  # not ascending
    ties = np.lexsort((np.arange(M), -S[5]))
    idx[5] = np.sort(np.concatenate([ties[:K - 1], ties[K:K + 1]]))  # another member of a tie
    want = np.array([check_selection_row(i, r, K) for i, r in zip(idx, S)])
    got = check_selection_rows(idx, S)
    assert np.array_equal(got, want)
    assert not got[60] and not got[61] and not got[62] and not got[63]
