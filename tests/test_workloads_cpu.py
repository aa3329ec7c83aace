"""The seeded input generator: its positional base is the feature product of the recipe, and the
inputs do not depend on how many threads build them."""
import hashlib
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import workloads as W  # noqa: E402


def _sha(x):
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()


def test_positional_base_is_the_feature_product():
    for grid in ((4, 32, 32), (15, 32, 64), (3, 5, 7)):
        F = W.positional_features(grid)
        assert F.shape[1] == W.N_FEATURES
        Wm = np.random.default_rng(5).standard_normal((W.N_FEATURES, 64))
        ref = F @ Wm
        got = W._positional_base(grid, Wm)
        assert got.shape == ref.shape
        assert np.abs(got - ref).max() <= 1e-13 * np.abs(ref).max()


def test_inputs_do_not_depend_on_the_thread_count():
    for name in ("tiny", "short"):
        wl = W.WORKLOADS[name]
        a = W.make_qkv(wl, threads=1)
        b = W.make_qkv(wl, threads=8)
        c = W.make_qkv(wl, threads=3)
        for x, y, z in zip(a, b, c):
            assert _sha(x) == _sha(y) == _sha(z)
