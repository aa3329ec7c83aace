"""Writes reblock_max.json: the SHA-256 of the oracle's Spark-Reblock permutation (int32,
little-endian, [B,H,N_v]) for seeded inputs at the largest sizes the partition accepts.  Only
`oracle` and the seeded generators in `workloads` are used; the oracle needs minutes per case on
one core (it runs one thread per (batch, head)), too long to recompute inside a test.

    python tests/golden/make_reblock_max.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as W  # noqa: E402

# (name, n_video, n_sink, d, block, seed): 2^20 video rows is the partition's largest size (its
# fixed-point second moment sums at most 2^20 products per entry); the other is the full clip's
# token count at d = 128, one head.
CASES = [
    ("max-rows-d64-b64", 1 << 20, 8, 64, 64, 20),
    ("fullclip-rows-d128-b128", 245952, 8, 128, 128, 21),
]


def main():
    out = {}
    for name, nv, ns, d, b, seed in CASES:
        Q, K, _ = W.gaussian_qkv(1, 1, nv, ns, d, seed=seed, dtype="bf16")
        perm = oracle.reblock(oracle.params(Q, ns, b), Q, K)
        assert perm.dtype == np.int32 and perm.shape == (1, 1, nv)
        out[name] = {"n_video": nv, "n_sink": ns, "d": d, "block": b, "seed": seed, "dtype": "bf16",
                     "perm_sha256": hashlib.sha256(perm.astype("<i4").tobytes()).hexdigest(),
                     "perm_head": perm[0, 0, :8].tolist(), "perm_tail": perm[0, 0, -8:].tolist()}
        print(name, out[name]["perm_sha256"], flush=True)
    with open(os.path.join(HERE, "reblock_max.json"), "w") as f:
        json.dump({"source": "oracle.reblock on workloads.gaussian_qkv inputs (tests/golden/make_reblock_max.py)",
                   "cases": out}, f, indent=1)


if __name__ == "__main__":
    main()
