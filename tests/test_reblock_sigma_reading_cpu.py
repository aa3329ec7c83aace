"""How much the partition depends on the reading of Sigma (CPU only, oracle only).

Spark-H3 page, section "Spark-Attnが変えるもの" (Spark-Reblock bullet): the cosine is taken in the
metric of the keys' second moment, with no formula or precision given.  The oracle reads it as
K^T K / N_v with every key entry first rounded onto the grid 2^(E-21) (E: max|k| < 2^E) and the
products summed exactly in fixed point.  The plainer reading keeps every product exact: the sum of
the exact products k_ia k_ib, exact, divided by N_v and rounded once.  Keys are bf16, so only
entries more than 13 binades below the largest are moved by the grid.

The test computes the exact-product Sigma independently of the oracle (keys scaled to integers,
split into 16-bit limbs, limb Gram matrices in binary64 where every partial sum is an integer
below 2^53, combined in Python integers, one correctly rounded division) and runs the oracle's
partition (readings R2..R6, unchanged) from both.  Measured on the 720p adaptive-block workload,
heads 0 and 1: every Sigma entry differs, by at most 3.3e-10 of max|Sigma|, and the two
partitions are identical.
"""
import os
import sys
from fractions import Fraction

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402


def exact_product_sigma(Kv):
    """sum_i K[i,a] K[i,b] / N_v, every product and the sum exact, rounded once to binary64."""
    Nv, d = Kv.shape
    x = Kv.astype(np.float64)
    _, e = np.frexp(np.abs(x[x != 0]))
    s_min = int((e - 24).min())  # binary32 values carry 24 significant bits
    X = np.ldexp(x, -s_min)
    assert np.array_equal(X, np.round(X))
    A, sg = np.abs(X).astype(np.int64), np.sign(X)
    L = (int(A.max()).bit_length() + 15) // 16
    limbs = [((A >> (16 * l)) & 0xFFFF).astype(np.float64) * sg for l in range(L)]
    tot = np.zeros((d, d), dtype=object)
    for p in range(L):
        for q in range(L):
            G = limbs[p].T @ limbs[q]  # terms below 2^32, N_v below 2^21: every partial sum exact
            assert np.abs(G).max() < 2.0 ** 53
            tot = tot + G.astype(np.int64).astype(object) * (1 << (16 * (p + q)))
    scale = Fraction(2) ** (2 * s_min) / Nv
    return np.array([[float(Fraction(int(tot[a, b])) * scale) for b in range(d)] for a in range(d)])


def leaves(perm, block):
    leaf = np.empty(perm.size, np.int64)
    leaf[perm] = np.arange(perm.size) // block
    return leaf


def test_given_sigma_reproduces_partition():
    """The Sigma-taking entry point runs the same partition: with R1's Sigma it returns orc_reblock's."""
    wl = W.Workload("rb_small", 91, B=1, H=2, d=64, grid=(3, 10, 16), n_sink=64, block=64, reblock=True)
    Q, K, _ = W.make_qkv(wl)
    p = oracle.params(Q, wl.n_sink, wl.block, 0.1, 1)
    Sg, _ = oracle.reblock_metric(p, Q, K)
    assert np.array_equal(oracle.reblock_given_sigma(p, Q, Sg), oracle.reblock(p, Q, K))


def test_exact_product_sigma_gives_the_same_partition_720p():
    wl = W.WORKLOADS["reblock720p"]
    heads = (0, 1)
    Q = np.empty((1, len(heads), wl.N, wl.d), np.float32)
    K = np.empty_like(Q)
    for j, h in enumerate(heads):
        q, k, _ = W._head(wl, 0, h, 0)
        Q[0, j], K[0, j] = q, k
    p = oracle.params(Q, wl.n_sink, wl.block, 0.1, 1)
    Sg, _ = oracle.reblock_metric(p, Q, K)
    Sx = np.stack([exact_product_sigma(K[0, j, :wl.n_video]) for j in range(len(heads))])[None]
    perm_g = oracle.reblock_given_sigma(p, Q, Sg)
    perm_x = oracle.reblock_given_sigma(p, Q, Sx)
    for j in range(len(heads)):
        rel = np.abs(Sx[0, j] - Sg[0, j]).max() / np.abs(Sx[0, j]).max()
        assert 0 < rel < 1e-9, rel
        moved = int((leaves(perm_g[0, j], wl.block) != leaves(perm_x[0, j], wl.block)).sum())
        print(f"head {heads[j]}: max |Sigma diff| / max |Sigma| = {rel:.2e}, tokens in another leaf: {moved}")
        assert moved == 0
        assert np.array_equal(perm_g[0, j], perm_x[0, j])
