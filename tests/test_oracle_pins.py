"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test ties one part of the oracle to a closed form, a special case that reduces to a
textbook routine, an invariant, a hand-worked example or a brute-force formulation:

  P-a  full density (K = M)           == dense softmax attention (torch SDPA, binary64)
  P-b  one-token blocks, any ratio    == dense attention, both compressed variants
  P-c  exp(s a.k~_J + beta_J)         == the block's exact mass at the anchor
  P-d  the compressed logit is a tangent lower bound of the block LSE, touching at q = a
  P-e  every query equal to the anchor: Reweight == dense, mean-pool != dense
  P-f  oracle == NumPy mask-matrix brute force (partial block, sinks, B > 1)
  P-g  selection == numpy.lexsort ranking
  P-h  reblocked forward at full density == dense (after un-permuting), with the keys reusing
       the query partition or partitioned on their own
  P-i  partition invariants; partition == score-vector brute force
  P-j  blocks of identical keys/values: compressed term exact, forward == dense
  P-k  hand-worked two-block example (tests/golden/hand_worked_example.json)
  P-l  adaptive-tau selection: the normal tail for Gaussian scores, NumPy mean/std threshold,
       keep-all == dense, forward == brute force (moderate, all kept, none kept)
  P-m  FP8 carrier: E4M3 rounding == torch.float8_e4m3fn cast and the format's closed form
       (every code maps to itself, midpoints go to the even mantissa); on-grid inputs at full
       density == dense; power-of-two rescalings act exactly; forward == brute force
  P-n  asymmetric route (query blocks of `block`, key blocks of `block_k`): one-token key blocks
       == dense for any budget; full density == dense; block_k = block changes nothing; forward
       == brute force (both pool modes, both orders of the sizes, FP8 carriers); selection ==
       lexsort over the rectangular score matrix
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa_dense(Q, K, V):
    """Library dense attention in binary64 on the CPU (torch's math path)."""
    q, k, v = (torch.from_numpy(np.asarray(x, np.float64)) for x in (Q, K, V))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()


def small(seed=0, B=1, H=2, nv=1000, ns=5, d=16, dtype="fp32"):
    return W.gaussian_qkv(B, H, nv, ns, d, seed=seed, dtype=dtype)


# ---------------------------------------------------------------- P-a
@pytest.mark.parametrize("pool_mode", [0, 1])
@pytest.mark.parametrize("nv,ns,block", [(1000, 5, 64), (1024, 0, 128), (77, 3, 16)])
def test_full_density_is_dense(orc, pool_mode, nv, ns, block):
    Q, K, V = small(seed=nv + ns, nv=nv, ns=ns)
    p = orc.params(Q, ns, block, 1.0, pool_mode)
    O, lse, idx = orc.forward(p, Q, K, V)
    ref = sdpa_dense(Q, K, V)
    assert np.abs(O - ref).max() < 1e-12
    M = orc.num_blocks(p)
    assert idx.shape[-1] == M
    assert (idx == np.arange(M)).all()


# ---------------------------------------------------------------- P-b
@pytest.mark.parametrize("pool_mode", [0, 1])
@pytest.mark.parametrize("ratio", [0.05, 0.3, 0.7])
def test_block_size_one_is_dense(orc, pool_mode, ratio):
    Q, K, V = small(seed=3, nv=200, ns=4)
    p = orc.params(Q, 4, 1, ratio, pool_mode)
    O, lse, _ = orc.forward(p, Q, K, V)
    ref = sdpa_dense(Q, K, V)
    assert np.abs(O - ref).max() < 1e-12
    # the dense LSE, computed directly
    s = 1.0 / math.sqrt(Q.shape[-1])
    z = s * np.einsum("bhid,bhjd->bhij", Q.astype(np.float64), K.astype(np.float64))
    assert np.abs(lse - np.log(np.exp(z).sum(-1))).max() < 1e-12


# ---------------------------------------------------------------- P-c, P-d
def test_log_mass_identity_at_anchor(orc):
    Q, K, V = small(seed=5, nv=1000, ns=7)
    p = orc.params(Q, 7, 64, 0.1, 1)
    pooled = orc.pool(p, Q, K, V)
    s = 1.0 / math.sqrt(Q.shape[-1])
    nv = 1000
    for h in range(Q.shape[1]):
        a = Q[0, h, :nv].astype(np.float64).mean(0)
        assert np.abs(pooled["anchor"][0, h] - a).max() < 1e-14
        for J in range(orc.num_blocks(p)):
            kb = K[0, h, J * 64:min(nv, J * 64 + 64)].astype(np.float64)
            exact = np.log(np.exp(s * kb @ a).sum())
            approx = s * a @ pooled["k_sum"][0, h, J] + pooled["bias"][0, h, J]
            assert abs(exact - approx) < 1e-12


def test_compressed_logit_is_tangent_lower_bound(orc):
    Q, K, V = small(seed=6, nv=640, ns=0)
    p = orc.params(Q, 0, 64, 0.1, 1)
    pooled = orc.pool(p, Q, K, V)
    s = 1.0 / math.sqrt(Q.shape[-1])
    rng = np.random.default_rng(0)
    for J in range(orc.num_blocks(p)):
        kb = K[0, 0, J * 64:J * 64 + 64].astype(np.float64)
        kt, beta = pooled["k_sum"][0, 0, J], pooled["bias"][0, 0, J]
        a = pooled["anchor"][0, 0]

        def lse(q):
            return np.logaddexp.reduce(s * kb @ q)

        for _ in range(50):
            q = a + rng.standard_normal(a.shape) * 0.3
            assert s * q @ kt + beta <= lse(q) + 1e-12
        # equal value and equal gradient (s * k~) at the anchor
        assert abs(s * a @ kt + beta - lse(a)) < 1e-12
        eps = 1e-6
        grad = np.array([(lse(a + eps * e) - lse(a - eps * e)) / (2 * eps)
                         for e in np.eye(a.size)])
        assert np.abs(grad - s * kt).max() < 1e-7


# ---------------------------------------------------------------- P-e
def test_queries_at_anchor(orc):
    Q, K, V = small(seed=7, nv=512, ns=3)
    Q[:, :, :512] = Q[:, :, :512].mean(axis=2, keepdims=True)  # every video query = the anchor
    ref = sdpa_dense(Q, K, V)
    for ratio in (0.1, 0.5):
        O, _, _ = orc.forward(orc.params(Q, 3, 32, ratio, 1), Q, K, V)
        assert np.abs(O - ref).max() < 1e-12
        O0, _, _ = orc.forward(orc.params(Q, 3, 32, ratio, 0), Q, K, V)
        rel = np.linalg.norm(O0 - ref) / np.linalg.norm(ref)
        assert rel > 1e-3  # the mean pool misses the Jensen gap


# ---------------------------------------------------------------- P-f
@pytest.mark.parametrize("pool_mode", [0, 1])
@pytest.mark.parametrize("ratio", [0.1, 0.25, 1.0])
def test_oracle_matches_brute_force(orc, pool_mode, ratio):
    Q, K, V = small(seed=11, B=2, H=2, nv=4096 - 40, ns=5, d=16)
    p = orc.params(Q, 5, 64, ratio, pool_mode)
    O, lse, idx = orc.forward(p, Q, K, V)
    Ob, lb, ib = brute.forward(Q, K, V, 5, 64, ratio, pool_mode)
    assert (idx == ib).all()
    assert np.abs(O - Ob).max() < 1e-12
    assert np.abs(lse - lb).max() < 1e-11


def test_oracle_matches_brute_force_structured(orc):
    wl = W.WORKLOADS["tiny"]
    Q, K, V = W.make_qkv(wl)
    for pm in (0, 1):
        O, lse, idx = orc.forward(orc.params(Q, 0, 64, 0.1, pm), Q, K, V)
        Ob, lb, ib = brute.forward(Q, K, V, 0, 64, 0.1, pm)
        assert (idx == ib).all()
        assert np.abs(O - Ob).max() < 1e-12


def test_attend_blocks_matches_forward(orc):
    Q, K, V = small(seed=12, B=1, H=2, nv=1000, ns=5)
    p = orc.params(Q, 5, 64, 0.2, 1)
    O, lse, idx = orc.forward(p, Q, K, V)
    pooled = orc.pool(p, Q, K, V)
    M = orc.num_blocks(p)
    qb = np.array([[0, 0], [1, 3], [1, M - 1], [0, M], [1, M + 4]])
    Os, ls = orc.attend_blocks(p, Q, K, V, pooled, idx, qb)
    for n, (bh, I) in enumerate(qb):
        if I < M:
            lo, hi = I * 64, min(1000, I * 64 + 64)
            assert np.abs(Os[n, :hi - lo] - O[0, bh, lo:hi]).max() < 1e-13
            assert np.abs(ls[n, :hi - lo] - lse[0, bh, lo:hi]).max() < 1e-12
        else:
            r = 1000 + I - M
            assert np.abs(Os[n, 0] - O[0, bh, r]).max() < 1e-13


# ---------------------------------------------------------------- P-g
def test_selection_is_lexsort_topk(orc):
    Q, K, V = small(seed=13, H=3, nv=3000, ns=0)
    p = orc.params(Q, 0, 64, 0.17, 1)
    pooled = orc.pool(p, Q, K, V)
    S = orc.scores(p, pooled["q_mean"], pooled["k_mean"])
    # scores: s * qbar . kbar with the block means taken directly
    s = 1.0 / math.sqrt(Q.shape[-1])
    qm = Q[0, 0, :46 * 64].astype(np.float64).reshape(46, 64, 16).mean(1)
    km = K[0, 0, :46 * 64].astype(np.float64).reshape(46, 64, 16).mean(1)
    assert np.abs(S[0, 0, :46, :46] - s * qm @ km.T).max() < 1e-13
    idx = orc.select(p, S)
    M = S.shape[-1]
    Kk = idx.shape[-1]
    assert Kk == math.floor(np.float32(0.17) * M + 0.5)
    for h in range(3):
        for I in range(M):
            ref = np.sort(np.lexsort((np.arange(M), -S[0, h, I]))[:Kk])
            assert (idx[0, h, I] == ref).all()


def test_selection_ties_take_lower_index(orc):
    p = orc.params(np.zeros((1, 1, 10 * 4, 4), np.float32), 0, 4, 0.3)
    M = 10
    S = np.zeros((1, 1, M, M))
    S[0, 0, 0] = [1, 2, 2, 2, 0, 2, 5, 2, 1, 0]  # K = 3: 6 then the two lowest of the 2's
    S[0, 0, 1] = -1.0  # all tied -> 0,1,2
    idx = orc.select(p, S)
    assert idx[0, 0, 0].tolist() == [1, 2, 6]
    assert idx[0, 0, 1].tolist() == [0, 1, 2]


# ---------------------------------------------------------------- budget
@pytest.mark.parametrize("M,ratio,K", [(64, 0.1, 6), (240, 0.1, 24), (591, 0.1, 59),
                                       (591, 0.2, 118), (591, 0.3, 177), (591, 1.0, 591),
                                       (1922, 0.1, 192), (10, 0.01, 1), (7, 0.5, 4),
                                       (5, 0.3, 2), (3, 1e-6, 1)])
def test_budget(orc, M, ratio, K):
    assert orc.topk_count(M, ratio) == K
    assert brute.budget(M, ratio) == K


# ---------------------------------------------------------------- P-h, P-i
def test_reblocked_full_density_is_dense(orc):
    Q, K, V = small(seed=21, nv=700, ns=6)
    p = orc.params(Q, 6, 32, 1.0, 1)
    perm = orc.reblock(p, Q, K)
    assert not (perm == np.arange(700)).all()
    O, _, _ = orc.forward(p, Q, K, V, perm=perm)
    assert np.abs(O - sdpa_dense(Q, K, V)).max() < 1e-12


def test_reblocked_forward_matches_brute_force(orc):
    Q, K, V = small(seed=22, nv=900, ns=4)
    p = orc.params(Q, 4, 64, 0.2, 1)
    perm = orc.reblock(p, Q, K)
    O, lse, idx = orc.forward(p, Q, K, V, perm=perm)
    Ob, lb, ib = brute.forward(Q, K, V, 4, 64, 0.2, 1, perm=perm)
    assert (idx == ib).all()
    assert np.abs(O - Ob).max() < 1e-12


def test_separate_key_partition_full_density_is_dense(orc):
    """Queries and keys each in their own partition (keys bisected under the queries' second
    moment): at full density the result is still dense attention, whatever the two orders."""
    Q, K, V = small(seed=23, nv=700, ns=6)
    p = orc.params(Q, 6, 32, 1.0, 1)
    perm_q = orc.reblock(p, Q, K)
    perm_k = orc.reblock(p, K, Q)
    assert not (perm_q == perm_k).all()
    O, _, _ = orc.forward(p, Q, K, V, perm=perm_q, perm_k=perm_k)
    assert np.abs(O - sdpa_dense(Q, K, V)).max() < 1e-12
    # only the key side partitioned
    O2, _, _ = orc.forward(p, Q, K, V, perm_k=perm_k)
    assert np.abs(O2 - sdpa_dense(Q, K, V)).max() < 1e-12


def test_separate_key_partition_matches_brute_force(orc):
    Q, K, V = small(seed=24, nv=900, ns=4)
    p = orc.params(Q, 4, 64, 0.2, 1)
    perm_q, perm_k = orc.reblock(p, Q, K), orc.reblock(p, K, Q)
    O, lse, idx = orc.forward(p, Q, K, V, perm=perm_q, perm_k=perm_k)
    Ob, lb, ib = brute.forward(Q, K, V, 4, 64, 0.2, 1, perm=perm_q, perm_k=perm_k)
    assert (idx == ib).all()
    assert np.abs(O - Ob).max() < 1e-12 and np.abs(lse - lb).max() < 1e-12
    # the key partition is the query partition with the roles of Q and K exchanged: the
    # score-vector brute force of the keys against the queries
    for h in range(2):
        assert (perm_k[0, h] == brute.reblock_head(K[0, h], Q[0, h], 900, 64)).all()


@pytest.mark.parametrize("nv,block,dtype", [(1000, 64, "fp32"), (1500, 128, "bf16"),
                                            (640, 64, "bf16"), (130, 64, "fp32")])
def test_reblock_matches_score_vector_brute_force(orc, nv, block, dtype):
    Q, K, V = small(seed=nv, H=2, nv=nv, ns=3, d=16, dtype=dtype)
    p = orc.params(Q, 3, block)
    perm = orc.reblock(p, Q, K)
    for h in range(2):
        ref = brute.reblock_head(Q[0, h], K[0, h], nv, block)
        assert (perm[0, h] == ref).all()


def test_reblock_invariants(orc):
    nv, b = 75 * 64 + 17, 64
    Q, K, V = small(seed=31, H=2, nv=nv, ns=2, d=32, dtype="bf16")
    p = orc.params(Q, 2, b)
    perm = orc.reblock(p, Q, K)
    M = orc.num_blocks(p)
    for h in range(2):
        pr = perm[0, h]
        assert (np.sort(pr) == np.arange(nv)).all()  # bijection
        for L in range(M):
            leaf = pr[L * b:(L + 1) * b]
            assert (np.diff(leaf) > 0).all()  # ascending inside every leaf
        assert len(pr[(M - 1) * b:]) == nv - (M - 1) * b
    # metric: Sigma = K^T K / N_v up to the fixed-point grid of the keys (entries rounded to
    # 2^(E-21), max|k| < 2^E): |error| <= 2^(2E-21); n_i = sqrt(q_i^T Sigma q_i)
    Sg, nrm = orc.reblock_metric(p, Q, K)
    kv = K[0, 0, :nv].astype(np.float64)
    qv = Q[0, 0, :nv].astype(np.float64)
    ref = kv.T @ kv / nv
    E = math.frexp(np.abs(kv).max())[1]
    assert np.abs(Sg[0, 0] - ref).max() <= 2.0 ** (2 * E - 21)
    assert np.allclose(nrm[0, 0], np.sqrt(np.einsum("ia,ab,ib->i", qv, Sg[0, 0], qv)), rtol=1e-12)
    # keys on the grid (|k| >= 2^(E-13) or 0, bf16): the fixed-point sum is the exact K^T K / N_v
    K4 = K.copy()
    K4[np.abs(K4) < 2.0 ** (E - 13)] = 0.0
    Sg4, nrm4 = orc.reblock_metric(p, Q, K4)
    kv4 = K4[0, 0, :nv].astype(np.float64)
    ref4 = kv4.T @ kv4 / nv
    assert np.abs(Sg4[0, 0] - ref4).max() <= 1e-13 * np.abs(ref4).max()
    assert np.allclose(nrm4[0, 0], np.linalg.norm(qv @ kv4.T, axis=1) / math.sqrt(nv), rtol=1e-12)
    # power-of-two scaling of query rows and of all keys leaves the partition unchanged
    Q2, K2 = Q.copy(), K.copy()
    Q2[0, 0, ::7] *= 8.0
    Q2[0, 1, 3::5] *= 0.25
    K2 *= 2.0 ** -5
    assert (orc.reblock(p, Q2, K2) == perm).all()
    # sink rows play no part
    Q3, K3 = Q.copy(), K.copy()
    Q3[:, :, nv:] = 100.0
    K3[:, :, nv:] = -100.0
    assert (orc.reblock(p, Q3, K3) == perm).all()


def test_reblock_recovers_planted_hierarchy(orc):
    """Queries drawn around 2^levels well separated centres (c = sum_l +-2^-l e_l); keys isotropic.
    Every leaf must be pure (one centre), whatever the raster order."""
    rng = np.random.default_rng(4)
    levels, per, d, b = 3, 64, 8, 64
    nv = per * 2 ** levels
    signs = np.array([[1 if (c >> l) & 1 else -1 for l in range(levels)]
                      for c in range(2 ** levels)], np.float64)
    centres = np.zeros((2 ** levels, d))
    centres[:, :levels] = signs * (2.0 ** -np.arange(levels))
    label = rng.permutation(np.repeat(np.arange(2 ** levels), per))
    q = centres[label] + 0.02 * rng.standard_normal((nv, d))
    k = rng.standard_normal((nv, d))
    Q = q[None, None].astype(np.float32)
    K = k[None, None].astype(np.float32)
    p = orc.params(Q, 0, b)
    perm = orc.reblock(p, Q, K)[0, 0]
    for L in range(nv // b):
        assert len(set(label[perm[L * b:(L + 1) * b]])) == 1


# ---------------------------------------------------------------- P-j
def test_constant_blocks_make_compression_exact(orc):
    rng = np.random.default_rng(8)
    d, b, nv, ns = 16, 32, 32 * 20, 4
    Q = rng.standard_normal((1, 2, nv + ns, d)).astype(np.float32)
    K = np.repeat(rng.standard_normal((1, 2, 20, d)), b, axis=2).astype(np.float32)
    V = np.repeat(rng.standard_normal((1, 2, 20, d)), b, axis=2).astype(np.float32)
    K = np.concatenate([K, rng.standard_normal((1, 2, ns, d)).astype(np.float32)], axis=2)
    V = np.concatenate([V, rng.standard_normal((1, 2, ns, d)).astype(np.float32)], axis=2)
    ref = sdpa_dense(Q, K, V)
    for pm in (0, 1):
        p = orc.params(Q, ns, b, 0.15, pm)
        pooled = orc.pool(p, Q, K, V)
        assert np.abs(pooled["bias"] - math.log(b)).max() < 1e-12
        assert np.abs(pooled["v_sum"] - V[:, :, :nv:b]).max() < 1e-12
        O, _, _ = orc.forward(p, Q, K, V)
        assert np.abs(O - ref).max() < 1e-12


# ---------------------------------------------------------------- P-k
@pytest.mark.parametrize("variant,pool_mode", [("mean", 0), ("reweight", 1)])
def test_hand_worked_example(orc, variant, pool_mode):
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_example.json")))
    Q = np.array(g["Q"], np.float32)[None, None]
    K = np.array(g["K"], np.float32)[None, None]
    V = np.array(g["V"], np.float32)[None, None]
    p = orc.params(Q, g["n_sink"], g["block"], g["topk_ratio"], pool_mode, g["scale"])
    O, lse, idx = orc.forward(p, Q, K, V)
    assert idx[0, 0].tolist() == g["idx"]
    e = math.e
    r = math.sqrt(e)
    env = dict(e=e, r=r, sig=r / (1 + r), exp=math.exp, log=math.log)
    expO = np.array([[eval(x, {}, env) for x in row] for row in g["expected"][variant]["O"]])
    expL = np.array([eval(x, {}, env) for x in g["expected"][variant]["lse"]])
    assert np.abs(O[0, 0] - expO).max() < 1e-14
    assert np.abs(lse[0, 0] - expL).max() < 1e-14


# ---------------------------------------------------------------- independence of units
def test_batches_and_heads_are_independent(orc):
    Q, K, V = small(seed=40, B=2, H=3, nv=500, ns=3)
    p = orc.params(Q, 3, 64, 0.2, 1)
    O, lse, idx = orc.forward(p, Q, K, V)
    p1 = orc.params(Q[1:2, 2:3], 3, 64, 0.2, 1)
    O1, l1, i1 = orc.forward(p1, Q[1:2, 2:3], K[1:2, 2:3], V[1:2, 2:3])
    assert (O1[0, 0] == O[1, 2]).all() and (i1[0, 0] == idx[1, 2]).all()


# ---------------------------------------------------------------- P-l adaptive-tau selection
def _normal_tail(t):
    return 0.5 * math.erfc(t / math.sqrt(2.0))


@pytest.mark.parametrize("tau", [1.0, 1.5, 2.0])
def test_tau_keeps_the_normal_tail_of_gaussian_scores(orc, tau):
    """For normally distributed block scores the kept fraction is the normal tail beyond tau
    (15.9% / 6.7% / 2.3%, the page's ~16 / ~7 / ~2.7%)."""
    Q, K, V = small(seed=61, H=2, nv=600 * 16, ns=0, d=16)
    p = orc.params(Q, 0, 16)
    M = orc.num_blocks(p)
    S = np.random.default_rng(62).standard_normal((1, 2, M, M)) * 3.0 + 0.7  # any mean and spread
    _, counts, stats = orc.select_tau(p, tau, S)
    frac = counts.sum(axis=2) / (M * M)
    assert np.abs(frac - _normal_tail(tau)).max() < 3e-3, (frac, _normal_tail(tau))
    assert np.allclose(stats[..., 0], S.mean(axis=(2, 3)), rtol=0, atol=1e-12)
    assert np.allclose(stats[..., 1], S.std(axis=(2, 3)), rtol=1e-12, atol=0)


@pytest.mark.parametrize("tau", [-0.5, 0.0, 0.7, 1.5])
def test_tau_selection_matches_numpy(orc, tau):
    Q, K, V = small(seed=63, H=2, nv=97 * 32 + 5, ns=0, d=16)
    p = orc.params(Q, 0, 32)
    M = orc.num_blocks(p)
    rng = np.random.default_rng(64)
    S = rng.standard_normal((1, 2, M, M))
    S[0, 1, :, ::3] = 0.25  # ties in every row
    idx, counts, _ = orc.select_tau(p, tau, S)
    for h in range(2):
        kept = brute.select_tau_head(S[0, h], tau)
        assert (counts[0, h] == kept.sum(axis=1)).all()
        for I in range(M):
            assert (idx[0, h, I, :counts[0, h, I]] == np.nonzero(kept[I])[0]).all()


def test_tau_keep_all_is_dense(orc):
    Q, K, V = small(seed=65, nv=700, ns=6)
    p = orc.params(Q, 6, 32, 0.1, 1)
    O, _, _, counts = orc.forward_tau(p, -1e30, Q, K, V)
    assert (counts == orc.num_blocks(p)).all()
    assert np.abs(O - sdpa_dense(Q, K, V)).max() < 1e-12


@pytest.mark.parametrize("tau", [0.8, -1e30, 1e30])
def test_tau_forward_matches_brute_force(orc, tau):
    """Moderate tau, everything kept, nothing kept (compressed branch and sinks only)."""
    Q, K, V = small(seed=66, B=2, nv=900, ns=4)
    p = orc.params(Q, 4, 64, 0.2, 1)
    O, lse, idx, counts = orc.forward_tau(p, tau, Q, K, V)
    Ob, lb, kept = brute.forward(Q, K, V, 4, 64, 0.2, 1, tau=tau)
    assert (counts == kept.sum(axis=3)).all()
    assert np.abs(O - Ob).max() < 1e-12 and np.abs(lse - lb).max() < 1e-12


# ---------------------------------------------------------------- P-m FP8 (E4M3) carrier
def _e4m3_codes():
    """Every finite E4M3 value from the format's definition (sign, 4-bit exponent with bias 7,
    3-bit mantissa; exponent 15 with mantissa 7 is NaN)."""
    vals = []
    for code in range(256):
        sgn, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        v = 2.0 ** (e - 7) * (1 + m / 8) if e else 2.0 ** -6 * (m / 8)
        vals.append(-v if sgn else v)
    return np.array(sorted(set(vals)), np.float64)


def test_e4m3_matches_torch_cast(orc):
    rng = np.random.default_rng(70)
    mag = np.exp2(rng.uniform(-14, np.log2(448), 200000))
    x = (mag * rng.choice([-1, 1], mag.size)).astype(np.float32)
    grid = _e4m3_codes()
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, grid.astype(np.float32), mids, np.float32([0, -0.0, 448, -448])])
    assert (orc.e4m3(x).view(np.uint32) == brute.e4m3_torch(x).view(np.uint32)).all()


def test_e4m3_closed_form(orc):
    grid = _e4m3_codes()
    assert grid.max() == 448 and np.sort(np.abs(grid))[1] == 2.0 ** -9
    g32 = grid.astype(np.float32)
    assert (orc.e4m3(g32) == g32).all()
    # a midpoint goes to the neighbour whose mantissa is even (its code is even)
    pos = grid[grid >= 0]
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = np.float32((lo + hi) / 2)
        got = float(orc.e4m3(np.float32([mid]))[0])
        lo_code = list(pos).index(lo)  # codes of non-negative values ascend with the value
        assert got == (lo if lo_code % 2 == 0 else hi), (lo, hi, got)
        # anything strictly inside rounds to the nearer neighbour
        q = np.float32(lo + 0.3 * (hi - lo))
        assert float(orc.e4m3(np.float32([q]))[0]) == lo


def _on_grid(rng, shape):
    """Random values on the E4M3 grid with 448 reached in every (batch, head) slab, so that every
    per-head scale is exactly 1."""
    grid = _e4m3_codes()
    grid = grid[np.abs(grid) >= 2.0 ** -3]
    x = rng.choice(grid, size=shape).astype(np.float32)
    x[..., 0, 0] = 448.0
    return x


def test_fp8_full_density_on_grid_is_dense(orc):
    rng = np.random.default_rng(71)
    B, H, nv, ns, d = 1, 2, 300, 3, 16
    Q, K, V = (_on_grid(rng, (B, H, nv + ns, d)) * np.float32(1) for _ in range(3))
    p = orc.params(Q, ns, 32, 1.0, 1)
    p.scale = 1.0 / 512  # keeps the logits of 448-sized rows moderate
    O, lse, idx, sc = orc.forward_fp8(p, Q, K, V)
    assert (sc[..., 1::2] == 1).all() and (sc[..., 0::2] == 1).all()
    Od, ld = orc.dense(p, Q, K, V)
    assert np.abs(O - Od).max() < 1e-12 * np.abs(Od).max()
    assert np.abs(lse - ld).max() < 1e-12


def test_fp8_power_of_two_rescaling_is_exact(orc):
    Q, K, V = small(seed=72, nv=600, ns=4)
    p = orc.params(Q, 4, 64, 0.2, 1)
    O, lse, idx, sc = orc.forward_fp8(p, Q, K, V)
    # V * 4: the same carrier, s_V four times larger
    O4, lse4, idx4, sc4 = orc.forward_fp8(p, Q, K, V * np.float32(4))
    assert (idx4 == idx).all() and (O4 == 4 * O).all() and (lse4 == lse).all()
    # Q * 2 and K / 2: the same carriers, the same s_Q s_K and route
    O2, lse2, idx2, sc2 = orc.forward_fp8(p, Q * np.float32(2), K * np.float32(0.5), V)
    assert (idx2 == idx).all()
    assert (sc2[..., 1] * sc2[..., 3] == sc[..., 1] * sc[..., 3]).all()
    assert np.abs(O2 - O).max() < 1e-12 and np.abs(lse2 - lse).max() < 1e-12


def test_fp8_quantization_changes_the_result(orc):
    """Off the grid the carrier is not the identity: the FP8 forward departs from the plain one by
    about the E4M3 rounding (3 mantissa bits), not more."""
    Q, K, V = small(seed=73, nv=800, ns=5)
    p = orc.params(Q, 5, 64, 0.2, 1)
    O8, _, idx8, _ = orc.forward_fp8(p, Q, K, V)
    O, _, idx = orc.forward(p, Q, K, V)
    assert (idx8 == idx).all()
    rel = np.linalg.norm(O8 - O) / np.linalg.norm(O)
    assert 1e-3 < rel < 2.0 ** -4


@pytest.mark.parametrize("pool_mode,block_k", [(1, 0), (0, 0), (1, 32)])
def test_fp8_forward_equals_plain_attention_on_decoded_carriers(orc, pool_mode, block_k):
    """The sampling route of the GPU tests: the oracle's plain attention of chosen blocks, fed the
    decoded carriers (parity.fp8_decoded_inputs), equals the oracle's FP8 forward on every video
    block and sink row (ragged blocks, sinks, B > 1, both pool modes, unequal key blocks)."""
    from parity import fp8_decoded_inputs

    Q, K, V = small(seed=75, B=2, nv=1000 - 24, ns=5)
    p = orc.params(Q, 5, 64, 0.2, pool_mode, block_k=block_k)
    O8, l8, idx, _ = orc.forward_fp8(p, Q, K, V)
    Qd, Kd, Vd, pd = fp8_decoded_inputs(orc, p, Q, K, V, orc.pool(p, Q, K, V))
    M, BH, nv, ns = orc.num_blocks(p), 2 * 2, 1000 - 24, 5
    qb = np.array([(bh, I) for bh in range(BH) for I in range(M + ns)])
    Os, ls = orc.attend_blocks(p, Qd, Kd, Vd, pd, idx, qb)
    O8f, l8f = O8.reshape(BH, -1, Q.shape[-1]), l8.reshape(BH, -1)
    for n, (bh, I) in enumerate(qb):
        lo, hi = (I * 64, min(nv, (I + 1) * 64)) if I < M else (nv + I - M, nv + I - M + 1)
        assert np.abs(Os[n, :hi - lo] - O8f[bh, lo:hi]).max() < 1e-6
        assert np.abs(ls[n, :hi - lo] - l8f[bh, lo:hi]).max() < 1e-6


@pytest.mark.parametrize("pool_mode,ratio", [(1, 0.2), (0, 0.2), (1, 1.0)])
def test_fp8_forward_matches_brute_force(orc, pool_mode, ratio):
    Q, K, V = small(seed=74, B=2, nv=1000 - 24, ns=5)
    perm = None
    p = orc.params(Q, 5, 64, ratio, pool_mode)
    O, lse, idx, _ = orc.forward_fp8(p, Q, K, V)
    Ob, lb, ib = brute.forward(Q, K, V, 5, 64, ratio, pool_mode, fp8=True)
    assert (idx == ib).all()
    assert np.abs(O - Ob).max() < 1e-12 and np.abs(lse - lb).max() < 1e-11


def test_fp8_reblocked_forward_matches_brute_force(orc):
    Q, K, V = small(seed=75, nv=640, ns=3)
    p = orc.params(Q, 3, 64, 0.25, 1)
    perm = orc.reblock(p, Q, K)
    O, lse, idx, _ = orc.forward_fp8(p, Q, K, V, perm=perm)
    Ob, lb, ib = brute.forward(Q, K, V, 3, 64, 0.25, 1, perm=perm, fp8=True)
    assert (idx == ib).all()
    assert np.abs(O - Ob).max() < 1e-12 and np.abs(lse - lb).max() < 1e-11


# ---------------------------------------------------------------- P-n asymmetric route (query blocks of
# `block` rows routed to key blocks of `block_k` keys)
@pytest.mark.parametrize("pool_mode", [0, 1])
def test_one_token_key_blocks_are_dense(orc, pool_mode):
    """One-token key blocks: every pseudo-key is its own token exactly, so any budget gives dense
    attention, whatever the query block size."""
    Q, K, V = small(seed=80, nv=300, ns=4)
    for ratio in (0.05, 0.3):
        p = orc.params(Q, 4, 32, ratio, pool_mode, block_k=1)
        O, lse, idx = orc.forward(p, Q, K, V)
        assert idx.shape[-1] == orc.topk_count(300, ratio)
        assert np.abs(O - sdpa_dense(Q, K, V)).max() < 1e-12


def test_asymmetric_full_density_is_dense(orc):
    Q, K, V = small(seed=81, nv=900, ns=7)
    p = orc.params(Q, 7, 64, 1.0, 1, block_k=32)
    O, lse, idx = orc.forward(p, Q, K, V)
    assert idx.shape[-2:] == (orc.num_blocks(p), orc.num_key_blocks(p))
    assert np.abs(O - sdpa_dense(Q, K, V)).max() < 1e-12


def test_equal_key_blocks_change_nothing(orc):
    Q, K, V = small(seed=82, nv=700, ns=3)
    a = orc.forward(orc.params(Q, 3, 64, 0.2, 1), Q, K, V)
    b = orc.forward(orc.params(Q, 3, 64, 0.2, 1, block_k=64), Q, K, V)
    for x, y in zip(a, b):
        assert (x == y).all()


@pytest.mark.parametrize("block,block_k", [(64, 32), (32, 64), (128, 64)])
@pytest.mark.parametrize("pool_mode", [0, 1])
def test_asymmetric_forward_matches_brute_force(orc, block, block_k, pool_mode):
    Q, K, V = small(seed=83, B=2, nv=2000 - 21, ns=5)
    p = orc.params(Q, 5, block, 0.15, pool_mode, block_k=block_k)
    O, lse, idx = orc.forward(p, Q, K, V)
    Ob, lb, ib = brute.forward(Q, K, V, 5, block, 0.15, pool_mode, block_k=block_k)
    assert (idx == ib).all()
    assert np.abs(O - Ob).max() < 1e-12 and np.abs(lse - lb).max() < 1e-11


def test_asymmetric_selection_is_lexsort_topk(orc):
    Q, K, V = small(seed=84, nv=1500, ns=0)
    p = orc.params(Q, 0, 128, 0.1, 1, block_k=64)
    pooled = orc.pool(p, Q, K, V)
    S = orc.scores(p, pooled["q_mean"], pooled["k_mean"])
    M, Mk = orc.num_blocks(p), orc.num_key_blocks(p)
    assert S.shape[-2:] == (M, Mk) == (12, 24)
    idx = orc.select(p, S)
    Kk = orc.topk_count(Mk, 0.1)
    for h in range(2):
        for I in range(M):
            ref = np.sort(np.lexsort((np.arange(Mk), -S[0, h, I]))[:Kk])
            assert (idx[0, h, I] == ref).all()


def test_asymmetric_fp8_matches_brute_force(orc):
    Q, K, V = small(seed=85, nv=1000 - 24, ns=5)
    p = orc.params(Q, 5, 128, 0.2, 1, block_k=64)
    O, lse, idx, _ = orc.forward_fp8(p, Q, K, V)
    Ob, lb, ib = brute.forward(Q, K, V, 5, 128, 0.2, 1, fp8=True, block_k=64)
    assert (idx == ib).all()
    assert np.abs(O - Ob).max() < 1e-12 and np.abs(lse - lb).max() < 1e-11


# ---------------------------------------------------------------- thread count
def test_results_do_not_depend_on_the_thread_count(orc):
    """OpenMP only splits independent (batch, head, block) units, so the forward, the pool and the
    partition are bit-identical on one thread and on all of them (the benchmark's single-core
    sample relies on this)."""
    Q, K, V = small(seed=11, B=2, H=2, nv=900, ns=7, d=32)
    p = orc.params(Q, 7, 64, 0.2, 1)
    n = orc.num_threads()
    try:
        orc.set_num_threads(1)
        O1, l1, i1 = orc.forward(p, Q, K, V)
        P1 = orc.reblock(p, Q, K)
    finally:
        orc.set_num_threads(n)
    On, ln, i_n = orc.forward(p, Q, K, V)
    Pn = orc.reblock(p, Q, K)
    assert np.array_equal(O1, On) and np.array_equal(l1, ln) and np.array_equal(i1, i_n)
    assert np.array_equal(P1, Pn)
