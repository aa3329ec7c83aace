"""The benchmark's own arithmetic, on the CPU: the algorithmic work it divides by the measured
times (one multiply-add for the logit and one for the value per query-key pair, counted from the
actual route), and its vectorised route check against the per-row rule of the parity tests."""
import types

import numpy as np
import pytest

import bench
from parity import check_selection


def brute_flops(wl, idx, counts, bk):
    """Query-key pairs of each branch counted one query block at a time."""
    b, nv, ns, d, N = wl.block, wl.n_video, wl.n_sink, wl.d, wl.N
    M, Mk = -(-nv // b), -(-nv // bk)
    qsize = [min(b, nv - I * b) for I in range(M)]
    ksize = [min(bk, nv - J * bk) for J in range(Mk)]
    sel = comp = 0
    for bh in range(wl.B * wl.H):
        for I in range(M):
            row = idx[0, bh, I] if counts is None else idx[0, bh, I, :counts[0, bh, I]]
            sel += qsize[I] * sum(ksize[J] for J in row)
            comp += qsize[I] * (Mk - len(row))
    BH = wl.B * wl.H
    return 4.0 * d * sel, 4.0 * d * nv * ns * BH, 4.0 * d * comp, 4.0 * d * ns * N * BH


def workload(nv, ns, d, b, H):
    return types.SimpleNamespace(block=b, n_video=nv, n_sink=ns, d=d, N=nv + ns, B=1, H=H)


@pytest.mark.parametrize("nv,ns,b,bk,K", [(1000, 7, 64, 64, 3), (1000, 0, 128, 64, 5), (513, 3, 64, 128, 2)])
def test_algorithmic_flops_fixed_route(nv, ns, b, bk, K):
    wl = workload(nv, ns, 32, b, 2)
    M, Mk = -(-nv // b), -(-nv // bk)
    rng = np.random.default_rng(nv + bk)
    idx = np.stack([np.sort(rng.choice(Mk, K, replace=False)) for _ in range(2 * M)]).reshape(1, 2, M, K)
    got = bench.algorithmic_flops(idx, wl, K, None, 0 if bk == b else bk)
    assert got == brute_flops(wl, idx, None, bk)


def test_algorithmic_flops_variable_route():
    nv, ns, b = 1000, 5, 64
    wl = workload(nv, ns, 32, b, 2)
    M = -(-nv // b)
    rng = np.random.default_rng(2)
    counts = rng.integers(0, M + 1, (1, 2, M)).astype(np.int32)
    counts[0, 0, 0], counts[0, 1, M - 1] = 0, M  # nothing kept; everything kept (the ragged block)
    idx = np.full((1, 2, M, M), -1, np.int32)
    for bh in range(2):
        for I in range(M):
            idx[0, bh, I, :counts[0, bh, I]] = np.sort(rng.choice(M, counts[0, bh, I], replace=False))
    got = bench.algorithmic_flops(idx, wl, None, counts, 0)
    assert got == brute_flops(wl, idx, counts, b)


def test_route_check_agrees_with_the_per_row_rule():
    rng = np.random.default_rng(3)
    R, M, K = 200, 40, 6
    S = rng.standard_normal((R, M))
    S[:20, 10] = S[:20, 11]  # exact ties at arbitrary ranks
    idx = np.sort(np.argsort(-S, axis=1, kind="stable")[:, :K], axis=1).astype(np.int32)
    assert bench.route_check(idx, S) == 0 == check_selection(idx, S)[0]
    bad = idx.copy()
    # a clearly lower block swapped in; an unsorted row; a duplicated entry
    for r, how in ((3, "swap"), (50, "order"), (120, "dup")):
        if how == "swap":
            worst = int(np.argmin(S[r]))
            bad[r] = np.sort(np.r_[bad[r, 1:], worst])
        elif how == "order":
            bad[r] = bad[r, ::-1]
        else:
            bad[r, 1] = bad[r, 0]
    assert bench.route_check(bad, S) == 3
    assert check_selection(bad, S)[0] == 3


def test_cpu_leg_checks_routes_and_sampled_rows(orc):
    """The benchmark's CPU leg accepts rows equal to the oracle's and a route equal to its top-K,
    and rejects a route with a demoted block or a sampled row off by more than the bounds (the
    GPU rows are stood in for by the oracle's own, so this runs on the CPU)."""
    import workloads as W

    wl = W.WORKLOADS["tiny"]
    Q, K, V = W.make_qkv(wl)
    p = orc.params(Q, wl.n_sink, wl.block, 0.1, 1)
    pooled = orc.pool(p, Q, K, V)
    idx = orc.select(p, orc.scores(p, pooled["q_mean"], pooled["k_mean"]))
    M = idx.shape[2]
    qb, sq = bench.cpu_sample(wl, M, 5)
    assert len(sq) == 0 and qb.shape == (5, 2)  # no sink rows in this workload
    O, L = orc.attend_blocks(p, Q, K, V, pooled, idx, qb)
    rows = bench.sample_rows(wl, M, qb)
    G = np.concatenate([O[n, :len(r)] for n, r in enumerate(rows)])
    GL = np.concatenate([L[n, :len(r)] for n, r in enumerate(rows)])
    _, chk = bench.cpu_baseline(wl, 0.1, Q, K, V, idx, 1.0, qb, sq, (G, GL), single_core_blocks=1)
    assert chk["ok"] and chk["route_rows_violating_near_tie_rule"] == 0 and chk["rel_l2"] == 0.0
    G2 = G.copy()
    G2[3, 7] += 0.05  # beyond the max-abs bound
    _, chk = bench.cpu_baseline(wl, 0.1, Q, K, V, idx, 1.0, qb, sq, (G2, GL), single_core_blocks=1)
    assert not chk["ok"] and chk["max_abs"] > bench.FWD_MAX_ABS
    bad_idx = idx.copy()  # replace the top-scoring block of one row by the lowest-scoring one
    S = orc.scores(p, pooled["q_mean"], pooled["k_mean"])
    row = S[0, 1, 3]
    top, low = int(np.argmax(row)), int(np.argmin(row))
    sel = [j for j in bad_idx[0, 1, 3] if j != top] + [low]
    bad_idx[0, 1, 3] = np.sort(sel)
    _, chk = bench.cpu_baseline(wl, 0.1, Q, K, V, bad_idx, 1.0, qb, sq, (G, GL), single_core_blocks=1)
    assert not chk["ok"] and chk["route_rows_violating_near_tie_rule"] == 1
