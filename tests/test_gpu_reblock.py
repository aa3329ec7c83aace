"""GPU parity of the Spark-Reblock partition and of the forward on the partitioned layout.

The permutation must equal the oracle's bit for bit (every decision is taken in binary64 with one
fixed operation order on both sides).  The forward with the partition is held to the attention
tolerances, with the oracle attending through the GPU's validated route.
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import block_sparse_attention_score_amd as sa
import workloads as W
from parity import FWD_MAX_ABS, FWD_REL_L2, check_selection, max_abs, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sa.lib()
    yield
    torch.cuda.synchronize()


def note(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16 if dt == "bf16" else torch.float32)


# (name, B, H, n_video, n_sink, d, block, dtype)
CASES = [
    ("bf16-d128-b128", 1, 3, 11 * 128 + 37, 5, 128, 128, "bf16"),
    ("bf16-d64-b64", 2, 2, 37 * 64 + 1, 0, 64, 64, "bf16"),
    ("bf16-d128-b64", 1, 2, 16 * 64, 64, 128, 64, "bf16"),
    ("fp32-d64-b128", 1, 2, 9 * 128 + 100, 7, 64, 128, "fp32"),
    ("fp32-d128-b64", 1, 1, 25 * 64 + 63, 3, 128, 64, "fp32"),
    ("one-block", 1, 2, 90, 4, 128, 128, "bf16"),
    ("two-blocks", 1, 2, 129, 1, 128, 128, "bf16"),
    # groups of several 2048-position chunks at the top levels, ragged last chunks
    ("bf16-d128-b128-chunked", 1, 2, 70 * 128 + 77, 3, 128, 128, "bf16"),
    ("fp32-d128-b64-chunked", 1, 1, 150 * 64 + 13, 2, 128, 64, "fp32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_reblock_bit_exact(orc, case):
    name, B, H, nv, ns, d, b, dt = case
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=nv + d, dtype=dt)
    note(f"reblock {name}")
    perm = sa.reblock(dev(Q, dt), dev(K, dt), ns, b)
    torch.cuda.synchronize()
    ref = orc.reblock(orc.params(Q, ns, b), Q, K)
    got = perm.cpu().numpy()
    assert (got == ref).all(), f"{(got != ref).sum()} positions differ"


def test_reblock_structured_input_bit_exact(orc):
    wl = W.WORKLOADS["tiny"].with_(dtype="bf16", d=64)
    Q, K, V = W.make_qkv(wl)
    note("reblock on the tiny positional workload")
    perm = sa.reblock(dev(Q, "bf16"), dev(K, "bf16"), 0, 64)
    torch.cuda.synchronize()
    assert (perm.cpu().numpy() == orc.reblock(orc.params(Q, 0, 64), Q, K)).all()


def test_reblock_degenerate_rows(orc):
    """Zero query rows (norm 0: every cosine 0, ties decided by index) and a zero key set."""
    Q, K, V = W.gaussian_qkv(1, 2, 6 * 64 + 10, 2, 64, seed=5, dtype="bf16")
    Q[0, 0, ::3] = 0.0
    K[0, 1, :] = 0.0
    note("reblock with zero rows")
    perm = sa.reblock(dev(Q, "bf16"), dev(K, "bf16"), 2, 64)
    torch.cuda.synchronize()
    assert (perm.cpu().numpy() == orc.reblock(orc.params(Q, 2, 64), Q, K)).all()


def test_reblock_is_deterministic():
    Q, K, V = W.gaussian_qkv(1, 4, 20 * 128 + 3, 8, 128, seed=8, dtype="bf16")
    Qd, Kd = dev(Q, "bf16"), dev(K, "bf16")
    note("reblock twice")
    a = sa.reblock(Qd, Kd, 8, 128)
    b = sa.reblock(Qd, Kd, 8, 128)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


REBLOCK_MAX = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "reblock_max.json")


def test_reblock_at_the_largest_sizes():
    """The partition at 2^20 video rows (its largest size: 16384 leaves of 64, 14 bisection levels)
    and at the full clip's 245,952 rows with d = 128.  The oracle needs minutes per case there, so
    its permutation is stored as a SHA-256 written by tests/golden/make_reblock_max.py (oracle and
    seeded generators only); the GPU's permutation must hash the same.  It is also checked to be a
    bijection with ascending original indices inside every leaf."""
    cases = json.load(open(REBLOCK_MAX))["cases"]
    for name, c in cases.items():
        nv, b = c["n_video"], c["block"]
        Q, K, _ = W.gaussian_qkv(1, 1, nv, c["n_sink"], c["d"], seed=c["seed"], dtype=c["dtype"])
        note(f"reblock at {name}: N_v={nv} d={c['d']} block={b}")
        perm = sa.reblock(dev(Q, "bf16"), dev(K, "bf16"), c["n_sink"], b)
        torch.cuda.synchronize()
        got = perm.cpu().numpy()
        flat = got[0, 0]
        assert np.array_equal(np.sort(flat), np.arange(nv, dtype=flat.dtype)), "not a bijection"
        full = nv // b * b  # leaves of b tokens, then the ragged remainder as the last leaf
        assert (np.diff(flat[:full].reshape(-1, b), axis=1) > 0).all() and (np.diff(flat[full:]) > 0).all(), \
            "a leaf is not in ascending index order"
        assert flat[:8].tolist() == c["perm_head"] and flat[-8:].tolist() == c["perm_tail"]
        assert hashlib.sha256(got.astype("<i4").tobytes()).hexdigest() == c["perm_sha256"], name


def test_reblock_720p_bit_exact_and_forward(orc):
    """The 720p-like latent (75,600 video + 512 sink tokens, 24 heads) in full on the GPU; the oracle
    checks the partition of 3 heads bit for bit, and the forward on sampled query blocks."""
    wl = W.WORKLOADS["reblock720p"]
    Q, K, V = W.make_qkv(wl)
    note("reblock 720p")
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    perm = sa.reblock(Qd, Kd, wl.n_sink, wl.block)
    O, lse, idx = sa.forward(Qd, Kd, Vd, wl.n_sink, wl.block, 0.1, perm=perm, return_lse=True, return_idx=True)
    torch.cuda.synchronize()
    heads = [0, 11, 23]
    Qs, Ks, Vs = (np.ascontiguousarray(x[:, heads]) for x in (Q, K, V))
    p = orc.params(Qs, wl.n_sink, wl.block, 0.1, 1)
    ref = orc.reblock(p, Qs, Ks)
    gperm = perm.cpu().numpy()[:, heads]
    assert (gperm == ref).all(), f"{(gperm != ref).sum()} positions differ"
    # forward: the route is checked in the partitioned layout; sampled blocks are attended by the oracle
    nv = wl.n_video

    def permuted(X):
        Y = X.copy()
        for h in range(len(heads)):
            Y[0, h, :nv] = X[0, h][ref[0, h]]
        return Y

    Qp, Kp, Vp = permuted(Qs), permuted(Ks), permuted(Vs)
    pooled = orc.pool(p, Qp, Kp, Vp)
    S = orc.scores(p, pooled["q_mean"], pooled["k_mean"])
    gidx = idx.cpu().numpy()[:, heads]
    bad, _ = check_selection(gidx, S)
    assert bad == 0
    M = gidx.shape[2]
    rng = np.random.default_rng(3)
    qb = np.array([(h, I) for h in range(len(heads)) for I in rng.choice(M, 4, replace=False)] + [(0, M - 1)])
    Os, ls = orc.attend_blocks(p, Qp, Kp, Vp, pooled, gidx, qb)
    Og, lg = O.float().cpu().numpy()[:, heads], lse.cpu().numpy()[:, heads]
    g_rows, r_rows, gl, rl = [], [], [], []
    for n, (h, I) in enumerate(qb):
        lo, hi = I * wl.block, min(nv, (I + 1) * wl.block)
        rows = ref[0, h, lo:hi]  # original token rows of this partitioned block
        g_rows.append(Og[0, h, rows]); r_rows.append(Os[n, :hi - lo])
        gl.append(lg[0, h, rows]); rl.append(ls[n, :hi - lo])
    g_rows, r_rows = np.concatenate(g_rows), np.concatenate(r_rows)
    e2, ea = rel_l2(g_rows, r_rows), max_abs(g_rows, r_rows)
    el = max_abs(np.concatenate(gl), np.concatenate(rl))
    print(f"reblocked forward: rel-L2 {e2:.3e} max-abs {ea:.3e} lse {el:.3e}")
    assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS and el <= FWD_MAX_ABS


def test_reblock_720p_every_head_as_if_alone():
    """Heads are partitioned independently: the 720p-like latent's 24-head partition equals, head
    by head, the partition of that head passed on its own.  Every head of the batch (with its
    offsets into the per-head workspace) is pinned against a single-head call, and the oracle pins
    the single-head path."""
    wl = W.WORKLOADS["reblock720p"]
    Q, K, _ = W.make_qkv(wl)
    note("reblock 720p: all heads vs each head alone")
    Qd, Kd = dev(Q, "bf16"), dev(K, "bf16")
    full = sa.reblock(Qd, Kd, wl.n_sink, wl.block)
    alone = [sa.reblock(Qd[:, h:h + 1].contiguous(), Kd[:, h:h + 1].contiguous(), wl.n_sink, wl.block)
             for h in range(Qd.shape[1])]
    torch.cuda.synchronize()
    for h, a in enumerate(alone):
        assert torch.equal(full[:, h:h + 1], a), f"head {h}"


# ---- separate key partition: keys bisected under the queries' second moment (the same
# partitioner with the roles of Q and K exchanged), keys and values in their own order
KV_CASES = [
    ("bf16-d128-b128", 1, 3, 11 * 128 + 37, 5, 128, 128, "bf16"),
    ("bf16-d64-b64", 2, 2, 37 * 64 + 1, 0, 64, 64, "bf16"),
    ("fp32-d64-b128", 1, 2, 9 * 128 + 100, 7, 64, 128, "fp32"),
]


@pytest.mark.parametrize("case", KV_CASES, ids=[c[0] for c in KV_CASES])
def test_key_partition_bit_exact_and_forward(orc, case):
    name, B, H, nv, ns, d, b, dt = case
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=nv + 7, dtype=dt)
    note(f"key partition {name}")
    Qd, Kd, Vd = dev(Q, dt), dev(K, dt), dev(V, dt)
    perm_q = sa.reblock(Qd, Kd, ns, b)
    perm_k = sa.reblock(Kd, Qd, ns, b)
    O, lse, idx = sa.forward(Qd, Kd, Vd, ns, b, 0.2, perm=perm_q, perm_k=perm_k, return_lse=True,
                             return_idx=True)
    torch.cuda.synchronize()
    p = orc.params(Q, ns, b, 0.2, 1)
    rq, rk = orc.reblock(p, Q, K), orc.reblock(p, K, Q)
    assert (perm_q.cpu().numpy() == rq).all()
    assert (perm_k.cpu().numpy() == rk).all()
    # route validated against the oracle's scores in the two block layouts
    Qp, Kp, Vp = Q.copy(), K.copy(), V.copy()
    for bb in range(B):
        for h in range(H):
            Qp[bb, h, :nv] = Q[bb, h][rq[bb, h]]
            Kp[bb, h, :nv], Vp[bb, h, :nv] = K[bb, h][rk[bb, h]], V[bb, h][rk[bb, h]]
    pooled = orc.pool(p, Qp, Kp, Vp)
    gidx = idx.cpu().numpy()
    bad, _ = check_selection(gidx, orc.scores(p, pooled["q_mean"], pooled["k_mean"]))
    assert bad == 0
    Oref, lref, _ = orc.forward(p, Q, K, V, perm=rq, perm_k=rk, idx=gidx)
    Og = O.float().cpu().numpy()
    e2, ea, el = rel_l2(Og, Oref), max_abs(Og, Oref), max_abs(lse.cpu().numpy(), lref)
    print(f"key-partitioned forward: rel-L2 {e2:.3e} max-abs {ea:.3e} lse {el:.3e}")
    assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS and el <= FWD_MAX_ABS


def test_key_partition_alone_equals_forward_kv_with_identity(orc):
    """Only the keys partitioned (no query partition): spark_attn_forward_kv with perm_q = NULL."""
    Q, K, V = W.gaussian_qkv(1, 2, 21 * 64 + 5, 3, 64, seed=41, dtype="bf16")
    ns, b = 3, 64
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    note("key partition only")
    perm_k = sa.reblock(Kd, Qd, ns, b)
    O, idx = sa.forward(Qd, Kd, Vd, ns, b, 0.25, perm_k=perm_k, return_idx=True)
    torch.cuda.synchronize()
    p = orc.params(Q, ns, b, 0.25, 1)
    rk = perm_k.cpu().numpy()
    gidx = idx.cpu().numpy()
    Oref, _, _ = orc.forward(p, Q, K, V, perm_k=rk, idx=gidx)
    Og = O.float().cpu().numpy()
    assert rel_l2(Og, Oref) <= FWD_REL_L2 and max_abs(Og, Oref) <= FWD_MAX_ABS


def test_key_partition_720p(orc):
    """The 720p-like latent: the key partition of 3 heads bit for bit, and the doubly
    partitioned forward on sampled query blocks."""
    wl = W.WORKLOADS["reblock720p"]
    Q, K, V = W.make_qkv(wl)
    note("key partition 720p")
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    perm_q = sa.reblock(Qd, Kd, wl.n_sink, wl.block)
    perm_k = sa.reblock(Kd, Qd, wl.n_sink, wl.block)
    O, lse, idx = sa.forward(Qd, Kd, Vd, wl.n_sink, wl.block, 0.1, perm=perm_q, perm_k=perm_k,
                             return_lse=True, return_idx=True)
    torch.cuda.synchronize()
    heads = [0, 11, 23]
    Qs, Ks, Vs = (np.ascontiguousarray(x[:, heads]) for x in (Q, K, V))
    p = orc.params(Qs, wl.n_sink, wl.block, 0.1, 1)
    rq, rk = orc.reblock(p, Qs, Ks), orc.reblock(p, Ks, Qs)
    assert (perm_q.cpu().numpy()[:, heads] == rq).all()
    assert (perm_k.cpu().numpy()[:, heads] == rk).all()
    nv = wl.n_video
    Qp, Kp, Vp = Qs.copy(), Ks.copy(), Vs.copy()
    for h in range(len(heads)):
        Qp[0, h, :nv] = Qs[0, h][rq[0, h]]
        Kp[0, h, :nv], Vp[0, h, :nv] = Ks[0, h][rk[0, h]], Vs[0, h][rk[0, h]]
    pooled = orc.pool(p, Qp, Kp, Vp)
    gidx = idx.cpu().numpy()[:, heads]
    bad, _ = check_selection(gidx, orc.scores(p, pooled["q_mean"], pooled["k_mean"]))
    assert bad == 0
    M = gidx.shape[2]
    rng = np.random.default_rng(4)
    qb = np.array([(h, I) for h in range(len(heads)) for I in rng.choice(M, 4, replace=False)] + [(0, M - 1)])
    Os, ls = orc.attend_blocks(p, Qp, Kp, Vp, pooled, gidx, qb)
    Og, lg = O.float().cpu().numpy()[:, heads], lse.cpu().numpy()[:, heads]
    g_rows, r_rows, gl, rl = [], [], [], []
    for n, (h, I) in enumerate(qb):
        lo, hi = I * wl.block, min(nv, (I + 1) * wl.block)
        rows = rq[0, h, lo:hi]
        g_rows.append(Og[0, h, rows]); r_rows.append(Os[n, :hi - lo])
        gl.append(lg[0, h, rows]); rl.append(ls[n, :hi - lo])
    g_rows, r_rows = np.concatenate(g_rows), np.concatenate(r_rows)
    e2, ea = rel_l2(g_rows, r_rows), max_abs(g_rows, r_rows)
    el = max_abs(np.concatenate(gl), np.concatenate(rl))
    print(f"doubly partitioned forward: rel-L2 {e2:.3e} max-abs {ea:.3e} lse {el:.3e}")
    assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS and el <= FWD_MAX_ABS
