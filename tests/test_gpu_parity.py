"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle on the same seeded
inputs.

  pool      fp32 summaries vs binary64, relative 2e-5
  select    route sets bit-exact except inside the near-tie window (tests/parity.py)
  forward   rel-L2 <= 1e-2 and max-abs <= 2e-2 (bf16 matrix-core stages vs binary64); the oracle
            attends with the GPU's validated route, so an accepted near-tie swap is not scored as
            an attention error
  gather    bit-exact
Sizes span several tiles with ragged tails; the full-size shapes are checked on sampled query
blocks, in the launch configuration the benchmark times.
"""
import math
import numpy as np
import pytest
import torch

import block_sparse_attention_score_amd as sa
import workloads as W
from parity import (FWD_MAX_ABS, FWD_REL_L2, POOL_RTOL, check_selection, check_selection_rows, max_abs,
                    rel_l2)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sa.lib()
    yield
    torch.cuda.synchronize()


def note(msg):
    print(f"\n[gpu-case] {msg}", flush=True)


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


# (name, B, H, n_video, n_sink, d, block, ratio, dtype)
SMALL = [
    ("ragged-bf16-d128-b128", 2, 2, 5 * 128 + 37, 70, 128, 128, 0.3, "bf16"),
    ("ragged-bf16-d64-b128", 1, 3, 7 * 128 + 1, 3, 64, 128, 0.2, "bf16"),
    ("ragged-bf16-d128-b64", 1, 2, 20 * 64 + 63, 130, 128, 64, 0.1, "bf16"),
    ("fp32-d64-b64", 1, 2, 33 * 64 - 5, 64, 64, 64, 0.1, "fp32"),
    ("fp32-d128-b128", 1, 1, 9 * 128 + 100, 17, 128, 128, 0.25, "fp32"),
    ("one-block-no-sink", 1, 2, 100, 0, 128, 128, 0.1, "bf16"),
    ("one-sink-row", 1, 2, 4 * 128, 1, 128, 128, 0.5, "bf16"),
    ("full-density", 1, 2, 6 * 128 + 9, 40, 128, 128, 1.0, "bf16"),
    ("many-blocks-b64", 1, 1, 150 * 64 + 11, 96, 64, 64, 0.07, "bf16"),
]


def small_inputs(case, seed=0):
    name, B, H, nv, ns, d, b, r, dt = case
    return W.gaussian_qkv(B, H, nv, ns, d, seed=seed + nv, dtype=dt)


@pytest.mark.parametrize("pool_mode", [0, 1])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_pool_parity(orc, case, pool_mode):
    name, B, H, nv, ns, d, b, r, dt = case
    Q, K, V = small_inputs(case)
    note(f"pool {name} mode={pool_mode} B={B} H={H} Nv={nv} Ns={ns} d={d} b={b}")
    out = sa.pool(to_dev(Q, dt), to_dev(K, dt), to_dev(V, dt), ns, b, pool_mode)
    torch.cuda.synchronize()
    ref = orc.pool(orc.params(Q, ns, b, r, pool_mode), Q, K, V)
    for key in ("q_mean", "k_mean", "k_sum", "v_sum", "anchor"):
        g, o = host(out[key]), ref[key]
        err = np.abs(g - o).max() / max(np.abs(o).max(), 1e-30)
        assert err < POOL_RTOL, (key, err)
    assert np.abs(host(out["bias"]) - ref["bias"]).max() < 1e-4


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_select_parity(orc, case):
    name, B, H, nv, ns, d, b, r, dt = case
    Q, K, V = small_inputs(case)
    note(f"select {name}")
    Qd = to_dev(Q, dt)
    pooled = sa.pool(Qd, to_dev(K, dt), to_dev(V, dt), ns, b)
    idx, S = sa.select(pooled["q_mean"], pooled["k_mean"], Qd, ns, b, r, with_scores=True)
    torch.cuda.synchronize()
    p = orc.params(Q, ns, b, r)
    ref = orc.pool(p, Q, K, V)
    S_ref = orc.scores(p, ref["q_mean"], ref["k_mean"])
    assert np.abs(host(S) - S_ref).max() <= 1e-5 * np.abs(S_ref).max()
    bad, differ = check_selection(host(idx), S_ref)
    assert bad == 0
    print(f"rows differing from the exact oracle set (inside the near-tie window): {differ}")


# (name, M, K ratio, kind): crafted block means drive the selection directly
TOPK_CASES = [
    ("random-1922", 1922, 0.1, "random"),
    ("random-500", 500, 0.3, "random"),
    ("ties-1922", 1922, 0.1, "ties"),
    ("all-equal-1000", 1000, 0.1, "zero-q"),
    ("few-values-700", 700, 0.2, "few"),
    ("random-5000", 5000, 0.1, "random"),
    ("ties-5000", 5000, 0.05, "ties"),
    ("one-block", 1, 0.1, "random"),
]


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_select_is_exact_topk_of_its_scores(case):
    """The route must be exactly the K largest of the GPU's own score row by (score desc, J asc),
    listed in ascending J, whatever the score distribution (ties decided by the lower index)."""
    name, M, r, kind = case
    B, H, d, b = 1, 2, 64, 64
    rng = np.random.default_rng(M)
    qm = rng.standard_normal((B, H, M, d)).astype(np.float32)
    km = rng.standard_normal((B, H, M, d)).astype(np.float32)
    if kind == "ties":  # key means drawn from five vectors: five distinct scores per row
        km = rng.standard_normal((B, H, 5, d)).astype(np.float32)[:, :, rng.integers(0, 5, M)]
    elif kind == "zero-q":  # every score 0: the K lowest indices
        qm[:] = 0.0
    elif kind == "few":  # small integer-valued means: many exact score ties
        qm = rng.integers(-2, 3, (B, H, M, d)).astype(np.float32)
        km = rng.integers(-1, 2, (B, H, M, d)).astype(np.float32)
    Q = torch.zeros(B, H, M * b, d, device="cuda", dtype=torch.bfloat16)  # shapes only
    note(f"topk {name}")
    qm, km = np.ascontiguousarray(qm), np.ascontiguousarray(km)
    idx, S = sa.select(torch.from_numpy(qm).cuda(), torch.from_numpy(km).cuda(), Q, 0, b, r, with_scores=True)
    torch.cuda.synchronize()
    Sh, gi = host(S), host(idx)
    K = gi.shape[-1]
    for bb in range(B):
        for h in range(H):
            for I in range(M):
                row = Sh[bb, h, I]
                top = np.sort(np.lexsort((np.arange(M), -row))[:K])
                assert (gi[bb, h, I] == top).all(), (bb, h, I)


def permute_rows(X, perm):
    Y = X.copy()
    nv = perm.shape[-1]
    for bb in range(X.shape[0]):
        for h in range(X.shape[1]):
            Y[bb, h, :nv] = X[bb, h][perm[bb, h]]
    return Y


def forward_check(orc, Q, K, V, ns, b, r, pool_mode, dt, perm=None, block_k=0):
    Qd, Kd, Vd = to_dev(Q, dt), to_dev(K, dt), to_dev(V, dt)
    permd = torch.from_numpy(perm).cuda() if perm is not None else None
    O, lse, idx = sa.forward(Qd, Kd, Vd, ns, b, r, pool_mode, perm=permd, return_lse=True, return_idx=True,
                             block_k=block_k)
    torch.cuda.synchronize()
    p = orc.params(Q, ns, b, r, pool_mode, block_k=block_k)
    gidx = host(idx)
    # validate the route against the oracle's scores (in the permuted layout when a perm is given)
    Qp, Kp, Vp = (permute_rows(x, perm) for x in (Q, K, V)) if perm is not None else (Q, K, V)
    ref = orc.pool(p, Qp, Kp, Vp)
    bad, _ = check_selection(gidx, orc.scores(p, ref["q_mean"], ref["k_mean"]))
    assert bad == 0
    Oref, lref, _ = orc.forward(p, Q, K, V, perm=perm, idx=gidx)
    Og = host(O)
    e2, ea = rel_l2(Og, Oref), max_abs(Og, Oref)
    el = max_abs(host(lse), lref)
    print(f"rel-L2 {e2:.3e} max-abs {ea:.3e} lse max-abs {el:.3e}")
    assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS and el <= FWD_MAX_ABS
    return Og, Oref


@pytest.mark.parametrize("pool_mode", [0, 1])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_forward_parity(orc, case, pool_mode):
    name, B, H, nv, ns, d, b, r, dt = case
    Q, K, V = small_inputs(case)
    note(f"forward {name} mode={pool_mode}")
    forward_check(orc, Q, K, V, ns, b, r, pool_mode, dt)


def test_forward_tiny_workload(orc):
    wl = W.WORKLOADS["tiny"]
    Q, K, V = W.make_qkv(wl)
    for pm in wl.pool_modes:
        note(f"forward tiny workload mode={pm}")
        forward_check(orc, Q, K, V, wl.n_sink, wl.block, wl.ratios[0], pm, wl.dtype)


def test_full_density_equals_dense(orc):
    Q, K, V = W.gaussian_qkv(1, 2, 5 * 128 + 3, 21, 128, seed=5, dtype="bf16")
    note("forward at K = M vs dense")
    O = sa.forward(to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16"), 21, 128, 1.0)
    torch.cuda.synchronize()
    Od, _ = orc.dense(orc.params(Q, 21, 128), Q, K, V)
    assert rel_l2(host(O), Od) <= FWD_REL_L2 and max_abs(host(O), Od) <= FWD_MAX_ABS


def test_forward_with_permutation(orc):
    B, H, nv, ns, d, b = 1, 2, 6 * 128 + 50, 33, 128, 128
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=17, dtype="bf16")
    rng = np.random.default_rng(3)
    perm = np.stack([[rng.permutation(nv) for _ in range(H)] for _ in range(B)]).astype(np.int32)
    note("forward with a permutation")
    forward_check(orc, Q, K, V, ns, b, 0.3, 1, "bf16", perm=perm)


# asymmetric route: query blocks of `block` rows, key blocks of `block_k` keys
ASYM = [
    ("q128-k64", 1, 2, 11 * 128 + 37, 5, 128, 128, 64, 0.15, "bf16"),
    ("q64-k128", 1, 2, 23 * 64 + 5, 70, 128, 64, 128, 0.2, "bf16"),
    ("q128-k64-d64", 2, 1, 6 * 128 + 1, 0, 64, 128, 64, 0.3, "bf16"),
    ("q128-k64-fp32", 1, 1, 5 * 128 + 90, 3, 128, 128, 64, 0.25, "fp32"),
]


@pytest.mark.parametrize("pool_mode", [0, 1])
@pytest.mark.parametrize("case", ASYM, ids=[c[0] for c in ASYM])
def test_forward_asymmetric_route(orc, case, pool_mode):
    name, B, H, nv, ns, d, b, bk, r, dt = case
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=nv + bk, dtype=dt)
    note(f"forward asymmetric {name} mode={pool_mode}")
    forward_check(orc, Q, K, V, ns, b, r, pool_mode, dt, block_k=bk)


def test_asymmetric_pool_and_scores(orc):
    B, H, nv, ns, d, b, bk = 1, 2, 9 * 128 + 40, 6, 128, 128, 64
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=31, dtype="bf16")
    Qd, Kd, Vd = to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16")
    note("asymmetric pool and block scores")
    out = sa.pool(Qd, Kd, Vd, ns, b, block_k=bk)
    idx, S = sa.select(out["q_mean"], out["k_mean"], Qd, ns, b, 0.2, with_scores=True, block_k=bk)
    torch.cuda.synchronize()
    p = orc.params(Q.astype(np.float32), ns, b, 0.2, 1, block_k=bk)
    ref = orc.pool(p, host(Qd), host(Kd), host(Vd))
    assert out["k_mean"].shape[2] == orc.num_key_blocks(p) and out["q_mean"].shape[2] == orc.num_blocks(p)
    for key in ("q_mean", "k_mean", "k_sum", "v_sum", "anchor"):
        g, o = host(out[key]), ref[key]
        assert np.abs(g - o).max() / np.abs(o).max() < POOL_RTOL, key
    Sref = orc.scores(p, ref["q_mean"], ref["k_mean"])
    assert np.abs(host(S) - Sref).max() <= 1e-5 * np.abs(Sref).max()
    bad, _ = check_selection(idx.cpu().numpy(), Sref)
    assert bad == 0


def test_gather_rows_bit_exact():
    B, H, nv, ns, d = 2, 3, 1000, 7, 128
    X = torch.randn(B, H, nv + ns, d, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(1)
    perm = np.stack([[rng.permutation(nv) for _ in range(H)] for _ in range(B)]).astype(np.int32)
    note("gather rows")
    Y = sa.gather_rows(X, torch.from_numpy(perm).cuda(), ns)
    torch.cuda.synchronize()
    Xh, Yh = X.view(torch.int16).cpu().numpy(), Y.view(torch.int16).cpu().numpy()
    for bb in range(B):
        for h in range(H):
            assert (Yh[bb, h, :nv] == Xh[bb, h][perm[bb, h]]).all()
            assert (Yh[bb, h, nv:] == Xh[bb, h, nv:]).all()


def test_forward_is_deterministic():
    Q, K, V = W.gaussian_qkv(1, 2, 9 * 128 + 5, 64, 128, seed=9, dtype="bf16")
    Qd, Kd, Vd = to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16")
    note("determinism")
    a = sa.forward(Qd, Kd, Vd, 64, 128, 0.2, return_lse=True, return_idx=True)
    b = sa.forward(Qd, Kd, Vd, 64, 128, 0.2, return_lse=True, return_idx=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------- full-size shapes, sampled
def sampled_check(orc, wl, ratio, n_blocks=24, n_sink_rows=8, seed=0, edges=False):
    """Full GPU forward at the workload's real shape (the benchmark's launch configuration); the
    oracle pools everything and validates every route row of every head (near-tie rule against
    binary64 scores from its block means), and attends sampled query blocks and sink rows.  With
    edges, the sample also holds, deterministically: one query block of every head; the blocks on
    both sides of each boundary between the runs of blocks the eight XCDs take (runs of ceil(M/8)
    blocks of one head); the first and the ragged last block; and the first and last row of every
    sink-query workgroup (128 rows each) of the first and last head."""
    Q, K, V = W.make_qkv(wl)
    note(f"sampled {wl.name} ratio={ratio} N={wl.N} H={wl.H}")
    Qd, Kd, Vd = to_dev(Q, wl.dtype), to_dev(K, wl.dtype), to_dev(V, wl.dtype)
    O, lse, idx = sa.forward(Qd, Kd, Vd, wl.n_sink, wl.block, ratio, return_lse=True, return_idx=True)
    pooled_g = sa.pool(Qd, Kd, Vd, wl.n_sink, wl.block)
    torch.cuda.synchronize()
    del Qd, Kd, Vd
    p = orc.params(Q, wl.n_sink, wl.block, ratio, 1)
    ref = orc.pool(p, Q, K, V)
    for key in ("q_mean", "k_mean", "k_sum", "v_sum", "anchor"):
        g, o = host(pooled_g[key]), ref[key]
        assert np.abs(g - o).max() / np.abs(o).max() < POOL_RTOL, key
    gidx = host(idx)
    M = gidx.shape[2]
    s = 1.0 / math.sqrt(wl.d)  # scores of every route row, from the oracle means
    qm, km = ref["q_mean"][0], ref["k_mean"][0]
    bad = 0
    for bh in range(wl.H):
        bad += int((~check_selection_rows(gidx[0, bh], s * (qm[bh] @ km[bh].T))).sum())
    print(f"{wl.name}: route rows checked {wl.H * M}, outside the near-tie rule {bad}", flush=True)
    assert bad == 0
    rng = np.random.default_rng(seed)
    qb = [(int(bh), int(I)) for bh, I in zip(rng.integers(0, wl.H, n_blocks), rng.integers(0, M, n_blocks))]
    qb += [(wl.H - 1, M - 1)]  # the ragged last block
    sinks = [(int(bh), int(j)) for bh, j in zip(rng.integers(0, wl.H, n_sink_rows),
                                                rng.integers(0, wl.n_sink, n_sink_rows))]
    if edges:
        C = -(-M // 8)
        qb += [(bh, (bh * 997 + 13) % M) for bh in range(wl.H)]
        qb += [(x % wl.H, I) for x in range(1, 8) for I in (x * C - 1, x * C) if I < M]
        qb += [(0, 0), (0, M - 1)]
        rows = sorted({min(j, wl.n_sink - 1) for t in range(0, wl.n_sink, wl.block) for j in (t, t + wl.block - 1)})
        sinks += [(bh, j) for bh in (0, wl.H - 1) for j in rows]
    qb = sorted(set(qb)) + sorted(set((bh, M + j) for bh, j in sinks))
    Os, ls = orc.attend_blocks(p, Q, K, V, ref, gidx, np.array(qb))
    Og, lg = host(O), host(lse)
    g_rows, r_rows, gl, rl = [], [], [], []
    for n, (bh, I) in enumerate(qb):
        if I < M:
            lo, hi = I * wl.block, min(wl.n_video, (I + 1) * wl.block)
            g_rows.append(Og[0, bh, lo:hi]); r_rows.append(Os[n, :hi - lo])
            gl.append(lg[0, bh, lo:hi]); rl.append(ls[n, :hi - lo])
        else:
            row = wl.n_video + I - M
            g_rows.append(Og[0, bh, row:row + 1]); r_rows.append(Os[n, :1])
            gl.append(lg[0, bh, row:row + 1]); rl.append(ls[n, :1])
    g_rows, r_rows = np.concatenate(g_rows), np.concatenate(r_rows)
    e2, ea, el = rel_l2(g_rows, r_rows), max_abs(g_rows, r_rows), max_abs(np.concatenate(gl), np.concatenate(rl))
    nblk = sum(1 for _, I in qb if I < M)
    print(f"{wl.name}: {nblk} query blocks, {len(qb) - nblk} sink rows: rel-L2 {e2:.3e} max-abs {ea:.3e} "
          f"lse {el:.3e}", flush=True)
    assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS and el <= FWD_MAX_ABS


def test_short_clip_sampled(orc):
    sampled_check(orc, W.WORKLOADS["short"], 0.1)


@pytest.mark.parametrize("ratio", [0.1, 0.3])
def test_720p_sampled(orc, ratio):
    sampled_check(orc, W.WORKLOADS["720p"], ratio, n_blocks=12, n_sink_rows=4)


def test_fullclip_sampled(orc):
    sampled_check(orc, W.WORKLOADS["fullclip"], 0.1, n_blocks=12, n_sink_rows=4, edges=True)


def max_size_check(orc, b, bk, seed):
    """One head at the largest key-block count the library accepts (16384 key blocks of bk tokens,
    the last one ragged; query blocks of b), d = 64, 40 sinks.  At this size the top-K re-reads
    each score row from memory instead of holding it in registers.  Sampled route rows are checked
    against the oracle's block means with the near-tie rule, and sampled query blocks (the ragged
    last one included) and sink rows against the oracle's attention."""
    B, H, d, ns, ratio = 1, 1, 64, 40, 0.1
    Mk = 16384
    nv = Mk * bk - 21
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=seed, dtype="bf16")
    note(f"maximum block count M_k={Mk} N_v={nv} d={d} block={b} block_k={bk}")
    Qd, Kd, Vd = to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16")
    O, lse, idx = sa.forward(Qd, Kd, Vd, ns, b, ratio, return_lse=True, return_idx=True,
                             block_k=0 if bk == b else bk)
    torch.cuda.synchronize()
    del Qd, Kd, Vd
    p = orc.params(Q, ns, b, ratio, 1, block_k=0 if bk == b else bk)
    M = -(-nv // b)
    assert orc.num_blocks(p) == M and idx.shape[2] == M and idx.shape[3] == sa.topk_count(Mk, ratio)
    ref = orc.pool(p, Q, K, V)
    assert ref["k_mean"].shape[2] == Mk
    gidx = host(idx)
    rng = np.random.default_rng(1)
    rows = sorted(set(rng.choice(M, 512, replace=False).tolist()) | {0, M - 1})
    s = 1.0 / math.sqrt(d)
    qm, km = ref["q_mean"][0, 0], ref["k_mean"][0, 0]
    S = np.stack([s * km @ qm[I] for I in rows])
    bad, differ = check_selection(gidx[0, 0, rows], S)
    print(f"route rows checked {len(rows)}, outside the near-tie rule {bad}, differing {differ}", flush=True)
    assert bad == 0
    qb = [(0, int(I)) for I in rng.choice(M - 1, 6, replace=False)] + [(0, M - 1)]
    qb += [(0, M + int(j)) for j in rng.choice(ns, 3, replace=False)]
    Os, ls = orc.attend_blocks(p, Q, K, V, ref, gidx, np.array(qb))
    Og, lg = host(O), host(lse)
    g_rows, r_rows, gl, rl = [], [], [], []
    for n, (bh, I) in enumerate(qb):
        lo, hi = (I * b, min(nv, (I + 1) * b)) if I < M else (nv + I - M, nv + I - M + 1)
        g_rows.append(Og[0, bh, lo:hi]); r_rows.append(Os[n, :hi - lo])
        gl.append(lg[0, bh, lo:hi]); rl.append(ls[n, :hi - lo])
    g_rows, r_rows = np.concatenate(g_rows), np.concatenate(r_rows)
    e2, ea, el = rel_l2(g_rows, r_rows), max_abs(g_rows, r_rows), max_abs(np.concatenate(gl), np.concatenate(rl))
    print(f"maximum M_k: rel-L2 {e2:.3e} max-abs {ea:.3e} lse {el:.3e}", flush=True)
    assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS and el <= FWD_MAX_ABS


def test_maximum_block_count(orc):
    """M = M_k = 16384 blocks of 64 (1,048,555 video tokens)."""
    max_size_check(orc, 64, 64, seed=16384)


def test_maximum_key_block_count_asymmetric(orc):
    """The asymmetric route at its largest size: 8192 query blocks of 128 against 16384 key blocks
    of 64."""
    max_size_check(orc, 128, 64, seed=8192)


def test_stage_entry_points_match_forward():
    """pool -> select -> pack -> attend through their own entry points gives exactly what
    spark_attn_forward gives (same kernels, same inputs)."""
    B, H, nv, ns, d, b, r = 1, 2, 7 * 128 + 19, 45, 128, 128, 0.2
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=31, dtype="bf16")
    Qd, Kd, Vd = to_dev(Q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16")
    note("stage entry points vs forward")
    O, lse, idx = sa.forward(Qd, Kd, Vd, ns, b, r, return_lse=True, return_idx=True)
    pooled = sa.pool(Qd, Kd, Vd, ns, b)
    idx2 = sa.select(pooled["q_mean"], pooled["k_mean"], Qd, ns, b, r)
    lse2 = torch.empty_like(lse)
    O2 = sa.attend(Qd, Kd, Vd, pooled, idx2, ns, b, r, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(O, O2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("d,b,dt", [(128, 128, "bf16"), (128, 64, "bf16"), (64, 64, "bf16"), (64, 128, "bf16"),
                                    (128, 64, "fp32"), (64, 64, "fp32")])
def test_attend_explicit_routes(orc, d, b, dt):
    """spark_attn_attend with routes chosen by the test: every selected-block position modulo 32
    (the compressed-branch mask bits), the first and the ragged last block, and K up to M."""
    B, H, ns = 1, 2, 37
    M = 70
    nv = (M - 1) * b + 13
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=d + b, dtype=dt)
    Qd, Kd, Vd = to_dev(Q, dt), to_dev(K, dt), to_dev(V, dt)
    pooled = sa.pool(Qd, Kd, Vd, ns, b)
    rng = np.random.default_rng(b + d)
    for Ksel, ratio in ((3, 3 / M), (9, 9 / M)):
        assert sa.topk_count(M, ratio) == Ksel
        idx = np.empty((B, H, M, Ksel), np.int32)
        for h in range(H):
            for I in range(M):
                fixed = [I % 32, (I * 7) % M, M - 1 if I % 3 == 0 else 0]
                rest = rng.permutation(np.setdiff1d(np.arange(M), fixed))[:Ksel]
                row = list(dict.fromkeys(fixed + list(rest)))[:Ksel]
                idx[0, h, I] = np.sort(row)
        note(f"attend explicit routes d={d} b={b} {dt} K={Ksel}")
        lse = torch.empty(B, H, nv + ns, device="cuda", dtype=torch.float32)
        O = sa.attend(Qd, Kd, Vd, pooled, torch.from_numpy(idx).cuda(), ns, b, ratio, lse=lse)
        torch.cuda.synchronize()
        Oref, lref, _ = orc.forward(orc.params(Q, ns, b, ratio, 1), Q, K, V, idx=idx)
        e2, ea, el = rel_l2(host(O), Oref), max_abs(host(O), Oref), max_abs(host(lse), lref)
        print(f"rel-L2 {e2:.3e} max-abs {ea:.3e} lse {el:.3e}")
        assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS and el <= FWD_MAX_ABS


POOL_PACK = [(c[0], c[1], c[2], c[3], c[4], c[5], c[6], 0, c[8]) for c in SMALL] + [
    (c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], c[9]) for c in ASYM]


@pytest.mark.parametrize("pool_mode", [0, 1])
@pytest.mark.parametrize("case", POOL_PACK, ids=[c[0] for c in POOL_PACK])
def test_pool_pack_equals_pool_then_pack(case, pool_mode):
    """spark_attn_pool_pack writes the same summaries and the same packed bytes as spark_attn_pool
    followed by spark_attn_pack (the fused kernel runs the pooling arithmetic unchanged)."""
    name, B, H, nv, ns, d, b, bk, dt = case
    note(f"pool_pack {name} mode={pool_mode}")
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=nv + 3 * bk + pool_mode, dtype=dt)
    Qd, Kd, Vd = (to_dev(x, dt) for x in (Q, K, V))
    p = sa.params(Qd, ns, b, 0.1, pool_mode, block_k=bk)
    ref = sa.pool(Qd, Kd, Vd, ns, b, pool_mode, block_k=bk)
    nbytes = sa.workspace_size(p, 4)
    packed_ref = torch.zeros(nbytes, device="cuda", dtype=torch.uint8)
    sa.spark_attn_pack(p, Kd, Vd, ref["k_sum"], ref["v_sum"], ref["bias"], packed_ref)
    got = {k: torch.full_like(v, float("nan")) for k, v in ref.items()}
    packed = torch.zeros(nbytes, device="cuda", dtype=torch.uint8)
    sa.spark_attn_pool_pack(p, Qd, Kd, Vd, got["q_mean"], got["k_mean"], got["k_sum"], got["v_sum"],
                            got["bias"], got["anchor"], packed)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), k
    assert torch.equal(packed, packed_ref)


def test_forward_is_deterministic_at_scale():
    """Two calls on the same inputs give the same bits: output, lse and route (bf16 in token order,
    bf16 through a reblock permutation, FP8 carriers).  Every reduction runs in a fixed order; the
    only atomics (max, integer sums, route bits) do not depend on their order."""
    wl = W.WORKLOADS["short"]
    note(f"determinism {wl.name}")
    Q, K, V = (to_dev(x, wl.dtype) for x in W.make_qkv(wl))
    perm = sa.reblock(Q, K, wl.n_sink, wl.block)
    runs = []
    for _ in range(2):
        a = sa.forward(Q, K, V, wl.n_sink, wl.block, 0.1, return_lse=True, return_idx=True)
        b = sa.forward(Q, K, V, wl.n_sink, wl.block, 0.1, perm=perm, return_lse=True, return_idx=True)
        c = sa.forward_fp8(Q, K, V, wl.n_sink, wl.block, 0.1, return_lse=True, return_idx=True)
        torch.cuda.synchronize()
        runs.append([t.clone() for t in (*a, *b, *c)])
    for x, y in zip(*runs):
        assert torch.equal(x, y)


@pytest.mark.parametrize("kind", ["every-tile", "mixed"])
def test_fixed_offset_exact_pass(orc, kind):
    """The attention stage subtracts a per-query Cauchy-Schwarz bound on the logits instead of a
    running maximum, and recomputes with the running maximum every query tile in which a row's
    normaliser falls below 2^-64 (its largest logit more than 64 log2 units under the bound).  A
    sink key of norm 100 along a dimension every query has zeroed puts the bound ~140 log2 units
    above every real logit, so without the exact pass each row's normaliser would underflow and O
    would not be finite.  'mixed': the queries of even video blocks are scaled by 2^-6 (exact in
    bf16), which keeps their bound close, so both passes write parts of one output."""
    B, H, nv, ns, d, b, r = 1, 2, 6 * 128 + 37, 9, 128, 128, 0.2
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=77, dtype="bf16")
    Q[..., 0] = 0.0
    K[:, :, nv + 3, :] = 0.0
    K[:, :, nv + 3, 0] = 100.0
    if kind == "mixed":
        for I in range(0, -(-nv // b), 2):
            Q[:, :, I * b:min(nv, (I + 1) * b)] *= np.float32(2.0 ** -6)
    note(f"fixed-offset exact pass {kind}")
    Og, _ = forward_check(orc, Q, K, V, ns, b, r, 1, "bf16")
    assert np.isfinite(Og).all()


ROUTE_CASES = [(c[0], c[1], c[2], c[3], d) for c in TOPK_CASES for d in (64, 128)]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=[f"{c[0]}-d{c[4]}" for c in ROUTE_CASES])
def test_select_route_against_binary64(orc, case):
    """spark_attn_select without a score matrix requested (the score matrix in the workspace), its
    route against binary64 scores of the same block means: exactly the lexsort top-K where the
    scores are exact in fp32 (integer-valued means, all-zero queries), and within the near-tie rule
    otherwise (including rows of tied key means, whose fp32 scores tie exactly too)."""
    name, M, r, kind, d = case
    B, H, b = 1, 2, 64
    rng = np.random.default_rng(M + d)
    qm = rng.standard_normal((B, H, M, d)).astype(np.float32)
    km = rng.standard_normal((B, H, M, d)).astype(np.float32)
    if kind == "ties":
        km = rng.standard_normal((B, H, 5, d)).astype(np.float32)[:, :, rng.integers(0, 5, M)]
    elif kind == "zero-q":
        qm[:] = 0.0
    elif kind == "few":
        qm = rng.integers(-2, 3, (B, H, M, d)).astype(np.float32)
        km = rng.integers(-1, 2, (B, H, M, d)).astype(np.float32)
    Q = torch.zeros(B, H, M * b, d, device="cuda", dtype=torch.bfloat16)  # shapes only
    note(f"select route {name} d={d}")
    qm, km = np.ascontiguousarray(qm), np.ascontiguousarray(km)
    idx = sa.select(torch.from_numpy(qm).cuda(), torch.from_numpy(km).cuda(), Q, 0, b, r)
    torch.cuda.synchronize()
    gi = host(idx)
    S = (qm.astype(np.float64) @ np.swapaxes(km.astype(np.float64), -1, -2)) / math.sqrt(d)
    K = gi.shape[-1]
    assert K == sa.topk_count(M, r)
    if kind in ("few", "zero-q"):  # every score exact in fp32
        for bb in range(B):
            for h in range(H):
                for I in range(M):
                    top = np.sort(np.lexsort((np.arange(M), -S[bb, h, I]))[:K])
                    assert (gi[bb, h, I] == top).all(), (bb, h, I)
    else:
        bad, differ = check_selection(gi, S)
        assert bad == 0
        print(f"rows differing from the binary64 top-K (inside the near-tie window): {differ}")
