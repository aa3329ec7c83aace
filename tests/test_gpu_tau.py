"""GPU parity of the adaptive-tau path: selection (threshold mu + tau*sigma per head), the
attention stage with a variable route, and the whole forward.

The GPU ranks in fp32 and the oracle in binary64, so a block whose score lies within the near-tie
window of the threshold may go either way; every other block must match.  The forward is held to
the attention tolerances, with the oracle attending through the GPU's validated route.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_score_amd as sa
import workloads as W
from parity import FWD_MAX_ABS, FWD_REL_L2, max_abs, rel_l2

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


def check_tau_route(idx, counts, S, tau, rel=1e-4, floor=1e-6):
    """Number of (row, block) decisions outside the near-threshold window that differ from the
    binary64 rule S_IJ > mean + tau*std, and rows whose list is not ascending."""
    bad = 0
    B, H, M, _ = S.shape
    for b in range(B):
        for h in range(H):
            Sh = S[b, h]
            thr = Sh.mean() + tau * Sh.std()
            delta = rel * abs(thr) + floor * np.abs(Sh).max()
            for I in range(M):
                c = counts[b, h, I]
                row = idx[b, h, I, :c]
                if c > 1 and not (np.diff(row) > 0).all():
                    bad += 1
                got = np.zeros(M, bool)
                got[row] = True
                must = Sh[I] > thr + delta
                may = Sh[I] >= thr - delta
                bad += int((must & ~got).sum() + (got & ~may).sum())
    return bad


# (name, B, H, n_video, n_sink, d, block, dtype)
CASES = [
    ("bf16-d128-b128", 1, 3, 13 * 128 + 37, 5, 128, 128, "bf16"),
    ("bf16-d64-b64", 2, 2, 37 * 64 + 1, 0, 64, 64, "bf16"),
    ("fp32-d64-b128", 1, 2, 9 * 128 + 100, 7, 64, 128, "fp32"),
    ("one-block", 1, 2, 90, 4, 128, 128, "bf16"),
]


@pytest.mark.parametrize("tau", [0.0, 1.0, 2.0])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_select_tau_and_forward(orc, case, tau):
    name, B, H, nv, ns, d, b, dt = case
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=nv + d, dtype=dt)
    note(f"tau {tau} {name}")
    Qd, Kd, Vd = dev(Q, dt), dev(K, dt), dev(V, dt)
    pooled = sa.pool(Qd, Kd, Vd, ns, b)
    idx, counts, stats = sa.select_tau(pooled["q_mean"], pooled["k_mean"], Qd, ns, b, tau, with_stats=True)
    O, lse, fidx, fcounts = sa.forward_tau(Qd, Kd, Vd, ns, b, tau, return_lse=True, return_route=True)
    torch.cuda.synchronize()
    p = orc.params(Q, ns, b, 0.1, 1)
    ref = orc.pool(p, Q, K, V)
    S = orc.scores(p, ref["q_mean"], ref["k_mean"])
    gi, gc = idx.cpu().numpy(), counts.cpu().numpy()
    assert check_tau_route(gi, gc, S, tau) == 0
    st = stats.cpu().numpy()
    assert np.abs(st[..., 0] - S.mean(axis=(2, 3))).max() <= 1e-5 * np.abs(S).max()
    assert np.abs(st[..., 1] - S.std(axis=(2, 3))).max() <= 1e-5 * max(S.std(axis=(2, 3)).max(), np.abs(S).max())
    # the forward's own route is the stage route
    assert (fcounts.cpu().numpy() == gc).all()
    for bb in range(B):
        for h in range(H):
            for I in range(gc.shape[2]):
                assert (fidx.cpu().numpy()[bb, h, I, :gc[bb, h, I]] == gi[bb, h, I, :gc[bb, h, I]]).all()
    Oref, lref, _, _ = orc.forward_tau(p, tau, Q, K, V, idx=gi, counts=gc)
    Og = O.float().cpu().numpy()
    e2, ea, el = rel_l2(Og, Oref), max_abs(Og, Oref), max_abs(lse.cpu().numpy(), lref)
    print(f"kept {gc.mean() / gc.shape[2]:.3f} of the blocks; rel-L2 {e2:.3e} max-abs {ea:.3e} lse {el:.3e}")
    assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS and el <= FWD_MAX_ABS


def test_attend_var_rows_keeping_nothing_and_everything(orc):
    """Hand-made variable routes: rows with no block, rows with every block, ragged rows."""
    B, H, nv, ns, d, b = 1, 2, 20 * 64 + 30, 6, 64, 64
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=77, dtype="bf16")
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    p_dev = sa.params(Qd, ns, b, 0.1, sa.POOL_REWEIGHT)
    M = sa.num_blocks(p_dev)
    rng = np.random.default_rng(5)
    counts = rng.integers(0, M + 1, (B, H, M)).astype(np.int32)
    counts[0, 0, 0], counts[0, 0, 1], counts[0, 1, M - 1] = 0, M, 0
    idx = np.full((B, H, M, M), -1, np.int32)
    for h in range(H):
        for I in range(M):
            idx[0, h, I, :counts[0, h, I]] = np.sort(rng.choice(M, counts[0, h, I], replace=False))
    note("attend_var hand-made routes")
    pooled = sa.pool(Qd, Kd, Vd, ns, b)
    packed = sa.pack(Kd, Vd, pooled, ns, b)
    O = torch.empty_like(Qd)
    lse = torch.empty(B, H, nv + ns, device="cuda", dtype=torch.float32)
    sa.spark_attn_attend_var(p_dev, Qd, packed, torch.from_numpy(idx).cuda(), torch.from_numpy(counts).cuda(),
                             None, O, lse)
    torch.cuda.synchronize()
    p = orc.params(Q, ns, b, 0.1, 1)
    Oref, lref, _, _ = orc.forward_tau(p, 0.0, Q, K, V, idx=idx, counts=counts)
    Og = O.float().cpu().numpy()
    e2, ea, el = rel_l2(Og, Oref), max_abs(Og, Oref), max_abs(lse.cpu().numpy(), lref)
    print(f"rel-L2 {e2:.3e} max-abs {ea:.3e} lse {el:.3e}")
    assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS and el <= FWD_MAX_ABS


def test_tau_on_the_short_clip(orc):
    """The short-clip workload (30,720 + 256 tokens, positional features) at tau = 1, two heads
    checked against the oracle in full."""
    wl = W.WORKLOADS["short"].with_(H=2)
    Q, K, V = W.make_qkv(wl)
    note("tau 1.0 short clip")
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    O, idx, counts = sa.forward_tau(Qd, Kd, Vd, wl.n_sink, wl.block, 1.0, return_route=True)
    torch.cuda.synchronize()
    p = orc.params(Q, wl.n_sink, wl.block, 0.1, 1)
    ref = orc.pool(p, Q, K, V)
    S = orc.scores(p, ref["q_mean"], ref["k_mean"])
    gi, gc = idx.cpu().numpy(), counts.cpu().numpy()
    assert check_tau_route(gi, gc, S, 1.0) == 0
    Oref, _, _, _ = orc.forward_tau(p, 1.0, Q, K, V, idx=gi, counts=gc)
    Og = O.float().cpu().numpy()
    e2, ea = rel_l2(Og, Oref), max_abs(Og, Oref)
    print(f"kept {gc.mean() / gc.shape[2]:.3f} of the blocks; rel-L2 {e2:.3e} max-abs {ea:.3e}")
    assert e2 <= FWD_REL_L2 and ea <= FWD_MAX_ABS


def test_tau_at_the_maximum_block_count(orc):
    """Adaptive-tau selection at the largest block count the library accepts (M = 16384 blocks of
    64, the last one ragged, one head): the statistics run over 2^28 scores and a row may keep up
    to M blocks.  The per-head (mu, sigma) and 512 sampled rows plus the first and last one are
    checked against the binary64 rule on the oracle's block means (the attention over such a
    route is covered at smaller sizes, where the oracle can run it)."""
    B, H, d, b, ns, tau = 1, 1, 64, 64, 0, 1.5
    M = 16384
    nv = M * b - 21
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=1234, dtype="bf16")
    note(f"tau {tau} at the maximum block count M={M}")
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    pooled = sa.pool(Qd, Kd, Vd, ns, b)
    idx, counts, stats = sa.select_tau(pooled["q_mean"], pooled["k_mean"], Qd, ns, b, tau, with_stats=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = sorted(set(rng.choice(M, 512, replace=False).tolist()) | {0, M - 1})
    gidx = idx[0, 0, rows].cpu().numpy()
    gcounts = counts[0, 0].cpu().numpy()
    gstats = stats[0, 0].cpu().numpy()
    del Qd, Kd, Vd, pooled, idx
    p = orc.params(Q, ns, b, 1.0, 1)
    ref = orc.pool(p, Q, K, V)
    qm, km = ref["q_mean"][0, 0].astype(np.float64), ref["k_mean"][0, 0].astype(np.float64)
    S = (qm @ km.T) / np.sqrt(d)
    mu, sd = S.mean(), S.std()
    assert abs(gstats[0] - mu) <= 1e-5 * abs(S).max() and abs(gstats[1] - sd) <= 1e-5 * sd, (gstats, mu, sd)
    sub_counts = gcounts[rows]
    # the threshold is the head's (all M x M scores), not that of the sampled rows
    thr = mu + tau * sd
    delta = 1e-4 * abs(thr) + 1e-6 * np.abs(S).max()
    bad = 0
    for n, I in enumerate(rows):
        row = gidx[n, :sub_counts[n]]
        bad += int(sub_counts[n] > 1 and not (np.diff(row) > 0).all())
        got = np.zeros(M, bool)
        got[row] = True
        bad += int(((S[I] > thr + delta) & ~got).sum() + (got & ~(S[I] >= thr - delta)).sum())
    kept = gcounts.mean() / M
    print(f"kept fraction {kept:.4f}, rows checked {len(rows)}, decisions outside the window {bad}", flush=True)
    assert bad == 0
    assert 0 <= gcounts.min() and gcounts.max() <= M
