"""GPU parity of the FP8 (E4M3) carrier path against the oracle's FP8 forward.

  scales    amax bit-exact (a maximum of exact values); s = amax/448 equal to the oracle's
  carriers  the packed key rows of real and compressed tiles bit-exact (e4m3 of x * r, ties to
            even); each value row holds exactly the 64 quantized values of its keys
  forward   the route is validated like the bf16 path's and handed to the oracle; O within
            FP8_REL_L2 / FP8_MAX_ABS (tests/parity.py: the probabilities are rounded to E4M3 on
            the GPU and not in the oracle)
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_score_amd as sa
import workloads as W
from parity import FP8_LSE_MAX_ABS, FP8_MAX_ABS, FP8_REL_L2, check_selection, max_abs, rel_l2

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


def host(t):
    return t.detach().float().cpu().numpy()


def permute_rows(X, perm):
    Y = X.copy()
    nv = perm.shape[-1]
    for b in range(X.shape[0]):
        for h in range(X.shape[1]):
            Y[b, h, :nv] = X[b, h, perm[b, h]]
    return Y


def rounded(x, dt):
    """The values the GPU sees (bf16 inputs rounded like the device copy)."""
    return host(dev(x, dt)) if dt == "bf16" else np.asarray(x, np.float32)


# (name, B, H, n_video, n_sink, d, block, ratio, dtype)
CASES = [
    ("bf16-d128-b128", 1, 3, 11 * 128 + 37, 5, 128, 128, 0.2, "bf16"),
    ("bf16-d64-b64", 2, 2, 37 * 64 + 1, 0, 64, 64, 0.1, "bf16"),
    ("bf16-d128-b64", 1, 2, 20 * 64 + 63, 130, 128, 64, 0.15, "bf16"),
    ("bf16-d64-b128", 1, 2, 7 * 128 + 1, 3, 64, 128, 0.3, "bf16"),
    ("fp32-d128-b128", 1, 1, 9 * 128 + 100, 17, 128, 128, 0.25, "fp32"),
    ("full-density", 1, 2, 6 * 128 + 9, 40, 128, 128, 1.0, "bf16"),
]


def fp8_check(orc, Q, K, V, ns, b, r, pool_mode, dt, perm=None, block_k=0):
    Q, K, V = (rounded(x, dt) for x in (Q, K, V))
    permd = torch.from_numpy(perm).cuda() if perm is not None else None
    O, lse, idx, amax = sa.forward_fp8(dev(Q, dt), dev(K, dt), dev(V, dt), ns, b, r, pool_mode, perm=permd,
                                       return_lse=True, return_idx=True, return_amax=True, block_k=block_k)
    torch.cuda.synchronize()
    p = orc.params(Q, ns, b, r, pool_mode, block_k=block_k)
    gidx = idx.cpu().numpy()
    Qp, Kp, Vp = (permute_rows(x, perm) for x in (Q, K, V)) if perm is not None else (Q, K, V)
    ref = orc.pool(p, Qp, Kp, Vp)
    bad, _ = check_selection(gidx, orc.scores(p, ref["q_mean"], ref["k_mean"]))
    assert bad == 0
    Oref, lref, _, sc = orc.forward_fp8(p, Q, K, V, perm=perm, idx=gidx)
    am = amax.cpu().numpy()
    assert (am == np.abs(np.stack([Q, K, V], axis=2)).reshape(*am.shape, -1).max(axis=-1)).all()
    assert (np.where(am > 0, am / np.float32(448), np.float32(1)) == sc[..., 1::2]).all()
    Og = host(O)
    e2, ea, el = rel_l2(Og, Oref), max_abs(Og, Oref), max_abs(host(lse), lref)
    print(f"fp8 rel-L2 {e2:.3e} max-abs {ea:.3e} lse max-abs {el:.3e}")
    assert e2 <= FP8_REL_L2 and ea <= FP8_MAX_ABS and el <= FP8_LSE_MAX_ABS
    return Og, Oref


@pytest.mark.parametrize("pool_mode", [0, 1])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_forward_parity(orc, case, pool_mode):
    name, B, H, nv, ns, d, b, r, dt = case
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=nv + 7, dtype=dt)
    note(f"fp8 forward {name} mode={pool_mode}")
    fp8_check(orc, Q, K, V, ns, b, r, pool_mode, dt)


def test_fp8_forward_reblocked(orc):
    B, H, nv, ns, d, b = 1, 2, 6 * 128 + 50, 33, 128, 128
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=19, dtype="bf16")
    note("fp8 forward on the reblocked layout")
    perm = sa.reblock(dev(Q, "bf16"), dev(K, "bf16"), ns, b).cpu().numpy()
    fp8_check(orc, Q, K, V, ns, b, 0.3, 1, "bf16", perm=perm)


@pytest.mark.parametrize("b,bk", [(128, 64), (64, 128)])
def test_fp8_asymmetric_route(orc, b, bk):
    Q, K, V = W.gaussian_qkv(1, 2, 10 * 128 + 33, 9, 128, seed=b + bk, dtype="bf16")
    note(f"fp8 forward, query blocks {b}, key blocks {bk}")
    fp8_check(orc, Q, K, V, 9, b, 0.2, 1, "bf16", block_k=bk)


def test_fp8_structured_workload(orc):
    wl = W.WORKLOADS["tiny"]
    Q, K, V = W.make_qkv(wl)
    note("fp8 forward on the tiny positional workload")
    fp8_check(orc, Q, K, V, wl.n_sink, wl.block, wl.ratios[0], 1, wl.dtype)


def test_fp8_packed_carriers_bit_exact(orc):
    B, H, nv, ns, d, b = 1, 2, 5 * 128 + 20, 70, 128, 128
    Q, K, V = (rounded(x, "bf16") for x in W.gaussian_qkv(B, H, nv, ns, d, seed=23, dtype="bf16"))
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    note("fp8 scales and packed carriers")
    amax = sa.fp8_scales(Qd, Kd, Vd, ns, b)
    pooled = sa.pool(Qd, Kd, Vd, ns, b)
    packed = sa.pack_fp8(Kd, Vd, pooled, amax, ns, b)
    torch.cuda.synchronize()
    p = orc.params(Q, ns, b)
    sc = orc.fp8_scales(p, Q, K, V)
    M = orc.num_blocks(p)
    Tv, Ts, Tc = M * b // 64, (ns + 63) // 64, (M + 63) // 64
    Tall = Tv + Ts + Tc
    tiles = packed[: B * H * Tall * 128 * d].view(torch.float8_e4m3fn).float().cpu().numpy()
    tiles = tiles.reshape(B * H, Tall, 128 * d)
    ks, vs = host(pooled["k_sum"]), host(pooled["v_sum"])
    for bh in range(B * H):
        bb, hh = divmod(bh, H)
        rk, rv = sc[bb, hh, 2], sc[bb, hh, 4]
        for t in range(Tall):
            if t < Tv:
                rows_k, rows_v = K[bb, hh, 64 * t:min(nv, 64 * t + 64)], V[bb, hh, 64 * t:min(nv, 64 * t + 64)]
            elif t < Tv + Ts:
                lo = nv + 64 * (t - Tv)
                rows_k, rows_v = K[bb, hh, lo:min(nv + ns, lo + 64)], V[bb, hh, lo:min(nv + ns, lo + 64)]
            else:
                lo = 64 * (t - Tv - Ts)
                rows_k, rows_v = ks[bb, hh, lo:min(M, lo + 64)], vs[bb, hh, lo:min(M, lo + 64)]
            n = rows_k.shape[0]
            kpart = tiles[bh, t, :64 * d].reshape(64, d)
            vpart = tiles[bh, t, 64 * d:].reshape(d, 64)
            assert (kpart[:n] == orc.e4m3(rows_k * rk)).all(), (bh, t)
            assert (kpart[n:] == 0).all()
            vq = orc.e4m3(np.asarray(rows_v, np.float32) * rv)
            full = np.zeros((64, d), np.float32)
            full[:n] = vq
            assert (np.sort(vpart, axis=1) == np.sort(full.T, axis=1)).all(), (bh, t)


@pytest.mark.parametrize("block_k", [0, 64])
@pytest.mark.parametrize("pool_mode", [0, 1])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pool_fp8_scales_equals_pool_and_scales(case, pool_mode, block_k):
    """spark_attn_pool_fp8_scales writes the same summaries as spark_attn_pool and the same amax as
    spark_attn_fp8_scales (maxima are exact and independent of their order)."""
    name, B, H, nv, ns, d, b, r, dt = case
    if block_k and b == 64:
        pytest.skip("64-row query blocks route to key blocks of 64 already")
    note(f"pool_fp8_scales {name} mode={pool_mode} block_k={block_k}")
    Q, K, V = W.gaussian_qkv(B, H, nv, ns, d, seed=nv + 7 * pool_mode + block_k, dtype=dt)
    Q[..., 0, 3] = -40.0  # a video row holds Q's largest |x|
    if ns:
        K[..., -1, 5] = 37.0  # a sink row holds K's
    Qd, Kd, Vd = (dev(x, dt) for x in (Q, K, V))
    p = sa.params(Qd, ns, b, r, pool_mode, block_k=block_k)
    ref = sa.pool(Qd, Kd, Vd, ns, b, pool_mode, block_k=block_k)
    amax_ref = torch.empty(B, H, 3, device="cuda", dtype=torch.float32)
    sa.spark_attn_fp8_scales(p, Qd, Kd, Vd, amax_ref)
    got = {k: torch.full_like(v, float("nan")) for k, v in ref.items()}
    amax = torch.full_like(amax_ref, float("nan"))
    sa.spark_attn_pool_fp8_scales(p, Qd, Kd, Vd, got["q_mean"], got["k_mean"], got["k_sum"], got["v_sum"],
                                  got["bias"], got["anchor"], amax)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), k
    assert torch.equal(amax, amax_ref)
    assert float(amax_ref[..., 0].max()) == 40.0
    if ns:
        assert float(amax_ref[..., 1].max()) == 37.0


def test_fp8_fullclip_sampled(orc):
    """The FP8 forward at the full clip's shape (245,952 video + 512 sink tokens, 24 heads, the
    benchmark's --fp8 launch).  For three heads the oracle checks the per-head maxima exactly,
    sampled route rows with the near-tie rule, and sampled query blocks (the ragged last one
    included) and sink rows through its plain attention on the decoded carriers (the oracle's
    full FP8 forward is too long at this size; tests/test_oracle_pins.py shows the two agree)."""
    import math

    from parity import fp8_decoded_inputs

    wl = W.WORKLOADS["fullclip"]
    Q, K, V = W.make_qkv(wl)
    note(f"fp8 forward, full clip N={wl.N} H={wl.H}")
    O, lse, idx, amax = sa.forward_fp8(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), wl.n_sink, wl.block,
                                       0.1, 1, return_lse=True, return_idx=True, return_amax=True)
    torch.cuda.synchronize()
    heads = [0, 11, 23]
    Qs, Ks, Vs = (np.ascontiguousarray(x[:, heads]) for x in (Q, K, V))
    del Q, K, V
    gidx = idx.cpu().numpy()[:, heads]
    am = amax.cpu().numpy()[:, heads]
    Og, lg = host(O)[:, heads], lse.cpu().numpy()[:, heads]
    del O, lse, idx
    assert (am == np.abs(np.stack([Qs, Ks, Vs], axis=2)).reshape(*am.shape, -1).max(axis=-1)).all()
    p = orc.params(Qs, wl.n_sink, wl.block, 0.1, 1)
    ref = orc.pool(p, Qs, Ks, Vs)
    M = gidx.shape[2]
    rng = np.random.default_rng(8)
    s = 1.0 / math.sqrt(wl.d)
    rows = [(h, int(I)) for h in range(len(heads)) for I in rng.choice(M, 16, replace=False)]
    S = np.stack([s * ref["k_mean"][0, h] @ ref["q_mean"][0, h, I] for h, I in rows])
    bad, _ = check_selection(np.stack([gidx[0, h, I] for h, I in rows]), S)
    assert bad == 0
    Qd, Kd, Vd, pd = fp8_decoded_inputs(orc, p, Qs, Ks, Vs, ref)
    qb = [(int(h), int(I)) for h, I in zip(rng.integers(0, len(heads), 9), rng.integers(0, M, 9))]
    qb += [(len(heads) - 1, M - 1)]
    qb += [(int(h), M + int(j)) for h, j in zip(rng.integers(0, len(heads), 3), rng.integers(0, wl.n_sink, 3))]
    Os, ls = orc.attend_blocks(p, Qd, Kd, Vd, pd, gidx, np.array(qb))
    nv = wl.n_video
    g_rows, r_rows, gl, rl = [], [], [], []
    for n, (h, I) in enumerate(qb):
        lo, hi = (I * wl.block, min(nv, (I + 1) * wl.block)) if I < M else (nv + I - M, nv + I - M + 1)
        g_rows.append(Og[0, h, lo:hi]); r_rows.append(Os[n, :hi - lo])
        gl.append(lg[0, h, lo:hi]); rl.append(ls[n, :hi - lo])
    g_rows, r_rows = np.concatenate(g_rows), np.concatenate(r_rows)
    e2, ea, el = rel_l2(g_rows, r_rows), max_abs(g_rows, r_rows), max_abs(np.concatenate(gl), np.concatenate(rl))
    print(f"fp8 full clip: rel-L2 {e2:.3e} max-abs {ea:.3e} lse max-abs {el:.3e}", flush=True)
    assert e2 <= FP8_REL_L2 and ea <= FP8_MAX_ABS and el <= FP8_LSE_MAX_ABS
