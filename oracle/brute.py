"""Brute-force NumPy (binary64) formulation for tiny inputs.  TEST INFRASTRUCTURE ONLY.

It pins the C oracle by computing the same method a different way:

* the forward builds, per (batch, head), one explicit logit matrix over N real keys plus M
  pseudo-keys (one per block) and an explicit boolean mask, then takes one masked softmax;
* block means use ``np.add.reduceat``, the anchor-weighted summary uses a within-block
  softmax and ``logaddexp.reduce``, the top-K uses ``np.lexsort``;
* the partition works on score vectors K q_i directly (the cosine of two queries' score
  patterns), never forming the second-moment matrix.

Sources: Spark-H3 news page, section "Spark-Attnが変えるもの" (exact/compressed branches,
Spark-Reblock and Spark-Reweight bullets) and section "ワークフロー" (topk_ratio, q_reuse_k);
core block-sparse node page, section "ブロックスパースアテンション" (per-query-block routing,
sink_conditioning); H3 Optimizations README, section "Nodes" (non-video queries dense).
"""
from __future__ import annotations

import math

import numpy as np


def _blocks(n_video, block):
    starts = np.arange(0, n_video, block)
    sizes = np.minimum(starts + block, n_video) - starts
    return starts, sizes


def budget(M, ratio):
    """K = round-half-up(r*M) in binary64 (ratio given as binary32), clamped to [1, M]."""
    k = math.floor(float(np.float32(ratio)) * M + 0.5)
    return int(min(M, max(1, k)))


def pool_head(q, k, v, n_video, block, pool_mode, s, block_k=None):
    """Query means over query blocks of `block` rows; key summaries over key blocks of `block_k`
    keys (default: `block`)."""
    qs, qz = _blocks(n_video, block)
    starts, sizes = _blocks(n_video, block_k or block)
    qv, kv, vv = q[:n_video], k[:n_video], v[:n_video]
    q_mean = np.add.reduceat(qv, qs, axis=0) / qz[:, None]
    k_mean = np.add.reduceat(kv, starts, axis=0) / sizes[:, None]
    anchor = qv.mean(axis=0)
    if pool_mode == 0:
        return dict(q_mean=q_mean, k_mean=k_mean, anchor=anchor, k_sum=k_mean,
                    v_sum=np.add.reduceat(vv, starts, axis=0) / sizes[:, None],
                    bias=np.log(sizes.astype(np.float64)))
    ks, vs, bias = [], [], []
    for st, n in zip(starts, sizes):
        x = s * (kv[st:st + n] @ anchor)
        lse = np.logaddexp.reduce(x)
        w = np.exp(x - lse)
        kt = w @ kv[st:st + n]
        ks.append(kt)
        vs.append(w @ vv[st:st + n])
        bias.append(lse - s * (anchor @ kt))
    return dict(q_mean=q_mean, k_mean=k_mean, anchor=anchor, k_sum=np.array(ks),
                v_sum=np.array(vs), bias=np.array(bias))


def select_head(q_mean, k_mean, s, K):
    S = s * (q_mean @ k_mean.T)
    M, Mk = S.shape
    idx = np.empty((M, K), np.int64)
    for I in range(M):
        order = np.lexsort((np.arange(Mk), -S[I]))
        idx[I] = np.sort(order[:K])
    return S, idx


def select_tau_head(S, tau):
    """Adaptive-tau route of one head from its block scores: kept[I, J] = S_IJ > mean + tau * std
    (NumPy's mean and population standard deviation over all entries)."""
    S = np.asarray(S, np.float64)
    return S > S.mean() + tau * S.std()


def e4m3_torch(x):
    """E4M3 rounding through PyTorch's float8_e4m3fn cast (a library routine, independent of the C
    oracle's own rounding)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).to(
        torch.float32).numpy()


def _fp8_carrier(x):
    """Per-head E4M3 carrier of a [N, d] binary32 array: (decoded carrier, s) with r = 448/amax and
    s = amax/448 in binary32."""
    x = np.asarray(x, np.float32)
    amax = np.float32(np.abs(x).max())
    if amax == 0:
        return x.copy(), np.float32(1)
    r = np.float32(448) / amax
    return e4m3_torch(x * r), amax / np.float32(448)


def forward(Q, K, V, n_sink, block, ratio, pool_mode=1, scale=None, perm=None, idx=None, perm_k=None,
            tau=None, fp8=False, block_k=None):
    """Q, K, V [B,H,N,d] (float arrays). Returns O, lse (binary64) and the route idx.
    perm: query partition (and output rows); perm_k: separate key partition of K and V (None:
    keys and values reuse perm).  tau: adaptive-tau routes instead of top-K (the returned idx is
    then the boolean kept matrix [B,H,M,M]).  fp8: queries, keys, values and the pseudo-keys on
    per-head E4M3 carriers (route and bias from the unquantized inputs).  block_k: key block size
    (default: block); the route, the budget and the compressed branch are per key block."""
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    B, H, N, d = Q.shape
    n_video = N - n_sink
    s = 1.0 / math.sqrt(d) if not scale else float(scale)
    bk = block_k or block
    starts, sizes = _blocks(n_video, block)
    kstarts, ksizes = _blocks(n_video, bk)
    M, Mk = len(starts), len(kstarts)
    if tau is not None and Mk != M:
        raise ValueError("adaptive tau is defined for equal query and key blocks")
    Ksel = budget(Mk, ratio)
    O = np.empty((B, H, N, d))
    LSE = np.empty((B, H, N))
    IDX = np.empty((B, H, M, Ksel), np.int64) if tau is None else np.empty((B, H, M, M), bool)
    blk = np.repeat(np.arange(M), sizes)  # video token -> query block
    kblk = np.repeat(np.arange(Mk), ksizes)  # video token -> key block
    for b in range(B):
        for h in range(H):
            q, k, v = Q[b, h].copy(), K[b, h].copy(), V[b, h].copy()
            if perm is not None:
                q[:n_video] = q[np.asarray(perm[b, h])]
            pk = perm_k if perm_k is not None else perm
            if pk is not None:
                pkm = np.asarray(pk[b, h])
                k[:n_video], v[:n_video] = k[pkm], v[pkm]
            pooled = pool_head(q, k, v, n_video, block, pool_mode, s, bk)
            if tau is not None:
                chosen = select_tau_head(s * (pooled["q_mean"] @ pooled["k_mean"].T), tau)
                IDX[b, h] = chosen
            else:
                if idx is None:
                    _, sel = select_head(pooled["q_mean"], pooled["k_mean"], s, Ksel)
                else:
                    sel = np.asarray(idx[b, h])
                IDX[b, h] = sel
                chosen = np.zeros((M, Mk), bool)  # chosen[I, J]
                chosen[np.repeat(np.arange(M), Ksel), sel.reshape(-1)] = True
            qa, ka, va, kt, vt, sl, sv = q, k, v, pooled["k_sum"], pooled["v_sum"], s, 1.0
            if fp8:
                qa, sq = _fp8_carrier(q)
                ka, sk = _fp8_carrier(k)
                va, sv = _fp8_carrier(v)
                # the pseudo-keys ride on the keys' and values' carriers
                kmax, vmax = np.float32(np.abs(np.asarray(k, np.float32)).max()), np.float32(
                    np.abs(np.asarray(v, np.float32)).max())
                rk = np.float32(448) / kmax if kmax > 0 else np.float32(1)
                rv = np.float32(448) / vmax if vmax > 0 else np.float32(1)
                kt = e4m3_torch(np.asarray(kt, np.float32) * rk).astype(np.float64)
                vt = e4m3_torch(np.asarray(vt, np.float32) * rv).astype(np.float64)
                qa, ka, va = (np.asarray(x, np.float64) for x in (qa, ka, va))
                sl = s * float(sq) * float(sk)
                sv = float(sv)
            logits = np.concatenate([sl * (qa @ ka.T), sl * (qa @ kt.T) + pooled["bias"]], axis=1)
            values = sv * np.concatenate([va, vt], axis=0)
            mask = np.zeros((N, N + Mk), bool)
            # video queries: keys of chosen blocks, all sinks, pseudo-keys of unchosen blocks
            mask[:n_video, :n_video] = chosen[blk][:, kblk]
            mask[:n_video, n_video:N] = True
            mask[:n_video, N:] = ~chosen[blk]
            # sink queries: every real key, no pseudo-key
            mask[n_video:, :N] = True
            z = np.where(mask, logits, -np.inf)
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            Z = e.sum(axis=1, keepdims=True)
            o = (e @ values) / Z
            lse = (m + np.log(Z))[:, 0]
            if perm is not None:
                pm = np.asarray(perm[b, h])
                o_video, l_video = o[:n_video].copy(), lse[:n_video].copy()
                o[pm], lse[pm] = o_video, l_video
            O[b, h], LSE[b, h] = o, lse
    return O, LSE, IDX


def dense(Q, K, V, scale=None):
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    d = Q.shape[-1]
    s = 1.0 / math.sqrt(d) if not scale else float(scale)
    z = s * (Q @ np.swapaxes(K, -1, -2))
    m = z.max(-1, keepdims=True)
    e = np.exp(z - m)
    Z = e.sum(-1, keepdims=True)
    return (e @ V) / Z, (m + np.log(Z))[..., 0]


def reblock_head(q, k, n_video, block):
    """Partition by score-vector cosines: u_i = K q_i / |K q_i|, cos(i, j) = u_i . u_j."""
    q = np.asarray(q[:n_video], np.float64)
    k = np.asarray(k[:n_video], np.float64)
    S = q @ k.T  # row i = score pattern of query i against every video key
    nrm = np.linalg.norm(S, axis=1)
    U = np.divide(S, nrm[:, None], out=np.zeros_like(S), where=nrm[:, None] > 0)
    M = -(-n_video // block)
    leaves = []

    def split(tok, c):
        if c == 1:
            leaves.append(np.sort(tok))
            return
        p0 = tok.min()
        cos0 = U[tok] @ U[p0]
        A = tok[np.lexsort((tok, cos0))[0]]
        cosA = U[tok] @ U[A]
        Bp = tok[np.lexsort((tok, cosA))[0]]
        key = cosA - U[tok] @ U[Bp]
        order = tok[np.lexsort((tok, -key))]
        cl = (c + 1) // 2
        split(order[:cl * block], cl)
        split(order[cl * block:], c - cl)

    split(np.arange(n_video), M)
    return np.concatenate(leaves)
