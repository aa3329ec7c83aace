"""Comparison rules shared by the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import numpy as np

# Forward tolerances for bf16 matrix-core attention against the binary64 oracle.
FWD_REL_L2 = 1e-2
FWD_MAX_ABS = 2e-2
# FP8 carrier forward against the oracle's FP8 forward.  Both use the same carriers; the GPU also
# rounds each probability to E4M3 (3 mantissa bits) for the value product, the normaliser sums them
# unrounded.  For a value x spread over a binade [2^k, 2^(k+1)) the rounding error is uniform on
# +-2^(k-4), so its relative RMS is sqrt(2^-9 / 3) = 0.0255; an output that sums zero-mean values
# with perturbed weights carries about that relative error (measured 0.025-0.027), and less where
# the values share a mean.  The bound is 1.5x that RMS.  Per element the error is a weighted average
# of independent roundings (measured <= 1.3e-2 on unit-scale values); the bound is 3e-2.  The log-sum-
# exp uses the unrounded normaliser: binary32 error only.
FP8_REL_L2 = 0.04
FP8_MAX_ABS = 3e-2
FP8_LSE_MAX_ABS = 1e-4
# Pooled fp32 summaries against binary64 (fp32 accumulation over <= 128 rows).
POOL_RTOL = 2e-5
# Selection near-tie window: relative 1e-4 of the K-th / (K+1)-th scores, plus an absolute floor
# of 1e-6 of the row's largest |score| where scores cross zero.
SEL_REL = 1e-4
SEL_FLOOR = 1e-6


def check_selection_row(sel, S_row, K):
    """True when `sel` (GPU, ascending) is a valid top-K of the oracle scores `S_row`: exactly K
    distinct ascending blocks, containing every block clearly above the K-th score and none
    clearly below it.  Where the K-th and (K+1)-th scores are further apart than the window the
    set is forced to be the oracle's exact one."""
    sel = np.asarray(sel)
    M = S_row.shape[0]
    if sel.shape != (K,) or not (np.diff(sel) > 0).all() or sel.min() < 0 or sel.max() >= M:
        return False
    order = np.lexsort((np.arange(M), -S_row))
    sK = S_row[order[K - 1]]
    sK1 = S_row[order[K]] if K < M else -np.inf
    delta = SEL_REL * max(abs(sK), abs(sK1) if np.isfinite(sK1) else 0.0) + SEL_FLOOR * np.abs(S_row).max()
    must = set(np.nonzero(S_row > sK + delta)[0].tolist())
    allowed = set(np.nonzero(S_row >= sK - delta)[0].tolist())
    G = set(sel.tolist())
    return must <= G <= allowed


def check_selection_rows(idx, S):
    """Vectorised form of check_selection_row over rows: idx [R, K] GPU routes, S [R, M] oracle
    scores; returns the boolean validity of every row."""
    idx = np.asarray(idx)
    S = np.asarray(S, np.float64)
    K, M = idx.shape[-1], S.shape[-1]
    part = -np.sort(-S, axis=1)
    sK = part[:, K - 1]
    sK1 = part[:, K] if K < M else np.full_like(sK, -np.inf)
    delta = SEL_REL * np.maximum(np.abs(sK), np.where(np.isfinite(sK1), np.abs(sK1), 0.0)) \
        + SEL_FLOOR * np.abs(S).max(1)
    inrange = (idx >= 0).all(1) & (idx < M).all(1)
    chosen = np.zeros(S.shape, dtype=bool)
    np.put_along_axis(chosen, np.clip(idx, 0, M - 1).astype(np.int64), True, axis=1)
    must = S > (sK + delta)[:, None]
    allowed = S >= (sK - delta)[:, None]
    ok = inrange & (chosen.sum(1) == K) & ~(must & ~chosen).any(1) & ~(chosen & ~allowed).any(1)
    if K > 1:
        ok &= (np.diff(idx, axis=1) > 0).all(1)
    return ok


def check_selection(idx, S):
    """idx [..., M, K] GPU route vs oracle scores S [..., M, M]; returns (#rows bad, #rows not
    equal to the oracle's exact top-K)."""
    idx = np.asarray(idx)
    S = np.asarray(S)
    K = idx.shape[-1]
    M = S.shape[-1]
    bad = differ = 0
    for sel, row in zip(idx.reshape(-1, K), S.reshape(-1, M)):
        if not check_selection_row(sel, row, K):
            bad += 1
        ref = np.sort(np.lexsort((np.arange(M), -row))[:K])
        differ += int(not np.array_equal(ref, sel))
    return bad, differ


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def max_abs(a, b):
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max())


def fp8_decoded_inputs(orc, p, Q, K, V, pooled):
    """Inputs on which the oracle's plain attention computes the FP8 forward: every carrier
    decoded, x -> e4m3(x * r) * s per (batch, head) and tensor (the product x * r in binary32),
    and the pseudo-keys and pseudo-values carried with the keys' and values' scales (their
    summaries rounded to binary32 first), as the oracle's FP8 forward defines them.  A logit
    scale * (q8 s_Q) . (k8 s_K) is then the FP8 logit scale * s_Q * s_K * (q8 . k8).  The decoded
    rows are handed to the oracle in binary32, a relative rounding of 2^-24 far inside the FP8
    tolerances; the decoded summaries stay binary64 (exact).  Used to sample the FP8 forward at
    sizes where the oracle's full FP8 forward would take too long."""
    sc = orc.fp8_scales(p, Q, K, V)  # [B, H, 6]: (r, s) for Q, K, V

    def carry(X, t):
        r = sc[..., 2 * t].astype(np.float32)[:, :, None, None]
        s = sc[..., 2 * t + 1].astype(np.float64)[:, :, None, None]
        return orc.e4m3((np.asarray(X, np.float32) * r).astype(np.float32)).astype(np.float64) * s

    Qd, Kd, Vd = carry(Q, 0), carry(K, 1), carry(V, 2)
    pd = dict(pooled)
    pd["k_sum"] = carry(pooled["k_sum"], 1)
    pd["v_sum"] = carry(pooled["v_sum"], 2)
    return Qd, Kd, Vd, pd
