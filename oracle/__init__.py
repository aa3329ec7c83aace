"""CPU oracle for the Spark-Attn forward and the Spark-Reblock partition.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import it.  It never touches the HIP library and the HIP library never
touches it: the two share no code.

``spark_oracle.c`` holds the binary64 reference (built with gcc, OpenMP over independent
(batch, head, block) units); ``brute.py`` holds a NumPy mask-matrix formulation for tiny inputs
that pins it.  This module is the ctypes wrapper of the C part.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spark_oracle.c")
_LIB = os.path.join(_HERE, "libspark_oracle.so")


class Params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("d", ctypes.c_int),
        ("n_sink", ctypes.c_int), ("block", ctypes.c_int), ("topk_ratio", ctypes.c_float),
        ("pool_mode", ctypes.c_int), ("scale", ctypes.c_double), ("block_k", ctypes.c_int),
    ]


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (binary64, no fp contraction, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", _SRC, "-o", _LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    """The loaded C oracle, built first when missing or stale.  SPARK_ORACLE_LIB names another
    build of spark_oracle.c to load instead (the sanitizer test loads an instrumented one)."""
    global _lib
    if _lib is None:
        path = os.environ.get("SPARK_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        P = ctypes.POINTER(Params)
        f32, f64, i32 = (np.ctypeslib.ndpointer(t, flags="C_CONTIGUOUS")
                         for t in (np.float32, np.float64, np.int32))
        vp = ctypes.c_void_p
        L.orc_num_blocks.argtypes = [P]
        L.orc_num_key_blocks.argtypes = [P]
        L.orc_topk_count.argtypes = [ctypes.c_int, ctypes.c_float]
        L.orc_num_threads.argtypes = []
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        L.orc_set_num_threads.restype = None
        L.orc_pool.argtypes = [P, f32, f32, f32, f64, f64, f64, f64, f64, f64]
        L.orc_scores.argtypes = [P, f64, f64, f64]
        L.orc_select.argtypes = [P, f64, i32]
        L.orc_dense.argtypes = [P, f32, f32, f32, f64, f64]
        L.orc_attend_blocks.argtypes = [P, f32, f32, f32, f64, f64, f64, i32, ctypes.c_int, i32,
                                        ctypes.c_int, f64, f64]
        L.orc_forward.argtypes = [P, f32, f32, f32, vp, vp, vp, f64, f64, vp]
        L.orc_select_tau.argtypes = [P, ctypes.c_double, f64, i32, i32, vp]
        L.orc_forward_tau.argtypes = [P, ctypes.c_double, f32, f32, f32, vp, vp, f64, f64, vp, vp]
        L.orc_e4m3.argtypes = [ctypes.c_float]
        L.orc_e4m3.restype = ctypes.c_float
        L.orc_e4m3_array.argtypes = [f32, f32, ctypes.c_size_t]
        L.orc_fp8_scales.argtypes = [P, f32, f32, f32, f32]
        L.orc_forward_fp8.argtypes = [P, f32, f32, f32, vp, vp, f64, f64, vp, vp]
        L.orc_reblock_metric.argtypes = [P, f32, f32, f64, f64]
        L.orc_reblock.argtypes = [P, f32, f32, i32]
        L.orc_reblock_given_sigma.argtypes = [P, f32, f64, i32]
        for fn in (L.orc_pool, L.orc_scores, L.orc_select, L.orc_dense, L.orc_attend_blocks,
                   L.orc_forward, L.orc_select_tau, L.orc_forward_tau, L.orc_reblock_metric,
                   L.orc_reblock, L.orc_reblock_given_sigma):
            fn.restype = None
        _lib = L
    return _lib


def params(Q, n_sink, block, ratio=0.1, pool_mode=1, scale=0.0, block_k=0) -> Params:
    """block: query block size; block_k: key block size (0: the same as block)."""
    B, H, N, d = Q.shape
    return Params(B, H, N, d, n_sink, block, float(ratio), int(pool_mode), float(scale), int(block_k))


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def num_blocks(p: Params) -> int:
    """Query blocks M."""
    return lib().orc_num_blocks(ctypes.byref(p))


def num_key_blocks(p: Params) -> int:
    """Key blocks M_k (M when the key block size equals the query block size)."""
    return lib().orc_num_key_blocks(ctypes.byref(p))


def _equal_blocks(p: Params, what):
    if p.block_k not in (0, p.block):
        raise ValueError(f"{what} is defined for equal query and key blocks")


def topk_count(M: int, ratio: float) -> int:
    return lib().orc_topk_count(M, ratio)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads for later calls (timing only: every result is independent of the thread count)."""
    lib().orc_set_num_threads(int(n))


def pool(p: Params, Q, K, V):
    """Returns dict q_mean [B,H,M,d]; k_mean, k_sum, v_sum [B,H,M_k,d], bias [B,H,M_k];
    anchor [B,H,d]."""
    M, Mk = num_blocks(p), num_key_blocks(p)
    out = {"q_mean": np.empty((p.B, p.H, M, p.d))}
    out.update({k: np.empty((p.B, p.H, Mk, p.d)) for k in ("k_mean", "k_sum", "v_sum")})
    out["bias"] = np.empty((p.B, p.H, Mk))
    out["anchor"] = np.empty((p.B, p.H, p.d))
    lib().orc_pool(ctypes.byref(p), _f32(Q), _f32(K), _f32(V), out["q_mean"], out["k_mean"],
                   out["k_sum"], out["v_sum"], out["bias"], out["anchor"])
    return out


def scores(p: Params, q_mean, k_mean):
    M, Mk = num_blocks(p), num_key_blocks(p)
    S = np.empty((p.B, p.H, M, Mk))
    lib().orc_scores(ctypes.byref(p), np.ascontiguousarray(q_mean, np.float64),
                     np.ascontiguousarray(k_mean, np.float64), S)
    return S


def select(p: Params, S):
    M = num_blocks(p)
    K = topk_count(num_key_blocks(p), p.topk_ratio)
    idx = np.empty((p.B, p.H, M, K), np.int32)
    lib().orc_select(ctypes.byref(p), np.ascontiguousarray(S, np.float64), idx)
    return idx


def dense(p: Params, Q, K, V):
    O = np.empty((p.B, p.H, p.N, p.d))
    lse = np.empty((p.B, p.H, p.N))
    lib().orc_dense(ctypes.byref(p), _f32(Q), _f32(K), _f32(V), O, lse)
    return O, lse


def forward(p: Params, Q, K, V, perm=None, idx=None, perm_k=None):
    """Full forward. Returns (O [B,H,N,d] f64, lse [B,H,N] f64, idx [B,H,M,K] int32).
    perm: query partition (and output rows); perm_k: separate key partition for K and V, or
    None for keys and values reusing perm."""
    M = num_blocks(p)
    Ksel = topk_count(num_key_blocks(p), p.topk_ratio)
    O = np.empty((p.B, p.H, p.N, p.d))
    lse = np.empty((p.B, p.H, p.N))
    idx_out = np.empty((p.B, p.H, M, Ksel), np.int32)
    keep = []

    def ptr(a, dt):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dt)
        keep.append(a)
        return a.ctypes.data

    lib().orc_forward(ctypes.byref(p), _f32(Q), _f32(K), _f32(V), ptr(perm, np.int32),
                      ptr(perm_k, np.int32), ptr(idx, np.int32), O, lse, idx_out.ctypes.data)
    return O, lse, idx_out


def select_tau(p: Params, tau, S):
    """Adaptive-tau routes from block scores S [B,H,M,M]: (idx [B,H,M,M] with row I's kept blocks
    ascending in its first counts[I] entries (the rest -1), counts [B,H,M], stats [B,H,2] =
    (mu, sigma))."""
    _equal_blocks(p, "adaptive-tau selection")
    M = num_blocks(p)
    idx = np.full((p.B, p.H, M, M), -1, np.int32)
    counts = np.empty((p.B, p.H, M), np.int32)
    stats = np.empty((p.B, p.H, 2))
    S = np.ascontiguousarray(S, dtype=np.float64)
    lib().orc_select_tau(ctypes.byref(p), float(tau), S, idx, counts, stats.ctypes.data)
    return idx, counts, stats


def forward_tau(p: Params, tau, Q, K, V, idx=None, counts=None):
    """Forward with adaptive-tau routes.  Returns (O, lse, idx [B,H,M,M], counts [B,H,M]); idx and
    counts, when given, replace the oracle's own selection."""
    _equal_blocks(p, "adaptive-tau selection")
    M = num_blocks(p)
    O = np.empty((p.B, p.H, p.N, p.d))
    lse = np.empty((p.B, p.H, p.N))
    idx_out = np.full((p.B, p.H, M, M), -1, np.int32)
    cnt_out = np.empty((p.B, p.H, M), np.int32)
    keep = []

    def ptr(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=np.int32)
        keep.append(a)
        return a.ctypes.data

    lib().orc_forward_tau(ctypes.byref(p), float(tau), _f32(Q), _f32(K), _f32(V), ptr(idx), ptr(counts),
                          O, lse, idx_out.ctypes.data, cnt_out.ctypes.data)
    return O, lse, idx_out, cnt_out


def e4m3(x):
    """E4M3 rounding (OCP 8-bit float, 3 mantissa bits, ties to even) of binary32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    lib().orc_e4m3_array(x.reshape(-1), y.reshape(-1), x.size)
    return y


def fp8_scales(p: Params, Q, K, V):
    """Per (batch, head): [r_Q, s_Q, r_K, s_K, r_V, s_V] (binary32), r = 448/amax, s = amax/448."""
    sc = np.empty((p.B, p.H, 6), np.float32)
    lib().orc_fp8_scales(ctypes.byref(p), _f32(Q), _f32(K), _f32(V), sc.reshape(-1))
    return sc


def forward_fp8(p: Params, Q, K, V, perm=None, idx=None):
    """Forward with Q, K, V and the pseudo-keys on per-head-scaled E4M3 carriers.  Returns
    (O, lse, idx [B,H,M,K], scales [B,H,6])."""
    M = num_blocks(p)
    Ksel = topk_count(num_key_blocks(p), p.topk_ratio)
    O = np.empty((p.B, p.H, p.N, p.d))
    lse = np.empty((p.B, p.H, p.N))
    idx_out = np.empty((p.B, p.H, M, Ksel), np.int32)
    sc = np.empty((p.B, p.H, 6), np.float32)
    keep = []

    def ptr(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=np.int32)
        keep.append(a)
        return a.ctypes.data

    lib().orc_forward_fp8(ctypes.byref(p), _f32(Q), _f32(K), _f32(V), ptr(perm), ptr(idx), O, lse,
                          idx_out.ctypes.data, sc.ctypes.data)
    return O, lse, idx_out, sc


def attend_blocks(p: Params, Q, K, V, pooled, idx, qblocks):
    """Attention rows of chosen query blocks. qblocks: int array [n, 2] of (b*H + h, I) where
    I < M is a video query block and I >= M the sink row N_v + I - M.  Inputs are in the
    (already permuted) block layout that ``idx`` refers to.  Returns O [n, block, d] and
    lse [n, block] (rows past a partial block / past row 0 of a sink entry are NaN)."""
    qb = np.ascontiguousarray(qblocks, dtype=np.int32).reshape(-1, 2)
    n = qb.shape[0]
    O = np.full((n, p.block, p.d), np.nan)
    lse = np.full((n, p.block), np.nan)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    lib().orc_attend_blocks(ctypes.byref(p), _f32(Q), _f32(K), _f32(V),
                            np.ascontiguousarray(pooled["k_sum"], np.float64),
                            np.ascontiguousarray(pooled["v_sum"], np.float64),
                            np.ascontiguousarray(pooled["bias"], np.float64), idx,
                            idx.shape[-1], qb, n, O, lse)
    return O, lse


def reblock_metric(p: Params, Q, K):
    Nv = p.N - p.n_sink
    Sigma = np.empty((p.B, p.H, p.d, p.d))
    nrm = np.empty((p.B, p.H, Nv))
    lib().orc_reblock_metric(ctypes.byref(p), _f32(Q), _f32(K), Sigma, nrm)
    return Sigma, nrm


def reblock(p: Params, Q, K):
    Nv = p.N - p.n_sink
    perm = np.empty((p.B, p.H, Nv), np.int32)
    lib().orc_reblock(ctypes.byref(p), _f32(Q), _f32(K), perm)
    return perm


def reblock_given_sigma(p: Params, Q, Sigma):
    """The partition (readings R2..R6) from a caller's Sigma [B,H,d,d] in place of R1's."""
    Nv = p.N - p.n_sink
    perm = np.empty((p.B, p.H, Nv), np.int32)
    lib().orc_reblock_given_sigma(ctypes.byref(p), _f32(Q), np.ascontiguousarray(Sigma, np.float64), perm)
    return perm
