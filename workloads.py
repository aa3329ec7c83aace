"""Seeded synthetic video-shaped Q/K/V, shared by the oracle tests, the GPU tests and the bench.

This module only draws inputs. It holds none of the attention method's arithmetic
(no pooling, no scores, no selection, no softmax), so the oracle and the HIP path can
both consume it without sharing any of the method.

Workloads stand in for the pages' MiniMax-H3 clips (Spark-H3 page, section
"ベンチマーク" (benchmarks): 1344x768, 240 frames). H3's weights, prompts and sampler are
not available, so the tensors only take the shapes and a spatially structured score
pattern:

* Tokens are the video latent grid T x Y x X in raster order, index (t*Y + y)*X + x.
* Features F (N_v x 48): per axis of length L and coordinate p, for f = 0..7 the
  frequency w = pi * L**((f - 7) / 7) (geometric ladder from pi/L to pi), and the pair
  sin(w p), cos(w p).
* Per head one Gaussian W_h (48 x d), shared by Q, K and V;
  X_h = (F @ W_h + 0.5 * E_X) / sqrt(d) with E_X i.i.d. N(0, 1) per tensor.
* Sink (conditioning) rows sit after the video rows and are i.i.d. N(0, 1), unscaled.
* bf16 workloads are rounded to bf16 (round to nearest even) here, so the float32
  arrays returned carry exactly the values the GPU receives.

Seeds: numpy.random.SeedSequence([config_id, batch, head, tensor_id]).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor ids used in the seed sequence
_T_W, _T_QN, _T_KN, _T_VN, _T_QS, _T_KS, _T_VS = range(7)


@dataclass(frozen=True)
class Workload:
    """One synthetic configuration. N = N_v + n_sink rows per (batch, head)."""

    name: str
    config_id: int
    B: int
    H: int
    d: int
    grid: tuple  # (T, Y, X) latent grid of the video tokens
    n_sink: int
    block: int
    ratios: tuple = (0.1,)
    dtype: str = "bf16"  # "bf16" or "fp32"
    pool_modes: tuple = (1,)  # 0 = plain mean pool, 1 = anchor-weighted summary + log-mass bias
    reblock: bool = False
    key_partition: bool = False  # with reblock: keys and values in their own partition
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def n_video(self) -> int:
        t, y, x = self.grid
        return t * y * x

    @property
    def N(self) -> int:
        return self.n_video + self.n_sink

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, B=1, H=2, d=64, grid=(4, 32, 32), n_sink=0, block=64, ratios=(0.1,),
        dtype="fp32", pool_modes=(0, 1),
        description="4x32x32 raster, fp32, d=64, 64-token blocks, no sinks, both compressed variants"),
    "short": Workload(
        "short", 2, B=1, H=24, d=128, grid=(15, 32, 64), n_sink=256, block=128, ratios=(0.1,),
        description="30,720 video + 256 sink tokens, bf16, d=128, 128-token blocks"),
    "720p": Workload(
        "720p", 3, B=1, H=24, d=128, grid=(21, 45, 80), n_sink=512, block=128,
        ratios=(0.1, 0.2, 0.3, 1.0),
        description="75,600 video + 512 sink tokens (720p-like latent), density sweep"),
    "fullclip": Workload(
        "fullclip", 4, B=1, H=24, d=128, grid=(61, 48, 84), n_sink=512, block=128, ratios=(0.1,),
        description="1344x768x240-frame clip: 245,952 video + 512 sink tokens, bf16, d=128"),
    "reblock720p": Workload(
        "reblock720p", 5, B=1, H=24, d=128, grid=(21, 45, 80), n_sink=512, block=128,
        ratios=(0.1,), reblock=True,
        description="720p-like latent with adaptive blocks (q_reuse_k layout)"),
    "reblockkv720p": Workload(
        "reblockkv720p", 6, B=1, H=24, d=128, grid=(21, 45, 80), n_sink=512, block=128,
        ratios=(0.1,), reblock=True, key_partition=True,
        description="720p-like latent with adaptive blocks, queries and keys each partitioned under "
                    "the other side's second moment"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32 holding them."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


N_FEATURES = 48  # 3 raster axes x 8 frequencies x (sin, cos)


def positional_features(grid) -> np.ndarray:
    """F (N_v x 48) float64: sin/cos of each raster coordinate at 8 frequencies per axis."""
    T, Y, X = grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    cols = []
    for L, p in ((T, t.reshape(-1)), (Y, y.reshape(-1)), (X, x.reshape(-1))):
        for f in range(8):
            w = math.pi * float(L) ** ((f - 7) / 7.0)
            cols.append(np.sin(w * p))
            cols.append(np.cos(w * p))
    return np.stack(cols, axis=1).astype(np.float64)


def _positional_base(grid, W: np.ndarray) -> np.ndarray:
    """positional_features(grid) @ W in binary64, in a fixed summation order.  Columns 16a ..
    16a+15 of the features depend on raster axis a alone, so the product is A_t[t] + A_y[y] +
    A_x[x] with A_a the product of axis a's 16 columns (taken per coordinate value, summed in
    column order), added as (A_t + A_y) + A_x.  Scalar libm sin/cos and elementwise IEEE
    operations only: the same bits on every run, thread count and machine with this C library (a
    BLAS product may split its sums differently from call to call, which flips the last bit of
    some values and now and then a bf16 rounding)."""
    parts = []
    for a, L in enumerate(grid):
        acc = None
        for f in range(8):
            w = math.pi * float(L) ** ((f - 7) / 7.0)
            # the C library's scalar sin and cos (a vectorised form may take CPU-specific paths)
            for j, fn in enumerate((math.sin, math.cos)):
                col = np.array([fn(w * v) for v in range(L)], np.float64)
                term = col[:, None] * W[16 * a + 2 * f + j]
                acc = term if acc is None else acc + term
        parts.append(acc)
    At, Ay, Ax = parts
    base = (At[:, None, None, :] + Ay[None, :, None, :]) + Ax[None, None, :, :]
    return base.reshape(-1, W.shape[1])


def _rng(cfg_id, b, h, tid):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, b, h, tid])))


def _head(wl: Workload, b: int, h: int, seed_offset: int):
    cid = wl.config_id + seed_offset
    d, nv, ns = wl.d, wl.n_video, wl.n_sink
    W = _rng(cid, b, h, _T_W).standard_normal((N_FEATURES, d))
    base = _positional_base(wl.grid, W).astype(np.float32)
    inv = np.float32(1.0 / math.sqrt(d))
    out = []
    for tn, ts in ((_T_QN, _T_QS), (_T_KN, _T_KS), (_T_VN, _T_VS)):
        x = np.empty((nv + ns, d), np.float32)
        noise = _rng(cid, b, h, tn).standard_normal((nv, d), dtype=np.float32)
        x[:nv] = (base + np.float32(0.5) * noise) * inv
        if ns:
            x[nv:] = _rng(cid, b, h, ts).standard_normal((ns, d), dtype=np.float32)
        if wl.dtype == "bf16":
            x = round_to_bf16(x)
        out.append(x)
    return out


def make_qkv(wl: Workload, seed_offset: int = 0, threads: int = 8):
    """Q, K, V as float32 numpy arrays [B, H, N, d] (bf16-exact values for bf16 workloads)."""
    shape = (wl.B, wl.H, wl.N, wl.d)
    Q = np.empty(shape, np.float32)
    K = np.empty(shape, np.float32)
    V = np.empty(shape, np.float32)

    def one(bh):
        b, h = bh
        q, k, v = _head(wl, b, h, seed_offset)
        Q[b, h], K[b, h], V[b, h] = q, k, v

    jobs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    with ThreadPoolExecutor(max_workers=max(1, min(threads, len(jobs)))) as ex:
        list(ex.map(one, jobs))
    return Q, K, V


def gaussian_qkv(B, H, n_video, n_sink, d, seed, dtype="fp32"):
    """Unstructured i.i.d. N(0, 1) inputs for edge-case tests (any N_v, including ragged); with
    softmax scale 1/sqrt(d) the logits have unit spread."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([97, seed])))
    N = n_video + n_sink
    out = []
    for _ in range(3):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if dtype == "bf16":
            x = round_to_bf16(x)
        out.append(x)
    return out
