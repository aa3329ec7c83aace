"""The block-score product's arithmetic (CPU): an fp32 value is exactly the sum of its three bf16
parts, and the three part products the matrix-core kernel drops stay below 2^-23 of sum |q||k|.

The block scores decide the route, so they must be fp32-accurate (near-tie window 1e-4 relative).
The kernel runs them on bf16 MFMA by splitting each fp32 mean x into h = bf16(x),
m = bf16(x - h), l = bf16(x - h - m) (round to nearest even at each step) and accumulating the six
part products h.h, h.m, m.h, h.l, m.m, l.h.  These tests check the facts that make the product
fp32-accurate, in binary64 where every sum below is exact.
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from workloads import round_to_bf16  # noqa: E402


def split3(x):
    x = np.asarray(x, dtype=np.float32)
    h = round_to_bf16(x)
    r1 = (x - h).astype(np.float32)
    m = round_to_bf16(r1)
    l_ = round_to_bf16((r1 - m).astype(np.float32))
    return h, m, l_


def wide_fp32(rng, n):
    """fp32 values over 2^-60 .. 2^60, both signs, every mantissa pattern likely."""
    mant = rng.integers(0, 1 << 23, n, dtype=np.uint64)
    exp = rng.integers(127 - 60, 127 + 60, n, dtype=np.uint64)
    sign = rng.integers(0, 2, n, dtype=np.uint64)
    return ((sign << 31) | (exp << 23) | mant).astype(np.uint32).view(np.float32)


def test_three_bf16_parts_are_exact():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        wide_fp32(rng, 1 << 20),
        np.float32([1.0, -1.0, 0.0, 2.0 ** -20, 3.0, 0.1, 1.0 - 2.0 ** -24, 1.0 + 2.0 ** -23]),
        # every mantissa bit set, and the rounding carry cases (low half 0x8000 and around it)
        (np.uint32(0x3FFFFFFF) - np.arange(4096, dtype=np.uint32)).view(np.float32),
        (np.uint32(0x3F808000) + np.arange(-2048, 2048, dtype=np.int64).astype(np.uint32)).view(np.float32),
    ])
    h, m, l_ = split3(x)
    for part in (h, m, l_):  # each part is a bf16 value
        assert np.array_equal(part, round_to_bf16(part))
    total = h.astype(np.float64) + m.astype(np.float64) + l_.astype(np.float64)
    assert np.array_equal(total, x.astype(np.float64))
    # the parts shrink by at least 2^-8 each: |m| <= 2^-8 |x|, |l| <= 2^-16 |x| (relative bound
    # on each part's magnitude, used by the dropped-term bound)
    ax = np.abs(x.astype(np.float64))
    nz = ax > 0
    assert (np.abs(m.astype(np.float64))[nz] <= 2.0 ** -8 * ax[nz]).all()
    assert (np.abs(l_.astype(np.float64))[nz] <= 2.0 ** -16 * ax[nz]).all()


def test_dropped_part_products_below_two_to_minus_23():
    rng = np.random.default_rng(12)
    n, d = 4096, 128
    q = (rng.standard_normal((n, d)) * np.exp2(rng.integers(-8, 8, (n, 1)))).astype(np.float32)
    k = (rng.standard_normal((n, d)) * np.exp2(rng.integers(-8, 8, (n, 1)))).astype(np.float32)
    qh, qm, ql = (p.astype(np.float64) for p in split3(q))
    kh, km, kl = (p.astype(np.float64) for p in split3(k))
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    exact = (q64 * k64).sum(axis=1)
    kept = (qh * kh + qh * km + qm * kh + qh * kl + qm * km + ql * kh).sum(axis=1)
    scale = (np.abs(q64) * np.abs(k64)).sum(axis=1)
    err = np.abs(kept - exact) / scale
    # worst case |m.l| + |l.m| + |l.l| <= (2 * 2^-24 + 2^-32) |q||k| per term
    assert err.max() <= 2.0 ** -23, err.max()
    # every dropped product, term by term, within its worst-case weight
    dropped = np.abs(qm * kl) + np.abs(ql * km) + np.abs(ql * kl)
    assert (dropped <= (2.0 ** -23) * np.abs(q64) * np.abs(k64) + 1e-300).all()
    # one bf16 rounding of the means (the shortcut the kernel does not take) is far outside
    single = (qh * kh).sum(axis=1)
    assert (np.abs(single - exact) / scale).max() > 2.0 ** -12


def test_integer_valued_means_need_only_the_high_part():
    # integer-valued means (the exact-score route tests use them) are bf16 values already
    x = np.arange(-256, 257, dtype=np.float32)
    h, m, l_ = split3(x)
    assert np.array_equal(h, x) and not m.any() and not l_.any()
