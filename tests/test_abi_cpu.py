"""C-ABI contract checks that need no GPU: the library loads, exports every declared symbol, its
host helpers agree with the oracle's budget rule, and invalid arguments are rejected with their
status before any device work (only fake, never-dereferenced addresses are passed)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_score_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spark_attn.h")

OK, INVALID, UNSUPPORTED, WS_SMALL, HIP_ERR, MISALIGNED = 0, -1, -2, -3, -4, -5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spark_attn_[a-z0-9_]+)\s*\(", text)))


def P(**kw):
    base = dict(B=1, H=2, N=1000, d=128, n_sink=8, block=128, topk_ratio=0.1, pool_mode=1,
                dtype=0, scale=0.0)
    base.update(kw)
    return sa.SparkAttnParams(**base)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(sa.EXPORTS)
    L = sa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_header_struct_matches_binding():
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} spark_attn_params;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\b(int|float)\s+([A-Za-z_, ]+);", body)
    names = [n.strip() for _, group in fields for n in group.split(",")]
    assert names == [f[0] for f in sa.SparkAttnParams._fields_]


@pytest.mark.parametrize("M,ratio,K", [(64, 0.1, 6), (240, 0.1, 24), (591, 0.1, 59), (591, 0.2, 118),
                                       (591, 0.3, 177), (591, 1.0, 591), (1922, 0.1, 192),
                                       (10, 0.01, 1), (7, 0.5, 4), (3, 1e-6, 1)])
def test_topk_count_matches_oracle(orc, M, ratio, K):
    assert sa.topk_count(M, ratio) == K == orc.topk_count(M, ratio)


def test_topk_count_rejects_bad_ratio():
    L = sa.lib()
    assert L.spark_attn_topk_count(10, 0.0) == INVALID
    assert L.spark_attn_topk_count(10, 1.5) == INVALID
    assert L.spark_attn_topk_count(10, float("nan")) == INVALID
    assert L.spark_attn_topk_count(0, 0.5) == INVALID


def test_num_blocks():
    L = sa.lib()
    assert L.spark_attn_num_blocks(ctypes.byref(P(N=1000, n_sink=8, block=128))) == 8
    assert L.spark_attn_num_blocks(ctypes.byref(P(N=30720 + 256, n_sink=256))) == 240
    assert L.spark_attn_num_blocks(ctypes.byref(P(N=245952 + 512, n_sink=512))) == 1922
    assert L.spark_attn_num_blocks(ctypes.byref(P(N=75600 + 512, n_sink=512))) == 591
    assert L.spark_attn_num_blocks(ctypes.byref(P(N=5, n_sink=0, block=64, d=64))) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), INVALID), (dict(H=0), INVALID), (dict(N=0), INVALID), (dict(n_sink=-1), INVALID),
    (dict(n_sink=1000), INVALID), (dict(topk_ratio=0.0), INVALID), (dict(topk_ratio=1.01), INVALID),
    (dict(topk_ratio=float("nan")), INVALID), (dict(pool_mode=2), INVALID),
    (dict(scale=-1.0), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(block=32), UNSUPPORTED),
    (dict(block=256), UNSUPPORTED), (dict(dtype=2), UNSUPPORTED),
    (dict(N=16384 * 128 + 2, n_sink=1, d=64, H=1), UNSUPPORTED),  # M > 16384
    (dict(B=64, H=64, N=8192, d=128), UNSUPPORTED),                # B*H*N*d >= 2^31
])
def test_invalid_params_rejected_before_launch(kw, status):
    L = sa.lib()
    p = P(**kw)
    fake = ctypes.c_void_p(0x100000)
    assert L.spark_attn_num_blocks(ctypes.byref(p)) == status
    assert L.spark_attn_workspace_size(ctypes.byref(p), 0) == 0
    assert L.spark_attn_pool(ctypes.byref(p), *([fake] * 9), None) == status
    assert L.spark_attn_select(ctypes.byref(p), fake, fake, fake, None, fake, 1 << 40, None) == status
    assert L.spark_attn_pack(ctypes.byref(p), *([fake] * 6), 1 << 40, None) == status
    assert L.spark_attn_attend(ctypes.byref(p), fake, fake, 1 << 40, fake, None, fake, None, None) == status
    assert L.spark_attn_forward(ctypes.byref(p), fake, fake, fake, None, fake, None, None, fake,
                                1 << 40, None) == status
    assert L.spark_attn_forward_kv(ctypes.byref(p), fake, fake, fake, None, fake, fake, None, None, fake,
                                   1 << 40, None) == status
    assert L.spark_attn_reblock(ctypes.byref(p), fake, fake, fake, fake, 1 << 40, None) == status
    assert L.spark_attn_gather_rows(ctypes.byref(p), fake, fake, ctypes.c_void_p(0x200000), None) == status


def test_null_and_misaligned_pointers_rejected():
    L = sa.lib()
    p = P()
    a = ctypes.c_void_p(0x100000)
    bad = ctypes.c_void_p(0x100008)
    assert L.spark_attn_pool(ctypes.byref(p), None, a, a, a, a, a, a, a, a, None) == INVALID
    assert L.spark_attn_pool(ctypes.byref(p), bad, a, a, a, a, a, a, a, a, None) == MISALIGNED
    assert L.spark_attn_select(ctypes.byref(p), a, a, None, None, a, 1 << 40, None) == INVALID
    assert L.spark_attn_select(ctypes.byref(p), bad, a, a, None, a, 1 << 40, None) == MISALIGNED
    assert L.spark_attn_select(ctypes.byref(p), a, a, a, None, None, 0, None) == WS_SMALL
    assert L.spark_attn_select(ctypes.byref(p), a, a, a, None, a, 10, None) == WS_SMALL
    assert L.spark_attn_attend(ctypes.byref(p), a, a, 1 << 40, None, None, a, None, None) == INVALID
    assert L.spark_attn_attend(ctypes.byref(p), a, a, 1 << 40, a, None, bad, None, None) == MISALIGNED
    assert L.spark_attn_attend(ctypes.byref(p), a, a, 10, a, None, a, None, None) == WS_SMALL
    assert L.spark_attn_attend(ctypes.byref(p), a, None, 1 << 40, a, None, a, None, None) == WS_SMALL
    assert L.spark_attn_pack(ctypes.byref(p), a, None, a, a, a, a, 1 << 40, None) == INVALID
    assert L.spark_attn_pack(ctypes.byref(p), a, a, a, bad, a, a, 1 << 40, None) == MISALIGNED
    assert L.spark_attn_pack(ctypes.byref(p), a, a, a, a, a, a, 10, None) == WS_SMALL
    assert L.spark_attn_forward(ctypes.byref(p), a, a, a, None, None, None, None, a, 1 << 40, None) == INVALID
    assert L.spark_attn_forward(ctypes.byref(p), a, bad, a, None, a, None, None, a, 1 << 40, None) == MISALIGNED
    assert L.spark_attn_forward_kv(ctypes.byref(p), a, a, None, None, None, a, None, None, a, 1 << 40, None) == INVALID
    assert L.spark_attn_forward_kv(ctypes.byref(p), a, a, a, None, None, bad, None, None, a, 1 << 40, None) == MISALIGNED
    assert L.spark_attn_gather_rows(ctypes.byref(p), a, a, a, None) == INVALID  # in place
    assert L.spark_attn_gather_rows(ctypes.byref(p), a, None, ctypes.c_void_p(0x200000), None) == INVALID
    assert L.spark_attn_reblock(ctypes.byref(p), a, a, None, a, 1 << 40, None) == INVALID


def test_workspace_sizes_and_too_small():
    L = sa.lib()
    p = P(N=245952 + 512, n_sink=512, H=24)
    w0 = L.spark_attn_workspace_size(ctypes.byref(p), 0)
    w2 = L.spark_attn_workspace_size(ctypes.byref(p), 2)
    M, K, d, BH = 1922, 192, 128, 24
    Tall = 1922 * 2 + 8 + 31  # video (2 per block), sink and compressed 64-key tiles per head
    NQT = 4 + M  # query tiles per head: 512 sink rows in 4 tiles of 128, then the video blocks
    # tiles (K rows | V^T, bf16) and their additive rows (fp32), per-tile norm/term maxima (2 fp32),
    # per-head bound constants (4 fp32), per-query-tile flags (int32), the attention pass's eight
    # tile counters (int32), each region 256-byte aligned
    packed = BH * Tall * 64 * (2 * d * 2 + 4) + BH * Tall * 8 + BH * 16 + BH * NQT * 4 + 8 * 4
    assert packed <= L.spark_attn_workspace_size(ctypes.byref(p), 4) < packed + 5 * 256
    need = 4 * BH * M * d * 4 + BH * M * 4 + BH * d * 4 + BH * M * K * 4 + BH * M * M * 4 + packed
    assert need <= w0 < need + 15 * 256
    assert L.spark_attn_workspace_size(ctypes.byref(p), 3) == BH * M * M * 4
    assert w2 - w0 >= 3 * BH * (245952 + 512) * d * 2
    a = ctypes.c_void_p(0x100000)
    assert L.spark_attn_forward(ctypes.byref(p), a, a, a, None, a, None, None, a, w0 - 1, None) == WS_SMALL
    assert L.spark_attn_forward(ctypes.byref(p), a, a, a, a, a, None, None, a, w2 - 1, None) == WS_SMALL
    assert L.spark_attn_forward(ctypes.byref(p), a, a, a, None, a, None, None, None, w0, None) == WS_SMALL
    # a separate key partition alone needs the permuted-layout workspace too
    assert L.spark_attn_forward_kv(ctypes.byref(p), a, a, a, None, a, a, None, None, a, w2 - 1, None) == WS_SMALL
    assert L.spark_attn_forward_kv(ctypes.byref(p), a, a, a, a, None, a, None, None, a, w2 - 1, None) == WS_SMALL
    assert L.spark_attn_forward_kv(ctypes.byref(p), a, a, a, None, None, a, None, None, a, w0 - 1, None) == WS_SMALL


def test_status_strings():
    for s in (OK, INVALID, UNSUPPORTED, WS_SMALL, HIP_ERR, MISALIGNED):
        assert sa.status_str(s) and sa.status_str(s) != "unknown status"
    assert sa.status_str(-99) == "unknown status"


def test_adaptive_tau_entry_points_validate_before_launch():
    L = sa.lib()
    p = P()
    a = ctypes.c_void_p(0x100000)
    bad = ctypes.c_void_p(0x100008)
    f = ctypes.c_float
    w5 = L.spark_attn_workspace_size(ctypes.byref(p), 5)
    w6 = L.spark_attn_workspace_size(ctypes.byref(p), 6)
    M = L.spark_attn_num_blocks(ctypes.byref(p))
    BH = p.B * p.H
    # select: the score matrix plus per-head partial sums
    assert w5 >= BH * M * M * 4
    assert w6 > w5
    for t in (float("nan"), float("inf"), float("-inf")):
        assert L.spark_attn_select_tau(ctypes.byref(p), f(t), a, a, a, a, None, a, w5, None) == INVALID
        assert L.spark_attn_forward_tau(ctypes.byref(p), f(t), a, a, a, a, None, None, None, a, w6, None) == INVALID
    assert L.spark_attn_select_tau(ctypes.byref(p), f(1.0), a, a, None, a, None, a, w5, None) == INVALID
    assert L.spark_attn_select_tau(ctypes.byref(p), f(1.0), a, a, a, None, None, a, w5, None) == INVALID
    assert L.spark_attn_select_tau(ctypes.byref(p), f(1.0), bad, a, a, a, None, a, w5, None) == MISALIGNED
    assert L.spark_attn_select_tau(ctypes.byref(p), f(1.0), a, a, a, a, None, a, w5 - 1, None) == WS_SMALL
    assert L.spark_attn_attend_var(ctypes.byref(p), a, a, 1 << 40, a, None, None, a, None, None) == INVALID
    assert L.spark_attn_attend_var(ctypes.byref(p), a, a, 10, a, a, None, a, None, None) == WS_SMALL
    assert L.spark_attn_forward_tau(ctypes.byref(p), f(1.0), a, a, a, a, None, None, None, a, w6 - 1, None) == WS_SMALL
    assert L.spark_attn_forward_tau(ctypes.byref(p), f(1.0), a, None, a, a, None, None, None, a, w6, None) == INVALID
    q = P(d=96)
    assert L.spark_attn_select_tau(ctypes.byref(q), f(1.0), a, a, a, a, None, a, 1 << 40, None) == UNSUPPORTED


def test_fp8_entry_points_validate_before_launch():
    L = sa.lib()
    p = P()
    a = ctypes.c_void_p(0x100000)
    bad = ctypes.c_void_p(0x100008)
    w7 = L.spark_attn_workspace_size(ctypes.byref(p), 7)
    w8 = L.spark_attn_workspace_size(ctypes.byref(p), 8)
    w9 = L.spark_attn_workspace_size(ctypes.byref(p), 9)
    # E4M3 tiles are half the bf16 tiles' key/value bytes (same bias rows)
    w4 = L.spark_attn_workspace_size(ctypes.byref(p), 4)
    M = L.spark_attn_num_blocks(ctypes.byref(p))
    Tall = M + (p.n_sink + 63) // 64 + (M + 63) // 64
    BH = p.B * p.H
    assert w9 >= BH * Tall * 128 * p.d and w9 < w4
    assert w8 > w7 > w9
    byref = ctypes.byref
    assert L.spark_attn_fp8_scales(byref(p), a, a, a, None, None) == INVALID
    assert L.spark_attn_fp8_scales(byref(p), a, bad, a, a, None) == MISALIGNED
    assert L.spark_attn_pack_fp8(byref(p), a, a, a, a, a, None, a, w9, None) == INVALID
    assert L.spark_attn_pack_fp8(byref(p), a, a, a, a, a, a, a, w9 - 1, None) == WS_SMALL
    assert L.spark_attn_attend_fp8(byref(p), a, a, w9, a, None, None, a, None, None) == INVALID
    assert L.spark_attn_attend_fp8(byref(p), a, a, w9 - 1, a, None, a, a, None, None) == WS_SMALL
    assert L.spark_attn_attend_fp8(byref(p), a, bad, w9, a, None, a, a, None, None) == MISALIGNED
    assert L.spark_attn_forward_fp8(byref(p), a, a, a, None, a, None, None, None, a, w7 - 1, None) == WS_SMALL
    assert L.spark_attn_forward_fp8(byref(p), a, a, a, a, a, None, None, None, a, w8 - 1, None) == WS_SMALL
    assert L.spark_attn_forward_fp8(byref(p), a, None, a, None, a, None, None, None, a, w7, None) == INVALID
    q = P(d=96)
    assert L.spark_attn_forward_fp8(byref(q), a, a, a, None, a, None, None, None, a, 1 << 40, None) == UNSUPPORTED


def test_key_block_size_validation_and_counts():
    L = sa.lib()
    byref = ctypes.byref
    p = P(N=1000, n_sink=8, block=128, block_k=64)
    nv = 1000 - 8
    assert L.spark_attn_num_blocks(byref(p)) == -(-nv // 128)
    assert L.spark_attn_num_key_blocks(byref(p)) == -(-nv // 64)
    assert L.spark_attn_num_key_blocks(byref(P())) == L.spark_attn_num_blocks(byref(P()))
    assert L.spark_attn_num_key_blocks(byref(P(block_k=32))) == UNSUPPORTED
    assert L.spark_attn_num_key_blocks(byref(P(block_k=-1))) == INVALID
    # the score matrix is query blocks x key blocks; the compressed tiles cover the key blocks
    M, Mk = -(-nv // 128), -(-nv // 64)
    assert L.spark_attn_workspace_size(byref(p), 3) == p.B * p.H * M * Mk * 4
    a = ctypes.c_void_p(0x100000)
    # adaptive tau is defined for equal query and key blocks
    assert L.spark_attn_select_tau(byref(p), ctypes.c_float(1.0), a, a, a, a, None, a, 1 << 40, None) == UNSUPPORTED
    assert L.spark_attn_forward_tau(byref(p), ctypes.c_float(1.0), a, a, a, a, None, None, None, a, 1 << 40,
                                    None) == UNSUPPORTED


def test_pool_pack_validates_before_launch():
    L = sa.lib()
    p = P()
    a = ctypes.c_void_p(0x100000)
    bad = ctypes.c_void_p(0x100008)
    byref = ctypes.byref
    w4 = L.spark_attn_workspace_size(byref(p), 4)
    args = [a] * 9  # Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor
    assert L.spark_attn_pool_pack(byref(p), *args, a, w4 - 1, None) == WS_SMALL
    assert L.spark_attn_pool_pack(byref(p), *args, None, w4, None) == WS_SMALL
    for i in range(9):
        miss = list(args)
        miss[i] = None
        assert L.spark_attn_pool_pack(byref(p), *miss, a, w4, None) == INVALID
    mis = list(args)
    mis[1] = bad
    assert L.spark_attn_pool_pack(byref(p), *mis, a, w4, None) == MISALIGNED
    assert L.spark_attn_pool_pack(byref(p), *args, bad, w4, None) == MISALIGNED
    assert L.spark_attn_pool_pack(byref(P(d=96)), *args, a, 1 << 40, None) == UNSUPPORTED


def test_pool_fp8_scales_validates_before_launch():
    L = sa.lib()
    p = P()
    a = ctypes.c_void_p(0x100000)
    bad = ctypes.c_void_p(0x100008)
    byref = ctypes.byref
    args = [a] * 10  # Q, K, V, q_mean, k_mean, k_sum, v_sum, bias, anchor, amax
    for i in range(10):
        miss = list(args)
        miss[i] = None
        assert L.spark_attn_pool_fp8_scales(byref(p), *miss, None) == INVALID
    mis = list(args)
    mis[0] = bad
    assert L.spark_attn_pool_fp8_scales(byref(p), *mis, None) == MISALIGNED
    assert L.spark_attn_pool_fp8_scales(byref(P(d=96)), *args, None) == UNSUPPORTED


def test_binding_checks_tensor_sizes_and_types():
    """The Python wrappers check every buffer against the parameters before handing bare pointers
    to the library.  CPU tensors are used: a buffer that passes the size and type check then
    fails the device-tensor check, so no call reaches the library's launch path."""
    import torch

    B, H, N, d, ns, b = 1, 2, 1000, 128, 8, 128
    p = sa.params(torch.empty(B, H, N, d, dtype=torch.bfloat16), ns, b, 0.1)
    M = sa.num_blocks(p)
    Kk = sa.topk_count(M, 0.1)
    f32, i32 = torch.float32, torch.int32
    good = dict(
        Q=torch.empty(B, H, N, d, dtype=torch.bfloat16), K=torch.empty(B, H, N, d, dtype=torch.bfloat16),
        V=torch.empty(B, H, N, d, dtype=torch.bfloat16), q_mean=torch.empty(B, H, M, d, dtype=f32),
        k_mean=torch.empty(B, H, M, d, dtype=f32), k_sum=torch.empty(B, H, M, d, dtype=f32),
        v_sum=torch.empty(B, H, M, d, dtype=f32), bias=torch.empty(B, H, M, dtype=f32),
        anchor=torch.empty(B, H, d, dtype=f32))
    order = ["Q", "K", "V", "q_mean", "k_mean", "k_sum", "v_sum", "bias", "anchor"]

    def pool(**over):
        t = dict(good, **over)
        sa.spark_attn_pool(p, *[t[k] for k in order])

    with pytest.raises(ValueError, match="device tensors"):
        pool()
    with pytest.raises(TypeError, match="Q: element type"):
        pool(Q=good["Q"].float())
    with pytest.raises(ValueError, match="bias: 1 elements"):
        pool(bias=torch.empty(1, dtype=f32))
    with pytest.raises(ValueError, match="anchor"):
        pool(anchor=torch.empty(B, H, d - 1, dtype=f32))
    O = torch.empty(B, H, N, d, dtype=torch.bfloat16)
    packed = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match=f"idx: {M * (Kk - 1) * 2} elements, expected {B * H * M * Kk}"):
        sa.spark_attn_attend(p, good["Q"], packed, torch.empty(B, H, M, Kk - 1, dtype=i32), None, O)
    with pytest.raises(TypeError, match="idx: element type"):
        sa.spark_attn_attend(p, good["Q"], packed, torch.empty(B, H, M, Kk, dtype=torch.int64), None, O)
    with pytest.raises(ValueError, match="perm"):
        sa.spark_attn_attend(p, good["Q"], packed, torch.empty(B, H, M, Kk, dtype=i32),
                             torch.empty(B, H, N - ns - 1, dtype=i32), O)
    with pytest.raises(ValueError, match="lse"):
        sa.spark_attn_attend(p, good["Q"], packed, torch.empty(B, H, M, Kk, dtype=i32), None, O,
                             torch.empty(B, H, N - 1, dtype=f32))
    with pytest.raises(ValueError, match="amax"):
        sa.spark_attn_fp8_scales(p, good["Q"], good["K"], good["V"], torch.empty(B, H, 2, dtype=f32))
    with pytest.raises(ValueError, match="Y"):
        sa.spark_attn_gather_rows(p, good["Q"], torch.empty(B, H, N - ns, dtype=i32),
                                  torch.empty(B, H, N - 1, d, dtype=torch.bfloat16))
    # invalid parameters are left to the library's own status
    bad = sa.params(good["Q"], N, b, 0.1)  # n_sink = N
    with pytest.raises(ValueError, match="device tensors"):
        sa.spark_attn_pool(bad, *[torch.empty(1, dtype=f32)] * 9)


def test_content_checks_of_index_inputs():
    """sa.check_contents (run before every launch under SPARK_ATTN_CHECK=1) accepts routes,
    variable routes and permutations as the header documents them and rejects entries the
    kernels would otherwise clamp or skip: route entries outside [0, M_k), rows not strictly
    ascending, counts outside [0, M_k], permutation entries outside [0, N_v).  CPU tensors."""
    import torch

    p = P(N=1000, n_sink=8, block=128, topk_ratio=0.3)  # N_v = 992: M = M_k = 8, K = 2
    M, K, Nv = 8, 2, 992
    idx = torch.tensor([[0, 5]] * M, dtype=torch.int32).expand(2, M, K).reshape(1, 2, M, K).contiguous()
    sa.check_contents(p, idx=idx)
    for bad, msg in ((7 + 1, "outside"), (-1, "outside")):
        b = idx.clone()
        b[0, 1, 3, 1] = bad
        with pytest.raises(ValueError, match=msg):
            sa.check_contents(p, idx=b)
    b = idx.clone()
    b[0, 0, 2] = torch.tensor([4, 4], dtype=torch.int32)
    with pytest.raises(ValueError, match="ascending"):
        sa.check_contents(p, idx=b)
    # variable route: entries past counts[I] are not looked at
    var = torch.full((1, 2, M, M), 99, dtype=torch.int32)
    counts = torch.zeros(1, 2, M, dtype=torch.int32)
    var[0, 0, 1, :3] = torch.tensor([1, 2, 7], dtype=torch.int32)
    counts[0, 0, 1] = 3
    sa.check_contents(p, idx=var, counts=counts)
    counts[0, 1, 0] = M + 1
    with pytest.raises(ValueError, match="counts"):
        sa.check_contents(p, idx=var, counts=counts)
    perm = torch.arange(Nv, dtype=torch.int32).flip(0).expand(2, Nv).reshape(1, 2, Nv).contiguous()
    sa.check_contents(p, perm=perm)
    b = perm.clone()
    b[0, 1, 10] = Nv
    with pytest.raises(ValueError, match="perm"):
        sa.check_contents(p, perm=b)


def test_noalloc_select_rejects_before_any_launch():
    """spark_attn_select_noalloc validates before touching the device: a score matrix larger than
    the static scratch (64 MiB) is SCRATCH_TOO_SMALL, null pointers INVALID_ARGUMENT (fake,
    never-dereferenced addresses)."""
    L = sa.lib()
    a = ctypes.c_void_p(0x100000)
    big = P(N=245952 + 512, n_sink=512, H=24)  # 24 x 1922 x 1922 scores = 355 MB
    assert L.spark_attn_select_noalloc(ctypes.byref(big), a, a, a, None) == -6
    assert L.spark_attn_status_str(-6) == b"problem exceeds the library's static scratch"
    small = P(N=75600 + 512, n_sink=512, H=24)  # 24 x 591 x 591 scores = 33.5 MB: fits
    assert L.spark_attn_select_noalloc(ctypes.byref(small), None, a, a, None) == INVALID
    assert L.spark_attn_select_noalloc(ctypes.byref(small), a, a, None, None) == INVALID
