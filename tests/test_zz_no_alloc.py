"""spark_attn_select_noalloc (the score matrix in the library's static scratch) against
spark_attn_select with a caller-owned workspace: the same kernels, so the routes must be
identical bit for bit, on consecutive calls of different sizes (the scratch keeps the previous
call's contents, which every call overwrites before reading)."""
import pytest
import torch

import block_sparse_attention_score_amd as sa

pytestmark = pytest.mark.gpu


def routes(B, H, M, d, ratio, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    qm = torch.randn(B, H, M, d, generator=g).cuda()
    km = torch.randn(B, H, M, d, generator=g).cuda()
    Q = torch.zeros(B, H, M * 64, d, device="cuda", dtype=torch.bfloat16)  # shapes only
    p = sa.params(Q, 0, 64, ratio)
    K = sa.topk_count(sa.num_key_blocks(p), ratio)
    ref = torch.empty(B, H, M, K, device="cuda", dtype=torch.int32)
    ws = torch.empty(sa.workspace_size(p, 3), device="cuda", dtype=torch.uint8)
    sa.spark_attn_select(p, qm, km, ref, None, ws)
    got = torch.full_like(ref, -1)
    sa.spark_attn_select_noalloc(p, qm, km, got)
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_select_matches_workspace_select():
    assert torch.cuda.is_available()
    # 8 x 591 x 591 scores (11 MB), then a smaller problem, then the large one again
    for B, H, M, d, ratio, seed in ((1, 8, 591, 128, 0.1, 1), (2, 1, 100, 64, 0.3, 2), (1, 8, 591, 128, 0.2, 3)):
        print(f"[gpu-case] noalloc select B={B} H={H} M={M} d={d} ratio={ratio}", flush=True)
        got, ref = routes(B, H, M, d, ratio, seed)
        assert torch.equal(got, ref), (B, H, M, d)
