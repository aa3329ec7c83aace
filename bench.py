#!/usr/bin/env python3
"""Benchmark of the two-branch block-sparse attention forward on one MI355X.

One step = one pass of the whole path over one batch of synthetic video-shaped input resident
in HBM: pool -> select -> pack -> attend, launched through the library's C entry points on the
current stream (the same launches spark_attn_forward makes without a partition).  HIP events on that
stream bracket every stage inside the timed region; the attention kernel's average duration gives
the roofline figure.

Order of a default run:
  1. warmup steps;
  2. the CPU leg, on the warmup step's outputs: the oracle pools the same input, scores every block
     pair and checks every route row against the near-tie rule, then attends a seeded sample of
     query blocks and sink rows through the GPU's route and compares them element by element with
     the GPU's O and LSE (the same bound as the parity tests).  Any route or parity violation ends
     the run with a non-zero exit status before anything is timed.  The same oracle calls, timed,
     are the CPU baseline (host cores, bounded sample, full forward extrapolated);
  3. the timed steps, after which the output and route must equal the checked ones bit for bit
     (exit status 4 otherwise);
  4. cold-cache steps, the single-call cross-check and a pooling-only timing.
--no-cpu-baseline skips step 2 (no oracle runs; the JSON then says the route was not checked).

Prints ONE JSON line.  Default workload: the full 1344x768x240-frame clip (245,952 video +
512 sink tokens, H=24, d=128, block 128, topk_ratio 0.1, anchor-weighted compressed branch).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (no sparsity)
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak (no sparsity)
HBM_PEAK_GBS = 8000.0
MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak
# the forward tolerances of the parity tests (bf16 matrix-core attention against the binary64 oracle)
FWD_REL_L2, FWD_MAX_ABS = 1e-2, 2e-2


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_flops(idx, wl, ratio_K, counts=None, block_k=0):
    """F_sel from the actual route, plus the sink, compressed and sink-query terms (4 d per
    query-key pair: one multiply-add for the logit and one for the value).  A variable route is
    idx [B,H,M,M] with counts [B,H,M].  block_k: key block size (0: the query block size)."""
    import numpy as np

    b, nv, ns, d, N = wl.block, wl.n_video, wl.n_sink, wl.d, wl.N
    bk = block_k or b
    M = idx.shape[2]
    Mk = -(-nv // bk)
    sizes = np.minimum(b, nv - np.arange(M) * b).astype(np.int64)  # query block sizes
    ksizes = np.minimum(bk, nv - np.arange(Mk) * bk).astype(np.int64)  # key block sizes
    BH = wl.B * wl.H
    if counts is None:
        n_sel = ksizes[idx].sum(axis=-1)  # [B,H,M] keys in the selected blocks of each query block
        n_unsel = float(BH * nv * (Mk - ratio_K))
    else:
        valid = np.arange(M)[None, None, None, :] < counts[..., None]
        n_sel = np.where(valid, sizes[np.clip(idx, 0, M - 1)], 0).sum(axis=-1)
        n_unsel = float(((M - counts) * sizes[None, None, :]).sum())
    F_sel = 4.0 * d * float((n_sel * sizes[None, None, :]).sum())
    F_sink = 4.0 * d * nv * ns * BH
    F_comp = 4.0 * d * n_unsel
    F_sinkq = 4.0 * d * ns * N * BH
    return F_sel, F_sink, F_comp, F_sinkq


def committed_traffic(workload, kernel="attn_fwd"):
    """HBM bytes per attention launch from the committed counter summary, or None when the kernel
    source has changed since the counters were taken (or no summary exists for the workload)."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(kernel + r"_kernel_source_sha256_16: ([0-9a-f]+)", text)
    t = re.search(kernel + r"_kernel_traffic_bytes_per_launch: ([0-9.]+)", text)
    if not h or not t or kernel_source_hash(kernel) != h.group(1):
        return None
    return float(t.group(1))


def kernel_source_hash(kernel):
    """sha256 (16 hex digits) of an attention kernel's source file and the headers it includes."""
    import hashlib

    csrc = os.path.join(ROOT, "block_sparse_attention_score_amd", "csrc")
    files = [f"{kernel}.hip", "common.hpp", "kernels.hpp"] + (["attn_tile.hpp"] if kernel == "attn_fwd" else [])
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def route_check(idx, S, rel=1e-4, floor=1e-6):
    """Rows whose GPU route violates the near-tie rule against oracle scores S (vectorised)."""
    import numpy as np

    K = idx.shape[-1]
    M = S.shape[-1]
    S2 = S.reshape(-1, M)
    I2 = idx.reshape(-1, K)
    part = -np.sort(-S2, axis=1)
    sK = part[:, K - 1]
    sK1 = part[:, K] if K < M else np.full_like(sK, -np.inf)
    delta = rel * np.maximum(np.abs(sK), np.where(np.isfinite(sK1), np.abs(sK1), 0)) + floor * np.abs(S2).max(1)
    chosen = np.zeros_like(S2, dtype=bool)
    np.put_along_axis(chosen, I2.astype(np.int64), True, axis=1)
    must = S2 > (sK + delta)[:, None]
    allowed = S2 >= (sK - delta)[:, None]
    ok = (chosen.sum(1) == K) & ~(must & ~chosen).any(1) & ~(chosen & ~allowed).any(1)
    ok &= (np.diff(I2, axis=1) > 0).all(1) if K > 1 else True
    return int((~ok).sum())


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_sample(wl, M, sample_blocks, n_sink_rows=16, seed=7):
    """Seeded sample of the CPU leg: (b*H + h, I) for video query blocks I < M and sink rows M + j."""
    import numpy as np

    rng = np.random.default_rng(seed)
    BH = wl.B * wl.H
    qb = np.stack([rng.integers(0, BH, sample_blocks), rng.integers(0, M, sample_blocks)], 1)
    sq = np.stack([rng.integers(0, BH, n_sink_rows), M + rng.integers(0, max(wl.n_sink, 1), n_sink_rows)], 1)
    return qb, (sq if wl.n_sink else sq[:0])


def sample_rows(wl, M, entries):
    """Row indices (within a (batch, head)) of each sample entry, in the layout the route refers to."""
    import numpy as np

    out = []
    for bh, I in entries:
        if I < M:
            out.append(np.arange(I * wl.block, min(wl.n_video, (I + 1) * wl.block)))
        else:
            out.append(np.array([wl.n_video + I - M]))
    return out


def cpu_baseline(wl, ratio, Qh, Kh, Vh, gidx, F_sel_total, qb, sq, g_rows, block_k=0, single_core_blocks=24):
    """The oracle as it stands, on a bounded sample: full pool, full block scores and top-K, and
    the attention of the sampled video query blocks and sink rows; the full forward time is
    extrapolated from the per-block time.  The same results check the GPU: every route row against
    the near-tie rule, and the sampled attention rows g_rows = (O rows, LSE rows) of the GPU in the
    sample's order."""
    import numpy as np
    import oracle

    p = oracle.params(Qh, wl.n_sink, wl.block, ratio, 1, block_k=block_k)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    pooled = oracle.pool(p, Qh, Kh, Vh)
    t1 = time.perf_counter()
    S = oracle.scores(p, pooled["q_mean"], pooled["k_mean"])
    oidx = oracle.select(p, S)
    t2 = time.perf_counter()
    bad = route_check(gidx, S)
    same = float((oidx == gidx).all(axis=-1).mean())
    M = S.shape[-2]  # query blocks
    BH = wl.B * wl.H
    t3 = time.perf_counter()
    Ob, lb = oracle.attend_blocks(p, Qh, Kh, Vh, pooled, gidx, qb)
    t4 = time.perf_counter()
    Os, ls = oracle.attend_blocks(p, Qh, Kh, Vh, pooled, gidx, sq) if len(sq) else (None, None)
    t5 = time.perf_counter()
    # element-by-element comparison with the GPU rows of the same entries
    r_rows, r_lse = [], []
    for O_, l_, ent in ((Ob, lb, qb), (Os, ls, sq)):
        for n, (bh, I) in enumerate(ent):
            m = (min(wl.n_video, (I + 1) * wl.block) - I * wl.block) if I < M else 1
            r_rows.append(O_[n, :m])
            r_lse.append(l_[n, :m])
    R, RL = np.concatenate(r_rows), np.concatenate(r_lse)
    G, GL = g_rows
    rel = float(np.linalg.norm(G - R) / np.linalg.norm(R))
    mab = float(np.abs(G - R).max())
    lab = float(np.abs(GL - RL).max())
    per_block = (t4 - t3) / len(qb)
    per_sink_row = (t5 - t4) / max(len(sq), 1)
    t_full = (t1 - t0) + (t2 - t1) + per_block * BH * M + per_sink_row * BH * wl.n_sink
    # one host core: the attention of a few of the same query blocks, scaled the same way
    n1 = max(1, min(len(qb), single_core_blocks))
    oracle.set_num_threads(1)
    try:
        t6 = time.perf_counter()
        oracle.attend_blocks(p, Qh, Kh, Vh, pooled, gidx, qb[:n1])
        t7 = time.perf_counter()
    finally:
        oracle.set_num_threads(threads)
    t_full_1 = (t7 - t6) / n1 * BH * M  # attention of every video query block on one core
    return {
        "value": F_sel_total / t_full / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"binary64 C oracle on the same {wl.name} input: full pool ({t1 - t0:.1f} s), full "
                   f"block scores + top-K ({t2 - t1:.1f} s), attention of {len(qb)} random video "
                   f"query blocks ({t4 - t3:.1f} s) and {len(sq)} sink query rows ({t5 - t4:.1f} s); "
                   f"full forward extrapolated to {t_full:.0f} s"),
        "est_forward_s": t_full,
        "cpu_model": cpu_model(),
        "single_core": {"query_blocks": n1, "seconds": round(t7 - t6, 2),
                        "attention_per_block_s": round((t7 - t6) / n1, 4),
                        "est_attention_s": round(t_full_1, 1),
                        "speedup_of_all_threads": round((t7 - t6) / n1 / per_block, 2)},
    }, {
        "route_rows_checked": int(gidx.shape[0] * gidx.shape[1] * gidx.shape[2]),
        "route_rows_violating_near_tie_rule": bad,
        "route_rows_equal_to_oracle": same,
        "sampled_query_blocks": int(len(qb)), "sampled_sink_rows": int(len(sq)),
        "rows_compared": int(R.shape[0]),
        "rel_l2": rel, "max_abs": mab, "lse_max_abs": lab,
        "bounds": {"rel_l2": FWD_REL_L2, "max_abs": FWD_MAX_ABS, "lse_max_abs": FWD_MAX_ABS},
        "ok": bool(bad == 0 and rel <= FWD_REL_L2 and mab <= FWD_MAX_ABS and lab <= FWD_MAX_ABS),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fullclip")
    ap.add_argument("--ratio", type=float, default=None)
    ap.add_argument("--tau", type=float, default=None,
                    help="adaptive-tau selection (per-head threshold mu + tau*sigma) instead of top-K")
    ap.add_argument("--block-k", type=int, default=0,
                    help="key block size of the route (0: the workload's block); 64 with block 128 is the "
                         "asymmetric 128Q x 64KV route")
    ap.add_argument("--fp8", action="store_true",
                    help="the exact branch, sinks and pseudo-keys on per-head E4M3 carriers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-blocks", type=int, default=600)
    ap.add_argument("--no-forward-check", action="store_true",
                    help="skip the spark_attn_forward cross-check launches (for counter runs)")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="after the timed steps, this many more steps each preceded by a 512 MiB device "
                         "write that evicts L2 and the MALL (reported under 'cold'; 0: none)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many MiB (a kernel of "
                         "known traffic, used to scale hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every (batch, head) is independent, so the path "
              "shards by heads with no exchange; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_score_amd as sa
    import workloads as W

    wl = W.WORKLOADS[args.workload]
    ratio = args.ratio if args.ratio is not None else wl.ratios[0]
    log(f"workload {wl.name}: B={wl.B} H={wl.H} N_v={wl.n_video} N_s={wl.n_sink} d={wl.d} "
        f"block={wl.block} ratio={ratio}")
    t = time.perf_counter()
    Qh, Kh, Vh = W.make_qkv(wl)
    log(f"inputs generated in {time.perf_counter() - t:.1f} s")
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    Q, K, V = (torch.from_numpy(x).to("cuda", dt) for x in (Qh, Kh, Vh))
    if args.no_cpu_baseline:
        Qh = Kh = Vh = None

    p = sa.params(Q, wl.n_sink, wl.block, ratio, sa.POOL_REWEIGHT, block_k=args.block_k)
    M, Mk = sa.num_blocks(p), sa.num_key_blocks(p)
    Kk = sa.topk_count(Mk, ratio)
    B, H, N, d = Q.shape
    f32 = dict(device="cuda", dtype=torch.float32)
    pooled = {"q_mean": torch.empty(B, H, M, d, **f32)}
    pooled.update({k: torch.empty(B, H, Mk, d, **f32) for k in ("k_mean", "k_sum", "v_sum")})
    pooled["bias"] = torch.empty(B, H, Mk, **f32)
    pooled["anchor"] = torch.empty(B, H, d, **f32)
    tau_mode = args.tau is not None
    fp8 = args.fp8
    if tau_mode and (wl.reblock or Mk != M):
        print("--tau runs on token-order workloads with equal query and key blocks", file=sys.stderr)
        sys.exit(2)
    if fp8 and (tau_mode or wl.key_partition):
        print("--fp8 runs with top-K routes on token-order or q_reuse_k layouts", file=sys.stderr)
        sys.exit(2)
    # adaptive tau: a variable route, row I of idx [B,H,M,M] holds counts[I] blocks
    idx = torch.empty(B, H, M, M if tau_mode else Kk, device="cuda", dtype=torch.int32)
    counts = torch.empty(B, H, M, device="cuda", dtype=torch.int32) if tau_mode else None
    O = torch.empty_like(Q)
    lse = torch.empty(B, H, N, **f32)
    sel_ws = torch.empty(sa.workspace_size(p, 5 if tau_mode else 3), device="cuda", dtype=torch.uint8)
    packed = torch.empty(sa.workspace_size(p, 9 if fp8 else 4), device="cuda", dtype=torch.uint8)
    amax = torch.empty(B, H, 3, **f32) if fp8 else None
    stream = torch.cuda.current_stream()
    perm = perm_k = None
    if wl.reblock:  # adaptive blocks: partition, gather, attend, scatter back
        perm = torch.empty(B, H, wl.n_video, device="cuda", dtype=torch.int32)
        # q_reuse_k: keys and values reuse the query partition; else keys get their own
        perm_k = torch.empty_like(perm) if wl.key_partition else perm
        rb_ws = torch.empty(sa.workspace_size(p, 1), device="cuda", dtype=torch.uint8)
        Qp, Kp, Vp = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    else:
        Qp, Kp, Vp = Q, K, V

    stage_names = ((["reblock"] + (["reblock_k"] if wl.key_partition else []) + ["gather"]) if wl.reblock else []) \
        + (["pool_scales", "select", "pack", "attend"] if fp8 else ["pool_pack", "select", "attend"])

    def step(ev=None):
        k = 1
        if wl.reblock:
            sa.spark_attn_reblock(p, Q, K, perm, rb_ws, stream)
            if ev: ev[k].record(stream)
            k += 1
            if wl.key_partition:  # keys bisected under the queries' second moment
                sa.spark_attn_reblock(p, K, Q, perm_k, rb_ws, stream)
                if ev: ev[k].record(stream)
                k += 1
            for X, Y, pm in ((Q, Qp, perm), (K, Kp, perm_k), (V, Vp, perm_k)):
                sa.spark_attn_gather_rows(p, X, pm, Y, stream)
            if ev: ev[k].record(stream)
            k += 1
        if fp8:  # pooling and the per-head E4M3 scales in one pass over Q, K, V
            sa.spark_attn_pool_fp8_scales(p, Qp, Kp, Vp, pooled["q_mean"], pooled["k_mean"], pooled["k_sum"],
                                          pooled["v_sum"], pooled["bias"], pooled["anchor"], amax, stream)
        else:  # pooling and packing in one pass over K and V
            sa.spark_attn_pool_pack(p, Qp, Kp, Vp, pooled["q_mean"], pooled["k_mean"], pooled["k_sum"],
                                    pooled["v_sum"], pooled["bias"], pooled["anchor"], packed, stream)
        if ev: ev[k].record(stream)
        k += 1
        if tau_mode:
            sa.spark_attn_select_tau(p, args.tau, pooled["q_mean"], pooled["k_mean"], idx, counts, None, sel_ws,
                                     stream)
        else:
            sa.spark_attn_select(p, pooled["q_mean"], pooled["k_mean"], idx, None, sel_ws, stream)
        if ev: ev[k].record(stream)
        k += 1
        if fp8:
            sa.spark_attn_pack_fp8(p, Kp, Vp, pooled["k_sum"], pooled["v_sum"], pooled["bias"], amax, packed, stream)
            if ev: ev[k].record(stream)
            k += 1
        if fp8:
            sa.spark_attn_attend_fp8(p, Qp, packed, idx, perm, amax, O, lse, stream)
        elif tau_mode:
            sa.spark_attn_attend_var(p, Qp, packed, idx, counts, perm, O, lse, stream)
        else:
            sa.spark_attn_attend(p, Qp, packed, idx, perm, O, lse, stream)
        if ev: ev[k].record(stream)

    log(f"M={M} K={Kk}; warmup {max(1, args.warmup)}")
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    # ---- the CPU leg, before anything is timed: route and sampled outputs of the warmup step
    # against the oracle, and the oracle's own time on that sample (the CPU baseline)
    run_cpu = not args.no_cpu_baseline and not tau_mode and not fp8
    if not args.no_cpu_baseline and (tau_mode or fp8):
        log("cpu baseline and route check: run for the bf16 top-K path only")
    gidx = idx.cpu().numpy()
    cpu_out, check = None, None
    O_ref, idx_ref = O.clone(), idx.clone()  # the timed steps must reproduce these bit for bit
    if run_cpu:
        qb, sq = cpu_sample(wl, M, args.cpu_sample_blocks)
        perm_h = perm.cpu().numpy() if wl.reblock else None
        perm_kh = perm_k.cpu().numpy() if wl.reblock else None
        # GPU rows of the sample: video rows of a permuted layout sit at perm[row] of the output
        g_rows, g_lse = [], []
        for ent, rows in zip(np.concatenate([qb, sq]), sample_rows(wl, M, np.concatenate([qb, sq]))):
            bh = int(ent[0])
            b_, h_ = divmod(bh, H)
            r = rows
            if wl.reblock and ent[1] < M:
                r = perm_h[b_, h_][rows]
            rt = torch.from_numpy(np.ascontiguousarray(r)).to("cuda", torch.int64)
            g_rows.append(O[b_, h_].index_select(0, rt).float().cpu().numpy())
            g_lse.append(lse[b_, h_].index_select(0, rt).cpu().numpy())
        if wl.reblock:  # the oracle runs on the partitioned layouts the route refers to
            for X, ph in ((Qh, perm_h), (Kh, perm_kh), (Vh, perm_kh)):
                for b_ in range(B):
                    for h_ in range(H):
                        X[b_, h_, :wl.n_video] = X[b_, h_][ph[b_, h_]]
        log("cpu leg (oracle): route check, sampled parity, CPU baseline ...")
        F_sel_w = algorithmic_flops(gidx, wl, Kk, None, args.block_k)[0]
        cpu_out, check = cpu_baseline(wl, ratio, Qh, Kh, Vh, gidx, F_sel_w, qb, sq,
                                      (np.concatenate(g_rows), np.concatenate(g_lse)), args.block_k)
        log(f"route rows violating the near-tie rule: {check['route_rows_violating_near_tie_rule']} of "
            f"{check['route_rows_checked']}; sampled parity rel-L2 {check['rel_l2']:.3e} max-abs "
            f"{check['max_abs']:.3e} lse {check['lse_max_abs']:.3e}")
        del Qh, Kh, Vh
        if not check["ok"]:
            print(json.dumps({"error": "route or sampled output outside the parity bounds; nothing timed",
                              "check": check}), flush=True)
            sys.exit(3)

    ns = len(stage_names)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        events[k][0].record(stream)
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    per_step = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(ns)] for e in events])
    stage_ms = {n: float(x) for n, x in zip(stage_names, per_step.mean(axis=0))}
    stage_spread = {"median": {n: round(float(x), 4) for n, x in zip(stage_names, np.median(per_step, axis=0))},
                    "min": {n: round(float(x), 4) for n, x in zip(stage_names, per_step.min(axis=0))}}
    ms_pool = stage_ms["pool_scales"] if fp8 else stage_ms["pool_pack"]
    ms_sel, ms_attn = stage_ms["select"], stage_ms["attend"]
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (" + ", ".join(f"{n} {v:.3f}" for n, v in stage_ms.items()) + ")")

    # cold caches: a 512 MiB write before each step evicts the 4 MB L2 of every XCD and the 256 MB
    # MALL, so the step starts with none of its inputs cached (the warm steps above keep whatever
    # the previous step left)
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, device="cuda", dtype=torch.uint8)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(args.cold_steps)]
        for k in range(args.cold_steps):
            flush.fill_(k & 0xFF)
            cev[k][0].record(stream)
            step(cev[k])
        torch.cuda.synchronize()
        cold_steps = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(ns)] for e in cev])
        cold = {"steps": args.cold_steps, "flush": "512 MiB device write before each step",
                "ms_per_step_median": round(float(np.median(cold_steps.sum(axis=1))), 4),
                "ms_per_step_min": round(float(cold_steps.sum(axis=1).min()), 4),
                "stages_ms_median": {n: round(float(x), 4)
                                     for n, x in zip(stage_names, np.median(cold_steps, axis=0))}}
        del flush
        log(f"cold caches, {args.cold_steps} steps: median {cold['ms_per_step_median']:.3f} ms/step")

    # cross-check: the single-call entry point over the same input
    ms_forward_call, same_out, ws, O2 = None, None, None, None
    if not args.no_forward_check:
        what = (8 if wl.reblock else 7) if fp8 else 6 if tau_mode else (2 if wl.reblock else 0)
        ws = torch.empty(sa.workspace_size(p, what), device="cuda", dtype=torch.uint8)
        O2 = torch.empty_like(Q)

        def fwd_call():
            if fp8:
                sa.spark_attn_forward_fp8(p, Q, K, V, perm, O2, None, None, None, ws, stream)
            elif tau_mode:
                sa.spark_attn_forward_tau(p, args.tau, Q, K, V, O2, None, None, None, ws, stream)
            else:
                sa.spark_attn_forward_kv(p, Q, K, V, perm, perm_k, O2, None, None, ws, stream)

        fwd_call()
        fe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fe[0].record(stream)
        for _ in range(3):
            fwd_call()
        fe[1].record(stream)
        torch.cuda.synchronize()
        ms_forward_call = round(fe[0].elapsed_time(fe[1]) / 3, 4)
        same_out = bool(torch.equal(O, O2))

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, device="cuda", dtype=torch.uint8)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the timed steps computed exactly what was checked
    timed_identical = bool(torch.equal(O, O_ref) and torch.equal(idx, idx_ref))
    del O_ref, idx_ref

    # pooling alone (no packing): what the pooling stage costs on its own, for its HBM roofline
    pool_only_ms = None
    if not fp8:
        pev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        sa.spark_attn_pool(p, Qp, Kp, Vp, pooled["q_mean"], pooled["k_mean"], pooled["k_sum"], pooled["v_sum"],
                           pooled["bias"], pooled["anchor"], stream)
        pev[0].record(stream)
        for _ in range(5):
            sa.spark_attn_pool(p, Qp, Kp, Vp, pooled["q_mean"], pooled["k_mean"], pooled["k_sum"],
                               pooled["v_sum"], pooled["bias"], pooled["anchor"], stream)
        pev[1].record(stream)
        torch.cuda.synchronize()
        pool_only_ms = pev[0].elapsed_time(pev[1]) / 5

    gcounts = counts.cpu().numpy() if tau_mode else None
    F_sel, F_sink, F_comp, F_sinkq = algorithmic_flops(gidx, wl, Kk, gcounts, args.block_k)
    F_attn = F_sel + F_sink + F_comp + F_sinkq
    value = F_sel / (ms_step * 1e-3) / 1e12
    achieved = F_attn / (ms_attn * 1e-3) / 1e12
    sel_flops = 2.0 * B * H * M * Mk * d
    # pooling's algorithmic bytes: Q, K, V video rows read once, the four fp32 summaries, the bias and
    # the anchor written
    esz = Q.element_size()
    pool_bytes = (3.0 * B * H * wl.n_video * d * esz + 4.0 * (B * H * M * d + 3 * B * H * Mk * d)
                  + 4.0 * B * H * Mk + 4.0 * B * H * d)
    stage_bytes = pool_bytes
    if fp8:  # the fused stage also reads the sink rows of Q, K, V for their maxima
        stage_bytes += 3.0 * B * H * wl.n_sink * d * esz
    else:  # the fused stage also reads the sink keys/values and writes every packed tile
        stage_bytes += 2.0 * B * H * wl.n_sink * d * esz + float(packed.numel())
    # select's compulsory bytes: the block means in, the route out (no score matrix: the score
    # product and the row selection run in one kernel)
    sel_bytes = 4.0 * B * H * (M + Mk) * d + 4.0 * float(idx.numel())

    peak = MFMA_FP8_PEAK_TFLOPS if fp8 else MFMA_BF16_PEAK_TFLOPS
    kernel = "attn_fwd_fp8" if fp8 else "attn_fwd"
    out = {
        "metric": ("selected-block TFLOP/s of the sparse-attention forward at 10% density"
                   + (", E4M3 carriers" if fp8 else "") if not tau_mode else
                   f"selected-block TFLOP/s of the sparse-attention forward with adaptive-tau selection (tau={args.tau})"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (bf16 in/out)" if fp8 else ("bf16" if wl.dtype == "bf16" else "f32"),
        "data": "synthetic (seeded positional-feature Q/K/V of the clip's shape; no model weights)",
        "config": {
            "workload": wl.name, "description": wl.description, "B": B, "H": H, "N_video": wl.n_video,
            "N_sink": wl.n_sink, "d": d, "block": wl.block, "M": M,
            **({"block_k": args.block_k, "M_k": Mk} if args.block_k not in (0, wl.block) else {}),
            **({"topk_ratio": ratio, "K": Kk} if not tau_mode else
               {"selection": "adaptive tau", "tau": args.tau, "kept_fraction": round(float(gcounts.mean()) / M, 4)}),
            "compressed_branch": "anchor-weighted summary + log-mass bias", "parallelism": "none (1 GPU)",
            "layout": ("separate key partition" if wl.key_partition else "q_reuse_k") if wl.reblock
            else "token order",
        },
        "stages_ms": dict({n: round(v, 4) for n, v in stage_ms.items()},
                          spark_attn_forward_call=ms_forward_call),
        "stages_ms_spread": stage_spread,
        "cold": cold,
        "forward_call_output_identical": same_out,
        "flops": {"F_sel": F_sel, "F_sink": F_sink, "F_comp": F_comp, "F_sinkq": F_sinkq},
        "roofline": {
            "kernel": f"{kernel}_kernel (exact + sink + compressed branches, sink queries)",
            "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            # the committed counters were taken on the workload's default route (top-K at its first
            # ratio, key blocks of `block` keys); any other route streams other tiles
            "traffic": (committed_traffic(wl.name, kernel)
                        if args.block_k == 0 and not tau_mode and ratio == wl.ratios[0] else None),
            "traffic_unit": "bytes per launch (FETCH+WRITE, scaled)",
            "exact_branch_frac": round((F_sel + F_sink) / (ms_attn * 1e-3) / 1e12 / peak, 4),
        },
        "pool_roofline": {
            "stage": "pool (pooling alone, spark_attn_pool: Q, K, V video rows read once, summaries written)",
            "bound": "hbm", "bytes": pool_bytes,
            "achieved": round(pool_bytes / (pool_only_ms * 1e-3) / 1e9, 1) if pool_only_ms else None,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(pool_bytes / (pool_only_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if pool_only_ms else None,
            "ms": round(pool_only_ms, 4) if pool_only_ms else None,
            "fused_stage": {
                "stage": "pool_scales (pooling + E4M3 amax, one pass over Q, K, V)" if fp8
                else "pool_pack (pooling + packed tiles, one pass over K, V)",
                "ms": round(ms_pool, 4), "bytes": stage_bytes,
                "frac_own_bytes": round(stage_bytes / (ms_pool * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "frac_pool_bytes": round(pool_bytes / (ms_pool * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        },
        # select = block-score product (2*M*M_k*d fp32-accurate flops per head, run as six bf16
        # part products on the matrix cores) + row top-K.  Its compulsory bytes (block means in,
        # route out) are small next to the product, so the roofline is the product's fp32 rate;
        # the score matrix the stage writes and reads back is reported beside it.
        "select_roofline": {"bound": "mfma", "achieved": round(sel_flops / (ms_sel * 1e-3) / 1e12, 2),
                            "peak": MFMA_FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(sel_flops / (ms_sel * 1e-3) / 1e12 / MFMA_FP32_PEAK_TFLOPS, 4),
                            "executed_bf16_TFLOPs": round(6 * sel_flops / (ms_sel * 1e-3) / 1e12, 2),
                            "bytes": sel_bytes,
                            "hbm_achieved_GBs": round(sel_bytes / (ms_sel * 1e-3) / 1e9, 1),
                            "hbm_frac": round(sel_bytes / (ms_sel * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "bytes_with_score_matrix": sel_bytes + 8.0 * B * H * M * Mk,
                            "hbm_frac_with_score_matrix": round((sel_bytes + 8.0 * B * H * M * Mk) / (ms_sel * 1e-3)
                                                                / 1e9 / HBM_PEAK_GBS, 4)},
        "check": check,
        "timed_output_identical_to_checked": timed_identical,
        "cpu_baseline": cpu_out,
    }
    print(json.dumps(out), flush=True)
    if not timed_identical:
        log("the timed steps did not reproduce the checked output bit for bit")
        sys.exit(4)


if __name__ == "__main__":
    main()
