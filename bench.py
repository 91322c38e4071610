#!/usr/bin/env python3
"""Benchmark of one PCP prefill step on one MI355X.

A step is the whole hot path on one batch: pcp_partition, pcp_kv_insert for every
virtual rank, mla_prefill_partial for every virtual rank (one after another, each at
its real shape), and pcp_lse_merge. Default workload: one 131072-token request, P = 4,
16 heads, latent 512 + rope 64 (bf16), per-head sink.

Prints ONE JSON line. ``value`` is the attention TFLOP/s of the whole step
(algorithmic flops of every token's key set, each token counted once even where its row
is replicated on every rank, / wall time of the step, inputs resident in HBM). ``roofline`` covers the dominant kernel (the partial attention), with its
average launch time from HIP events on the launch stream. ``cpu_baseline`` times the
fp64 oracle on a bounded sample of query rows of the same workload.

``--paged`` keeps the KV in a paged cache of 64-row blocks behind a seeded random block
table; with the fp8 top-k workload (``--workload 4``) the step then inserts the new rows
as bf16 and quantises them on insert, in one call for the all-gathered rows of every rank.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0


def attn_flops(positions: np.ndarray, H: int, Dl: int, Dr: int) -> float:
    """Algorithmic flops of causal MLA attention: 2*(Dqk + Dv) per (query, head, key)."""
    return float(2 * (Dl + Dr + Dl) * H) * float((positions.astype(np.int64) + 1).sum())


def sparse_set_sizes(topk_rows: np.ndarray, w) -> np.ndarray:
    """|key set| per global token: selected indices in [0, p] outside the window, plus the
    window keys [max(0, p-window+1), p]."""
    cu = np.zeros(w.n_req + 1, np.int64)
    cu[1:] = np.cumsum(w.q_lens)
    t = np.arange(w.T_glob)
    b = np.searchsorted(cu, t, side="right") - 1
    p = (w.kv_lens[b] - w.q_lens[b] + (t - cu[b])).astype(np.int64)
    lo = np.maximum(0, p - w.window + 1)
    out = np.empty(w.T_glob, np.int64)
    for a in range(0, w.T_glob, 8192):
        e = topk_rows[a:a + 8192].astype(np.int64)
        pp_, lo_ = p[a:a + 8192, None], lo[a:a + 8192, None]
        ok = (e >= 0) & (e <= pp_) & ((e < lo_) if w.window > 0 else True)
        out[a:a + 8192] = ok.sum(1) + (p[a:a + 8192] - lo[a:a + 8192] + 1 if w.window > 0 else 0)
    return out


def merge_bytes(merge_src: np.ndarray, H: int, Dv: int, kv_splits: int = 1, ranges=None) -> float:
    """Bytes the merge must move: each contributor row's LSE (fp32, every key split) and the O
    (bf16) of each split that holds keys -- all kv_splits, or ranges[row] of them under a
    per-row split plan -- read, each output row written, plus the map."""
    src = merge_src[merge_src >= 0]
    n_o = len(src) * kv_splits if ranges is None else int(ranges[src].sum())
    T, P = merge_src.shape
    return float(n_o * H * 2 * Dv + len(src) * kv_splits * H * 4 + T * H * (2 * Dv + 4) + T * P * 4)


def row_ranges(pl, splits: np.ndarray) -> np.ndarray:
    """Key ranges of every rank-concatenated partial row under a per-row split plan."""
    out = np.empty(pl.T_total, np.int64)
    for r in range(pl.P):
        cu = pl.cu_q[r].cpu().numpy()
        out[pl.rank_rows(r)] = np.repeat(splits[r], np.diff(cu))
    return out


# sources the benchmarked dense attention kernel (dense_wide_kernel) is compiled from; its
# traffic record names their hash
ATTN_SOURCES = ("attn_dense_wide.hip", "attn_core.h", "wide_tile.h", "work_order.h")


def measured_traffic(workload: int):
    """HBM bytes per launch of the attention and merge kernels from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by a plain copy kernel), or None when the kernel
    sources have changed since those counters were taken (or for other workloads)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "dense_attention_128k_p4_traffic.json")
    if workload != 3 or not os.path.exists(path):
        return None, None
    rec = json.load(open(path))

    def sha(*names):
        h = hashlib.sha256()
        for name in names:
            with open(os.path.join(ROOT, "context_mla_prefill_amd", "csrc", name), "rb") as f:
                h.update(f.read())
        return h.hexdigest()[:16]

    att = rec["bytes_per_launch"] if sha(*ATTN_SOURCES) == rec["kernel_source_sha256_prefix"] else None
    mer = rec["merge_bytes_per_launch"] if sha("merge.hip") == rec["merge_source_sha256_prefix"] else None
    return att, mer


def cpu_baseline(w, n_tokens: int, seconds: float):
    """Time the oracle on a bounded sample of query tokens (their full key sets)."""
    from oracle import attention as oa
    from oracle import numerics as on
    from oracle import partition as op
    from context_mla_prefill_amd import synth

    plan = op.partition(w.q_lens, w.kv_lens, w.kv_start, w.P)

    rng = np.random.default_rng(12345)
    pos_all = np.concatenate([rp.positions for rp in plan.ranks])
    gid_all = np.concatenate([rp.local_gidx for rp in plan.ranks])
    pos = np.full(plan.T_glob, -1, np.int64)
    pos[gid_all] = pos_all
    toks = np.sort(rng.choice(plan.T_glob, size=min(n_tokens, plan.T_glob), replace=False))
    n_keys = int(pos[toks].max()) + 1
    lat = on.bf16_to_f64(synth.latent_rows(w, 0, n_keys))
    rope = on.bf16_to_f64(synth.rope_rows(w, 0, n_keys))
    sink = synth.sink(w).astype(np.float64)
    done, flops, t0 = 0, 0.0, time.perf_counter()
    for t in toks:
        qt = on.bf16_to_f64(synth.q_rows(w, int(t), int(t) + 1))
        oa.dense_causal_block(qt, pos[[t]], lat, rope, float(w.scale), sink)
        done += 1
        flops += 2.0 * (w.Dl + w.Dr + w.Dl) * w.H * (pos[t] + 1)
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    cores = threads or len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} random query tokens of the workload (all {w.H} heads, full causal key sets, "
                      f"fp64), {dt:.1f} s"}


def box_reference(dev):
    """Rates this box delivers outside the library, for context (timed after the step): a bf16
    GEMM through torch.matmul (the BLAS library torch prefers on this device, recorded), 8192^3,
    and a 1 GiB device-to-device copy."""
    import torch
    n = 8192
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)

    def timed(fn, reps):
        for _ in range(3):
            fn()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return float(np.median(t))

    t_gemm = timed(lambda: torch.matmul(a, b, out=c), 20)
    del a, b, c
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    nbytes = src.numel() * 2
    del src, dst
    try:
        blas = str(torch.backends.cuda.preferred_blas_library()).split(".")[-1]
    except Exception:  # older torch: not exposed
        blas = "unknown"
    return {"gemm_bf16_tflops": round(2.0 * n ** 3 / (t_gemm * 1e-3) / 1e12, 1),
            "gemm": f"torch.matmul bf16 8192^3, preferred BLAS backend {blas}",
            "copy_GB/s": round(2.0 * nbytes / (t_copy * 1e-3) / 1e9, 1), "copy": "1 GiB device-to-device"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--heads", type=int, default=0, help="query heads per GPU (default: the workload's)")
    ap.add_argument("--kv-splits", type=int, default=1,
                    help="cut every row's keys into this many ranges (split-KV partials, merged with the ranks)")
    ap.add_argument("--split-plan", action="store_true",
                    help="with --kv-splits S: each virtual row gets its own range count (at most S) and the rows "
                         "their launch order from the library's host planner (pcp_plan_splits)")
    ap.add_argument("--paged", action="store_true",
                    help="keep the KV in a paged cache of 64-row blocks (seeded random block table); the fp8 "
                         "workload then quantises its new bf16 rows on insert, in one call for all ranks")
    ap.add_argument("--select", action="store_true",
                    help="top-k workload: the step also selects every rank's top-k indices on the GPU from "
                         "hashed index scores (sparse_topk_select), instead of taking them as an input")
    ap.add_argument("--in-kernel-dequant", action="store_true",
                    help="top-k workload: the sparse kernel dequantises the fp8 rows of every tile itself, instead "
                         "of reading a bf16 workspace that pcp_kv_dequant_fp8 fills once per step")
    ap.add_argument("--no-box-reference", action="store_true",
                    help="skip the on-box bf16 GEMM and device-copy reference rates")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device-to-device copy three times "
                         "(a kernel of known byte count for scaling HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the virtual PCP ranks run "
              "one after another on that GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    from context_mla_prefill_amd import _lib, synth
    from context_mla_prefill_amd import pipeline as pp

    _lib.load()
    w = synth.workload(args.workload)
    if args.heads:  # a per-GPU share of the heads (e.g. 16 of 64 under TP4)
        w = dataclasses.replace(w, H=args.heads)
    dev = "cuda"
    sparse = w.topk > 0

    def upload(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t_setup = time.perf_counter()
    q = upload(synth.q_rows(w))
    quantise = sparse and args.paged  # new rows arrive as bf16 and are quantised on insert
    if sparse and not quantise:
        lat_full = torch.from_numpy(synth.latent_rows(w)).to(dev)
        kv_scale = torch.from_numpy(synth.kv_scales(w)).to(dev)
    else:
        # the same N(0, std) draws as the fp8 codes of a sparse workload, kept in bf16
        lat_full = upload(synth.latent_rows(dataclasses.replace(w, kv_dtype="bf16")))
        kv_scale = None
    select = sparse and args.select
    if select:  # filled by the selection inside the step
        topk_host = None
        topk = torch.full((w.T_glob, w.topk), -1, dtype=torch.int32, device=dev)
    elif sparse:
        topk_host = synth.topk_rows(w)
        topk = torch.from_numpy(topk_host).to(dev)
    else:
        topk, topk_host = None, None
    rope_full = upload(synth.rope_rows(w))
    sink = torch.from_numpy(synth.sink(w)).to(dev)
    block_table = None
    if args.paged:
        rng = np.random.default_rng(2024)
        nb = (w.kv_lens.astype(np.int64) + 63) // 64
        perm = rng.permutation(int(nb.sum())).astype(np.int32)
        block_table = np.zeros((w.n_req, int(nb.max())), np.int32)
        for b, k0 in enumerate(np.concatenate([[0], np.cumsum(nb)[:-1]])):
            block_table[b, :nb[b]] = perm[k0:k0 + nb[b]]
    pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P, block_table=block_table)
    pp.run_partition(pl)
    ranks = [pp.rank_inputs(pl, r, q, lat_full, rope_full, topk) for r in range(w.P)]
    del q
    if select:  # per rank: fp32 index scores [T_loc][ld] of its rows, built on the device
        ld_s = (int(w.kv_lens.max()) + 3) // 4 * 4
        scores_r = [synth.index_scores_device(w, pl.local_gidx[pl.rank_rows(r)].long(), ld_s) for r in range(w.P)]
    if args.paged:
        # every key of every request in its block before the step (context rows stay, the step
        # re-inserts the new ones)
        n_cache = int(nb.sum()) * 64
        # every key's cache row and its packed source row, both from the library's slot map
        dst = pp.cache_rows(w.kv_lens, w.kv_lens, w.kv_start, block_table=block_table, device=dev)
        src = pp.cache_rows(w.kv_lens, w.kv_lens, w.kv_start, device=dev)
        kv_rope = torch.empty(n_cache, w.Dr, dtype=torch.bfloat16, device=dev)
        kv_rope[dst] = rope_full[src]
        if quantise:
            kv_lat = torch.empty(n_cache, w.Dl, dtype=torch.uint8, device=dev)
            kv_scale = torch.empty(n_cache // 64, dtype=torch.float32, device=dev)
            lat_src = lat_full[src].contiguous()
            _lib.pcp_kv_insert_fp8(lat_src, kv_rope[dst].contiguous(), dst.int(), w.N_kv, w.Dl, w.Dr, n_cache,
                                   kv_lat, kv_rope, kv_scale)
            del lat_src
        else:
            kv_lat = torch.empty(n_cache, w.Dl, dtype=torch.bfloat16, device=dev)
            kv_lat[dst] = lat_full[src]
        del dst, src
    else:
        kv_lat = lat_full.clone()  # context rows present before the step; new rows are re-inserted
        kv_rope = rope_full.clone()
    n_cache = int(kv_lat.shape[0])
    if quantise:  # one insert of the all-gathered new rows (rank order)
        lat_new = torch.cat([ri.latent for ri in ranks])
        rope_new = torch.cat([ri.rope for ri in ranks])
        for ri in ranks:
            ri.latent = ri.rope = None
    S = args.kv_splits
    bufs = pp.alloc_step(pl, w.H, w.Dl, kv_splits=S)
    sp = pp.plan_splits(pl, w.H, w.Dl, S) if args.split_plan and S > 1 else None
    plan_note = None
    if sp is not None and sp.split_rows == 0:  # the planner splits nothing: launch unsplit
        plan_note = f"per row (pcp_plan_splits, at most {S} ranges): no row split, launched unsplit"
        sp, S = None, 1
        bufs = pp.alloc_step(pl, w.H, w.Dl, kv_splits=1)
    kv_dtype = _lib.MLA_KV_FP8_E4M3 if sparse else _lib.MLA_KV_BF16
    use_ws = sparse and not args.in_kernel_dequant
    if use_ws:  # the fp8 cache's blocks dequantised once per step into a bf16 workspace
        ws = torch.empty(n_cache, w.Dl, dtype=torch.bfloat16, device=dev)
        ws_blocks = torch.arange((n_cache + 63) // 64, dtype=torch.int32, device=dev)
        args_r = [pp.partial_args(pl, r, ranks[r], ws, kv_rope, bufs, w.H, w.Dl, w.Dr, w.scale, topk=w.topk,
                                  window=w.window, kv_splits=S, split_plan=sp) for r in range(w.P)]
    else:
        args_r = [pp.partial_args(pl, r, ranks[r], kv_lat, kv_rope, bufs, w.H, w.Dl, w.Dr, w.scale, kv_dtype=kv_dtype,
                                  kv_scale=kv_scale, topk=w.topk, window=w.window, kv_splits=S, split_plan=sp)
                  for r in range(w.P)]
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    stream = torch.cuda.current_stream()
    n_ev = w.P + 4
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
              for _ in range(args.steps)]

    def step(ev=None):
        pp.run_partition(pl)
        if select:
            if ev:
                ev[w.P + 2][0].record(stream)
            for r in range(w.P):
                _lib.sparse_topk_select(scores_r[r], ld_s, pl.positions[pl.rank_rows(r)], pl.T_loc[r], w.topk,
                                        ranks[r].topk)
            if ev:
                ev[w.P + 2][1].record(stream)
        if ev:
            ev[w.P + 1][0].record(stream)
        if quantise:
            _lib.pcp_kv_insert_fp8(lat_new, rope_new, pl.slot, pl.T_total, w.Dl, w.Dr, n_cache, kv_lat, kv_rope,
                                   kv_scale)
        else:
            for r in range(w.P):
                _lib.pcp_kv_insert(ranks[r].latent, ranks[r].rope, pl.slot[pl.rank_rows(r)], pl.T_loc[r], w.Dl,
                                   w.Dr, kv_dtype, n_cache, kv_lat, kv_rope)
        if ev:
            ev[w.P + 1][1].record(stream)
        if use_ws:
            if ev:
                ev[w.P + 3][0].record(stream)
            _lib.pcp_kv_dequant_fp8(kv_lat, kv_scale, n_cache, w.Dl, ws_blocks, int(ws_blocks.numel()), ws)
            if ev:
                ev[w.P + 3][1].record(stream)
        for r in range(w.P):
            if ev:
                ev[r][0].record(stream)
            _lib.mla_prefill_partial(args_r[r])
            if ev:
                ev[r][1].record(stream)
        if ev:
            ev[w.P][0].record(stream)
        pp.run_merge(pl, bufs, sink, w.H, w.Dl, kv_splits=S)
        if ev:
            ev[w.P][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3

    # algorithmic work from the device plan's own positions
    pos_r = [pl.positions[pl.rank_rows(r)].cpu().numpy() for r in range(w.P)]
    if sparse:
        if select:  # the selected sets of the last step, gathered back to global token order
            topk_host = np.empty((w.T_glob, w.topk), np.int32)
            for r in range(w.P):
                topk_host[pl.local_gidx[pl.rank_rows(r)].cpu().numpy()] = ranks[r].topk.cpu().numpy()
        n_keys = sparse_set_sizes(topk_host, w)
        gidx_r = [pl.local_gidx[pl.rank_rows(r)].cpu().numpy() for r in range(w.P)]
        flops_r = [float(2 * (w.Dl + w.Dr + w.Dl) * w.H) * float(n_keys[g].sum()) for g in gidx_r]
        flops_step = float(2 * (w.Dl + w.Dr + w.Dl) * w.H) * float(n_keys.sum())
    else:
        flops_r = [attn_flops(p, w.H, w.Dl, w.Dr) for p in pos_r]
        pos_glob = np.empty(w.T_glob, np.int64)
        for r in range(w.P):
            pos_glob[pl.local_gidx[pl.rank_rows(r)].cpu().numpy()] = pos_r[r]
        flops_step = attn_flops(pos_glob, w.H, w.Dl, w.Dr)
    # flops_r: what each rank's launch computes (rows replicated on every rank -- decode rows
    # and short prefills -- count on each); flops_step: every global token once, the step's value
    flops_launch = float(sum(flops_r))
    t_rank_all = [[events[k][r][0].elapsed_time(events[k][r][1]) for k in range(args.steps)] for r in range(w.P)]
    t_rank = [float(np.mean(x)) for x in t_rank_all]
    t_merge = float(np.mean([events[k][w.P][0].elapsed_time(events[k][w.P][1]) for k in range(args.steps)]))
    t_insert = float(np.mean([events[k][w.P + 1][0].elapsed_time(events[k][w.P + 1][1]) for k in range(args.steps)]))
    avg_launch_ms = float(np.mean(t_rank))
    achieved = (flops_launch / w.P) / (avg_launch_ms * 1e-3) / 1e12
    mbytes = merge_bytes(pl.merge_src.cpu().numpy(), w.H, w.Dl, S,
                         None if sp is None else row_ranges(pl, sp.splits.cpu().numpy()))
    att_traffic, merge_traffic = measured_traffic(args.workload) if not args.paged else (None, None)

    out = {
        "metric": "PCP-shard MLA prefill attention TFLOP/s + MFMA% at 1 GPU; merge GB/s",
        "value": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 KV dequantised to bf16, bf16 MFMA" if sparse else "bf16",
        "data": "synthetic (seeded N(0,1)*0.5 bf16 q/latent/rope, N(0,1) sink)",
        "config": {"workload": w.name, "T": w.T_glob, "pcp": w.P, "heads": w.H, "d_latent": w.Dl,
                   "d_rope": w.Dr, "parallelism": f"{w.P} virtual PCP ranks, serial on 1 GPU",
                   **({"kv_splits": S} if S > 1 else {}),
                   **({"split_plan": f"per row (pcp_plan_splits): {sp.split_rows} of {w.P * pl.n_vrows} "
                                     "virtual rows split"} if sp is not None else {}),
                   **({"split_plan": plan_note} if plan_note else {}),
                   **({"kv_cache": "paged, 64-row blocks" + (", fp8 quantise-on-insert" if quantise else "")}
                      if args.paged else {})},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": att_traffic},
        "attention": {"rank_ms": [round(x, 3) for x in t_rank],
                      "rank_ms_min": [round(float(np.min(r_)), 3) for r_ in t_rank_all],
                      "rank_ms_p90": [round(float(np.percentile(r_, 90)), 3) for r_ in t_rank_all],
                      "rank_tflops": [round(f / (t * 1e-3) / 1e12, 2) for f, t in zip(flops_r, t_rank)],
                      "balance_last_over_first": round(t_rank[-1] / t_rank[0], 4),
                      "tokens_per_s": round(w.T_glob / (ms_step * 1e-3), 1)},
        "merge": {"ms": round(t_merge, 4), "GB/s": round(mbytes / (t_merge * 1e-3) / 1e9, 1),
                  "frac_hbm": round(mbytes / (t_merge * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bytes": mbytes,
                  "traffic": merge_traffic},
        "insert": {"ms": round(t_insert, 4),
                   "kind": "fp8 quantise-on-insert, one call" if quantise else f"byte copy, {w.P} calls"},
        "setup_s": round(setup_s, 1),
    }
    if sparse:
        # algorithmic gather: every key of a query's set once per workgroup of up to 64 heads, as the
        # method stores it: the fp8 latent row, the bf16 rope row and the row's fp32 scale. The
        # workspace path reads a bf16 latent row instead (its own bytes, reported beside).
        alg_key = w.Dl + 2 * w.Dr + 4
        path_key = 2 * w.Dl + 2 * w.Dr if use_ws else alg_key
        keys_r = [float(n_keys[g].sum()) * -(-w.H // 64) for g in gidx_r]
        gbs = float(np.mean([k * alg_key / (t * 1e-3) / 1e9 for k, t in zip(keys_r, t_rank)]))
        pbs = float(np.mean([k * path_key / (t * 1e-3) / 1e9 for k, t in zip(keys_r, t_rank)]))
        out["gather"] = {"bytes_per_key": alg_key, "bytes_per_rank": [round(k * alg_key) for k in keys_r],
                         "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                         "path_bytes_per_key": path_key, "path_GB/s": round(pbs, 1)}
    if use_ws:
        t_dq = float(np.mean([events[k][w.P + 3][0].elapsed_time(events[k][w.P + 3][1]) for k in range(args.steps)]))
        dq_bytes = float(n_cache) * (w.Dl + 2 * w.Dl) + (n_cache + 63) // 64 * 4
        out["dequant"] = {"ms": round(t_dq, 4), "GB/s": round(dq_bytes / (t_dq * 1e-3) / 1e9, 1),
                          "kind": "fp8 cache -> bf16 workspace, once per step"}
        out["config"]["sparse_kv_read"] = "bf16 workspace dequantised once per step"
    elif sparse:
        out["config"]["sparse_kv_read"] = "fp8 rows dequantised inside the sparse kernel"
    if select:
        t_sel = float(np.mean([events[k][w.P + 2][0].elapsed_time(events[k][w.P + 2][1]) for k in range(args.steps)]))
        n_scores = float(sum((pos_r[r].astype(np.int64) + 1).sum() for r in range(w.P)))
        sel_bytes = n_scores * 4 + w.T_glob * w.topk * 4  # every prefix score read once, indices written
        out["topk_select"] = {"ms": round(t_sel, 3), "GB/s": round(sel_bytes / (t_sel * 1e-3) / 1e9, 1),
                              "frac_hbm": round(sel_bytes / (t_sel * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                              "bytes": sel_bytes}
        out["config"]["topk_source"] = "selected on the GPU from hashed index scores"
    if not args.no_box_reference:
        ref = box_reference(dev)
        ref["attention_frac_of_gemm"] = round(achieved / ref["gemm_bf16_tflops"], 4)
        ref["merge_frac_of_copy"] = round(out["merge"]["GB/s"] / ref["copy_GB/s"], 4)
        out["box_reference"] = ref
    if args.calib_copy:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = {"read": src.numel() * 2, "write": dst.numel() * 2}
    if not args.no_cpu_baseline and not sparse:  # the oracle baseline is timed on the dense workload
        out["cpu_baseline"] = cpu_baseline(w, 2048, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
