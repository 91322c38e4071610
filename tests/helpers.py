"""Shared test plumbing: run the HIP path on a workload and get the oracle's answer.

The two sides meet only at the seeded input bytes from ``context_mla_prefill_amd.synth``.
"""
from __future__ import annotations

import numpy as np

from oracle import attention as oa
from oracle import numerics as on
from oracle import partition as op


def oracle_plan(w):
    return op.partition(w.q_lens, w.kv_lens, w.kv_start, w.P)


def token_maps(plan):
    """Global token -> (position, request), from the oracle's own partition."""
    pos = np.full(plan.T_glob, -1, dtype=np.int64)
    for rp in plan.ranks:
        pos[rp.local_gidx] = rp.positions
    req = np.searchsorted(plan.cu_seqlens_glob, np.arange(plan.T_glob), side="right") - 1
    return pos, req


def oracle_dense(w, plan, q_bits, lat_bits, rope_bits, sink, tokens):
    """fp64 (O0, LSE0, O, LSE) per token, dense causal."""
    pos, req = token_maps(plan)
    return oa.attention_tokens(
        tokens, q_of=lambda ts: on.bf16_to_f64(q_bits[ts]), pos_of=lambda ts: pos[ts],
        req_of=lambda ts: req[ts], kv_start=w.kv_start,
        lat_rows=lambda a, b: on.bf16_to_f64(lat_bits[a:b]),
        rope_rows=lambda a, b: on.bf16_to_f64(rope_bits[a:b]),
        scale=float(w.scale), sink=np.asarray(sink, dtype=np.float64))


def oracle_sparse(w, plan, q_bits, lat_codes, kv_scale, rope_bits, topk_rows, sink, tokens, rows_of=None):
    """fp64 (O0, LSE0, O, LSE) per token for the top-k + window key set over fp8 latent.

    ``rows_of(b, keys)`` gives the cache rows of request b's keys (default: the packed
    rows kv_start[b] + keys); latent codes and scales are read at those rows, rope at the
    packed rows of ``rope_bits``."""
    pos, req = token_maps(plan)
    out = {}
    for t in np.asarray(tokens, dtype=np.int64):
        b = int(req[t])
        p = int(pos[t])
        keys = oa.sparse_keyset(p, topk_rows[t], w.window)
        packed = int(w.kv_start[b]) + keys
        rows = packed if rows_of is None else rows_of(b, keys)
        lat = on.dequant_fp8_rows(lat_codes[rows], rows, kv_scale)
        rope = on.bf16_to_f64(rope_bits[packed])
        out[int(t)] = oa.attend_keyset(on.bf16_to_f64(q_bits[t]), lat, rope, float(w.scale),
                                       np.asarray(sink, dtype=np.float64))
    return out


def compare(name, got_o, got_lse, ref_o, ref_lse, o_tol, lse_tol):
    """Element-wise check plus relative diagnostics. Returns a dict of the errors."""
    got_o = np.asarray(got_o, dtype=np.float64)
    got_lse = np.asarray(got_lse, dtype=np.float64)
    e_o = float(np.max(np.abs(got_o - ref_o))) if got_o.size else 0.0
    e_l = float(np.max(np.abs(got_lse - ref_lse))) if got_lse.size else 0.0
    nrm = float(np.linalg.norm(ref_o))
    rel = float(np.linalg.norm(got_o - ref_o) / nrm) if nrm > 0 else 0.0
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_lse)), f"{name}: non-finite output"
    info = dict(max_abs_o=e_o, max_abs_lse=e_l, rel_o=rel)
    print(f"{name}: {info}", flush=True)
    assert e_o <= o_tol, f"{name}: max|O-O_ref| = {e_o} > {o_tol}"
    assert e_l <= lse_tol, f"{name}: max|LSE-LSE_ref| = {e_l} > {lse_tol}"
    assert rel <= 2e-2, f"{name}: relative O error {rel} > 2e-2"
    return info


def sample_tokens(w, plan, n_random=512, seed=None):
    """First and last token of every DualChunkSwap chunk (every virtual row of every rank;
    a decode row is a virtual row of one token), and n_random uniform tokens."""
    toks = set()
    for rp in plan.ranks:
        for v in range(rp.n_vrows):
            a, e = rp.cu_seqlens_q[v], rp.cu_seqlens_q[v + 1]
            if e > a:
                toks.add(int(rp.local_gidx[a]))
                toks.add(int(rp.local_gidx[e - 1]))
    rng = np.random.default_rng(w.cfg if seed is None else seed)
    if plan.T_glob:
        toks.update(int(x) for x in rng.integers(0, plan.T_glob, size=n_random))
    return np.array(sorted(toks), dtype=np.int64)


def mixed_split_counts(w, S, seed):
    """A per-row split plan for tests: key-range counts cycling through 1..S (shifted per rank,
    with a 0 and an S+3 among them, which the kernels clamp) and a random row order per rank.
    Returns int32 arrays [P][n_vrows] (counts, order)."""
    n_vrows = oracle_plan(w).ranks[0].n_vrows
    rng = np.random.default_rng(seed)
    splits = np.array([[(v + r) % S + 1 for v in range(n_vrows)] for r in range(w.P)], np.int32)
    splits[0, 0], splits[-1, -1] = 0, S + 3
    order = np.stack([rng.permutation(n_vrows) for _ in range(w.P)]).astype(np.int32)
    return splits, order
