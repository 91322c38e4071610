"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Integer maps (partition, positions, slots, merge map) and the KV insert are bit-exact;
partial and merged O / LSE meet max|O-O_ref| <= 1e-2 and max|LSE-LSE_ref| <= 1e-3
(3e-2 on O for the fp8 sparse workload), plus a relative-error sanity bound.
"""
import dataclasses

import numpy as np
import pytest
import torch

import helpers as hp
from context_mla_prefill_amd import _lib, synth
from context_mla_prefill_amd import pipeline as pp
from oracle import attention as oa
from oracle import merge as om
from oracle import numerics as on
from oracle import partition as op

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL = 1e-2, 1e-3


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def poison_partials(bufs):
    """NaN in every partial output and LSE before the kernels run."""
    bufs.o_cat.view(torch.int16).fill_(0x7FC0)
    bufs.lse_cat.fill_(float("nan"))


def check_plan(pl, plan):
    """Bit-exact comparison of the device plan with the oracle's partition."""
    torch.cuda.synchronize()
    assert pl.T_glob == plan.T_glob
    assert np.array_equal(pl.cu_glob.cpu().numpy(), plan.cu_seqlens_glob)
    for r, rp in enumerate(plan.ranks):
        rows = pl.rank_rows(r)
        assert pl.T_loc[r] == rp.T_loc and pl.row_off[r] == plan.row_off[r]
        assert np.array_equal(pl.local_gidx[rows].cpu().numpy(), rp.local_gidx)
        assert np.array_equal(pl.positions[rows].cpu().numpy(), rp.positions)
        assert np.array_equal(pl.slot[rows].cpu().numpy(), rp.slot)
        assert np.array_equal(pl.cu_q[r].cpu().numpy(), rp.cu_seqlens_q)
        assert np.array_equal(pl.vrow_req[r].cpu().numpy(), rp.vrow_req)
        assert np.array_equal(pl.vrow_kv_start[r].cpu().numpy(), rp.vrow_kv_start)
        assert np.array_equal(pl.vrow_kv_len[r].cpu().numpy(), rp.vrow_kv_len)
    assert np.array_equal(pl.merge_src.cpu().numpy(), plan.merge_src)


class DenseRun:
    """Runs partition -> insert -> P partials -> merge for a bf16 dense workload."""

    def __init__(self, w, kv_splits=1, split_plan=None):
        """split_plan: per-row split KV (pipeline.SplitPlan, max_splits == kv_splits); the
        partial buffers then start as NaN, so a slice the kernels leave unwritten and the merge
        read would poison the result."""
        self.w = w
        self.kv_splits = kv_splits
        self.split_plan = split_plan
        self.plan = hp.oracle_plan(w)
        print(f"[run] workload {w.cfg} {w.name} T={w.T_glob} N_kv={w.N_kv} kv_splits={kv_splits}", flush=True)
        self.q_bits = synth.q_rows(w)
        self.lat_bits = synth.latent_rows(w)
        self.rope_bits = synth.rope_rows(w)
        self.sink = synth.sink(w)
        q = dev_bf16(self.q_bits)
        lat_full, rope_full = dev_bf16(self.lat_bits), dev_bf16(self.rope_bits)
        self.pl = pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P)
        pp.run_partition(pl)
        # Full KV with every new-token row poisoned (NaN); the inserts must restore it.
        self.kv_lat, self.kv_rope = lat_full.clone(), rope_full.clone()
        new_rows = torch.unique(pl.slot.long())
        self.kv_lat.view(torch.int16)[new_rows] = 0x7FC0
        self.kv_rope.view(torch.int16)[new_rows] = 0x7FC0
        self.bufs = pp.alloc_step(pl, w.H, w.Dl, kv_splits=kv_splits)
        if split_plan is not None:
            poison_partials(self.bufs)
        self.sink_d = torch.from_numpy(self.sink).cuda()
        ranks = [pp.rank_inputs(pl, r, q, lat_full, rope_full) for r in range(w.P)]
        # every rank's rows reach the full KV (the all-gather) before any rank attends
        for r, ri in enumerate(ranks):
            _lib.pcp_kv_insert(ri.latent, ri.rope, pl.slot[pl.rank_rows(r)], pl.T_loc[r], w.Dl, w.Dr,
                               _lib.MLA_KV_BF16, w.N_kv, self.kv_lat, self.kv_rope)
        for r, ri in enumerate(ranks):
            args = pp.partial_args(pl, r, ri, self.kv_lat, self.kv_rope, self.bufs, w.H, w.Dl, w.Dr, w.scale,
                                   kv_splits=kv_splits, split_plan=split_plan)
            _lib.mla_prefill_partial(args)
        pp.run_merge(pl, self.bufs, self.sink_d, w.H, w.Dl, kv_splits=kv_splits)
        torch.cuda.synchronize()
        self.lat_full, self.rope_full = lat_full, rope_full

    def check_insert(self):
        assert torch.equal(self.kv_lat.view(torch.int16), self.lat_full.view(torch.int16))
        assert torch.equal(self.kv_rope.view(torch.int16), self.rope_full.view(torch.int16))

    def check_values(self, tokens):
        w, plan = self.w, self.plan
        ref = hp.oracle_dense(w, plan, self.q_bits, self.lat_bits, self.rope_bits, self.sink, tokens)
        o_cat = on.bf16_to_f64(host_bits(self.bufs.o_cat))
        lse_cat = self.bufs.lse_cat.cpu().numpy()
        tokset = set(int(t) for t in tokens)
        for r, rp in enumerate(plan.ranks):
            rows = [i for i, g in enumerate(rp.local_gidx) if int(g) in tokset]
            if not rows:
                continue
            gi = [int(rp.local_gidx[i]) for i in rows]
            cat = plan.row_off[r] + np.asarray(rows)
            hp.compare(f"workload {w.cfg} rank {r} partial", o_cat[cat], lse_cat[cat],
                       np.stack([ref[g][0] for g in gi]), np.stack([ref[g][1] for g in gi]), O_TOL, LSE_TOL)
        toks = np.asarray(sorted(tokset))
        o = on.bf16_to_f64(host_bits(self.bufs.o))[toks]
        lse = self.bufs.lse.cpu().numpy()[toks]
        hp.compare(f"workload {w.cfg} merged", o, lse, np.stack([ref[g][2] for g in toks]),
                   np.stack([ref[g][3] for g in toks]), O_TOL, LSE_TOL)
        return ref


@pytest.fixture(scope="module")
def tiny(gpu_lib):
    return DenseRun(synth.workload(1))


def test_tiny_plan(tiny):
    check_plan(tiny.pl, tiny.plan)


def test_tiny_insert(tiny):
    tiny.check_insert()


def test_tiny_values(tiny):
    tiny.check_values(np.arange(tiny.w.T_glob))


def test_tiny_sink_once_negative(tiny):
    """Partials with the sink already applied per rank, merged with the sink again,
    must miss the oracle: the test is sensitive to a doubled sink."""
    w = tiny.w
    o = tiny.bufs.o_cat.float()
    lse = tiny.bufs.lse_cat.clone()
    s = tiny.sink_d[None, :]
    o_bad = (o * torch.sigmoid(lse - s)[..., None]).to(torch.bfloat16)
    lse_bad = torch.logaddexp(lse, s)
    out = torch.empty_like(tiny.bufs.o)
    _lib.pcp_lse_merge(o_bad, lse_bad, tiny.pl.merge_src, w.P, w.T_glob, w.H, w.Dl, tiny.pl.T_total,
                       tiny.sink_d, out, None)
    torch.cuda.synchronize()
    ref = hp.oracle_dense(w, tiny.plan, tiny.q_bits, tiny.lat_bits, tiny.rope_bits, tiny.sink,
                          np.arange(w.T_glob))
    got = on.bf16_to_f64(host_bits(out))
    want = np.stack([ref[t][2] for t in range(w.T_glob)])
    assert np.max(np.abs(got - want)) > 3 * O_TOL


@pytest.fixture(scope="module")
def dense8k(gpu_lib):
    return DenseRun(synth.workload(2))


def test_dense8k_plan(dense8k):
    check_plan(dense8k.pl, dense8k.plan)


def test_dense8k_insert(dense8k):
    dense8k.check_insert()


def test_dense8k_values_full(dense8k):
    dense8k.check_values(np.arange(dense8k.w.T_glob))


EDGE = [
    # (seed, q_lens, kv_lens, P, H, Dl, Dr)
    (101, [1000], [1000], 3, 16, 512, 64),  # ragged chunks and tiles
    (102, [37, 3, 1, 1, 200, 9], [37, 3, 50, 7, 260, 9], 2, 16, 512, 64),  # short prefill, decodes, continuation
    (103, [77], [77], 1, 16, 512, 64),  # P = 1 is the identity
    (104, [130, 5, 1], [130, 5, 300], 4, 4, 64, 16),  # tiny dims, replicated rows
    (105, [64, 64], [64, 64], 2, 2, 64, 16),  # two requests, H = 2
    (106, [600, 1], [700, 900], 2, 64, 512, 64),  # H = 64
    (108, [300, 1], [300, 500], 2, 128, 512, 64),  # H = 128 (the largest)
    (109, [200, 50, 7], [200, 90, 7], 3, 3, 512, 64),  # H = 3: row tiles mix tokens of a virtual row
    (110, [1000, 16, 15], [1000, 16, 15], 8, 16, 512, 64),  # P = 8: 16 new tokens split, 15 replicated
    (111, [300, 128, 127, 1], [300, 128, 127, 40], 64, 4, 64, 16),  # P = 64, the largest: 1-token chunks
]


@pytest.mark.parametrize("case", EDGE, ids=[str(c[0]) for c in EDGE])
def test_edge_cases(gpu_lib, case):
    seed, q, kv, P, H, Dl, Dr = case
    w = synth.custom(seed, q, kv, P=P, H=H, Dl=Dl, Dr=Dr)
    run = DenseRun(w)
    check_plan(run.pl, run.plan)
    run.check_insert()
    run.check_values(np.arange(w.T_glob))


def test_empty_batch(gpu_lib):
    pl = pp.alloc_plan(np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32), 2)
    pp.run_partition(pl)
    torch.cuda.synchronize()
    assert pl.T_glob == 0 and pl.cu_glob.cpu().tolist() == [0]


def test_replicas_merged_once_negative(gpu_lib):
    """Merging every replica of a replicated row (instead of rank 0's only) must fail."""
    w = synth.custom(107, [3, 1, 16], [3, 40, 16], P=4, H=16, Dl=512, Dr=64)
    run = DenseRun(w)
    run.check_values(np.arange(w.T_glob))
    src = run.pl.merge_src.clone()
    plan = run.plan
    for r, rp in enumerate(plan.ranks):
        for i, g in enumerate(rp.local_gidx):
            if w.q_lens[int(np.searchsorted(plan.cu_seqlens_glob, g, side="right") - 1)] < 2 * w.P:
                src[int(g), r] = plan.row_off[r] + i
    out = torch.empty_like(run.bufs.o)
    _lib.pcp_lse_merge(run.bufs.o_cat, run.bufs.lse_cat, src, w.P, w.T_glob, w.H, w.Dl, run.pl.T_total,
                       run.sink_d, out, None)
    torch.cuda.synchronize()
    ref = hp.oracle_dense(w, plan, run.q_bits, run.lat_bits, run.rope_bits, run.sink, np.arange(w.T_glob))
    got = on.bf16_to_f64(host_bits(out))
    want = np.stack([ref[t][2] for t in range(w.T_glob)])
    assert np.max(np.abs(got - want)) > O_TOL


@pytest.mark.parametrize("T,P", [(64, 2), (96, 4), (45, 3)])
def test_merge_of_oracle_key_split_partials(gpu_lib, T, P):
    """The general <=P-contributor merge, fed with oracle-made partials of a DualChunkSwap
    key split (each rank attends only its own chunks' keys)."""
    rng = np.random.default_rng(T * 10 + P)
    H, Dl, Dr = 4, 64, 16
    q = rng.standard_normal((T, H, Dl + Dr)) * 0.5
    lat = rng.standard_normal((T, Dl)) * 0.5
    rope = rng.standard_normal((T, Dr)) * 0.5
    sink = rng.standard_normal(H).astype(np.float32)
    plan = op.partition([T], [T], [0], P)
    o_cat = np.zeros((T * P, H, Dl))
    lse_cat = np.full((T * P, H), -np.inf)
    src = np.full((T, P), -1, np.int32)
    for t in range(T):
        for r in range(P):
            keys = plan.ranks[r].positions
            keys = keys[keys <= t]
            if len(keys) == 0:
                continue
            o0, l0, _, _ = oa.attend_keyset(q[t], lat[keys], rope[keys], 0.3)
            o_cat[t * P + r], lse_cat[t * P + r] = o0, l0
            src[t, r] = t * P + r
    o_bits = synth.bf16_bits(o_cat.astype(np.float32))
    lse32 = lse_cat.astype(np.float32)
    o_out = torch.empty(T, H, Dl, dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty(T, H, dtype=torch.float32, device="cuda")
    _lib.pcp_lse_merge(dev_bf16(o_bits), torch.from_numpy(lse32).cuda(), torch.from_numpy(src).cuda(), P, T,
                       H, Dl, T * P, torch.from_numpy(sink).cuda(), o_out, lse_out)
    torch.cuda.synchronize()
    # oracle merge of the same stored partials
    want_o, want_l = om.merge(on.bf16_to_f64(o_bits), lse32.astype(np.float64), src, sink.astype(np.float64))
    got_o = on.bf16_to_f64(host_bits(o_out))
    np.testing.assert_allclose(got_o, want_o, atol=4e-3, rtol=1e-2)
    np.testing.assert_allclose(lse_out.cpu().numpy(), want_l, atol=1e-5, rtol=1e-6)
    # and it equals unsharded attention with the sink once
    for t in range(T):
        _, _, o, l = oa.attend_keyset(q[t], lat[:t + 1], rope[:t + 1], 0.3, sink.astype(np.float64))
        assert np.max(np.abs(got_o[t] - o)) < O_TOL and np.max(np.abs(lse_out[t].cpu().numpy() - l)) < LSE_TOL


MERGE_SHAPES = [
    # (D_v, H, P, kv_splits): head groups of a workgroup are 1024 / (D_v / 8) heads
    (1024, 16, 2, 1),  # 8 heads per group, two groups
    (136, 5, 4, 1),    # odd sizes: 60 heads per group, one partial group
    (8, 128, 3, 2),    # one group of 128 heads, split slices
    (512, 64, 2, 3),   # the sparse workload's heads with three split slices
]


@pytest.mark.parametrize("Dv,H,P,S", MERGE_SHAPES)
def test_merge_shapes(gpu_lib, Dv, H, P, S):
    """The merge over head groups and split slices against the oracle merge, with 0..P
    contributing ranks per token (none: O = 0, LSE = sink) and some empty partials."""
    rng = np.random.default_rng(Dv + 7 * H + 31 * P + S)
    T = 37
    stride = T * P  # rows from one split slice to the next
    R = S * stride
    o_bits = synth.bf16_bits((rng.standard_normal((R, H, Dv)) * 0.5).astype(np.float32))
    lse = (rng.standard_normal((R, H)) * 3).astype(np.float32)
    lse[rng.random((R, H)) < 0.05] = -np.inf  # a partial with no key
    src = np.full((T, P), -1, np.int32)
    for t in range(T):
        for r in rng.permutation(P)[:int(rng.integers(0, P + 1))]:
            src[t, r] = t * P + r
    sink = rng.standard_normal(H).astype(np.float32)
    o_out = torch.empty(T, H, Dv, dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty(T, H, dtype=torch.float32, device="cuda")
    _lib.pcp_lse_merge(dev_bf16(o_bits), torch.from_numpy(lse).cuda(), torch.from_numpy(src).cuda(), P, T, H, Dv, R,
                       torch.from_numpy(sink).cuda(), o_out, lse_out, kv_splits=S, split_stride=stride)
    torch.cuda.synchronize()
    # the contributors the API defines: every rank's row in each split slice
    src_x = np.full((T, P * S), -1, np.int64)
    for t in range(T):
        for k in range(P):
            if src[t, k] >= 0:
                for sl in range(S):
                    src_x[t, k * S + sl] = src[t, k] + sl * stride
    want_o, want_l = om.merge(on.bf16_to_f64(o_bits), lse.astype(np.float64), src_x, sink.astype(np.float64))
    np.testing.assert_allclose(on.bf16_to_f64(host_bits(o_out)), want_o, atol=4e-3, rtol=1e-2)
    np.testing.assert_allclose(lse_out.cpu().numpy(), want_l, atol=1e-5, rtol=1e-6)


def _sampled_run(cfg, n_random):
    w = synth.workload(cfg)
    run = DenseRun(w)
    check_plan(run.pl, run.plan)
    run.check_insert()
    toks = hp.sample_tokens(w, run.plan, n_random=n_random)
    print(f"[check] workload {cfg}: {len(toks)} sampled tokens", flush=True)
    run.check_values(toks)
    # every output row finite, on the GPU
    assert bool(torch.isfinite(run.bufs.o_cat.float()).all()) and bool(torch.isfinite(run.bufs.lse_cat).all())
    assert bool(torch.isfinite(run.bufs.o.float()).all()) and bool(torch.isfinite(run.bufs.lse).all())
    return run


def test_dense128k_p4_sampled(gpu_lib):
    """128K tokens, P=4: plan and insert in full, values on the first/last token of every
    chunk plus random tokens."""
    _sampled_run(3, n_random=512)


def test_mixed_varlen_decode_sampled(gpu_lib):
    """8 long prefills + 64 replicated decode rows, P=4: every decode row, the ends of
    every chunk, and random tokens."""
    _sampled_run(5, n_random=512)


def test_chunked_prefill_sampled(gpu_lib):
    """One chunked-prefill step of 32768 tokens, P=4: continuation chunks over 114688 and
    40960 cached keys, a fresh prefill, prefills at the replication threshold (8 = 2P new
    tokens split, 7 and 5 replicated) and 64 decode rows. Plan and insert in full; the ends
    of every virtual row and random tokens against the oracle."""
    run = _sampled_run(6, n_random=512)
    # the threshold: a request with q_len >= 2P is split into 2P chunks, a shorter one replicated
    for b, split in ((3, True), (4, False), (5, False)):
        n = sum(int(np.sum(rp.vrow_req == b)) for rp in run.plan.ranks)
        assert n == (2 * run.w.P if split else run.w.P), (b, n)


# ----------------------------------------------------------------------------- sparse fp8

SPARSE_O_TOL = 3e-2


class SparseRun:
    """partition -> fp8 insert -> P sparse partials -> merge for an fp8 top-k workload."""

    def __init__(self, w, lat_codes=None, kv_scale=None, topk_rows=None, kv_splits=1, workspace=False,
                 split_plan=None):
        """workspace: dequantise the cache once into a bf16 workspace (pcp_kv_dequant_fp8) and
        run the sparse partials on bf16 rows instead of dequantising inside the kernel.
        split_plan: per-row split KV, partial buffers poisoned first (as DenseRun)."""
        self.w = w
        self.kv_splits = kv_splits
        self.split_plan = split_plan
        self.workspace = workspace
        self.plan = hp.oracle_plan(w)
        print(f"[run] sparse workload {w.cfg} {w.name} T={w.T_glob} N_kv={w.N_kv}", flush=True)
        self.q_bits = synth.q_rows(w)
        self.lat_codes = synth.latent_rows(w) if lat_codes is None else lat_codes
        self.kv_scale = synth.kv_scales(w) if kv_scale is None else kv_scale
        self.rope_bits = synth.rope_rows(w)
        self.topk = synth.topk_rows(w) if topk_rows is None else topk_rows
        self.sink = synth.sink(w)
        q = dev_bf16(self.q_bits)
        lat_full = torch.from_numpy(np.ascontiguousarray(self.lat_codes)).cuda()
        rope_full = dev_bf16(self.rope_bits)
        topk_d = torch.from_numpy(np.ascontiguousarray(self.topk)).cuda()
        scale_d = torch.from_numpy(np.ascontiguousarray(self.kv_scale, dtype=np.float32)).cuda()
        self.pl = pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P)
        pp.run_partition(pl)
        # Full KV with every new-token row poisoned (NaN codes); the inserts must restore it.
        self.kv_lat, self.kv_rope = lat_full.clone(), rope_full.clone()
        new_rows = torch.unique(pl.slot.long())
        self.kv_lat[new_rows] = 0x7F
        self.kv_rope.view(torch.int16)[new_rows] = 0x7FC0
        self.bufs = pp.alloc_step(pl, w.H, w.Dl, kv_splits=kv_splits)
        if split_plan is not None:
            poison_partials(self.bufs)
        self.sink_d = torch.from_numpy(self.sink).cuda()
        ranks = [pp.rank_inputs(pl, r, q, lat_full, rope_full, topk_d) for r in range(w.P)]
        for r, ri in enumerate(ranks):
            _lib.pcp_kv_insert(ri.latent, ri.rope, pl.slot[pl.rank_rows(r)], pl.T_loc[r], w.Dl, w.Dr,
                               _lib.MLA_KV_FP8_E4M3, w.N_kv, self.kv_lat, self.kv_rope)
        if workspace:
            self.ws = torch.empty(w.N_kv, w.Dl, dtype=torch.bfloat16, device="cuda")
            n_blk = (w.N_kv + 63) // 64
            blocks = torch.arange(n_blk, dtype=torch.int32, device="cuda")
            _lib.pcp_kv_dequant_fp8(self.kv_lat, scale_d, w.N_kv, w.Dl, blocks, n_blk, self.ws)
        for r, ri in enumerate(ranks):
            if workspace:
                args = pp.partial_args(pl, r, ri, self.ws, self.kv_rope, self.bufs, w.H, w.Dl, w.Dr, w.scale,
                                       topk=w.topk, window=w.window, kv_splits=kv_splits, split_plan=split_plan)
            else:
                args = pp.partial_args(pl, r, ri, self.kv_lat, self.kv_rope, self.bufs, w.H, w.Dl, w.Dr, w.scale,
                                       kv_dtype=_lib.MLA_KV_FP8_E4M3, kv_scale=scale_d, topk=w.topk,
                                       window=w.window, kv_splits=kv_splits, split_plan=split_plan)
            _lib.mla_prefill_partial(args)
        pp.run_merge(pl, self.bufs, self.sink_d, w.H, w.Dl, kv_splits=kv_splits)
        torch.cuda.synchronize()
        self.lat_full, self.rope_full = lat_full, rope_full

    def check_insert(self):
        assert torch.equal(self.kv_lat, self.lat_full)
        assert torch.equal(self.kv_rope.view(torch.int16), self.rope_full.view(torch.int16))

    def check_values(self, tokens, o_tol=SPARSE_O_TOL):
        w, plan = self.w, self.plan
        ref = hp.oracle_sparse(w, plan, self.q_bits, self.lat_codes, self.kv_scale, self.rope_bits, self.topk,
                               self.sink, tokens)
        o_cat = on.bf16_to_f64(host_bits(self.bufs.o_cat))
        lse_cat = self.bufs.lse_cat.cpu().numpy()
        tokset = set(int(t) for t in tokens)
        for r, rp in enumerate(plan.ranks):
            rows = [i for i, g in enumerate(rp.local_gidx) if int(g) in tokset]
            if not rows:
                continue
            gi = [int(rp.local_gidx[i]) for i in rows]
            cat = plan.row_off[r] + np.asarray(rows)
            hp.compare(f"sparse workload {w.cfg} rank {r} partial", o_cat[cat], lse_cat[cat],
                       np.stack([ref[g][0] for g in gi]), np.stack([ref[g][1] for g in gi]), o_tol, LSE_TOL)
        toks = np.asarray(sorted(tokset))
        o = on.bf16_to_f64(host_bits(self.bufs.o))[toks]
        lse = self.bufs.lse.cpu().numpy()[toks]
        hp.compare(f"sparse workload {w.cfg} merged", o, lse, np.stack([ref[g][2] for g in toks]),
                   np.stack([ref[g][3] for g in toks]), o_tol, LSE_TOL)


@pytest.mark.parametrize("scale", [0.3713, 2.0 ** -5, 2.0 ** -117, 2.0 ** -118, 2.0 ** 6])
def test_fp8_dequant_bit_exact(gpu_lib, scale):
    """A query whose key set is one key returns that key's dequantised latent row exactly:
    every finite E4M3FN code times the block scale, rounded to bf16. Powers of two from 2^-117
    up take the kernel's scaled conversion (products exact and normal), the others (2^-118:
    subnormal products; 0.3713) its multiply."""
    w = synth.custom(201, [1], [1], P=1, H=64, Dl=512, Dr=64, topk=64, window=128, kv_dtype="fp8",
                     latent_std=1.0)
    codes = np.arange(512, dtype=np.int64) % 256
    codes[(codes & 0x7F) == 0x7F] = 0  # the two NaN codes
    lat = codes.astype(np.uint8)[None, :]
    scale = np.array([scale], np.float32)
    run = SparseRun(w, lat_codes=lat, kv_scale=scale, topk_rows=np.full((1, 64), -1, np.int32))
    got = on.bf16_to_f64(host_bits(run.bufs.o_cat)[0])  # [H, 512]
    want = on.dequant_fp8_rows(lat, np.array([0]), scale)[0]
    bad = np.nonzero(got != want[None, :])
    assert len(bad[0]) == 0, f"codes {codes[bad[1][:8]]}: got {got[bad][:8]} want {want[bad[1][:8]]}"
    # exact equality of values (the sign of a zero is not carried through P V: +0 + -0 = +0)


SCALE_KINDS = ("pow2_varied", "arbitrary", "mixed")


@pytest.mark.parametrize("kind", SCALE_KINDS)
def test_sparse_fp8_scale_kinds(gpu_lib, kind):
    """Block scales beyond the quantiser's: powers of two that vary by block (2^-3 .. 2^0
    times the drawn ones), arbitrary positive fp32 scales (0.3 .. 1 times them), and
    alternating blocks of both (tiles then mix rows of either kind); no larger than the drawn
    ones, so the values stay in the range the absolute bounds are set for. The in-kernel fp8
    path against the oracle on every row, and bit-identical to the bf16 workspace path."""
    w = synth.custom(231, [1200, 500], [1200, 800], P=2, H=64, Dl=512, Dr=64, topk=256, window=64,
                     kv_dtype="fp8", latent_std=1.0)
    rng = np.random.default_rng(231)
    base = synth.kv_scales(w)
    p2 = (base * np.exp2(rng.integers(-3, 1, base.shape))).astype(np.float32)
    arb = (base * rng.uniform(0.3, 1.0, base.shape)).astype(np.float32)
    scale = {"pow2_varied": p2, "arbitrary": arb,
             "mixed": np.where(np.arange(base.size) % 2 == 0, p2, arb).astype(np.float32)}[kind]
    run = SparseRun(w, kv_scale=scale)
    run.check_values(np.arange(w.T_glob))
    ws = SparseRun(w, kv_scale=scale, workspace=True)
    check_paths_identical(ws, run)


def test_sparse_small_all_rows(gpu_lib):
    """Selected keys + window on a small fp8 workload: every row of both ranks."""
    w = synth.custom(202, [1500, 700], [1500, 900], P=2, H=64, Dl=512, Dr=64, topk=256, window=64,
                     kv_dtype="fp8", latent_std=1.0)
    run = SparseRun(w)
    check_plan(run.pl, run.plan)
    run.check_insert()
    run.check_values(np.arange(w.T_glob))


def check_paths_identical(a, b, merged=False):
    """The bf16 workspace path and the in-kernel fp8 path on the same inputs give the same
    partials (or, split, the same merged outputs) bit for bit: the fp8 kernel dequantises each
    tile with the workspace's arithmetic and then runs the same tile compute."""
    if merged:
        assert torch.equal(a.bufs.o.view(torch.int16), b.bufs.o.view(torch.int16))
        assert torch.equal(a.bufs.lse.view(torch.int32), b.bufs.lse.view(torch.int32))
    else:
        assert torch.equal(a.bufs.o_cat.view(torch.int16), b.bufs.o_cat.view(torch.int16))
        assert torch.equal(a.bufs.lse_cat.view(torch.int32), b.bufs.lse_cat.view(torch.int32))


SPARSE_EDGE = {
    # seed: (q_lens, kv_lens, P, H, topk, window, shuffle the selected indices)
    211: ([900, 1, 300], [900, 700, 300], 2, 128, 128, 32, False),  # 2 head groups, a decode row
    212: ([1000], [1000], 2, 64, 192, 0, True),                      # top-k only, unsorted rows
    213: ([640, 5], [640, 5], 3, 64, 1, 96, False),                  # window only (one pad column), short prefill
    214: ([777], [1200], 2, 64, 64, 200, True),                      # continuation, wide window overlapping top-k
}


@pytest.mark.parametrize("seed", sorted(SPARSE_EDGE))
def test_sparse_edge_cases(gpu_lib, seed):
    """Sparse shapes beyond the two workloads: several head groups, decode and short-prefill
    rows, top-k only, window only, unsorted selected indices (the kernel may not depend on
    their order), kv_len > q_len; every row of every rank and the merge."""
    q, kv, P, H, topk, window, shuffle = SPARSE_EDGE[seed]
    w = synth.custom(seed, q, kv, P=P, H=H, Dl=512, Dr=64, topk=topk, window=window, kv_dtype="fp8",
                     latent_std=1.0)
    rows = synth.topk_rows(w)
    if topk == 1:
        rows[:] = -1  # window only
    if shuffle:
        rng = np.random.default_rng(seed)
        rows = np.stack([rng.permutation(r) for r in rows]).astype(np.int32)
    run = SparseRun(w, topk_rows=rows)
    check_plan(run.pl, run.plan)
    run.check_insert()
    run.check_values(np.arange(w.T_glob))
    # the same batch on the bf16 workspace
    ws = SparseRun(w, topk_rows=rows, workspace=True)
    ws.check_values(np.arange(w.T_glob))
    check_paths_identical(ws, run)


def split_ranges(L, S):
    """Key ranges of the split-KV call for a virtual row whose last position is L-1:
    n = ceil(L/64) tiles, range s = request-relative keys [64*floor(s*n/S), 64*floor((s+1)*n/S))."""
    n = -(-L // 64)
    return [(64 * (s * n // S), 64 * ((s + 1) * n // S)) for s in range(S)]


def row_split_counts(run, r):
    """Key ranges of each virtual row of rank r: the split plan's (clamped into 1..S), else S."""
    nv = run.plan.ranks[r].vrow_kv_len.shape[0]
    if getattr(run, "split_plan", None) is None:
        return np.full(nv, run.kv_splits)
    return np.clip(run.split_plan.splits[r].cpu().numpy(), 1, run.kv_splits)


def check_split_partials(run, tokens, key_rows, o_tol):
    """Every split slice of every rank's partial rows of the given tokens against the oracle
    restricted to that split's keys (no sink); a split with no key of the row must give
    O = 0 and LSE = -inf, and a slice past the row's own range count (per-row split plan)
    LSE = -inf. key_rows(t) -> (request-relative keys, latent fp64, rope fp64)."""
    w, plan, S = run.w, run.plan, run.kv_splits
    o_cat = on.bf16_to_f64(host_bits(run.bufs.o_cat))
    lse_cat = run.bufs.lse_cat.cpu().numpy()
    q = on.bf16_to_f64(run.q_bits)
    tokset = set(int(t) for t in tokens)
    for r, rp in enumerate(plan.ranks):
        vrow = np.searchsorted(rp.cu_seqlens_q, np.arange(rp.T_loc), side="right") - 1
        ns = row_split_counts(run, r)
        for i, g in enumerate(rp.local_gidx):
            g = int(g)
            if g not in tokset:
                continue
            keys, lat, rope = key_rows(g)
            n_v = int(ns[vrow[i]])
            for s in range(n_v, S):  # slices the row does not use: LSE -inf (O unspecified)
                assert np.all(np.isneginf(lse_cat[s * run.pl.T_total + plan.row_off[r] + i])), (g, s)
            for s, (lo, hi) in enumerate(split_ranges(int(rp.vrow_kv_len[vrow[i]]), n_v)):
                row = s * run.pl.T_total + plan.row_off[r] + i
                sel = (keys >= lo) & (keys < hi)
                if not sel.any():
                    assert np.all(o_cat[row] == 0) and np.all(np.isneginf(lse_cat[row])), (g, s)
                    continue
                o0, lse0, _, _ = oa.attend_keyset(q[g], lat[sel], rope[sel], float(w.scale))
                hp.compare(f"token {g} rank {r} split {s}", o_cat[row][None], lse_cat[row][None], o0[None],
                           lse0[None], o_tol, LSE_TOL)


def check_merged(run, ref, tokens, o_tol):
    toks = np.asarray(sorted(set(int(t) for t in tokens)))
    o = on.bf16_to_f64(host_bits(run.bufs.o))[toks]
    lse = run.bufs.lse.cpu().numpy()[toks]
    hp.compare(f"workload {run.w.cfg} merged over splits", o, lse, np.stack([ref[g][2] for g in toks]),
               np.stack([ref[g][3] for g in toks]), o_tol, LSE_TOL)


SPLIT_DENSE = {
    # seed: (q_lens, kv_lens, P, H, kv_splits)
    301: ([700, 1, 130], [700, 3000, 900], 2, 16, 3),  # prefill, a long decode row, a continuation
    302: ([2048], [2048], 4, 16, 2),
    303: ([64, 300, 1], [64, 300, 200], 1, 8, 5),       # more splits than some rows have tiles
}


@pytest.mark.parametrize("seed", sorted(SPLIT_DENSE))
def test_split_kv_dense(gpu_lib, seed):
    """Split-KV partials: each key range's partial matches the oracle on those keys, and the
    merge of all (rank, split) partials with the sink once reproduces unsharded attention."""
    q, kv, P, H, S = SPLIT_DENSE[seed]
    w = synth.custom(seed, q, kv, P=P, H=H, Dl=512, Dr=64)
    run = DenseRun(w, kv_splits=S)
    toks = np.arange(w.T_glob)
    ref = hp.oracle_dense(w, run.plan, run.q_bits, run.lat_bits, run.rope_bits, run.sink, toks)
    check_merged(run, ref, toks, O_TOL)
    pos, req = hp.token_maps(run.plan)
    lat_all, rope_all = on.bf16_to_f64(run.lat_bits), on.bf16_to_f64(run.rope_bits)

    def key_rows(g):
        keys = np.arange(int(pos[g]) + 1)
        rows = int(w.kv_start[req[g]]) + keys
        return keys, lat_all[rows], rope_all[rows]
    sample = hp.sample_tokens(w, run.plan, n_random=24)
    check_split_partials(run, sample, key_rows, O_TOL)


def custom_split_plan(w, S, seed):
    """helpers.mixed_split_counts on the device."""
    splits, order = hp.mixed_split_counts(w, S, seed)
    return pp.SplitPlan(S, torch.from_numpy(splits).cuda(), torch.from_numpy(order).cuda())


SPLIT_PER_ROW = {
    # seed: (q_lens, kv_lens, P, H, Dl, Dr, kv_splits)
    321: ([700, 1, 130, 1, 5], [700, 3000, 900, 5000, 40], 2, 16, 512, 64, 4),  # prefill, decodes, continuations
    322: ([300, 1, 9, 1], [300, 2000, 700, 100], 2, 4, 64, 16, 3),              # the 64+16 kernel
    323: ([2048, 1, 1], [2048, 4000, 20], 4, 16, 512, 64, 8),                    # more ranges than short rows have
}


@pytest.mark.parametrize("seed", sorted(SPLIT_PER_ROW))
def test_split_kv_dense_per_row(gpu_lib, seed):
    """Per-row split KV on the dense kernels: every virtual row its own range count (1..S, out of
    range counts clamped) in a random row order, partial buffers poisoned with NaN first. Every
    used slice against the oracle on its range's keys, every unused slice LSE = -inf, and the
    merge (which must not read the unused slices' outputs) against unsharded attention."""
    q, kv, P, H, Dl, Dr, S = SPLIT_PER_ROW[seed]
    w = synth.custom(seed, q, kv, P=P, H=H, Dl=Dl, Dr=Dr)
    run = DenseRun(w, kv_splits=S, split_plan=custom_split_plan(w, S, seed))
    check_plan(run.pl, run.plan)
    toks = np.arange(w.T_glob)
    ref = hp.oracle_dense(w, run.plan, run.q_bits, run.lat_bits, run.rope_bits, run.sink, toks)
    check_merged(run, ref, toks, O_TOL)
    pos, req = hp.token_maps(run.plan)
    lat_all, rope_all = on.bf16_to_f64(run.lat_bits), on.bf16_to_f64(run.rope_bits)

    def key_rows(g):
        keys = np.arange(int(pos[g]) + 1)
        rows = int(w.kv_start[req[g]]) + keys
        return keys, lat_all[rows], rope_all[rows]
    check_split_partials(run, hp.sample_tokens(w, run.plan, n_random=48), key_rows, O_TOL)


def test_split_plan_decode_heavy(gpu_lib):
    """The library's split plan (pcp_plan_splits) on a decode-heavy batch -- 24 decode rows over
    contexts of 2K-12K beside a short prefill, P=2 -- splits the decode rows; with NaN-poisoned
    partial buffers the merged output of every token matches unsharded attention."""
    rng = np.random.default_rng(331)
    ctx = rng.integers(2048, 12288, size=24)
    q = [256] + [1] * 24
    kv = [256] + [int(c) for c in ctx]
    w = synth.custom(331, q, kv, P=2, H=16, Dl=512, Dr=64)
    pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P)
    sp = pp.plan_splits(pl, w.H, w.Dl, max_splits=8)
    assert sp.split_rows >= 2 * 24  # every decode row on both ranks
    run = DenseRun(w, kv_splits=8, split_plan=sp)
    toks = np.arange(w.T_glob)
    ref = hp.oracle_dense(w, run.plan, run.q_bits, run.lat_bits, run.rope_bits, run.sink, toks)
    check_merged(run, ref, toks, O_TOL)


def test_split_plan_at_most_64_ranges(gpu_lib):
    """The largest split count (64 ranges, P = 1, the merge's limit P * kv_splits = 64): the
    planner's plan for four decode rows over 3K-100K keys, poisoned partial buffers, every
    token's merge against unsharded attention."""
    w = synth.custom(332, [1, 1, 1, 1], [100000, 70000, 50000, 3000], P=1, H=16, Dl=512, Dr=64)
    pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P)
    sp = pp.plan_splits(pl, w.H, w.Dl, max_splits=64)
    counts = sp.splits.cpu().numpy()
    print(f"[check] plan ranges {counts.tolist()}", flush=True)
    assert counts.max() > 8  # long rows cut into many ranges
    run = DenseRun(w, kv_splits=64, split_plan=sp)
    toks = np.arange(w.T_glob)
    ref = hp.oracle_dense(w, run.plan, run.q_bits, run.lat_bits, run.rope_bits, run.sink, toks)
    check_merged(run, ref, toks, O_TOL)


def test_dense128k_p4_split_kv_sampled(gpu_lib):
    """The 128K P=4 workload with each virtual row's keys cut into two ranges (the launch
    bench.py --kv-splits 2 times): on sampled tokens, the merge of all eight (rank, split)
    contributors against unsharded attention with the sink once, and for a subset both split
    partials against the oracle restricted to each range's keys; every partial row finite."""
    w = synth.workload(3)
    S = 2
    run = DenseRun(w, kv_splits=S)
    toks = np.asarray(sorted(set(int(t) for t in hp.sample_tokens(w, run.plan, n_random=512))))
    print(f"[check] split KV 128K: {len(toks)} sampled tokens", flush=True)
    ref = hp.oracle_dense(w, run.plan, run.q_bits, run.lat_bits, run.rope_bits, run.sink, toks)
    sel_d = torch.from_numpy(toks).cuda()
    hp.compare("128K merged over splits", on.bf16_to_f64(host_bits(run.bufs.o.index_select(0, sel_d))),
               run.bufs.lse.index_select(0, sel_d).cpu().numpy(), np.stack([ref[g][2] for g in toks]),
               np.stack([ref[g][3] for g in toks]), O_TOL, LSE_TOL)
    pos, req = hp.token_maps(run.plan)
    sub = set(int(t) for t in toks[::16])
    for r, rp in enumerate(run.plan.ranks):
        vrow = np.searchsorted(rp.cu_seqlens_q, np.arange(rp.T_loc), side="right") - 1
        for i in np.nonzero(np.isin(rp.local_gidx, list(sub)))[0]:
            g = int(rp.local_gidx[i])
            keys = np.arange(int(pos[g]) + 1)
            base = int(w.kv_start[req[g]])
            q = on.bf16_to_f64(run.q_bits[g])
            for s_, (lo, hi) in enumerate(split_ranges(int(rp.vrow_kv_len[vrow[i]]), S)):
                row = s_ * run.pl.T_total + run.plan.row_off[r] + int(i)
                o_row = on.bf16_to_f64(host_bits(run.bufs.o_cat[row]))
                lse_row = run.bufs.lse_cat[row].cpu().numpy()
                k = keys[(keys >= lo) & (keys < hi)]
                if len(k) == 0:
                    assert np.all(o_row == 0) and np.all(np.isneginf(lse_row)), (g, s_)
                    continue
                o0, lse0, _, _ = oa.attend_keyset(q, on.bf16_to_f64(run.lat_bits[base + k]),
                                                  on.bf16_to_f64(run.rope_bits[base + k]), float(w.scale))
                hp.compare(f"token {g} rank {r} split {s_}", o_row[None], lse_row[None], o0[None], lse0[None],
                           O_TOL, LSE_TOL)
    assert bool(torch.isfinite(run.bufs.o_cat.float()).all())


def test_dense128k_p4_per_row_split_sampled(gpu_lib):
    """The 128K P=4 workload under a per-row split plan (range counts 1..3 per virtual row,
    clamped, rows in a random order) with NaN-poisoned partial buffers: on sampled tokens the
    merge against unsharded attention, and for a subset every used slice against the oracle on
    its keys and every unused slice LSE = -inf."""
    w = synth.workload(3)
    S = 3
    run = DenseRun(w, kv_splits=S, split_plan=custom_split_plan(w, S, 333))
    toks = np.asarray(sorted(set(int(t) for t in hp.sample_tokens(w, run.plan, n_random=512))))
    print(f"[check] per-row split 128K: {len(toks)} sampled tokens", flush=True)
    ref = hp.oracle_dense(w, run.plan, run.q_bits, run.lat_bits, run.rope_bits, run.sink, toks)
    sel_d = torch.from_numpy(toks).cuda()
    hp.compare("128K merged over per-row splits", on.bf16_to_f64(host_bits(run.bufs.o.index_select(0, sel_d))),
               run.bufs.lse.index_select(0, sel_d).cpu().numpy(), np.stack([ref[g][2] for g in toks]),
               np.stack([ref[g][3] for g in toks]), O_TOL, LSE_TOL)
    pos, req = hp.token_maps(run.plan)
    sub = set(int(t) for t in toks[::16])
    for r, rp in enumerate(run.plan.ranks):
        ns = row_split_counts(run, r)
        vrow = np.searchsorted(rp.cu_seqlens_q, np.arange(rp.T_loc), side="right") - 1
        for i in np.nonzero(np.isin(rp.local_gidx, list(sub)))[0]:
            g = int(rp.local_gidx[i])
            keys = np.arange(int(pos[g]) + 1)
            base = int(w.kv_start[req[g]])
            q = on.bf16_to_f64(run.q_bits[g])
            n_v = int(ns[vrow[i]])
            for s_ in range(S):
                row = s_ * run.pl.T_total + run.plan.row_off[r] + int(i)
                lse_row = run.bufs.lse_cat[row].cpu().numpy()
                if s_ >= n_v:
                    assert np.all(np.isneginf(lse_row)), (g, s_)
                    continue
                lo, hi = split_ranges(int(rp.vrow_kv_len[vrow[i]]), n_v)[s_]
                o_row = on.bf16_to_f64(host_bits(run.bufs.o_cat[row]))
                k = keys[(keys >= lo) & (keys < hi)]
                if len(k) == 0:
                    assert np.all(o_row == 0) and np.all(np.isneginf(lse_row)), (g, s_)
                    continue
                o0, lse0, _, _ = oa.attend_keyset(q, on.bf16_to_f64(run.lat_bits[base + k]),
                                                  on.bf16_to_f64(run.rope_bits[base + k]), float(w.scale))
                hp.compare(f"token {g} rank {r} split {s_}", o_row[None], lse_row[None], o0[None], lse0[None],
                           O_TOL, LSE_TOL)


def test_split_kv_sparse(gpu_lib):
    """Split-KV on the sparse fp8 path: per-split partials and the merge over splits."""
    w = synth.custom(311, [900, 400], [900, 1300], P=2, H=64, Dl=512, Dr=64, topk=256, window=64,
                     kv_dtype="fp8", latent_std=1.0)
    run = SparseRun(w, kv_splits=3)
    toks = np.arange(w.T_glob)
    ref = hp.oracle_sparse(w, run.plan, run.q_bits, run.lat_codes, run.kv_scale, run.rope_bits, run.topk,
                           run.sink, toks)
    check_merged(run, ref, toks, SPARSE_O_TOL)
    pos, req = hp.token_maps(run.plan)

    def key_rows(g):
        keys = oa.sparse_keyset(int(pos[g]), run.topk[g], w.window)
        rows = int(w.kv_start[req[g]]) + keys
        return keys, on.dequant_fp8_rows(run.lat_codes[rows], rows, run.kv_scale), on.bf16_to_f64(run.rope_bits[rows])
    sample = hp.sample_tokens(w, run.plan, n_random=24)
    check_split_partials(run, sample, key_rows, SPARSE_O_TOL)


def test_split_kv_sparse_per_row(gpu_lib):
    """Per-row split KV on both sparse paths: row range counts 1..3 (clamped) with NaN-poisoned
    partials; used slices against the oracle on their keys, unused slices LSE = -inf, the
    merge against unsharded sparse attention, on both paths, which are bit-identical."""
    w = synth.custom(312, [900, 1, 400], [900, 2500, 1300], P=2, H=64, Dl=512, Dr=64, topk=256, window=64,
                     kv_dtype="fp8", latent_std=1.0)
    sp = custom_split_plan(w, 3, 312)
    run = SparseRun(w, kv_splits=3, split_plan=sp)
    ws = SparseRun(w, kv_splits=3, split_plan=sp, workspace=True)
    check_paths_identical(ws, run, merged=True)
    toks = np.arange(w.T_glob)
    ref = hp.oracle_sparse(w, run.plan, run.q_bits, run.lat_codes, run.kv_scale, run.rope_bits, run.topk,
                           run.sink, toks)
    pos, req = hp.token_maps(run.plan)

    def key_rows(g):
        keys = oa.sparse_keyset(int(pos[g]), run.topk[g], w.window)
        rows = int(w.kv_start[req[g]]) + keys
        return keys, on.dequant_fp8_rows(run.lat_codes[rows], rows, run.kv_scale), on.bf16_to_f64(run.rope_bits[rows])
    sample = hp.sample_tokens(w, run.plan, n_random=24)
    for r in (run, ws):
        check_merged(r, ref, toks, SPARSE_O_TOL)
        check_split_partials(r, sample, key_rows, SPARSE_O_TOL)


def test_dequant_workspace_bit_exact(gpu_lib):
    """pcp_kv_dequant_fp8 writes exactly the listed blocks, each row the oracle's
    bf16_rne(fp32(e4m3) * scale) of every code (a partial last block, ids outside the cache
    skipped, unlisted rows untouched)."""
    rng = np.random.default_rng(77)
    N, D = 64 * 5 + 17, 512
    codes = rng.integers(0, 256, size=(N, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0  # no NaN codes
    codes[0] = np.arange(512) % 256 & 0xFF
    codes[0][(codes[0] & 0x7F) == 0x7F] = 0
    scales = (rng.random(6) * 3 + 0.01).astype(np.float32)
    blocks = np.array([0, 2, 5, 99, -1, 2], np.int32)
    ws = torch.full((N, D), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    _lib.pcp_kv_dequant_fp8(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), N, D,
                            torch.from_numpy(blocks).cuda(), len(blocks), ws)
    torch.cuda.synchronize()
    got = host_bits(ws)
    for B in range(6):
        rows = np.arange(64 * B, min(64 * B + 64, N))
        if B in (0, 2, 5):
            want = on.dequant_fp8_rows(codes[rows], rows, scales)
            assert np.array_equal(on.bf16_to_f64(got[rows]), want), B
        else:
            assert np.all(got[rows] == 0x7FC0), B


SPARSE_WS = {
    # seed: (q_lens, kv_lens, P, H, topk, window, kv_splits)
    221: ([1500, 700], [1500, 900], 2, 64, 256, 64, 1),
    222: ([900, 1, 300], [900, 700, 300], 2, 128, 128, 32, 1),  # 2 head groups, a decode row
    223: ([777], [1200], 2, 64, 64, 200, 3),                      # continuation, wide window, split KV
}


@pytest.mark.parametrize("seed", sorted(SPARSE_WS))
def test_sparse_workspace_path(gpu_lib, seed):
    """The sparse path on a bf16 workspace dequantised once (pcp_kv_dequant_fp8) matches the
    oracle and gives the in-kernel dequantisation's partials (with split KV its merge) bit for
    bit."""
    q, kv, P, H, topk, window, S = SPARSE_WS[seed]
    w = synth.custom(seed, q, kv, P=P, H=H, Dl=512, Dr=64, topk=topk, window=window, kv_dtype="fp8",
                     latent_std=1.0)
    fp8 = SparseRun(w, kv_splits=S)
    ws = SparseRun(w, kv_splits=S, workspace=True)
    check_paths_identical(ws, fp8, merged=S > 1)
    if S == 1:
        ws.check_values(np.arange(w.T_glob))
    else:
        toks = np.arange(w.T_glob)
        ref = hp.oracle_sparse(w, ws.plan, ws.q_bits, ws.lat_codes, ws.kv_scale, ws.rope_bits, ws.topk, ws.sink,
                               toks)
        check_merged(ws, ref, toks, SPARSE_O_TOL)


def test_sparse_largest_window_and_topk(gpu_lib):
    """The largest key sets the API takes, top-k 2048 and a 4096-key window, on a prefill where
    early queries see the window cover their whole prefix (every selected index falls inside it
    and counts once) and late ones see 2048 selected keys before a full window: the fp8 kernel
    and the bf16 workspace path bit-identical, each on sampled tokens against the oracle, all finite."""
    w = synth.custom(221, [7000], [7000], P=2, H=64, Dl=512, Dr=64, topk=2048, window=4096, kv_dtype="fp8",
                     latent_std=1.0)
    fp8 = SparseRun(w)
    ws = SparseRun(w, workspace=True)
    check_paths_identical(ws, fp8)
    toks = hp.sample_tokens(w, fp8.plan, n_random=48)
    print(f"[check] largest key sets: {len(toks)} sampled tokens", flush=True)
    for r in (fp8, ws):
        r.check_values(toks)
        assert bool(torch.isfinite(r.bufs.o_cat.float()).all()) and bool(torch.isfinite(r.bufs.lse_cat).all())


def test_sparse128k_p2_sampled(gpu_lib):
    """128K tokens, P=2, 64 heads, top-2048 + window 128, fp8 KV: plan and insert in full,
    values on the ends of every chunk plus random tokens, all rows finite."""
    w = synth.workload(4)
    run = SparseRun(w)
    check_plan(run.pl, run.plan)
    run.check_insert()
    toks = hp.sample_tokens(w, run.plan)
    print(f"[check] sparse workload 4: {len(toks)} sampled tokens", flush=True)
    run.check_values(toks)
    assert bool(torch.isfinite(run.bufs.o_cat.float()).all()) and bool(torch.isfinite(run.bufs.lse_cat).all())


def test_sparse128k_p2_workspace_sampled(gpu_lib):
    """The 128K top-2048 workload on the bf16 workspace path (the one the benchmark times):
    sampled tokens against the oracle, all rows finite."""
    w = synth.workload(4)
    run = SparseRun(w, workspace=True)
    toks = hp.sample_tokens(w, run.plan)
    print(f"[check] sparse workload 4 on the workspace: {len(toks)} sampled tokens", flush=True)
    run.check_values(toks)
    assert bool(torch.isfinite(run.bufs.o_cat.float()).all()) and bool(torch.isfinite(run.bufs.lse_cat).all())


SPARSE_HEADS = {
    # seed: (q_lens, kv_lens, P, H, topk, window)
    231: ([1200, 1, 400], [1200, 900, 700], 2, 16, 256, 64),  # a per-GPU share under TP4 of 64 heads
    232: ([900, 300], [900, 500], 2, 32, 192, 128),           # TP2
    233: ([700], [700], 2, 80, 128, 64),                      # one full group and a partial one
}


@pytest.mark.parametrize("seed", sorted(SPARSE_HEADS))
def test_sparse_head_counts_under_64(gpu_lib, seed):
    """The sparse path at head counts that are not a multiple of 64 (per-GPU shares under
    tensor parallelism): the last head group's rows past H stay idle. Every row of every rank
    and the merge against the oracle, on both the in-kernel fp8 path and the bf16 workspace,
    which agree bit for bit."""
    q, kv, P, H, topk, window = SPARSE_HEADS[seed]
    w = synth.custom(seed, q, kv, P=P, H=H, Dl=512, Dr=64, topk=topk, window=window, kv_dtype="fp8",
                     latent_std=1.0)
    fp8 = SparseRun(w)
    ws = SparseRun(w, workspace=True)
    check_paths_identical(ws, fp8)
    fp8.check_values(np.arange(w.T_glob))
    ws.check_values(np.arange(w.T_glob))


def test_sparse128k_p2_h16_workspace_sampled(gpu_lib):
    """The 128K top-2048 workload at 16 heads (the per-GPU share of 64 heads under TP4) on the
    workspace path: sampled tokens against the oracle, every row finite."""
    w = dataclasses.replace(synth.workload(4), H=16)
    run = SparseRun(w, workspace=True)
    toks = hp.sample_tokens(w, run.plan)
    print(f"[check] sparse workload 4 at 16 heads: {len(toks)} sampled tokens", flush=True)
    run.check_values(toks)
    assert bool(torch.isfinite(run.bufs.o_cat.float()).all()) and bool(torch.isfinite(run.bufs.lse_cat).all())
