"""GPU parity of the paged latent-KV cache (block table of 64-row blocks) and of fp8
quantise-on-insert, against the oracle.

Slots, copied rows, fp8 codes and block scales are compared bit for bit; attention values
meet the same bounds as the packed path (max|O-O_ref| <= 1e-2, 3e-2 for fp8 latent;
max|LSE-LSE_ref| <= 1e-3). A paged dense run is also bit-identical to the packed run of
the same workload: paging changes addresses only.
"""
import dataclasses

import numpy as np
import pytest
import torch

import helpers as hp
from paged_tables import corrupt_table, make_block_table, rank_order, request_rows
import paged_tables as pt
from context_mla_prefill_amd import _lib, synth
from context_mla_prefill_amd import pipeline as pp
from oracle import kvcache as ok
from oracle import numerics as on

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL, SPARSE_O_TOL = 1e-2, 1e-3, 3e-2
NAN_BF16 = 0x7FC0


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def context_rows(w):
    """(request, position) of every key written before this step (kv_len > q_len)."""
    reqs, poss = [], []
    for b in range(w.n_req):
        ctx = int(w.kv_lens[b] - w.q_lens[b])
        reqs.append(np.full(ctx, b, np.int64))
        poss.append(np.arange(ctx, dtype=np.int64))
    return np.concatenate(reqs), np.concatenate(poss)


def check_paged_plan(pl, plan, bt):
    """Integer outputs bit-exact; slots are the oracle's positions through the block table."""
    torch.cuda.synchronize()
    pos, req = hp.token_maps(plan)
    assert pl.T_glob == plan.T_glob
    assert np.array_equal(pl.merge_src.cpu().numpy(), plan.merge_src)
    for r, rp in enumerate(plan.ranks):
        rows = pl.rank_rows(r)
        g = rp.local_gidx.astype(np.int64)
        assert np.array_equal(pl.local_gidx[rows].cpu().numpy(), rp.local_gidx)
        assert np.array_equal(pl.positions[rows].cpu().numpy(), rp.positions)
        assert np.array_equal(pl.cu_q[r].cpu().numpy(), rp.cu_seqlens_q)
        assert np.array_equal(pl.vrow_req[r].cpu().numpy(), rp.vrow_req)
        assert np.array_equal(pl.vrow_kv_start[r].cpu().numpy(), rp.vrow_kv_start)
        assert np.array_equal(pl.vrow_kv_len[r].cpu().numpy(), rp.vrow_kv_len)
        want = ok.paged_rows(bt, req[g], pos[g])
        assert np.array_equal(pl.slot[rows].cpu().numpy(), want)


class DenseCacheRun:
    """partition -> bf16 insert -> P dense partials -> merge, on a packed or a paged cache."""

    def __init__(self, w, seed=0, paged=True, kv_splits=1, table=None, split_plan=None):
        self.w, self.paged, self.kv_splits = w, paged, kv_splits
        self.plan = plan = hp.oracle_plan(w)
        print(f"[run] dense {'paged' if paged else 'packed'} {w.name} T={w.T_glob} kv_splits={kv_splits}",
              flush=True)
        self.q_bits, self.lat_bits, self.rope_bits = synth.q_rows(w), synth.latent_rows(w), synth.rope_rows(w)
        self.sink = synth.sink(w)
        q, lat_full, rope_full = dev_bf16(self.q_bits), dev_bf16(self.lat_bits), dev_bf16(self.rope_bits)
        if paged:
            self.bt, n_blocks = table if table is not None else make_block_table(w, seed)
            N = n_blocks * 64
        else:
            self.bt, N = None, w.N_kv
        self.pl = pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P, block_table=self.bt)
        pp.run_partition(pl)
        pos, req = hp.token_maps(plan)
        self.kv_lat = torch.full((N, w.Dl), NAN_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        self.kv_rope = torch.full((N, w.Dr), NAN_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        # keys written by earlier steps, placed where the cache layout puts them
        cr, cp = context_rows(w)
        self.key_rows = lambda b, p: ok.paged_rows(self.bt, b, p) if paged else w.kv_start[b] + p
        if len(cr):
            dst = torch.from_numpy(self.key_rows(cr, cp)).cuda()
            src = torch.from_numpy(w.kv_start[cr] + cp).cuda()
            self.kv_lat[dst] = lat_full[src]
            self.kv_rope[dst] = rope_full[src]
        self.bufs = pp.alloc_step(pl, w.H, w.Dl, kv_splits=kv_splits)
        self.sink_d = torch.from_numpy(self.sink).cuda()
        ranks = []
        for r, rp in enumerate(plan.ranks):
            g = torch.from_numpy(rp.local_gidx.astype(np.int64)).cuda()
            src = torch.from_numpy((w.kv_start[req] + pos)[rp.local_gidx.astype(np.int64)]).cuda()
            ranks.append(pp.RankInputs(q=q.index_select(0, g).contiguous(), topk=None,
                                       latent=lat_full.index_select(0, src).contiguous(),
                                       rope=rope_full.index_select(0, src).contiguous()))
        for r, ri in enumerate(ranks):
            _lib.pcp_kv_insert(ri.latent, ri.rope, pl.slot[pl.rank_rows(r)], pl.T_loc[r], w.Dl, w.Dr,
                               _lib.MLA_KV_BF16, N, self.kv_lat, self.kv_rope)
        for r, ri in enumerate(ranks):
            args = pp.partial_args(pl, r, ri, self.kv_lat, self.kv_rope, self.bufs, w.H, w.Dl, w.Dr, w.scale,
                                   kv_splits=kv_splits, split_plan=split_plan)
            _lib.mla_prefill_partial(args)
        pp.run_merge(pl, self.bufs, self.sink_d, w.H, w.Dl, kv_splits=kv_splits)
        torch.cuda.synchronize()

    def check_cache(self):
        """Every key of every request sits bit-exact at its row."""
        w = self.w
        reqs = np.concatenate([np.full(int(k), b, np.int64) for b, k in enumerate(w.kv_lens)])
        poss = np.concatenate([np.arange(int(k), dtype=np.int64) for k in w.kv_lens])
        rows = self.key_rows(reqs, poss)
        got_l = host_bits(self.kv_lat)[rows]
        got_r = host_bits(self.kv_rope)[rows]
        assert np.array_equal(got_l, self.lat_bits[w.kv_start[reqs] + poss])
        assert np.array_equal(got_r, self.rope_bits[w.kv_start[reqs] + poss])

    def check_values(self):
        w, plan = self.w, self.plan
        toks = np.arange(w.T_glob)
        ref = hp.oracle_dense(w, plan, self.q_bits, self.lat_bits, self.rope_bits, self.sink, toks)
        if self.kv_splits == 1:
            o_cat = on.bf16_to_f64(host_bits(self.bufs.o_cat))
            lse_cat = self.bufs.lse_cat.cpu().numpy()
            for r, rp in enumerate(plan.ranks):
                cat = plan.row_off[r] + np.arange(rp.T_loc)
                gi = rp.local_gidx.astype(np.int64)
                hp.compare(f"paged dense rank {r} partial", o_cat[cat], lse_cat[cat],
                           np.stack([ref[g][0] for g in gi]), np.stack([ref[g][1] for g in gi]), O_TOL, LSE_TOL)
        o = on.bf16_to_f64(host_bits(self.bufs.o))
        hp.compare("paged dense merged", o, self.bufs.lse.cpu().numpy(), np.stack([ref[g][2] for g in toks]),
                   np.stack([ref[g][3] for g in toks]), O_TOL, LSE_TOL)


PAGED_DENSE = {
    # seed: (q_lens, kv_lens, P, H, Dl, Dr, kv_splits)
    401: ([700, 1, 130, 64], [700, 3000, 900, 64], 2, 16, 512, 64, 1),  # prefill, long decode, continuations
    402: ([300, 5, 1], [300, 77, 200], 3, 4, 64, 16, 1),                # small dims, ragged blocks
    403: ([1500, 1, 200], [1500, 2100, 333], 2, 16, 512, 64, 3),        # paged + split KV
}


@pytest.mark.parametrize("seed", sorted(PAGED_DENSE))
def test_paged_dense(gpu_lib, seed):
    """Paged bf16 cache: plan slots through the block table, the cache after the inserts,
    every token against the oracle, and bit-identical partials to the packed run."""
    q, kv, P, H, Dl, Dr, S = PAGED_DENSE[seed]
    w = synth.custom(seed, q, kv, P=P, H=H, Dl=Dl, Dr=Dr)
    run = DenseCacheRun(w, seed=seed, paged=True, kv_splits=S)
    check_paged_plan(run.pl, run.plan, run.bt)
    run.check_cache()
    run.check_values()
    packed = DenseCacheRun(w, paged=False, kv_splits=S)
    assert torch.equal(run.bufs.o_cat.view(torch.int16), packed.bufs.o_cat.view(torch.int16))
    assert torch.equal(run.bufs.lse_cat.view(torch.int32), packed.bufs.lse_cat.view(torch.int32))


def test_paged_dense_per_row_split(gpu_lib):
    """Paged cache with per-row split KV (row range counts 1..4, clamped, in a random row order):
    the merge of every token against the oracle, and every partial slice bit-identical to the
    packed run with the same plan (the unused slices' LSE = -inf on both)."""
    w = synth.custom(404, [1500, 1, 200, 1], [1500, 2100, 333, 4100], P=2, H=16, Dl=512, Dr=64)
    splits, order = hp.mixed_split_counts(w, 4, 404)
    sp = pp.SplitPlan(4, torch.from_numpy(splits).cuda(), torch.from_numpy(order).cuda())
    run = DenseCacheRun(w, seed=404, paged=True, kv_splits=4, split_plan=sp)
    run.check_values()
    packed = DenseCacheRun(w, paged=False, kv_splits=4, split_plan=sp)
    lse_p, lse_k = run.bufs.lse_cat.cpu().numpy(), packed.bufs.lse_cat.cpu().numpy()
    assert np.array_equal(lse_p.view(np.int32), lse_k.view(np.int32))
    used = torch.from_numpy(np.isfinite(lse_p).all(axis=1)).cuda()  # slices a row's ranges wrote
    assert torch.equal(run.bufs.o_cat[used].view(torch.int16), packed.bufs.o_cat[used].view(torch.int16))
    assert np.isneginf(lse_p).any()  # some rows leave slices unused


# ------------------------------------------------------------------ fp8 quantise-on-insert


@pytest.mark.parametrize("cfg", [3, 5, 6])
def test_dense_full_size_paged_sampled(gpu_lib, cfg):
    """The full-size dense workloads on a paged cache (a random table of 64-row blocks, the cache
    layout bench.py --paged times): 128K tokens at P=4, the mixed 8-prefill + 64-decode batch,
    and the chunked-prefill step whose cached context sits in its blocks before the step. Every
    rank's partials bit-identical to the packed run of the same inputs (itself checked against
    the oracle), sampled merged rows against the oracle, every row finite."""
    w = synth.workload(cfg)
    paged = DenseCacheRun(w, seed=2024, paged=True)
    packed = DenseCacheRun(w, paged=False)
    assert torch.equal(paged.bufs.o_cat.view(torch.int16), packed.bufs.o_cat.view(torch.int16))
    assert torch.equal(paged.bufs.lse_cat.view(torch.int32), packed.bufs.lse_cat.view(torch.int32))
    del packed
    toks = hp.sample_tokens(w, paged.plan)
    print(f"[check] paged workload {cfg}: {len(toks)} sampled tokens", flush=True)
    ref = hp.oracle_dense(w, paged.plan, paged.q_bits, paged.lat_bits, paged.rope_bits, paged.sink, toks)
    o = on.bf16_to_f64(host_bits(paged.bufs.o))[toks]
    hp.compare(f"paged workload {cfg} merged", o, paged.bufs.lse.cpu().numpy()[toks], np.stack([ref[g][2] for g in toks]),
               np.stack([ref[g][3] for g in toks]), O_TOL, LSE_TOL)
    assert bool(torch.isfinite(paged.bufs.o.float()).all()) and bool(torch.isfinite(paged.bufs.lse).all())

def test_fp8_insert_scale_edges(gpu_lib):
    """The power-of-two block scale at its edges, codes and scales bit for bit against the
    oracle: amax / 448 exactly a power of two (2^-3, and 2^-117), one bf16 ulp above one
    (the next power), below 2^-126 (the floor 2^-126), an all-zero block (1) and amax 2^100
    (2^92). The other elements of a block are 0 or normal bf16 values below its maximum."""
    Dl, Dr, N = 64, 16, 64 * 6
    rng = np.random.default_rng(64016)
    top = [56.0, 56.25, 2.0 ** -125, 0.0, 2.0 ** 100, 448.0 * 2.0 ** -117]  # block maxima
    x = np.zeros((N, Dl), np.float32)
    for b, a in enumerate(top):
        if a == 0.0:
            continue
        if a < 2.0 ** -120:  # only 0 and normal values in the tiny block
            blk = rng.choice([0.0, 2.0 ** -126, 1.5 * 2.0 ** -126], size=(64, Dl))
        else:
            blk = rng.uniform(-1, 1, (64, Dl)) * a
            blk[np.abs(blk) < 2.0 ** -120] = 0.0  # no subnormal inputs
        blk[rng.integers(64), rng.integers(Dl)] = -a
        x[64 * b:64 * b + 64] = blk
    lat_bits = synth.bf16_bits(x)
    assert np.max(np.abs(on.bf16_to_f64(lat_bits[64:128]))) == 56.25  # the ulp above 56 survives bf16
    rope_bits = synth.bf16_bits(rng.standard_normal((N, Dr)).astype(np.float32))
    codes_d = torch.full((N, Dl), 0x7F, dtype=torch.uint8, device="cuda")
    scales_d = torch.full((N // 64,), float("nan"), dtype=torch.float32, device="cuda")
    rope_d = torch.zeros((N, Dr), dtype=torch.bfloat16, device="cuda")
    slot = np.arange(N, dtype=np.int32)
    _lib.pcp_kv_insert_fp8(dev_bf16(lat_bits), dev_bf16(rope_bits), torch.from_numpy(slot).cuda(), N, Dl, Dr, N,
                           codes_d, rope_d, scales_d)
    torch.cuda.synchronize()
    codes_o, scales_o = ok.quantize_insert_fp8(np.full((N, Dl), 0x7F, np.uint8), np.full(N // 64, np.nan, np.float32),
                                               lat_bits, slot)
    want = np.array([2.0 ** -3, 2.0 ** -2, 2.0 ** -126, 1.0, 2.0 ** 92, 2.0 ** -117], np.float32)
    assert np.array_equal(scales_o.view(np.uint32), want.view(np.uint32)), scales_o
    got = scales_d.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), got
    bad = np.argwhere(codes_d.cpu().numpy() != codes_o)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("dims", [(512, 64), (64, 16)])
def test_fp8_insert_bit_exact(gpu_lib, dims):
    """Two insert calls on one cache: fresh blocks, a block opened by the first call and
    continued by the second, rows into a block opened before both (stored scale, values
    that saturate), an all-zero block, and slots outside the cache. Codes, scales and rope
    rows match the oracle bit for bit after each call."""
    Dl, Dr = dims
    N = 64 * 8
    nblk = N // 64
    rng = np.random.default_rng(Dl)
    print(f"[run] fp8 insert dims {Dl}+{Dr}", flush=True)
    codes_o = np.full((N, Dl), 0x7F, np.uint8)
    scales_o = np.full(nblk, np.nan, np.float32)
    scales_o[2] = np.float32(0.01)  # block 2 was opened earlier
    rope_o = np.full((N, Dr), NAN_BF16, np.uint16)
    codes_d = torch.from_numpy(codes_o).cuda()
    scales_d = torch.from_numpy(scales_o).cuda()
    rope_d = torch.from_numpy(rope_o.view(np.int16)).cuda().view(torch.bfloat16)
    calls = [
        np.concatenate([rng.permutation(64), 64 + np.arange(10), 128 + np.arange(5, 21), [192, 255, -1, N],
                        320 + np.arange(64)]),
        np.concatenate([64 + np.arange(10, 64), 256 + rng.permutation(64)]),
    ]
    for ci, slot in enumerate(calls):
        T = len(slot)
        x = rng.standard_normal((T, Dl)).astype(np.float32) * np.exp(rng.normal(0, 2, (T, 1))).astype(np.float32)
        x[np.isin(slot, 320 + np.arange(64))] = 0.0  # block 5 all zero
        if ci == 0:
            x[np.isin(slot, 128 + np.arange(5, 21))] *= 10  # saturates against the stored 0.01
        lat_bits = synth.bf16_bits(x)
        rope_bits = synth.bf16_bits(rng.standard_normal((T, Dr)).astype(np.float32))
        slot32 = slot.astype(np.int32)
        _lib.pcp_kv_insert_fp8(dev_bf16(lat_bits), dev_bf16(rope_bits), torch.from_numpy(slot32).cuda(), T, Dl, Dr,
                               N, codes_d, rope_d, scales_d)
        torch.cuda.synchronize()
        codes_o, scales_o = ok.quantize_insert_fp8(codes_o, scales_o, lat_bits, slot)
        keep = (slot >= 0) & (slot < N)
        rope_o[slot[keep]] = rope_bits[keep]
        got_c = codes_d.cpu().numpy()
        bad = np.argwhere(got_c != codes_o)
        assert len(bad) == 0, f"call {ci}: {len(bad)} codes differ, first {bad[:4].tolist()}"
        assert np.array_equal(scales_d.cpu().numpy().view(np.uint32), scales_o.view(np.uint32)), \
            f"call {ci}: scales {scales_d.cpu().numpy()} vs {scales_o}"
        assert np.array_equal(host_bits(rope_d), rope_o)
    assert np.all(codes_o[320:384] == 0) and scales_o[5] == 1.0
    assert np.any(codes_o[133:149] & 0x7F == 0x7E)  # saturated codes present


class PagedSparseRun:
    """partition (paged) -> fp8 quantise-on-insert of context and new rows -> P sparse
    partials -> merge. The oracle quantises the same bf16 rows itself."""

    def __init__(self, w, seed, kv_splits=1, workspace=False, table=None):
        self.w, self.kv_splits = w, kv_splits
        self.plan = plan = hp.oracle_plan(w)
        print(f"[run] sparse paged {w.name} T={w.T_glob} kv_splits={kv_splits}", flush=True)
        # the library quantises bf16 rows on insert: a workload drawn as fp8 codes would hand
        # the insert one byte per element where it reads two
        assert w.kv_dtype == "bf16", "PagedSparseRun inserts bf16 latent rows"
        self.q_bits, self.lat_bits, self.rope_bits = synth.q_rows(w), synth.latent_rows(w), synth.rope_rows(w)
        self.topk = synth.topk_rows(w)
        self.sink = synth.sink(w)
        self.bt, n_blocks = table if table is not None else make_block_table(w, seed)
        N = n_blocks * 64
        q, lat_full, rope_full = dev_bf16(self.q_bits), dev_bf16(self.lat_bits), dev_bf16(self.rope_bits)
        topk_d = torch.from_numpy(self.topk).cuda()
        self.pl = pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P, block_table=self.bt)
        pp.run_partition(pl)
        pos, req = hp.token_maps(plan)
        self.codes_d = torch.full((N, w.Dl), 0x7F, dtype=torch.uint8, device="cuda")
        self.scales_d = torch.full((n_blocks,), float("nan"), dtype=torch.float32, device="cuda")
        self.rope_d = torch.full((N, w.Dr), NAN_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        self.codes_o = np.full((N, w.Dl), 0x7F, np.uint8)
        self.scales_o = np.full(n_blocks, np.nan, np.float32)
        # 1. the context keys, written by one earlier call
        cr, cp = context_rows(w)
        if len(cr):
            src = w.kv_start[cr] + cp
            slot = ok.paged_rows(self.bt, cr, cp)
            _lib.pcp_kv_insert_fp8(dev_bf16(self.lat_bits[src]), dev_bf16(self.rope_bits[src]),
                                   torch.from_numpy(slot.astype(np.int32)).cuda(), len(src), w.Dl, w.Dr, N,
                                   self.codes_d, self.rope_d, self.scales_d)
            self.codes_o, self.scales_o = ok.quantize_insert_fp8(self.codes_o, self.scales_o, self.lat_bits[src],
                                                                 slot)
        # 2. this step's rows of every rank in one call (the all-gathered latent KV)
        g = rank_order(plan)
        src = w.kv_start[req[g]] + pos[g]
        _lib.pcp_kv_insert_fp8(lat_full[torch.from_numpy(src).cuda()].contiguous(),
                               rope_full[torch.from_numpy(src).cuda()].contiguous(), pl.slot, pl.T_total, w.Dl,
                               w.Dr, N, self.codes_d, self.rope_d, self.scales_d)
        self.codes_o, self.scales_o = ok.quantize_insert_fp8(self.codes_o, self.scales_o, self.lat_bits[src],
                                                             ok.paged_rows(self.bt, req[g], pos[g]))
        self.bufs = pp.alloc_step(pl, w.H, w.Dl, kv_splits=kv_splits)
        self.sink_d = torch.from_numpy(self.sink).cuda()
        if workspace:  # the batch's blocks dequantised once into a bf16 workspace
            self.ws = torch.empty(N, w.Dl, dtype=torch.bfloat16, device="cuda")
            used = np.unique(self.bt[(self.bt >= 0) & (self.bt < n_blocks)]).astype(np.int32)
            _lib.pcp_kv_dequant_fp8(self.codes_d, self.scales_d, N, w.Dl, torch.from_numpy(used).cuda(), len(used),
                                    self.ws)
        for r, rp in enumerate(plan.ranks):
            gi = torch.from_numpy(rp.local_gidx.astype(np.int64)).cuda()
            ri = pp.RankInputs(q=q.index_select(0, gi).contiguous(), topk=topk_d.index_select(0, gi).contiguous(),
                               latent=None, rope=None)
            if workspace:
                args = pp.partial_args(pl, r, ri, self.ws, self.rope_d, self.bufs, w.H, w.Dl, w.Dr, w.scale,
                                       topk=w.topk, window=w.window, kv_splits=kv_splits)
            else:
                args = pp.partial_args(pl, r, ri, self.codes_d, self.rope_d, self.bufs, w.H, w.Dl, w.Dr, w.scale,
                                       kv_dtype=_lib.MLA_KV_FP8_E4M3, kv_scale=self.scales_d, topk=w.topk,
                                       window=w.window, kv_splits=kv_splits)
            _lib.mla_prefill_partial(args)
        pp.run_merge(pl, self.bufs, self.sink_d, w.H, w.Dl, kv_splits=kv_splits)
        torch.cuda.synchronize()

    def check_cache(self):
        assert np.array_equal(self.codes_d.cpu().numpy(), self.codes_o)
        assert np.array_equal(self.scales_d.cpu().numpy().view(np.uint32), self.scales_o.view(np.uint32))

    def check_values(self):
        w, plan = self.w, self.plan
        toks = np.arange(w.T_glob)
        ref = hp.oracle_sparse(w, plan, self.q_bits, self.codes_o, self.scales_o, self.rope_bits, self.topk,
                               self.sink, toks, rows_of=lambda b, keys: ok.paged_rows(self.bt, b, keys))
        if self.kv_splits == 1:
            o_cat = on.bf16_to_f64(host_bits(self.bufs.o_cat))
            lse_cat = self.bufs.lse_cat.cpu().numpy()
            for r, rp in enumerate(plan.ranks):
                cat = plan.row_off[r] + np.arange(rp.T_loc)
                gi = rp.local_gidx.astype(np.int64)
                hp.compare(f"paged sparse rank {r} partial", o_cat[cat], lse_cat[cat],
                           np.stack([ref[g][0] for g in gi]), np.stack([ref[g][1] for g in gi]), SPARSE_O_TOL,
                           LSE_TOL)
        o = on.bf16_to_f64(host_bits(self.bufs.o))
        hp.compare("paged sparse merged", o, self.bufs.lse.cpu().numpy(), np.stack([ref[g][2] for g in toks]),
                   np.stack([ref[g][3] for g in toks]), SPARSE_O_TOL, LSE_TOL)


PAGED_SPARSE = {
    # seed: (q_lens, kv_lens, P, topk, window, kv_splits)
    # fresh prefill; a decode row over 640 cached keys; a continuation of 512 cached keys;
    # a continuation whose first new rows land in a block the cached keys opened
    501: ([700, 1, 300, 200], [700, 641, 812, 300], 2, 128, 64, 1),
    502: ([900, 1], [1000, 1300], 2, 192, 32, 3),  # paged + split KV, unaligned continuation
}


@pytest.mark.parametrize("seed", sorted(PAGED_SPARSE))
def test_paged_sparse_quantize_on_insert(gpu_lib, seed):
    """fp8 sparse path on a paged cache that the library quantised itself: codes and block
    scales bit-exact against the oracle's quantiser, slots through the block table, and every
    token's partials and merged output against the oracle on the oracle's own codes."""
    q, kv, P, topk, window, S = PAGED_SPARSE[seed]
    w = synth.custom(seed, q, kv, P=P, H=64, Dl=512, Dr=64, topk=topk, window=window, latent_std=1.0)
    run = PagedSparseRun(w, seed, kv_splits=S)
    check_paged_plan(run.pl, run.plan, run.bt)
    run.check_cache()
    run.check_values()


@pytest.mark.parametrize("seed", sorted(PAGED_SPARSE))
def test_paged_sparse_workspace(gpu_lib, seed):
    """The same paged batches with the quantised blocks dequantised once into a bf16
    workspace: partials bit-identical to the in-kernel dequantisation, every token against the
    oracle."""
    q, kv, P, topk, window, S = PAGED_SPARSE[seed]
    w = synth.custom(seed, q, kv, P=P, H=64, Dl=512, Dr=64, topk=topk, window=window, latent_std=1.0)
    fp8 = PagedSparseRun(w, seed, kv_splits=S)
    ws = PagedSparseRun(w, seed, kv_splits=S, workspace=True)
    assert torch.equal(ws.bufs.o_cat.view(torch.int16), fp8.bufs.o_cat.view(torch.int16))
    assert torch.equal(ws.bufs.lse_cat.view(torch.int32), fp8.bufs.lse_cat.view(torch.int32))
    ws.check_values()


def test_sparse128k_p2_paged_quantised_sampled(gpu_lib):
    """The 128K top-2048 workload in the layout bench.py --workload 4 --paged times: bf16 rows
    quantised to fp8 on insert into a paged cache (a random table of 64-row blocks), dequantised
    once into the bf16 workspace, sparse partials on it. Codes and block scales bit-exact against
    the oracle's quantiser; sampled tokens (merged) against the oracle run on the oracle's own
    codes; every row finite. The oracle's quantiser over all 131,072 rows takes 1-2 minutes of
    host time."""
    w = dataclasses.replace(synth.workload(4), kv_dtype="bf16")  # the fp8 workload's draws, kept in bf16
    run = PagedSparseRun(w, 2024, workspace=True)
    run.check_cache()
    toks = hp.sample_tokens(w, run.plan)
    print(f"[check] paged quantised 128K sparse: {len(toks)} sampled tokens", flush=True)
    ref = hp.oracle_sparse(w, run.plan, run.q_bits, run.codes_o, run.scales_o, run.rope_bits, run.topk, run.sink,
                           toks, rows_of=lambda b, keys: ok.paged_rows(run.bt, b, keys))
    o = on.bf16_to_f64(host_bits(run.bufs.o))[toks]
    hp.compare("paged quantised 128K sparse merged", o, run.bufs.lse.cpu().numpy()[toks],
               np.stack([ref[g][2] for g in toks]), np.stack([ref[g][3] for g in toks]), SPARSE_O_TOL, LSE_TOL)
    assert bool(torch.isfinite(run.bufs.o.float()).all()) and bool(torch.isfinite(run.bufs.lse).all())


# ------------------------------------------------------------------ block ids outside the cache

def test_paged_block_ids_outside_the_cache(gpu_lib):
    """Block-table entries outside the cache give wrong values for the keys they map, never an
    access outside the cache: the dense kernel clamps block ids into the cache as it loads them,
    the sparse kernels clamp every key row into the cache before forming an offset, and the
    inserts skip slots outside the cache (every access of this test is modelled on the CPU in
    test_paged_access_model.py). Request 1's table holds such entries; request 0's
    partials equal those of the run with the valid table bit for bit, on the dense path and on
    the sparse path (bf16 workspace and fp8 in the kernel)."""
    wd = synth.custom(**pt.OUT_OF_CACHE_DENSE)
    bt, nb = make_block_table(wd, 404)
    rows = torch.from_numpy(request_rows(hp.oracle_plan(wd), 0, 600)).cuda()
    good = DenseCacheRun(wd, table=(bt, nb))
    bad = DenseCacheRun(wd, table=(corrupt_table(bt, nb, 1), nb))
    assert torch.equal(good.bufs.o_cat[rows].view(torch.int16), bad.bufs.o_cat[rows].view(torch.int16))
    assert torch.equal(good.bufs.lse_cat[rows].view(torch.int32), bad.bufs.lse_cat[rows].view(torch.int32))
    ws = synth.custom(**pt.OUT_OF_CACHE_SPARSE)
    bt, nb = make_block_table(ws, 504)
    rows = torch.from_numpy(request_rows(hp.oracle_plan(ws), 0, 700)).cuda()
    for workspace in (True, False):
        good = PagedSparseRun(ws, 504, workspace=workspace, table=(bt, nb))
        bad = PagedSparseRun(ws, 504, workspace=workspace, table=(corrupt_table(bt, nb, 1), nb))
        assert torch.equal(good.bufs.o_cat[rows].view(torch.int16), bad.bufs.o_cat[rows].view(torch.int16))
        assert torch.equal(good.bufs.lse_cat[rows].view(torch.int32), bad.bufs.lse_cat[rows].view(torch.int32))


def test_cache_rows_from_the_slot_map(gpu_lib):
    """The set-up helper that places every key of a batch in a cache (the benchmark's paged
    pre-fill, and the source rows of a paged plan's new tokens) takes its rows from the library's
    slot map: bit-exact against the oracle's paged addressing and the packed rows."""
    w = synth.custom(405, [300, 1, 70], [300, 900, 200], P=2, H=16, Dl=512, Dr=64)
    bt, nb = make_block_table(w, 405)
    reqs = np.concatenate([np.full(int(k), b, np.int64) for b, k in enumerate(w.kv_lens)])
    poss = np.concatenate([np.arange(int(k), dtype=np.int64) for k in w.kv_lens])
    got = pp.cache_rows(w.kv_lens, w.kv_lens, w.kv_start, block_table=bt).cpu().numpy()
    assert np.array_equal(got, ok.paged_rows(bt, reqs, poss))
    got = pp.cache_rows(w.kv_lens, w.kv_lens, w.kv_start).cpu().numpy()
    assert np.array_equal(got, w.kv_start[reqs] + poss)
    # a paged plan's new-token source rows come from its packed twin
    pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P, block_table=bt)
    pp.run_partition(pl)
    plan = hp.oracle_plan(w)
    pos, req = hp.token_maps(plan)
    for r, rp in enumerate(plan.ranks):
        g = rp.local_gidx.astype(np.int64)
        assert np.array_equal(pp.packed_rows(pl, r).cpu().numpy(), w.kv_start[req[g]] + pos[g])
