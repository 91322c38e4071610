"""CPU model of every device access of the paged out-of-cache block-id test.

The model restates, launch by launch, the index arithmetic of the kernels that the test
``test_gpu_paged.py::test_paged_block_ids_outside_the_cache`` runs, with the exact inputs
that test builds (valid and corrupted block tables), and checks every byte range against
the size of the buffer it touches:

* the harness's set-up tensors (the local latent / rope rows handed to the inserts);
* ``plan_tokens`` (block-table reads forming the slots);
* ``kv_insert_kernel`` and the fp8 quantise-on-insert launches (``fp8_block_reset``,
  ``fp8_block_amax``, ``fp8_quantize_rows``);
* ``fp8_dequant_blocks`` with the harness's list of blocks;
* the paged dense kernel's 64-tile window of block ids, its tile rows and the latent and
  rope loads (including the loads issued after a row's last tile);
* the sparse key sets (selected rows through the table, window blocks, the pad row) and the
  row clamps, latent / rope / scale offsets of the sparse kernels (the bf16 kernel reads the
  table only at the blocks of keys of the set and of key 0, a subset of what is modelled);
* the merge's contributor rows.

It also shows the cause of the fault that test met: built on an fp8 workload, the sparse
half of the test handed E4M3 codes (one byte per element) viewed as bf16 to the fp8 insert,
whose amax and quantise launches read two bytes per element, i.e. twice the buffer. The
kernels' own accesses stay inside the cache for every table the test uses.
"""
from __future__ import annotations

import numpy as np
import pytest

import helpers as hp
import paged_tables as pt
from context_mla_prefill_amd import synth

BN = 64  # keys per tile = rows per cache block
BM = 64  # rows (token x head) per dense workgroup


class Bufs:
    """Allocation sizes in bytes; every modelled access is checked against them."""

    def __init__(self, **sizes):
        self.size = dict(sizes)

    def touch(self, name, lo, hi):
        lo = np.atleast_1d(np.asarray(lo, dtype=np.int64))
        hi = np.atleast_1d(np.asarray(hi, dtype=np.int64))
        if lo.size == 0:
            return
        n = self.size[name]
        bad = (lo < 0) | (hi > n) | (hi < lo)
        assert not bad.any(), (f"{name}: {int(bad.sum())} accesses outside [0, {n}), first "
                               f"[{int(lo[bad][0])}, {int(hi[bad][0])})")


def i32(x):
    """The kernels form these values in 32-bit ints: they must not wrap."""
    x = np.asarray(x, dtype=np.int64)
    assert np.all((x >= -(1 << 31)) & (x < (1 << 31))), "int32 overflow"
    return x


# ------------------------------------------------------------------------------- launches

def model_plan_tokens(bufs, w, plan, bt):
    """plan_tokens: the slot of token t of request b at position p reads table column
    min(p / 64, bt_stride - 1) of row b."""
    pos, req = hp.token_maps(plan)
    bt_stride = bt.shape[1]
    col = np.minimum(pos >> 6, bt_stride - 1)
    idx = req * bt_stride + col
    bufs.touch("block_table", idx * 4, idx * 4 + 4)
    slot = i32(bt[req, col].astype(np.int64) * 64 + (pos & 63))
    return slot, pos, req


def model_kv_insert(bufs, src_name, rope_name, slot, T, N_kv, Dl, Dr):
    """kv_insert_kernel: reads local rows 0..T-1, writes cache rows s only for 0 <= s < N_kv."""
    r = np.arange(T, dtype=np.int64)
    bufs.touch(src_name, r * Dl * 2, r * Dl * 2 + Dl * 2)
    bufs.touch(rope_name, r * Dr * 2, r * Dr * 2 + Dr * 2)
    s = slot[(slot >= 0) & (slot < N_kv)].astype(np.int64)
    bufs.touch("kv_lat", s * Dl * 2, s * Dl * 2 + Dl * 2)
    bufs.touch("kv_rope", s * Dr * 2, s * Dr * 2 + Dr * 2)


def model_fp8_insert(bufs, src_name, rope_name, slot, T, N_kv, Dl, Dr):
    """fp8_block_reset / fp8_block_amax / fp8_quantize_rows: each reads the local row's
    Dl bf16 values (2 bytes each) and its rope row; cache codes, rope and the block's scale
    word are written only for slots inside the cache."""
    r = np.arange(T, dtype=np.int64)
    bufs.touch("slot", r * 4, r * 4 + 4)
    bufs.touch(src_name, r * Dl * 2, r * Dl * 2 + Dl * 2)  # amax and quantise: bf16x8 per lane
    bufs.touch(rope_name, r * Dr * 2, r * Dr * 2 + Dr * 2)
    s = slot[(slot >= 0) & (slot < N_kv)].astype(np.int64)
    bufs.touch("kv_scale", (s >> 6) * 4, (s >> 6) * 4 + 4)
    bufs.touch("kv_lat", s * Dl, s * Dl + Dl)  # one fp8 byte per element
    bufs.touch("kv_rope", s * Dr * 2, s * Dr * 2 + Dr * 2)


def model_dequant(bufs, blocks, N_kv, Dl):
    """fp8_dequant_blocks: a listed block outside the cache is skipped; rows past N_kv too."""
    blocks = np.asarray(blocks, dtype=np.int64)
    bufs.touch("blocks", np.arange(len(blocks)) * 4, np.arange(len(blocks)) * 4 + 4)
    b = blocks[(blocks >= 0) & (blocks * 64 < N_kv)]
    rows = (b[:, None] * 64 + np.arange(64)[None, :]).ravel()
    rows = rows[rows < N_kv]
    bufs.touch("kv_scale", b * 4, b * 4 + 4)
    bufs.touch("kv_lat", rows * Dl, rows * Dl + Dl)
    bufs.touch("ws", rows * Dl * 2, rows * Dl * 2 + Dl * 2)


def model_dense_paged(bufs, w, rp, bt, N_kv):
    """The paged dense kernel of one rank: per workgroup (64 rows of one virtual row) the KV
    extent (largest position + 1), the 64-entry window of clamped block ids, the rows of every
    tile it loads (tiles kt0 .. n_tiles, the last being the loads issued after the final tile,
    whose key is clamped to the last one), and the latent / rope byte ranges of those loads
    (latent: scalar offset min(n, rows-1) * 1024 plus 16 bytes per lane; rope: rows of 128
    bytes in 16-byte chunks). Returns the number of tiles checked."""
    H, DL, DR = w.H, w.Dl, w.Dr
    blk_max = (N_kv >> 6) - 1
    bt_stride = bt.shape[1]
    n = 0
    for v in range(rp.n_vrows):
        tok0, tok1 = int(rp.cu_seqlens_q[v]), int(rp.cu_seqlens_q[v + 1])
        nrows = (tok1 - tok0) * H
        b = int(rp.vrow_req[v])
        for tile in range((nrows + BM - 1) // BM):
            rl = np.arange(tile * BM, min(nrows, tile * BM + BM))
            kv_hi = int(rp.positions[tok0 + rl // H].max()) + 1
            last = kv_hi - 1
            nblk = (last >> 6) + 1
            n_tiles = (kv_hi + BN - 1) // BN
            win = {}

            def bw_load(base):
                win["base"] = base
                col = np.minimum(base + np.arange(64), min(nblk, bt_stride) - 1)
                idx = b * bt_stride + col
                bufs.touch("block_table", idx * 4, idx * 4 + 4)
                win["ids"] = np.clip(bt[b, col], 0, blk_max)

            def tile_rows(kt):
                tb = min(kt * BN, last)
                rows = min(BN, last - tb + 1)
                t = tb >> 6
                row0 = int(win["ids"][(t - win["base"]) & 63]) * 64 + (tb & 63)  # readlane: lane mod 64
                if t == win["base"] + 63:
                    bw_load(win["base"] + 64)
                return row0, rows

            bw_load(min(0, nblk - 1) & ~63)
            for kt in range(0, n_tiles + 1):
                row0, rows = tile_rows(kt)
                assert 1 <= rows <= BN
                r = row0 + np.minimum(np.arange(BN), rows - 1)
                bufs.touch("kv_lat", r * DL * 2, r * DL * 2 + DL * 2)
                bufs.touch("kv_rope", r * DR * 2, r * DR * 2 + DR * 2)
                n += 1
    return n


def model_sparse(bufs, w, rp, bt, N_kv, topk_rows, row_bytes):
    """The sparse kernels of one rank (one workgroup per token and 64 heads): the selected
    index row, the table reads of sparse_keys (clamped columns; the pad row is block 0's first
    row; the window's blocks), every key row clamped into [0, N_kv - 1] before an offset is
    formed, and the latent (row_bytes per row), rope and scale reads of those rows. Returns
    the number of key rows that the clamp moved (keys mapped through out-of-cache ids)."""
    bt_stride = bt.shape[1]
    k = w.topk
    moved = 0
    for v in range(rp.n_vrows):
        b = int(rp.vrow_req[v])
        for tok in range(int(rp.cu_seqlens_q[v]), int(rp.cu_seqlens_q[v + 1])):
            p = int(rp.positions[tok])
            bufs.touch("topk", (tok * k + np.arange(k)) * 4, (tok * k + np.arange(k)) * 4 + 4)
            e = topk_rows[tok].astype(np.int64)
            col = np.minimum(np.maximum(e, 0) >> 6, bt_stride - 1)
            bufs.touch("block_table", (b * bt_stride + col) * 4, (b * bt_stride + col) * 4 + 4)
            sel_rows = i32(bt[b, col].astype(np.int64) * BN + (e & (BN - 1)))
            win_lo = max(0, p - w.window + 1)
            keep = (e >= 0) & (e <= p) & (e < win_lo)
            sel_rows = sel_rows[keep]
            sel_rows = sel_rows[sel_rows >= 0]  # a negative row is a pad (-1) for slot_key
            wcol = np.arange(win_lo >> 6, (p >> 6) + 1)
            assert len(wcol) <= 4096 // BN + 1
            wcol_c = np.minimum(wcol, bt_stride - 1)
            bufs.touch("block_table", (b * bt_stride + wcol_c) * 4, (b * bt_stride + wcol_c) * 4 + 4)
            wk = np.arange(win_lo, p + 1)
            win_rows = i32(bt[b, np.minimum(wk >> 6, bt_stride - 1)].astype(np.int64) * BN + (wk & (BN - 1)))
            pad_row = i32(int(bt[b, 0]) * BN)
            rows = np.concatenate([sel_rows, win_rows, [pad_row]])
            clamped = np.clip(rows, 0, N_kv - 1)
            moved += int((clamped != rows).sum())
            bufs.touch("kv_lat", clamped * row_bytes, clamped * row_bytes + row_bytes)
            bufs.touch("kv_rope", clamped * w.Dr * 2, clamped * w.Dr * 2 + w.Dr * 2)
            bufs.touch("kv_scale", (clamped >> 6) * 4, (clamped >> 6) * 4 + 4)
    return moved


def model_merge(bufs, plan, H, Dl):
    R_total = sum(rp.T_loc for rp in plan.ranks)
    rows = plan.merge_src[plan.merge_src >= 0].astype(np.int64)
    assert np.all(rows < R_total)
    bufs.touch("o_cat", rows * H * Dl * 2, rows * H * Dl * 2 + H * Dl * 2)
    bufs.touch("lse_cat", rows * H * 4, rows * H * 4 + H * 4)


# ------------------------------------------------------------------------------- the runs

def dense_run(w, table):
    """DenseCacheRun: partition, per-rank bf16 inserts, per-rank paged dense partials, merge."""
    bt, n_blocks = table
    plan = hp.oracle_plan(w)
    N = n_blocks * 64
    T_tot = sum(rp.T_loc for rp in plan.ranks)
    bufs = Bufs(block_table=bt.size * 4, kv_lat=N * w.Dl * 2, kv_rope=N * w.Dr * 2,
                o_cat=T_tot * w.H * w.Dl * 2, lse_cat=T_tot * w.H * 4)
    slot, _, _ = model_plan_tokens(bufs, w, plan, bt)
    tiles = 0
    for rp in plan.ranks:
        lat_local = synth.latent_rows(w)[:rp.T_loc]  # the harness's per-rank index_select
        bufs.size["lat_local"] = lat_local.nbytes
        bufs.size["rope_local"] = rp.T_loc * w.Dr * 2
        rslot = plan_slots_of(plan, rp, slot)
        model_kv_insert(bufs, "lat_local", "rope_local", rslot, rp.T_loc, N, w.Dl, w.Dr)
        tiles += model_dense_paged(bufs, w, rp, bt, N)
    model_merge(bufs, plan, w.H, w.Dl)
    return tiles


def plan_slots_of(plan, rp, slot_glob):
    """Slots of a rank's rows (the plan writes the token's slot to every row holding it)."""
    return slot_glob[rp.local_gidx.astype(np.int64)]


def sparse_run(w, table, workspace):
    """PagedSparseRun: partition, one fp8 insert of every rank's rows, (workspace: the used
    blocks dequantised), per-rank sparse partials, merge. The local latent buffer is what the
    harness builds: the workload's latent rows as bf16 values, gathered per row."""
    bt, n_blocks = table
    plan = hp.oracle_plan(w)
    N = n_blocks * 64
    T_tot = sum(rp.T_loc for rp in plan.ranks)
    lat_rows = synth.latent_rows(w)
    row_view = np.ascontiguousarray(lat_rows).view(np.int16)  # what dev_bf16 uploads
    bufs = Bufs(block_table=bt.size * 4, kv_lat=N * w.Dl, kv_rope=N * w.Dr * 2, kv_scale=n_blocks * 4,
                slot=T_tot * 4, lat_new=T_tot * row_view.shape[1] * 2, rope_new=T_tot * w.Dr * 2,
                o_cat=T_tot * w.H * w.Dl * 2, lse_cat=T_tot * w.H * 4)
    slot, _, _ = model_plan_tokens(bufs, w, plan, bt)
    rank_slots = np.concatenate([plan_slots_of(plan, rp, slot) for rp in plan.ranks])
    model_fp8_insert(bufs, "lat_new", "rope_new", rank_slots, T_tot, N, w.Dl, w.Dr)
    if workspace:
        used = np.unique(bt[(bt >= 0) & (bt < n_blocks)])
        bufs.size["blocks"] = used.size * 4
        bufs.size["ws"] = N * w.Dl * 2
        model_dequant(bufs, used, N, w.Dl)
        bufs.size["kv_lat"] = N * w.Dl * 2  # the partials read the workspace
    topk = synth.topk_rows(w)
    moved = 0
    for rp in plan.ranks:
        bufs.size["topk"] = rp.T_loc * w.topk * 4
        moved += model_sparse(bufs, w, rp, bt, N, topk[rp.local_gidx.astype(np.int64)],
                              w.Dl * 2 if workspace else w.Dl)
    model_merge(bufs, plan, w.H, w.Dl)
    return moved


@pytest.mark.parametrize("bad", [False, True])
def test_dense_run_stays_in_bounds(bad):
    w = synth.custom(**pt.OUT_OF_CACHE_DENSE)
    bt, nb = pt.make_block_table(w, 404)
    if bad:
        bt = pt.corrupt_table(bt, nb, 1)
    assert dense_run(w, (bt, nb)) > 0


@pytest.mark.parametrize("bad", [False, True])
@pytest.mark.parametrize("workspace", [True, False])
def test_sparse_run_stays_in_bounds(bad, workspace):
    w = synth.custom(**pt.OUT_OF_CACHE_SPARSE)
    bt, nb = pt.make_block_table(w, 504)
    if bad:
        bt = pt.corrupt_table(bt, nb, 1)
    moved = sparse_run(w, (bt, nb), workspace)
    # the corrupted table maps some keys through out-of-cache ids: the clamp moves them
    assert (moved > 0) == bad


def test_fp8_workload_overreads_the_insert_source():
    """The cause of the fault: on a workload drawn as fp8 codes, the harness's local latent
    rows hold one byte per element, and the fp8 insert reads two bytes per element from them,
    so its reads run past the end of that buffer (the valid-table run, before any corrupted
    table is used)."""
    w = synth.custom(**{**pt.OUT_OF_CACHE_SPARSE, "kv_dtype": "fp8"})
    bt, nb = pt.make_block_table(w, 504)
    with pytest.raises(AssertionError, match="lat_new"):
        sparse_run(w, (bt, nb), workspace=True)
