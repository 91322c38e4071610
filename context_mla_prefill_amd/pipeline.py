"""Device plumbing for one PCP prefill step on one GPU.

Allocates the caller-owned buffers the C ABI expects and issues the calls in order:
``pcp_partition`` -> ``pcp_kv_insert`` (per rank; or one ``pcp_kv_insert_fp8`` of every
rank's rows) -> ``mla_prefill_partial`` (per rank, one after another) -> ``pcp_lse_merge``.
The KV cache is packed per request or paged (a block table of 64-row blocks). Tensors are
torch device tensors (memory and streams only); every step runs in the library's HIP
kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import _lib

BF16 = torch.bfloat16


@dataclass
class DevicePlan:
    P: int
    n_req: int
    T_glob: int
    n_vrows: int
    T_loc: list
    row_off: list
    q_lens: torch.Tensor
    kv_lens: torch.Tensor
    kv_start: torch.Tensor
    cu_glob: torch.Tensor  # [n_req+1]
    cu_q: torch.Tensor  # [P, n_vrows+1]
    vrow_req: torch.Tensor  # [P, n_vrows]
    vrow_kv_start: torch.Tensor
    vrow_kv_len: torch.Tensor
    local_gidx: torch.Tensor  # [sum T_loc]
    positions: torch.Tensor
    slot: torch.Tensor
    merge_src: torch.Tensor  # [T_glob, P]
    block_table: torch.Tensor | None = None  # [n_req, bt_stride] 64-row cache blocks (paged KV)

    @property
    def T_total(self) -> int:
        return int(sum(self.T_loc))

    def rank_rows(self, r: int) -> slice:
        return slice(self.row_off[r], self.row_off[r] + self.T_loc[r])


def alloc_plan(q_lens, kv_lens, kv_start, P: int, device="cuda", block_table=None) -> DevicePlan:
    """Plan buffers for the given lengths; ``block_table`` (host or device int32
    [n_req, bt_stride]) switches the KV addressing to paged."""
    q_h = np.ascontiguousarray(q_lens, dtype=np.int32)
    kv_h = np.ascontiguousarray(kv_lens, dtype=np.int32)
    T_loc, n_vrows, T_glob = _lib.pcp_plan_sizes(q_h, kv_h, P)
    row_off = [int(x) for x in np.concatenate([[0], np.cumsum(T_loc)[:-1]])]
    i32 = dict(dtype=torch.int32, device=device)
    n_req = len(q_h)
    tot = int(sum(T_loc))
    return DevicePlan(
        P=P, n_req=n_req, T_glob=T_glob, n_vrows=n_vrows, T_loc=T_loc, row_off=row_off,
        q_lens=torch.from_numpy(q_h).to(device), kv_lens=torch.from_numpy(kv_h).to(device),
        kv_start=torch.as_tensor(np.asarray(kv_start, dtype=np.int32)).to(device),
        cu_glob=torch.empty(n_req + 1, **i32), cu_q=torch.empty(P, n_vrows + 1, **i32),
        vrow_req=torch.empty(P, max(n_vrows, 0), **i32), vrow_kv_start=torch.empty(P, n_vrows, **i32),
        vrow_kv_len=torch.empty(P, n_vrows, **i32), local_gidx=torch.empty(tot, **i32),
        positions=torch.empty(tot, **i32), slot=torch.empty(tot, **i32),
        merge_src=torch.empty(T_glob, P, **i32),
        block_table=None if block_table is None else torch.as_tensor(block_table, dtype=torch.int32).to(device))


def run_partition(pl: DevicePlan, stream=None):
    _lib.pcp_partition(pl.q_lens, pl.kv_lens, pl.kv_start, pl.P, pl.T_glob, pl.n_vrows, pl.T_total,
                       pl.cu_glob, pl.cu_q, pl.vrow_req, pl.vrow_kv_start, pl.vrow_kv_len, pl.local_gidx,
                       pl.positions, pl.slot, pl.merge_src, stream, block_table=pl.block_table,
                       bt_stride=0 if pl.block_table is None else int(pl.block_table.shape[1]))


@dataclass
class RankInputs:
    """One rank's local query rows (and selected keys), gathered during set-up."""
    q: torch.Tensor  # [T_loc, H, Dqk] bf16
    topk: torch.Tensor | None  # [T_loc, topk] int32
    latent: torch.Tensor  # [T_loc, Dl] local KV rows to insert
    rope: torch.Tensor  # [T_loc, Dr]


def packed_rows(pl: DevicePlan, r: int) -> torch.Tensor:
    """Row of each of rank r's local tokens in the packed per-request KV layout of the inputs
    (where its latent/rope source row sits): the slots pcp_partition writes for a packed
    cache. A paged plan gets them from a packed twin plan of the same batch (same requests,
    no block table), made once."""
    if pl.block_table is None:
        return pl.slot[pl.rank_rows(r)].long()
    if getattr(pl, "_packed_twin", None) is None:
        twin = alloc_plan(pl.q_lens.cpu().numpy(), pl.kv_lens.cpu().numpy(), pl.kv_start.cpu().numpy(), pl.P,
                          device=pl.slot.device)
        run_partition(twin)
        pl._packed_twin = twin
    return pl._packed_twin.slot[pl.rank_rows(r)].long()


def cache_rows(q_lens, kv_lens, kv_start, block_table=None, device="cuda") -> torch.Tensor:
    """Cache row of every key of every request (request-major, positions 0..kv_len-1): the
    slots pcp_partition writes when every key is new and P = 1 (packed rows kv_start + j, or
    rows through the block table). Set-up of a cache whose earlier keys are already in place."""
    kv = np.ascontiguousarray(kv_lens, dtype=np.int32)
    pl = alloc_plan(kv, kv, kv_start, 1, device=device, block_table=block_table)
    run_partition(pl)
    return pl.slot.long()


def rank_inputs(pl: DevicePlan, r: int, q_glob, latent_full, rope_full, topk_glob=None) -> RankInputs:
    """Rank r's query rows (and selected keys) and the new KV rows it contributes, gathered
    from packed global inputs (set-up, not part of the step)."""
    rows = pl.rank_rows(r)
    gidx = pl.local_gidx[rows].long()
    src = packed_rows(pl, r)
    return RankInputs(q=q_glob.index_select(0, gidx).contiguous(),
                      topk=None if topk_glob is None else topk_glob.index_select(0, gidx).contiguous(),
                      latent=latent_full.index_select(0, src).contiguous(),
                      rope=rope_full.index_select(0, src).contiguous())


@dataclass
class StepBuffers:
    o_cat: torch.Tensor  # [sum T_loc, H, Dl] bf16
    lse_cat: torch.Tensor  # [sum T_loc, H] fp32
    o: torch.Tensor  # [T_glob, H, Dl] bf16
    lse: torch.Tensor  # [T_glob, H] fp32


def alloc_step(pl: DevicePlan, H: int, Dl: int, device="cuda", kv_splits: int = 1) -> StepBuffers:
    """Partial outputs of every rank (kv_splits slices of T_total rows each) and the merged output."""
    return StepBuffers(o_cat=torch.empty(kv_splits * pl.T_total, H, Dl, dtype=BF16, device=device),
                       lse_cat=torch.empty(kv_splits * pl.T_total, H, dtype=torch.float32, device=device),
                       o=torch.empty(pl.T_glob, H, Dl, dtype=BF16, device=device),
                       lse=torch.empty(pl.T_glob, H, dtype=torch.float32, device=device))


@dataclass
class SplitPlan:
    """Per-row split KV for the dense partials (pcp_plan_splits), on the device."""
    max_splits: int
    splits: torch.Tensor  # [P, n_vrows] key ranges of each virtual row
    order: torch.Tensor  # [P, n_vrows] order in which the workgroups take the rows

    @property
    def split_rows(self) -> int:
        return int((self.splits > 1).sum())


def plan_splits(pl: DevicePlan, H: int, Dl: int, max_splits: int, n_workers: int | None = None,
                device="cuda") -> SplitPlan:
    """Host planning of the per-row key-range counts (set-up; the host knows the lengths)."""
    if n_workers is None:
        n_workers = torch.cuda.get_device_properties(torch.device(device)).multi_processor_count
    splits, order = _lib.pcp_plan_splits(pl.q_lens.cpu().numpy(), pl.kv_lens.cpu().numpy(), pl.P, H, Dl,
                                         max_splits, n_workers)
    return SplitPlan(max_splits=max_splits, splits=torch.from_numpy(splits).to(device),
                     order=torch.from_numpy(order).to(device))


def partial_args(pl: DevicePlan, r: int, ri: RankInputs, kv_latent, kv_rope, bufs: StepBuffers, H, Dl, Dr,
                 scale, kv_dtype=_lib.MLA_KV_BF16, kv_scale=None, topk=0, window=0, kv_splits=1,
                 split_plan: SplitPlan | None = None):
    """Arguments of rank r's mla_prefill_partial; with split_plan, kv_splits must be its max_splits."""
    rows = pl.rank_rows(r)
    if split_plan is not None:
        assert kv_splits == split_plan.max_splits, "kv_splits must match the split plan"
    return _lib.make_partial_args(
        q=ri.q, latent_kv=kv_latent, rope_k=kv_rope, cu_seqlens_q=pl.cu_q[r], vrow_kv_start=pl.vrow_kv_start[r],
        positions=pl.positions[rows], n_vrows=pl.n_vrows, T_loc=pl.T_loc[r], H=H, D_latent=Dl, D_rope=Dr,
        scale=scale, o_partial=bufs.o_cat[rows], lse=bufs.lse_cat[rows], N_kv=int(kv_latent.shape[0]),
        kv_dtype=kv_dtype, kv_scale=kv_scale, topk_idx=ri.topk, topk=topk, window=window,
        kv_splits=kv_splits, split_stride=pl.T_total if kv_splits > 1 else 0,
        vrow_kv_len=pl.vrow_kv_len[r] if kv_splits > 1 else None, block_table=pl.block_table,
        bt_stride=0 if pl.block_table is None else int(pl.block_table.shape[1]),
        vrow_req=None if pl.block_table is None else pl.vrow_req[r],
        vrow_splits=None if split_plan is None else split_plan.splits[r],
        vrow_order=None if split_plan is None else split_plan.order[r])


def run_merge(pl: DevicePlan, bufs: StepBuffers, sink, H: int, Dl: int, stream=None, kv_splits: int = 1):
    _lib.pcp_lse_merge(bufs.o_cat, bufs.lse_cat, pl.merge_src, pl.P, pl.T_glob, H, Dl, kv_splits * pl.T_total, sink,
                       bufs.o, bufs.lse, stream, kv_splits=kv_splits, split_stride=pl.T_total)
