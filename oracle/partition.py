"""DualChunkSwap prefill-context-parallel partition (oracle; test infrastructure only).

Source: "[Core] Add MRV2 virtual-batch PCP for MLA", section "PCP algorithm" and
"DualChunkSwap partitioning" with its PCP=4 figure:

* the scheduler produces one global batch; the PCP manager turns it into rank-local
  virtual rows holding a portion of each prefill;
* each prefill request is partitioned on its own into 2*P contiguous chunks, and
  rank r receives chunks r and 2*P-1-r;
* decode rows are replicated on every PCP rank.

Readings where the pages are silent (each listed in the design notes):

* chunk sizes when 2P does not divide the prefill: numpy.array_split sizes, i.e.
  chunk i holds q//(2P) + (i < q % 2P) tokens, contiguous and in order ("arbitrary PCP
  chunk boundaries", "[Feature][PCP] Add DeepSeek-V4.1-Flash support", "Supported
  Scope");
* a request with fewer than 2P new tokens is replicated like a decode row
  ("replicated short prefills", same page, "Rank-local Compressor Revision");
  rank 0 owns replicated rows for the merge, so the sink and the row are counted once;
* rank-local order: requests in batch order; a split request contributes its chunk r
  then its chunk 2P-1-r, each as one virtual row; a replicated request is one virtual
  row at its batch position;
* global order: requests in batch order, tokens by position;
* position of the i-th new token = kv_len - q_len + i (the new tokens end the KV);
  slot = kv_start + position in the packed KV.
"""
from dataclasses import dataclass

import numpy as np


@dataclass
class RankPlan:
    local_gidx: np.ndarray  # [T_loc] global packed token of each local row
    positions: np.ndarray  # [T_loc]
    slot: np.ndarray  # [T_loc] packed KV row written by / attended up to by the token
    cu_seqlens_q: np.ndarray  # [n_vrows+1] local token offsets of the virtual rows
    vrow_req: np.ndarray  # [n_vrows] request of each virtual row
    vrow_kv_start: np.ndarray  # [n_vrows] packed KV offset of the row's request
    vrow_kv_len: np.ndarray  # [n_vrows] last position of the row + 1

    @property
    def T_loc(self) -> int:
        return int(len(self.local_gidx))

    @property
    def n_vrows(self) -> int:
        return int(len(self.vrow_req))


@dataclass
class Plan:
    P: int
    T_glob: int
    cu_seqlens_glob: np.ndarray  # [n_req+1]
    ranks: list  # list[RankPlan]
    row_off: np.ndarray  # [P] first row of each rank in the rank-concatenated buffers
    merge_src: np.ndarray  # [T_glob, P] rank-concatenated row contributed by rank r, or -1


def chunk_sizes(q_len: int, n_chunks: int) -> list:
    """Sizes of n_chunks contiguous chunks of q_len tokens, larger chunks first."""
    base, extra = divmod(q_len, n_chunks)
    return [base + (1 if i < extra else 0) for i in range(n_chunks)]


def partition(q_lens, kv_lens, kv_start, P: int) -> Plan:
    """DualChunkSwap plan for a batch of requests over P ranks (plain Python loops)."""
    q_lens = [int(x) for x in q_lens]
    kv_lens = [int(x) for x in kv_lens]
    kv_start = [int(x) for x in kv_start]
    n_req = len(q_lens)
    assert P >= 1 and len(kv_lens) == n_req and len(kv_start) == n_req
    cu = [0]
    for q in q_lens:
        cu.append(cu[-1] + q)
    T_glob = cu[-1]

    # per rank: lists of (global token, position, slot) and virtual rows
    toks = [[] for _ in range(P)]
    vrows = [[] for _ in range(P)]  # (req, kv_start, kv_len, n_tokens)
    owner = {}  # global token -> (rank, local index)

    for b in range(n_req):
        q, kv = q_lens[b], kv_lens[b]
        assert 0 <= q <= kv
        p0 = kv - q  # position of the first new token
        if q >= 2 * P:
            sizes = chunk_sizes(q, 2 * P)
            starts = [sum(sizes[:i]) for i in range(2 * P)]
            for r in range(P):
                for c in (r, 2 * P - 1 - r):
                    first = len(toks[r])
                    for i in range(starts[c], starts[c] + sizes[c]):
                        toks[r].append((cu[b] + i, p0 + i, kv_start[b] + p0 + i))
                    vrows[r].append((b, kv_start[b], p0 + starts[c] + sizes[c], sizes[c]))
                    for j in range(sizes[c]):
                        owner[cu[b] + starts[c] + j] = (r, first + j)
        else:
            for r in range(P):
                first = len(toks[r])
                for i in range(q):
                    toks[r].append((cu[b] + i, p0 + i, kv_start[b] + p0 + i))
                vrows[r].append((b, kv_start[b], p0 + q, q))
                if r == 0:
                    for i in range(q):
                        owner[cu[b] + i] = (0, first + i)

    ranks = []
    for r in range(P):
        t = np.asarray(toks[r], dtype=np.int64).reshape(-1, 3)
        v = vrows[r]
        cuq = np.zeros(len(v) + 1, dtype=np.int64)
        cuq[1:] = np.cumsum([x[3] for x in v]) if v else []
        ranks.append(RankPlan(
            local_gidx=t[:, 0].copy(), positions=t[:, 1].copy(), slot=t[:, 2].copy(),
            cu_seqlens_q=cuq,
            vrow_req=np.asarray([x[0] for x in v], dtype=np.int64),
            vrow_kv_start=np.asarray([x[1] for x in v], dtype=np.int64),
            vrow_kv_len=np.asarray([x[2] for x in v], dtype=np.int64)))
    row_off = np.zeros(P, dtype=np.int64)
    for r in range(1, P):
        row_off[r] = row_off[r - 1] + ranks[r - 1].T_loc
    merge_src = np.full((T_glob, P), -1, dtype=np.int64)
    for g, (r, i) in owner.items():
        merge_src[g, r] = row_off[r] + i
    return Plan(P=P, T_glob=T_glob, cu_seqlens_glob=np.asarray(cu, dtype=np.int64),
                ranks=ranks, row_off=row_off, merge_src=merge_src)


def causal_pairs(plan: Plan, r: int) -> int:
    """Number of (query, key) pairs rank r attends under the causal rule."""
    return int((plan.ranks[r].positions + 1).sum())
