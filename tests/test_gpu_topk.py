"""GPU parity of the top-k selection kernel against the oracle (bit-exact index lists),
and the selection feeding the sparse partial."""
import time

import numpy as np
import pytest
import torch

import helpers as hp
from context_mla_prefill_amd import _lib, synth
from context_mla_prefill_amd import pipeline as pp
from oracle import topk as ot

pytestmark = pytest.mark.gpu


def _pattern_row(pat, n, rng, w):
    if pat == "hash":
        return synth.index_scores(w, [n * 7 % 131072], n)[0]
    if pat == "asc":
        return np.arange(n, dtype=np.float32)
    if pat == "desc":
        return -np.arange(n, dtype=np.float32)
    if pat == "equal":
        return np.full(n, 0.5, np.float32)
    if pat == "few":
        return rng.integers(0, 16, n).astype(np.float32)
    if pat == "zeros":  # +0 and -0 mixed (equal scores), a few ones
        z = np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0))
        return (z + (rng.random(n) < 0.01).astype(np.float32)).astype(np.float32)
    if pat == "normal":
        return rng.standard_normal(n).astype(np.float32)
    row = np.where(rng.random(n) < 0.02, np.float32(np.inf), rng.standard_normal(n).astype(np.float32))
    row[::97] = -np.inf
    return row.astype(np.float32)


PATTERNS = ["hash", "asc", "desc", "equal", "few", "zeros", "normal", "inf"]
LENGTHS = [1, 5, 2047, 2048, 2049, 3000, 6143, 6144, 6145, 9000, 50000, 131072]


@pytest.mark.parametrize("k", [2048, 64, 1])
def test_topk_select_edge_rows(gpu_lib, k):
    """Every length regime (a prefix shorter than k, rows held whole in LDS, sampled
    threshold, the in-memory fallback for sorted, constant and heavily tied rows), +-0 and
    +-inf scores; scores past a row's prefix are NaN and must never be read; one row's
    position lies past ld (its prefix is cut at ld)."""
    rng = np.random.default_rng(k)
    w = synth.workload(4)
    ld = 131072
    rows, ns = [], []
    for n in LENGTHS:
        for pat in PATTERNS:
            r = np.full(ld, np.nan, np.float32)
            r[:n] = _pattern_row(pat, n, rng, w)
            rows.append(r)
            ns.append(n)
    rows.append(synth.index_scores(w, [99], ld)[0])
    ns.append(ld + 5000)  # position past ld
    scores = np.stack(rows)
    pos = np.asarray(ns, np.int64) - 1
    T = len(rows)
    print(f"[run] top-k edge rows T={T} k={k}", flush=True)
    s_d = torch.from_numpy(scores).cuda()
    p_d = torch.from_numpy(pos.astype(np.int32)).cuda()
    out = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    _lib.sparse_topk_select(s_d, ld, p_d, T, k, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i in range(T):
        want = ot.topk_select(scores[i], min(int(pos[i]) + 1, ld), k)
        assert np.array_equal(got[i], want), f"row {i} n={ns[i]}: first differences " \
            f"{np.nonzero(got[i] != want)[0][:5]}"


def test_topk_select_rows_past_the_bitmap(gpu_lib):
    """Rows longer than the LDS bitmap covers (more than 196,608 scores): the sampled threshold
    and the LDS select, then the ordered pass over the row writes the indices."""
    w = synth.workload(4)
    ns = [196609, 200000, 250000, 262144]
    ld = max(ns)
    scores = synth.index_scores(w, [5, 6, 7, 8], ld)
    scores[1, 100:3000] = 0.999999  # a long tie band near the top
    pos = np.asarray(ns, np.int32) - 1
    print(f"[run] top-k long rows {ns}", flush=True)
    out = torch.empty(len(ns), 2048, dtype=torch.int32, device="cuda")
    _lib.sparse_topk_select(torch.from_numpy(scores).cuda(), ld, torch.from_numpy(pos).cuda(), len(ns), 2048, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i, n in enumerate(ns):
        assert np.array_equal(got[i], ot.topk_select(scores[i], n, 2048)), n


def test_topk_select_full_size_sampled(gpu_lib):
    """One rank of the 128K top-2048 workload: 65536 query rows of up to 131072 hashed scores
    (34 GB). Every row checked for its invariants on the GPU (increasing, in the prefix, no
    pads once the prefix exceeds k); the first and last row of every chunk and 192 random
    rows against the oracle, bit-exact."""
    w = synth.workload(4)
    pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P)
    pp.run_partition(pl)
    r = 0
    rows = pl.rank_rows(r)
    T = pl.T_loc[r]
    ld = int(w.kv_lens.max())
    gidx = pl.local_gidx[rows].long()
    pos = pl.positions[rows]
    print(f"[run] top-k full size rank {r}: T={T} ld={ld}", flush=True)
    scores = synth.index_scores_device(w, gidx, ld)
    out = torch.empty(T, w.topk, dtype=torch.int32, device="cuda")
    _lib.sparse_topk_select(scores, ld, pos, T, w.topk, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _lib.sparse_topk_select(scores, ld, pos, T, w.topk, out)
    torch.cuda.synchronize()
    print(f"[time] selection {1e3 * (time.perf_counter() - t0):.2f} ms", flush=True)
    n = (pos.long() + 1)[:, None]
    o = out.long()
    full = n[:, 0] > w.topk
    assert bool(((o >= 0) & (o < n)).all(dim=1)[full].all())
    assert bool((o[:, 1:] > o[:, :-1])[full].all())
    short = ~full
    if bool(short.any()):
        ar = torch.arange(w.topk, device="cuda")[None, :]
        want_short = torch.where(ar < n, ar, torch.full_like(ar, -1))
        assert bool((o[short] == want_short[short]).all())
    # sampled rows against the oracle on host-built scores
    rng = np.random.default_rng(4)
    g_host = gidx.cpu().numpy()
    p_host = pos.cpu().numpy()
    cu = pl.cu_q[r].cpu().numpy()
    pick = set(int(x) for x in rng.integers(0, T, size=192))
    for v in range(pl.n_vrows):
        if cu[v + 1] > cu[v]:
            pick.update([int(cu[v]), int(cu[v + 1] - 1)])
    got = out.cpu().numpy()
    for i in sorted(pick):
        row = synth.index_scores(w, [g_host[i]], int(p_host[i]) + 1)[0]
        want = ot.topk_select(row, int(p_host[i]) + 1, w.topk)
        assert np.array_equal(got[i], want), f"row {i} (token {g_host[i]}, position {p_host[i]})"


def test_topk_select_feeds_sparse_partial(gpu_lib):
    """Selected indices made on the GPU from hashed scores equal the oracle's, and the sparse
    path on them (top-k 128 + window 64, fp8, P = 2) matches the oracle on every row."""
    from test_gpu_parity import SparseRun

    w = synth.custom(601, [1500, 700], [1500, 900], P=2, H=64, Dl=512, Dr=64, topk=128, window=64,
                     kv_dtype="fp8", latent_std=1.0)
    pl = pp.alloc_plan(w.q_lens, w.kv_lens, w.kv_start, w.P)
    pp.run_partition(pl)
    ld = int(w.kv_lens.max())
    sel = np.full((w.T_glob, w.topk), -9, np.int32)
    for r in range(w.P):
        rows = pl.rank_rows(r)
        gidx = pl.local_gidx[rows].long()
        scores = synth.index_scores_device(w, gidx, ld)
        out = torch.empty(pl.T_loc[r], w.topk, dtype=torch.int32, device="cuda")
        _lib.sparse_topk_select(scores, ld, pl.positions[rows], pl.T_loc[r], w.topk, out)
        torch.cuda.synchronize()
        sel[gidx.cpu().numpy()] = out.cpu().numpy()
    plan = hp.oracle_plan(w)
    pos, _ = hp.token_maps(plan)
    host_scores = synth.index_scores(w, np.arange(w.T_glob), ld)
    for t in range(w.T_glob):
        assert np.array_equal(sel[t], ot.topk_select(host_scores[t], int(pos[t]) + 1, w.topk)), t
    run = SparseRun(w, topk_rows=sel)
    run.check_values(np.arange(w.T_glob))
