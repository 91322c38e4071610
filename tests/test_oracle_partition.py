"""Pins of the oracle's DualChunkSwap partition against the pages and independent checks."""
import os

import numpy as np
import pytest

from oracle import partition as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split(":")
        rows[int(k)] = v.split()
    return rows


def _single(T, P, kv=None):
    kv = T if kv is None else kv
    return op.partition([T], [kv], [0], P)


def test_pcp4_figure():
    """The PCP=4 picture: rank r holds C_r then C_{7-r}."""
    g = _read_golden("dualchunkswap_pcp4.txt")
    c = 5
    plan = _single(8 * c, 4)
    for r in range(4):
        want = np.concatenate([np.arange(int(x) * c, (int(x) + 1) * c) for x in g[r]])
        assert np.array_equal(plan.ranks[r].positions, want)
        assert plan.ranks[r].n_vrows == 2


def test_tiny_p2_positions():
    g = _read_golden("tiny_p2_positions.txt")
    plan = _single(256, 2)
    for r in range(2):
        want = np.concatenate([np.arange(int(a), int(b) + 1)
                               for a, b in (s.split("-") for s in g[r])])
        assert np.array_equal(plan.ranks[r].positions, want)
        assert np.array_equal(plan.ranks[r].local_gidx, want)


@pytest.mark.parametrize("q", list(range(0, 40)))
@pytest.mark.parametrize("n", [1, 2, 4, 6, 8])
def test_chunk_sizes_match_array_split(q, n):
    want = [len(a) for a in np.array_split(np.arange(q), n)]
    assert op.chunk_sizes(q, n) == want


def _random_batch(rng, max_tok=64):
    n_req = int(rng.integers(1, 6))
    q, kv = [], []
    for _ in range(n_req):
        kind = rng.integers(0, 3)
        if kind == 0:  # decode row
            ctx = int(rng.integers(1, 20))
            q.append(1), kv.append(ctx)
        elif kind == 1:  # short or long prefill
            t = int(rng.integers(0, max_tok))
            q.append(t), kv.append(t)
        else:  # chunked-prefill continuation
            t = int(rng.integers(1, max_tok))
            q.append(t), kv.append(t + int(rng.integers(0, 10)))
    ks = np.concatenate([[0], np.cumsum(kv)[:-1]]).astype(np.int64)
    return q, kv, ks


@pytest.mark.parametrize("seed", range(40))
@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_brute_force_assignment(seed, P):
    """Independent per-token enumeration: chunk by array_split membership, rank by the
    pairing rule, coverage exactly once, replicas owned by rank 0 only."""
    rng = np.random.default_rng(seed * 7 + P)
    q, kv, ks = _random_batch(rng)
    plan = op.partition(q, kv, ks, P)
    cu = np.concatenate([[0], np.cumsum(q)])
    # every rank row points to a real token with the right position and slot
    seen = {}
    for r in range(P):
        rp = plan.ranks[r]
        assert rp.cu_seqlens_q[-1] == rp.T_loc
        for i, g in enumerate(rp.local_gidx):
            b = int(np.searchsorted(cu, g, side="right") - 1)
            pos = kv[b] - q[b] + (g - cu[b])
            assert rp.positions[i] == pos and rp.slot[i] == ks[b] + pos
            seen.setdefault(int(g), []).append(r)
    for b in range(len(q)):
        toks = np.arange(cu[b], cu[b + 1])
        if q[b] >= 2 * P:
            chunks = np.array_split(toks, 2 * P)
            for c, ch in enumerate(chunks):
                want_rank = c if c < P else 2 * P - 1 - c
                for g in ch:
                    assert seen[int(g)] == [want_rank]
                    row = plan.merge_src[g]
                    assert (row >= 0).sum() == 1 and row[want_rank] >= 0
        else:
            for g in toks:
                assert seen[int(g)] == list(range(P))
                row = plan.merge_src[g]
                assert (row >= 0).sum() == 1 and row[0] >= 0
    # merge_src points at the row that holds that token
    for g in range(plan.T_glob):
        for r in range(P):
            m = plan.merge_src[g, r]
            if m >= 0:
                i = m - plan.row_off[r]
                assert plan.ranks[r].local_gidx[i] == g
    # virtual rows: contiguous positions ending at kv_len
    for r in range(P):
        rp = plan.ranks[r]
        for v in range(rp.n_vrows):
            a, e = rp.cu_seqlens_q[v], rp.cu_seqlens_q[v + 1]
            if e > a:
                pos = rp.positions[a:e]
                assert np.array_equal(pos, np.arange(pos[0], pos[0] + (e - a)))
                assert rp.vrow_kv_len[v] == pos[-1] + 1
            assert rp.vrow_kv_start[v] == ks[rp.vrow_req[v]]


@pytest.mark.parametrize("T,P", [(256, 2), (8192, 2), (4096, 4), (131072, 4), (48, 3)])
def test_pair_count_closed_form(T, P):
    """With 2P | T every rank attends exactly c(T+1) causal pairs, c = T/(2P)."""
    assert T % (2 * P) == 0
    plan = _single(T, P)
    c = T // (2 * P)
    for r in range(P):
        assert op.causal_pairs(plan, r) == c * (T + 1)
    if (T, P) == (131072, 4):
        assert c * (T + 1) == 2_147_500_032


def test_contiguous_split_is_unbalanced():
    """Contrast: a contiguous quarter split would give ranks 1:7 pair counts."""
    T, P = 131072, 4
    q = T // P
    pairs = [sum(range(r * q + 1, (r + 1) * q + 1)) for r in range(P)]
    assert pairs[0] == 536_887_296 and pairs[3] == 3_758_112_768


@pytest.mark.parametrize("T", [0, 1, 2, 3, 7, 8, 64])
def test_p1_is_identity(T):
    plan = _single(T, 1)
    assert np.array_equal(plan.ranks[0].local_gidx, np.arange(T))
    assert np.array_equal(plan.merge_src[:, 0], np.arange(T))


def test_short_prefill_replicated():
    plan = op.partition([3, 9], [3, 9], [0, 3], 2)  # 3 < 2P=4: replicated; 9: split
    for r in range(2):
        assert list(plan.ranks[r].local_gidx[:3]) == [0, 1, 2]
    assert plan.ranks[0].n_vrows == 3 and plan.ranks[1].n_vrows == 3
    assert list(plan.ranks[0].local_gidx[3:]) == [3, 4, 5, 10, 11]
    assert list(plan.ranks[1].local_gidx[3:]) == [6, 7, 8, 9]


def test_empty_batch():
    plan = op.partition([], [], [], 3)
    assert plan.T_glob == 0 and all(rp.T_loc == 0 and rp.n_vrows == 0 for rp in plan.ranks)
