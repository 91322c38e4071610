"""Pins of the oracle's LSE merge: merging disjoint partials reproduces unsharded
attention with the sink counted once; negative cases fail."""
import math

import numpy as np
import pytest

from oracle import attention as oa
from oracle import merge as om
from oracle import partition as op


def _problem(rng, n, H=3, Dl=8, Dr=4):
    q = rng.standard_normal((H, Dl + Dr)) * 0.5
    lat = rng.standard_normal((n, Dl)) * 0.5
    rope = rng.standard_normal((n, Dr)) * 0.5
    return q, lat, rope


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_merge_of_disjoint_parts_is_unsharded(seed, P):
    rng = np.random.default_rng(seed * 10 + P)
    n = int(rng.integers(P, 60))
    q, lat, rope = _problem(rng, n)
    sink = rng.standard_normal(q.shape[0]) * 2
    _, _, o_ref, l_ref = oa.attend_keyset(q, lat, rope, 0.3, sink)
    owner = rng.integers(0, P, size=n)  # random disjoint split of the key set
    parts = []
    for k in range(P):
        idx = np.nonzero(owner == k)[0]
        if len(idx):
            o0, l0, _, _ = oa.attend_keyset(q, lat[idx], rope[idx], 0.3)
            parts.append((o0, l0))
    for h in range(q.shape[0]):
        perm = rng.permutation(len(parts))  # contributor order is irrelevant
        o, l = om.merge_row([parts[i][0][h] for i in perm], [parts[i][1][h] for i in perm], sink[h])
        np.testing.assert_allclose(o, o_ref[h], atol=1e-13)
        np.testing.assert_allclose(l, l_ref[h], atol=1e-13)


@pytest.mark.parametrize("T,P", [(64, 2), (96, 4), (45, 3)])
def test_dualchunkswap_key_split(T, P):
    """Key-split variant: each rank attends only the keys of its own two chunks."""
    rng = np.random.default_rng(T)
    q, lat, rope = _problem(rng, T)
    sink = np.array([0.5, -1.0, 3.0])
    plan = op.partition([T], [T], [0], P)
    p = T - 1  # last query sees every key
    _, _, o_ref, l_ref = oa.attend_keyset(q, lat, rope, 0.3, sink)
    parts = []
    for r in range(P):
        keys = plan.ranks[r].positions
        o0, l0, _, _ = oa.attend_keyset(q, lat[keys], rope[keys], 0.3)
        parts.append((o0, l0))
    for h in range(3):
        o, l = om.merge_row([x[0][h] for x in parts], [x[1][h] for x in parts], sink[h])
        np.testing.assert_allclose(o, o_ref[h], atol=1e-13)
        np.testing.assert_allclose(l, l_ref[h], atol=1e-13)
    assert p == T - 1


def test_no_contributor_and_no_sink():
    o, l = om.merge_row([], [], 1.5)
    assert o is None and l == 1.5
    o, l = om.merge_row([np.ones(4)], [2.0], -math.inf)
    np.testing.assert_allclose(o, np.ones(4)) and math.isclose(l, 2.0)


def test_merge_array_form_global_order():
    """merge() follows merge_src into global order and skips -1 entries."""
    rng = np.random.default_rng(2)
    o_cat = rng.standard_normal((5, 2, 3))
    lse_cat = rng.standard_normal((5, 2))
    src = np.array([[4, -1], [-1, 0], [1, 2]])
    sink = np.array([0.1, -0.2])
    O, L = om.merge(o_cat, lse_cat, src, sink)
    o, l = om.merge_row([o_cat[1, 1], o_cat[2, 1]], [lse_cat[1, 1], lse_cat[2, 1]], -0.2)
    np.testing.assert_allclose(O[2, 1], o) and np.testing.assert_allclose(L[2, 1], l)
    o, l = om.merge_row([o_cat[4, 0]], [lse_cat[4, 0]], 0.1)
    np.testing.assert_allclose(O[0, 0], o)


def test_sink_per_rank_is_wrong():
    """Applying the sink on every rank and again in the merge misses by a wide margin
    when the sink is large (sigma = ln n + 2)."""
    rng = np.random.default_rng(11)
    n = 16
    q, lat, rope = _problem(rng, n, H=1)
    lat = lat * 8  # O of order one, so the absolute miss is visible too
    sig = math.log(n) + 2
    _, _, o_ref, _ = oa.attend_keyset(q, lat, rope, 0.3, np.array([sig]))
    halves = [np.arange(0, n // 2), np.arange(n // 2, n)]
    parts_sink = [oa.attend_keyset(q, lat[i], rope[i], 0.3, np.array([sig])) for i in halves]
    o_bad, _ = om.merge_row([p[2][0] for p in parts_sink], [p[3][0] for p in parts_sink], sig)
    assert np.max(np.abs(o_bad - o_ref[0])) > 1e-2 * 3
    assert np.linalg.norm(o_bad - o_ref[0]) > 0.5 * np.linalg.norm(o_ref[0])


def test_replicas_merged_once():
    """A replicated row merged from all P copies gives P e^L / (e^s + P e^L) weights."""
    rng = np.random.default_rng(12)
    q, lat, rope = _problem(rng, 4, H=1)
    sig = 1.0
    o0, l0, o_ref, l_ref = oa.attend_keyset(q, lat, rope, 0.3, np.array([sig]))
    o_once, l_once = om.merge_row([o0[0]], [l0[0]], sig)
    np.testing.assert_allclose(o_once, o_ref[0], atol=1e-14)
    o_all, _ = om.merge_row([o0[0]] * 4, [l0[0]] * 4, sig)
    w_all = 4 * math.exp(l0[0]) / (math.exp(sig) + 4 * math.exp(l0[0]))
    np.testing.assert_allclose(o_all, o0[0] * w_all, atol=1e-14)
    assert np.max(np.abs(o_all - o_ref[0])) > 1e-2
