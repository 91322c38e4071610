"""Pins of the oracle's top-k selection, and of the hashed index-score inputs."""
import numpy as np
import pytest
import torch

from context_mla_prefill_amd import synth
from oracle import topk as ot


def _brute(scores, n, k):
    """Repeatedly take the largest remaining score, the smallest index among equal ones."""
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    left = list(range(n))
    chosen = []
    for _ in range(k):
        best = left[0]
        for j in left[1:]:
            if float(scores[j]) > float(scores[best]):
                best = j
        chosen.append(best)
        left.remove(best)
    return sorted(chosen)


@pytest.mark.parametrize("seed", range(40))
def test_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 40))
    k = int(rng.integers(1, 12))
    vals = np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 1.0, np.inf], np.float32)
    row = vals[rng.integers(0, len(vals), size=max(n, 1))]
    assert list(ot.topk_select(row, n, k)) == _brute(row, n, k)


def test_matches_torch_topk_on_distinct_scores():
    """A library routine: the set torch.topk returns when no two scores are equal."""
    rng = np.random.default_rng(5)
    for n, k in [(3000, 2048), (50000, 2048), (100, 7), (2049, 2048)]:
        row = rng.permutation(n).astype(np.float32) * np.float32(0.37) - np.float32(11)
        want = np.sort(torch.topk(torch.from_numpy(row), k).indices.numpy())
        assert np.array_equal(ot.topk_select(row, n, k), want)


def test_closed_forms():
    n, k = 5000, 2048
    assert np.array_equal(ot.topk_select(np.full(n, 0.25, np.float32), n, k), np.arange(k))
    assert np.array_equal(ot.topk_select(np.arange(n, dtype=np.float32), n, k), np.arange(n - k, n))
    assert np.array_equal(ot.topk_select(-np.arange(n, dtype=np.float32), n, k), np.arange(k))
    # a short prefix is taken whole; scores past the prefix are never read
    row = np.concatenate([np.zeros(10, np.float32), np.full(90, 9.0, np.float32)])
    assert list(ot.topk_select(row, 10, 16)) == list(range(10)) + [-1] * 6
    assert list(ot.topk_select(row, 12, 3)) == [0, 10, 11]
    # -0 and +0 are equal scores: the smaller index wins
    z = np.array([1.0, 0.0, -0.0, -0.0, 0.0], np.float32)
    assert list(ot.topk_select(z, 5, 3)) == [0, 1, 2]


def test_invariants_on_hashed_rows():
    w = synth.workload(4)
    toks = [3000, 70000, 131071]
    rows = synth.index_scores(w, toks, 131072)
    for t, row in zip(toks, rows):
        n = t + 1
        sel = ot.topk_select(row, n, 2048)
        assert len(sel) == 2048 and np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < n
        mask = np.zeros(n, bool)
        mask[sel] = True
        lo, hi = row[:n][mask].min(), row[:n][~mask].max()
        assert lo >= hi
        if lo == hi:  # a tie at the threshold: the selected equal keys precede the others
            assert np.nonzero(mask & (row[:n] == lo))[0].max() < np.nonzero(~mask & (row[:n] == lo))[0].min()


def test_index_scores_host_device_identical():
    w = synth.workload(4)
    toks = np.array([0, 1, 77, 65535, 131071])
    host = synth.index_scores(w, toks, 9000)
    dev = synth.index_scores_device(w, torch.from_numpy(toks), 9000, rows_per_chunk=2).numpy()
    assert np.array_equal(host, dev)
    assert host.min() >= 0 and host.max() < 1 and np.all(host * 2 ** 24 == np.floor(host * 2 ** 24))
    # another workload draws other scores
    assert not np.array_equal(host, synth.index_scores(synth.workload(3), toks, 9000))
