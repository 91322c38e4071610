"""pcp_plan_splits (host only): the per-row split-KV plan is well formed, follows the
virtual-row layout of the partition, splits long decode rows and leaves batches that already
fill the GPU unsplit. Any well-formed plan gives the same merged attention (the GPU tests check
that); these tests pin the plan's shape and its decisions on clear-cut batches."""
import os

import numpy as np
import pytest

from context_mla_prefill_amd import _lib, synth
from oracle import partition as op

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")

CUS = 256


def _well_formed(splits, order, q, kv, P, S):
    _, nv, _ = _lib.pcp_plan_sizes(q, kv, P)
    assert splits.shape == (P, nv) and order.shape == (P, nv)
    assert np.all((splits >= 1) & (splits <= S))
    for r in range(P):
        assert sorted(order[r].tolist()) == list(range(nv))


@pytest.mark.parametrize("seed", range(12))
def test_plans_are_well_formed(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 20))
    q = rng.integers(0, 3000, size=n) * (rng.random(n) < 0.6) + (rng.random(n) < 0.4)
    kv = q + rng.integers(0, 60000, size=n)
    P = int(rng.choice([1, 2, 3, 4, 8]))
    S = int(rng.choice([1, 2, 3, 5, 8, 64]))
    H = int(rng.choice([1, 16, 64, 128]))
    Dl = int(rng.choice([64, 512]))
    splits, order = _lib.pcp_plan_splits(q, kv, P, H, Dl, S, CUS)
    _well_formed(splits, order, q, kv, P, S)


def test_one_range_gives_the_default_plan():
    q, kv = [5000, 1, 1], [5000, 90000, 70000]
    splits, order = _lib.pcp_plan_splits(q, kv, 2, 16, 512, 1, CUS)
    assert np.all(splits == 1)
    assert np.array_equal(order, np.tile(np.arange(4)[::-1], (2, 1)))


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_batches_that_fill_the_gpu_stay_unsplit(cfg):
    """The 8K and 128K prefills and the mixed 8-prefill + 64-decode batch already give every
    compute unit many similar work items: no row is split, rows keep the default order."""
    w = synth.workload(cfg)
    for S in (2, 4, 8):
        splits, order = _lib.pcp_plan_splits(w.q_lens, w.kv_lens, w.P, w.H, w.Dl, S, CUS)
        assert np.all(splits == 1), (cfg, S)
        nv = splits.shape[1]
        assert np.array_equal(order, np.tile(np.arange(nv)[::-1], (w.P, 1)))


def test_long_decode_rows_are_split():
    """A batch of 64 decode rows over 32K-128K contexts and one 4K prefill, P=4: 64 one-tile
    rows cannot fill 256 compute units, so every decode row is split, and rows with more
    ranges' worth of keys come first."""
    rng = np.random.default_rng(1)
    ctx = np.floor(np.exp(rng.uniform(np.log(32768), np.log(131072), 64))).astype(np.int64)
    q = np.array([4096] + [1] * 64)
    kv = np.concatenate([[4096], ctx])
    splits, order = _lib.pcp_plan_splits(q, kv, 4, 16, 512, 8, CUS)
    _well_formed(splits, order, q, kv, 4, 8)
    plan = op.partition(q, kv, np.zeros(len(q), int), 4)
    for r, rp in enumerate(plan.ranks):
        dec = np.arange(2, rp.n_vrows)  # rows 0, 1: the prefill's two chunks
        assert np.all(splits[r, dec] > 1)
        # rows taken in order of their longest range, longest first
        per_range = rp.vrow_kv_len[order[r]] / splits[r, order[r]]
        assert np.all(np.diff(per_range[np.isin(order[r], dec)]) <= 0)


def test_split_rows_follow_the_partition_layout():
    """Virtual rows are numbered as pcp_partition lays them out (requests in batch order, a split
    request's chunk r then chunk 2P-1-r): the long decode row is the one split."""
    q = [4096, 3, 1, 1]
    kv = [4096, 10, 120000, 64]
    P = 2
    splits, _ = _lib.pcp_plan_splits(q, kv, P, 16, 512, 8, CUS)
    plan = op.partition(q, kv, np.zeros(4, int), P)
    for r, rp in enumerate(plan.ranks):
        longest = int(np.argmax(rp.vrow_kv_len))
        assert rp.vrow_req[longest] == 2
        assert splits[r, longest] > 1
        assert np.all(np.delete(splits[r], longest) == 1)


def test_chunked_prefill_step_is_split():
    """The chunked-prefill step (continuations over 115K and 41K cached keys, 64 decode rows):
    its longest tiles are a large share of a compute unit's work, so some rows are split."""
    w = synth.workload(6)
    splits, _ = _lib.pcp_plan_splits(w.q_lens, w.kv_lens, w.P, w.H, w.Dl, 4, CUS)
    assert np.all((splits > 1).sum(axis=1) > 0)


def test_plan_splits_errors():
    ok = dict(q_lens=[8], kv_lens=[8], P=2, H=16, D_latent=512, max_splits=4, n_workers=CUS)

    def call(**kw):
        a = dict(ok, **kw)
        try:
            _lib.pcp_plan_splits(a["q_lens"], a["kv_lens"], a["P"], a["H"], a["D_latent"], a["max_splits"],
                                 a["n_workers"])
        except _lib.MlaError as e:
            return e.status
        return 0

    assert call() == 0
    assert call(q_lens=[9]) == _lib.MLA_ERR_INVALID_ARG  # q_len > kv_len
    assert call(P=0) == _lib.MLA_ERR_INVALID_ARG
    assert call(H=0) == _lib.MLA_ERR_INVALID_ARG
    assert call(H=129) == _lib.MLA_ERR_INVALID_ARG
    assert call(D_latent=128) == _lib.MLA_ERR_UNSUPPORTED
    assert call(max_splits=0) == _lib.MLA_ERR_INVALID_ARG
    assert call(max_splits=65) == _lib.MLA_ERR_INVALID_ARG
    assert call(n_workers=0) == _lib.MLA_ERR_INVALID_ARG
